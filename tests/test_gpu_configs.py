"""The five workloads at full size, in the launch configuration the benchmark
times, against the fp64 oracle: every matrix where the oracle is cheap,
sampled batch members (first and last) where it is not."""
import numpy as np
import pytest
import torch

from gpu_common import NS5, TOL_F32, TOL_HALF, need_gpu, per_matrix_rel, rel_err, say, oracle_gram
from gram_newton_schulz_amd import synth

pytestmark = pytest.mark.gpu


def test_config2_logspectrum_f16_compute():
    """16 x 1024x4096, singular values log-uniform in [1e-4, 1].  Forming X X^T
    squares the condition number, so bf16 products lose the small singular
    values; fp16 products (the pages' default precision) keep the error
    within the bound."""
    gns = need_gpu()
    X = synth.workload_batch(2)
    X64 = synth.as_f64(X)
    say("config2 f16 compute")
    out16 = gns.gram_ns_batched(X.cuda(), NS5, compute_dtype=torch.float16)
    out_bf = gns.gram_ns_batched(X.cuda(), NS5, compute_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = np.stack([oracle_gram(X64[b]) for b in range(X.shape[0])])
    e16 = per_matrix_rel(synth.as_f64(out16), ref)
    ebf = per_matrix_rel(synth.as_f64(out_bf), ref)
    say(f"  f16 max {max(e16):.4g}  bf16 max {max(ebf):.4g}")
    assert max(e16) <= TOL_HALF
    assert max(ebf) < 0.5          # bf16 products: degraded but not diverged


def test_config3_dense_mlp():
    """8 x 4096x16384 bf16 (aspect ratio 4): Gram NS and standard NS, matrices 0 and 7."""
    gns = need_gpu()
    X = synth.workload_batch(3)
    say("config3 upload")
    Xd = X.cuda()
    say("config3 gram")
    g = gns.gram_ns_batched(Xd, NS5, restarts=(2,))
    say("config3 standard")
    s = gns.standard_ns_batched(Xd, NS5)
    torch.cuda.synchronize()
    for b in (0, X.shape[0] - 1):
        say(f"  oracle matrix {b}")
        ref = oracle_gram(synth.as_f64(X[b]))
        eg = rel_err(synth.as_f64(g[b]), ref)
        es = rel_err(synth.as_f64(s[b]), ref)
        say(f"  matrix {b}: gram {eg:.4g} standard {es:.4g}")
        assert eg <= TOL_HALF and es <= TOL_HALF
    assert torch.isfinite(g).all()


def test_config4_moe_stack():
    """64 x 2048x7168 Student-t experts in one grouped launch; four members."""
    gns = need_gpu()
    X = synth.workload_batch(4)
    say("config4 gram")
    g = gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,))
    torch.cuda.synchronize()
    for b in (0, 21, 42, 63):
        ref = oracle_gram(synth.as_f64(X[b]))
        e = rel_err(synth.as_f64(g[b]), ref)
        say(f"  matrix {b}: {e:.4g}")
        assert e <= TOL_HALF
    assert torch.isfinite(g).all()


def test_config5_fractional_rows():
    """8 x 4096x16384 N(0,1), 1024 seeded rows per matrix: gather, Gram NS on
    1024 x 16384, scatter; the other rows untouched."""
    gns = need_gpu()
    X = synth.workload_batch(5)
    rows = synth.workload_rows(5)
    init = torch.zeros_like(X)
    out = init.cuda()
    say("config5 gram rows")
    gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,), row_idx=rows.cuda(), out=out)
    torch.cuda.synchronize()
    oc = out.cpu()
    for b in range(X.shape[0]):
        sel = rows[b].numpy()
        ref = oracle_gram(synth.as_f64(X[b][sel]))
        e = rel_err(synth.as_f64(oc[b][sel]), ref)
        mask = torch.ones(X.shape[1], dtype=torch.bool)
        mask[rows[b]] = False
        assert torch.count_nonzero(oc[b][mask]).item() == 0
        say(f"  matrix {b}: {e:.4g}")
        assert e <= TOL_HALF
