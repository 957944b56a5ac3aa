"""Dion3 selection step on the GPU (the k rows of largest l1 norm) against
the oracle: indices are integers, so they must match exactly."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import NS5, TOL_HALF, need_gpu, rel_err, say
from gram_newton_schulz_amd import synth

pytestmark = pytest.mark.gpu


def _oracle_sel(M, k):
    M64 = synth.as_f64(M)
    return np.stack([oracle.dion3_select(M64[b], k) for b in range(M.shape[0])])


def test_select_fractional_rows_workload():
    """8 x 4096x16384 bf16 N(0,1) momentum, f = 1/4 (k = 1024), the Dion3
    shape; every index of every matrix equals the oracle's."""
    gns = need_gpu()
    X = synth.workload_batch(5)
    k = gns.select_count(X.shape[1], 0.25)
    say(f"select l1 8x4096x16384 k={k}")
    got = gns.select_rows_l1(X.cuda(), k)
    torch.cuda.synchronize()
    ref = _oracle_sel(X, k)
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16, torch.float16])
def test_select_ragged_and_ties(dt):
    """Ragged row length (scalar path for m = 37), many exactly equal rows
    (duplicates), k cutting through a group of ties, fp32/bf16/fp16."""
    gns = need_gpu()
    B, n, m = 3, 1000, 37
    g = torch.Generator().manual_seed(31)
    X = torch.randn(B, n, m, generator=g)
    X[:, 500:700] = X[:, 100:101]           # 200 rows with one norm
    X[:, 800:900] = -X[:, 5:6]              # same norm, opposite signs
    X = X.to(dt)
    for k in (1, 37, 250, 500, 999, 1000):
        say(f"select ties dt={dt} k={k}")
        got = gns.select_rows_l1(X.cuda(), k)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), _oracle_sel(X, k)), k


def test_select_then_orthogonalise():
    """The whole Dion3 orthogonalisation of Algorithm 4 (select
    the top rows, orthogonalise them as one k x m matrix, write them back)
    against the oracle's selection and row update."""
    gns = need_gpu()
    B, n, m = 2, 512, 2048
    X = synth.batch(B, n, m, seed=32, dtype=torch.bfloat16)
    init = torch.zeros_like(X)
    k = gns.select_count(n, 0.25)
    say("select + gram rows")
    idx = gns.select_rows_l1(X.cuda(), k)
    out = init.cuda()
    gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,), row_idx=idx, out=out)
    torch.cuda.synchronize()
    X64 = synth.as_f64(X)
    for b in range(B):
        sel = oracle.dion3_select(X64[b], k)
        assert np.array_equal(idx[b].cpu().numpy(), sel)
        ref = oracle.dion3_rows(X64[b], np.zeros((n, m)), sel, NS5)
        got = synth.as_f64(out[b].cpu())
        assert rel_err(got[sel], ref[sel]) <= TOL_HALF
        keep = np.setdiff1d(np.arange(n), sel)
        assert np.count_nonzero(got[keep]) == 0
