"""gns_gram_batched_noalloc (the entry point for callers that cannot
allocate) through the C ABI against gns_gram_batched on the same inputs:
two calls in a row, the second smaller, each bit-identical to the existing
entry point's result (same kernels on one stream) and within the bf16 bar
of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import NS5, TOL_HALF, need_gpu, rel_err, say
from gram_newton_schulz_amd import synth

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_entry_point():
    gns = need_gpu()
    from gram_newton_schulz_amd import binding
    cases = [(2, 1024, 4096, (2,), 140), (3, 300, 700, (), 141)]     # the second smaller, ragged
    for B, n, m, rs, seed in cases:
        assert gns.gram_workspace_bytes(torch.bfloat16, B, n, m) <= binding.NOALLOC_SCRATCH_BYTES
        X = synth.batch(B, n, m, seed=seed, dtype=torch.bfloat16)
        Xd = X.cuda()
        say(f"noalloc {B}x{n}x{m} restarts={rs}")
        want = gns.gram_ns_batched(Xd, NS5, restarts=rs, split_batch=False)
        out = torch.full_like(Xd, float("nan"))
        torch.cuda.synchronize()
        got = binding.gram_ns_batched_noalloc(Xd, out, NS5, restarts=rs)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(out, want)
        X64 = synth.as_f64(X)
        for b in (0, B - 1):
            assert rel_err(synth.as_f64(out[b]), oracle.gram_ns(X64[b], NS5, restarts=rs)) <= TOL_HALF


def test_noalloc_refusals():
    gns = need_gpu()
    from gram_newton_schulz_amd import binding
    X = torch.zeros(4, 1024, 4096, dtype=torch.bfloat16, device="cuda")   # 156 MiB of workspace
    out = torch.empty_like(X)
    say("noalloc refusals")
    with pytest.raises(gns.GnsError) as e:
        binding.gram_ns_batched_noalloc(X, out, NS5)
    assert e.value.name == "GNS_E_WORKSPACE"
    with pytest.raises(gns.GnsError) as e:
        binding.gram_ns_batched_noalloc(X[:1], out[:1], NS5, tile="auto")
    assert e.value.name == "GNS_E_FLAGS"
    with pytest.raises(gns.GnsError) as e:
        binding.gram_ns_batched_noalloc(X[:1], out[:1], NS5, restarts=(7,))
    assert e.value.name == "GNS_E_RESTART"
