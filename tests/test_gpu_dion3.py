"""The Dion3 update around the orthogonalisation ("Dion3: Full-Stack
Orthogonal Updates", §6, Algorithm 4, with the NorMuon steps of §2.1
eq. (2)) through the C ABI, against the fp64 oracle and plain fp32 torch.

Each stage is checked on its own, on the same seeded state:
* run A (W = 0, lr = 1, no decay, no NorMuon) exposes the orthogonalised
  update exactly (W[S] becomes -O): the selection must equal the oracle's,
  O must meet the orthogonalisation tolerance against the oracle, and the
  momentum rows must equal plain fp32 torch arithmetic bit for bit;
* run B (W = 0, lr = 1, NorMuon) exposes the NorMuon output, which must
  equal the oracle's NorMuon steps applied to run A's O to fp32 rounding,
  with v updated at the selected rows only;
* run C (realistic lr and decay) must equal decay * W - lr * (run B's
  update) to fp32 rounding, rows outside S bit-identical to torch's
  W * decay.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import NS5, TOL_F32, TOL_HALF, need_gpu, rel_err, say
from gram_newton_schulz_amd import synth

pytestmark = pytest.mark.gpu


def _run(gns, W, G, M, v, k, **kw):
    Wd, Gd, Md = W.cuda(), G.cuda(), M.cuda()
    vd = None if v is None else v.cuda()
    S = gns.dion3_step(Wd, Gd, Md, vd, k, NS5, restarts=(2,), **kw)
    torch.cuda.synchronize()
    return Wd.cpu(), Md.cpu(), (None if vd is None else vd.cpu()), S.cpu()


def _check_step(gns, count, n, m, k, seed, grad_dtype, compute_dtype, tol, members, tile=None):
    W, G, M, v = synth.dion3_state(count, n, m, seed=seed, grad_dtype=grad_dtype)
    Z = torch.zeros_like(W)
    Msum = (M + G.float())                               # plain fp32 torch
    mu = 0.5
    say(f"dion3 run A {count}x{n}x{m} k={k} {grad_dtype} {compute_dtype} tile={tile}")
    WA, MA, _, SA = _run(gns, Z, G, M, None, k, lr=1.0, weight_decay=0.0, mu=mu, normuon=False,
                         compute_dtype=compute_dtype, tile=tile)
    say(f"dion3 run B")
    WB, MB, vB, SB = _run(gns, Z, G, M, v, k, lr=1.0, weight_decay=0.0, mu=mu, beta2=0.9, eps=1e-8,
                          normuon=True, compute_dtype=compute_dtype, tile=tile)
    lr, wd = 0.02, 0.1
    say(f"dion3 run C")
    WC, MC, vC, SC = _run(gns, W, G, M, v, k, lr=lr, weight_decay=wd, mu=mu, beta2=0.9, eps=1e-8,
                          normuon=True, compute_dtype=compute_dtype, tile=tile)
    assert torch.equal(SA, SB) and torch.equal(SA, SC)
    decay = np.float32(1.0 - lr * wd)
    for b in members:
        S = SA[b].numpy()
        rest = np.setdiff1d(np.arange(n), S)
        # selection: the oracle's, from the same fp32 momentum sum
        S_ref = oracle.dion3_select(synth.as_f64(Msum[b]), k)
        assert np.array_equal(S, S_ref), f"matrix {b}: selection differs"
        # momentum: fp32 sum kept outside S, error feedback inside (bit-exact)
        for Mx in (MA, MB, MC):
            assert torch.equal(Mx[b][rest], Msum[b][rest])
            assert torch.equal(Mx[b][S], Msum[b][S] * torch.tensor(mu, dtype=torch.float32))
        # orthogonalised update against the oracle
        O = -synth.as_f64(WA[b][S])
        assert not WA[b][rest].any()
        ref = oracle.gram_ns(synth.as_f64(Msum[b])[S], NS5, restarts=(2,))
        e = rel_err(O, ref)
        say(f"  matrix {b}: update rel err {e:.3g}")
        assert e <= tol
        # NorMuon: the oracle's steps on the GPU's own update
        On_ref, v_ref = oracle.normuon_rows(O, synth.as_f64(v[b])[S], beta2=0.9, eps=1e-8)
        On = -synth.as_f64(WB[b][S])
        en = rel_err(On, On_ref)
        ev = rel_err(synth.as_f64(vB[b])[S], v_ref)
        say(f"  matrix {b}: normuon rel err {en:.3g}, v rel err {ev:.3g}")
        assert en <= 1e-6 and ev <= 1e-6
        assert torch.equal(vB[b][rest], v[b][rest]) and torch.equal(vC[b], vB[b])
        # and the whole update end to end against the oracle's Algorithm 4
        full = oracle.dion3_step(synth.as_f64(W[b]), synth.as_f64(G[b]), synth.as_f64(M[b]),
                                 synth.as_f64(v[b]), k, NS5, restarts=(2,), lr=1.0, weight_decay=0.0,
                                 momentum=mu, beta2=0.9, eps=1e-8, normuon=True)
        ee = rel_err(On, full["O"])
        say(f"  matrix {b}: end-to-end NorMuon update rel err {ee:.3g}")
        assert ee <= 2 * tol
        # decay and the fp32 update of the weights
        assert torch.equal(WC[b][rest], W[b][rest] * torch.tensor(decay))
        Wref = np.float64(decay) * synth.as_f64(W[b][S]) - lr * On
        scale = float(np.max(np.abs(synth.as_f64(W[b][S])))) + 1e-30
        assert np.max(np.abs(synth.as_f64(WC[b][S]) - Wref)) <= 4 * 2.0 ** -23 * scale


def test_dion3_step_small_ragged():
    """3 x 150x520 (ragged against every tile), k = 40, bf16 gradient."""
    gns = need_gpu()
    _check_step(gns, 3, 150, 520, 40, 31, torch.bfloat16, torch.bfloat16, TOL_HALF, range(3))


@pytest.mark.parametrize("tile", [256, "mixed"])
def test_dion3_step_256_tiles(tile):
    """3 x 300x1030 with k = 211 on forced 256-edge (or mixed) tiles: the
    fp32 update leaves the last product through the staged fp32 epilogue
    (ragged rows) or, with m not a multiple of 4, element by element."""
    gns = need_gpu()
    _check_step(gns, 3, 300, 1030, 211, 39, torch.bfloat16, torch.bfloat16, TOL_HALF, range(3), tile=tile)
    _check_step(gns, 2, 300, 1032, 211, 40, torch.bfloat16, torch.bfloat16, TOL_HALF, range(2), tile=tile)


def test_dion3_step_fp32_compute():
    """2 x 64x256 fp32 gradient and fp32 products: the fp32 tolerance."""
    gns = need_gpu()
    _check_step(gns, 2, 64, 256, 16, 32, torch.float32, torch.float32, TOL_F32, range(2))


def test_dion3_step_every_row_and_square():
    """k = n selects every row (f = 1 is Muon); k = m = n runs the square
    fallback (standard Newton-Schulz)."""
    gns = need_gpu()
    _check_step(gns, 2, 96, 300, 96, 33, torch.bfloat16, torch.bfloat16, TOL_HALF, range(2))
    _check_step(gns, 2, 128, 128, 128, 34, torch.bfloat16, torch.float32, TOL_F32, range(2))


def test_dion3_step_full_size():
    """8 x 4096x16384, f = 1/4 (k = 1024), bf16 gradient: the shape of the
    fractional-row workload, in the launch configuration the benchmark uses;
    matrices 0 and 7 checked against the oracle."""
    gns = need_gpu()
    _check_step(gns, 8, 4096, 16384, 1024, 35, torch.bfloat16, torch.bfloat16, TOL_HALF, (0, 7))


def test_dion3_step_graph_replay():
    """The whole step captured in a HIP graph: every replay on restored
    state equals the eager step bit for bit."""
    gns = need_gpu()
    W, G, M, v = synth.dion3_state(2, 256, 1024, seed=36)
    Wd, Gd, Md, vd = W.cuda(), G.cuda(), M.cuda(), v.cuda()
    k = 64
    ws = torch.empty(gns.dion3_workspace_bytes(torch.bfloat16, 2, 256, 1024, k), dtype=torch.uint8,
                     device="cuda")
    S = torch.empty(2, k, dtype=torch.int64, device="cuda")
    kw = dict(lr=0.02, weight_decay=0.1, mu=0.9, beta2=0.95, eps=1e-8, normuon=True, row_idx=S, workspace=ws)
    say("dion3 eager")
    gns.dion3_step(Wd, Gd, Md, vd, k, NS5, restarts=(2,), **kw)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (Wd, Md, vd, S)]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    for t, src in zip((Wd, Md, vd), (W, M, v)):
        t.copy_(src)
    torch.cuda.synchronize()
    say("dion3 capture")
    with torch.cuda.graph(g, stream=s):
        gns.dion3_step(Wd, Gd, Md, vd, k, NS5, restarts=(2,), stream=s, **kw)
    for rep in range(3):
        for t, src in zip((Wd, Md, vd), (W, M, v)):
            t.copy_(src)
        S.fill_(-1)
        torch.cuda.synchronize()
        say(f"dion3 replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((Wd, Md, vd, S), eager):
            assert torch.equal(got, want)
