"""The boundary on the GPU: in-place calls, stray writes, the debug checks
(row subset and Inf/NaN), scale, threads, and the half-precision stability
behaviour the pages describe ("Dion3: Full-Stack Orthogonal Updates",
Appendix B.1-B.2), all through the C ABI against the fp64 oracle."""
import threading

import numpy as np
import pytest
import torch

import oracle
from gpu_common import NS5, TOL_HALF, need_gpu, per_matrix_rel, rel_err, say, oracle_gram
from gram_newton_schulz_amd import synth

pytestmark = pytest.mark.gpu

# the stability study's schedule (Dion3 App. B.1.1; the minus sign of b that
# Fig. 12's caption drops is forced by h(x) = 15/8 - 10/8 x + 3/8 x^2, B.1.2)
STAB = (15 / 8, -10 / 8, 3 / 8)


def _bf16(B, n, m, seed, dist="normal"):
    X = synth.batch(B, n, m, seed=seed, dist=dist, dtype=torch.bfloat16)
    return X, synth.as_f64(X)


def test_longest_rows_at_the_addressing_limit():
    """The longest rows the library accepts: a 256-row panel of 4194048 bf16
    columns spans 2^31 - 2^17 bytes, just under the 32-bit offsets of the
    buffer loads (a longer row is refused; see the host tests).  1 x 256 x
    4194048 bf16 with the size rule (128-edge tiles, X transposed) and with
    256-edge tiles (one workgroup contracting the whole rows for the Gram
    matrix, Q X reading X row-major as one 2 GiB operand), against the fp64
    oracle."""
    gns = need_gpu()
    n, m = 256, 4194048
    say(f"longest rows 1 x {n} x {m}: inputs")
    X = synth.batch(1, n, m, seed=43, dtype=torch.bfloat16)
    Xd = X.cuda()
    got = {}
    for tile in (None, 256):
        say(f"longest rows: tile {tile}")
        got[tile] = gns.gram_ns_batched(Xd, NS5, restarts=(2,), tile=tile).cpu()
        torch.cuda.synchronize()
    del Xd
    say("longest rows: oracle")
    ref = oracle_gram(synth.as_f64(X)[0])
    for tile, o in got.items():
        assert rel_err(synth.as_f64(o)[0], ref) <= TOL_HALF, tile


def test_batch_beyond_one_grid_dimension():
    """70000 matrices, more than 65535 (the batch is a grid dimension of the
    input pass): 70000 x 8 x 24 bf16 in one call; the members around 65535
    and a seeded sample of the rest against the fp64 oracle."""
    gns = need_gpu()
    B, n, m = 70000, 8, 24
    say(f"batch {B} x {n} x {m}")
    g = torch.Generator().manual_seed(44)
    X = (torch.randn(B, n, m, generator=g) * 0.1).to(torch.bfloat16)
    out = gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,)).cpu()
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    picks = sorted({0, 1, 65534, 65535, 65536, B - 1, *rng.choice(B, 24, replace=False).tolist()})
    X64 = synth.as_f64(X[picks])
    got = synth.as_f64(out[picks])
    for i, b in enumerate(picks):
        assert rel_err(got[i], oracle_gram(X64[i])) <= TOL_HALF, b


@pytest.mark.parametrize("tile,shape", [(256, (3, 512, 1536)), (None, (3, 512, 1536)),
                                        (None, (2, 2048, 4096))])
@pytest.mark.parametrize("T", [5, 1])
def test_in_place_whole_tiles_no_restart(tile, shape, T):
    """out = X on whole 256-edge tiles with no restart: the final Q X would
    read X itself, so the input pass copies it first.  Bit-identical to the
    out-of-place call and within the bf16 bar of the oracle (Dion3 §4.2,
    Algorithm 3: X <- Q_T X is the only write of the output)."""
    gns = need_gpu()
    B, n, m = shape
    X, X64 = _bf16(B, n, m, seed=60 + n)
    co = NS5[:T]
    say(f"in place {shape} tile={tile} T={T}")
    ref_gpu = gns.gram_ns_batched(X.cuda(), co, restarts=(), tile=tile)
    Xd = X.cuda()
    got = gns.gram_ns_batched(Xd, co, restarts=(), tile=tile, out=Xd)
    torch.cuda.synchronize()
    assert got.data_ptr() == Xd.data_ptr()
    assert torch.equal(got, ref_gpu)
    for b in (0, B - 1):
        assert rel_err(synth.as_f64(got[b]), oracle.gram_ns(X64[b], co, restarts=())) <= TOL_HALF


@pytest.mark.parametrize("split", [True, False])
def test_in_place_restart_and_standard(split):
    """In place with a restart (the final product reads a workspace copy) and
    for standard NS (X read only by the first product), both stream layouts."""
    gns = need_gpu()
    X, X64 = _bf16(3, 512, 1536, seed=64)
    say(f"in place restart/standard split={split}")
    for algo in ("gram", "standard"):
        fn = (lambda x, **kw: gns.gram_ns_batched(x, NS5, restarts=(2,), tile=256, split_batch=split, **kw)) \
            if algo == "gram" else \
            (lambda x, **kw: gns.standard_ns_batched(x, NS5, tile=256, split_batch=split, **kw))
        ref = fn(X.cuda())
        Xd = X.cuda()
        fn(Xd, out=Xd)
        torch.cuda.synchronize()
        assert torch.equal(Xd, ref), algo


def test_autotune_in_place():
    """tile="auto" with out = X never times (each timed run would
    orthogonalise the previous output): on a fresh shape it runs the size
    rule and keeps nothing; on a tuned shape it runs the kept choice.  Both
    equal the out-of-place call of the same plan bit for bit."""
    gns = need_gpu()
    B, n, m = 3, 512, 1536
    X, X64 = _bf16(B, n, m, seed=65)
    gns.autotune_clear()
    say("autotune in place, fresh shape")
    Xd = X.cuda()
    gns.gram_ns_batched(Xd, NS5, restarts=(), tile="auto", out=Xd)
    torch.cuda.synchronize()
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m) == 0      # nothing kept
    rule = gns.gram_ns_batched(X.cuda(), NS5, restarts=())                   # the size rule
    assert torch.equal(Xd, rule)
    say("autotune in place, tuned shape")
    tuned = gns.gram_ns_batched(X.cuda(), NS5, restarts=(), tile="auto")     # times and keeps
    torch.cuda.synchronize()
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m) in (128, 256)
    Xd2 = X.cuda()
    gns.gram_ns_batched(Xd2, NS5, restarts=(), tile="auto", out=Xd2)
    torch.cuda.synchronize()
    assert torch.equal(Xd2, tuned)
    assert rel_err(synth.as_f64(Xd2[0]), oracle.gram_ns(X64[0], NS5, restarts=())) <= TOL_HALF
    gns.autotune_clear()


@pytest.mark.parametrize("algo", ["gram", "standard"])
def test_unselected_rows_keep_canaries(algo):
    """A row subset written into an out whose other rows hold NaN canaries
    (every batch member, ragged shape): the canaries survive bit for bit, so
    no kernel writes outside its matrix's selected rows (Dion3 §6,
    Algorithm 4: the other rows are not updated)."""
    gns = need_gpu()
    B, n, m, k = 4, 600, 1400, 300
    X, X64 = _bf16(B, n, m, seed=66)
    rows = np.stack([synth.row_subset(n, k, seed=66, index=b) for b in range(B)])
    out = torch.full((B, n, m), float("nan"), dtype=torch.bfloat16, device="cuda")
    say(f"canaries {algo}")
    ri = torch.from_numpy(rows).cuda()
    if algo == "gram":
        gns.gram_ns_batched(X.cuda(), NS5, row_idx=ri, out=out)
    else:
        gns.standard_ns_batched(X.cuda(), NS5, row_idx=ri, out=out)
    torch.cuda.synchronize()
    got = out.cpu()
    for b in range(B):
        mask = np.ones(n, bool)
        mask[rows[b]] = False
        assert torch.isnan(got[b][torch.from_numpy(mask)]).all(), f"matrix {b}: an unselected row was written"
        sel = got[b][torch.from_numpy(rows[b])]
        assert not torch.isnan(sel).any()
        x = X64[b][rows[b]]
        ref = oracle.gram_ns(x, NS5, restarts=(2,)) if algo == "gram" else oracle.standard_ns(x, NS5)
        assert rel_err(synth.as_f64(sel), ref) <= TOL_HALF


@pytest.mark.parametrize("k", [-40, 40])
@pytest.mark.parametrize("tile", [256, 128])
def test_power_of_two_scale_on_direct_path(k, tile):
    """out(2^k X) on the direct path, which forms X X^T and Q X of the
    unnormalised input in fp32 and applies 1/(||X|| + eps) in the epilogues:
    within the bf16 bar of the oracle for k = +-40 (Dion3 §4.2, Algorithm 3,
    normalisation step; the oracle normalises in fp64)."""
    gns = need_gpu()
    B, n, m = 2, 512, 1536
    X, _ = _bf16(B, n, m, seed=67)
    Xs = (X.float() * 2.0 ** k).to(torch.bfloat16)            # exact: a power of two
    assert torch.equal(Xs.float() * 2.0 ** -k, X.float())
    X64 = synth.as_f64(Xs)
    say(f"scale 2^{k} tile={tile}")
    plan = gns.call_plan(False, 1 << 32, 2 << 32, B, n, m, torch.bfloat16, torch.bfloat16, NS5, (2,),
                         opts=0x20 if tile == 256 else 0x10)
    assert plan.direct_input == 1
    out = gns.gram_ns_batched(Xs.cuda(), NS5, restarts=(2,), tile=tile)
    torch.cuda.synchronize()
    ref = np.stack([oracle_gram(X64[b]) for b in range(B)])
    assert max(per_matrix_rel(synth.as_f64(out), ref)) <= TOL_HALF


def test_debug_checks_nonfinite_and_rowidx():
    """GNS_OPT_DEBUG_CHECKS: an Inf in the input gives GNS_E_NONFINITE, a
    finite call gives GNS_OK, a repeated row index GNS_E_ROWIDX before any
    compute; gns_check_finite reports the same flag enqueue-only."""
    gns = need_gpu()
    X, _ = _bf16(2, 256, 768, seed=68)
    say("debug checks")
    out = gns.gram_ns_batched(X.cuda(), NS5, debug_checks=True)
    assert gns.check_finite(out)
    Xi = X.clone()
    Xi[1, 7, 9] = float("inf")
    with pytest.raises(gns.GnsError) as e:
        gns.gram_ns_batched(Xi.cuda(), NS5, debug_checks=True)
    assert e.value.name == "GNS_E_NONFINITE"
    with pytest.raises(gns.GnsError) as e:
        gns.standard_ns_batched(Xi.cuda(), NS5, debug_checks=True)
    assert e.value.name == "GNS_E_NONFINITE"
    # without the bit the same call returns normally, the output carries the NaNs
    bad = gns.gram_ns_batched(Xi.cuda(), NS5)
    assert not gns.check_finite(bad) and gns.check_finite(bad[:1])
    dup = torch.tensor([[1, 5, 5], [0, 2, 3]], dtype=torch.int64, device="cuda")
    with pytest.raises(gns.GnsError) as e:
        gns.gram_ns_batched(X.cuda(), NS5, row_idx=dup, debug_checks=True)
    assert e.value.name == "GNS_E_ROWIDX"
    # rows of a NaN-holding out that are not selected are not checked
    canary = torch.full_like(X, float("nan")).cuda()
    ri = torch.tensor([[1, 5, 9], [0, 2, 3]], dtype=torch.int64, device="cuda")
    gns.gram_ns_batched(X.cuda(), NS5, row_idx=ri, out=canary, debug_checks=True)
    assert gns.check_finite(canary, row_idx=ri) and not gns.check_finite(canary)


def test_debug_checks_refused_in_capture():
    gns = need_gpu()
    X, _ = _bf16(2, 256, 768, seed=69)
    Xd = X.cuda()
    out = torch.empty_like(Xd)
    ws = torch.empty(gns.gram_workspace_bytes(torch.bfloat16, 2, 256, 768), dtype=torch.uint8, device="cuda")
    gns.gram_ns_batched(Xd, NS5, out=out, workspace=ws)
    torch.cuda.synchronize()
    say("debug checks under capture")
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g):
        try:
            gns.gram_ns_batched(Xd, NS5, out=out, workspace=ws, debug_checks=True,
                                stream=torch.cuda.current_stream())
        except gns.GnsError as e:
            err = e
    assert err is not None and err.name == "GNS_E_FLAGS"


def test_dion3_debug_check_keeps_weights():
    """A non-finite update is reported before it reaches W or v."""
    gns = need_gpu()
    B, n, m, k = 2, 256, 768, 64
    W, G, M, v = (t.cuda() for t in synth.dion3_state(B, n, m, seed=70))
    G[0, 3, 4] = float("inf")
    W0, v0 = W.clone(), v.clone()
    say("dion3 debug check")
    with pytest.raises(gns.GnsError) as e:
        gns.dion3_step(W, G, M, v, k, NS5, (2,), lr=0.02, weight_decay=0.1, debug_checks=True)
    assert e.value.name == "GNS_E_NONFINITE"
    torch.cuda.synchronize()
    assert torch.equal(W, W0) and torch.equal(v, v0)


def test_threads_with_own_streams():
    """Two host threads, each with its own stream and workspace, call the
    library at the same time (each thread gets its own fan-out streams):
    every result equals the single-thread result bit for bit."""
    gns = need_gpu()
    Xs = [_bf16(4, 512, 1536, seed=71 + i)[0].cuda() for i in range(2)]
    want = [gns.gram_ns_batched(x, NS5) for x in Xs]
    torch.cuda.synchronize()
    got = [[None] * 4 for _ in range(2)]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            ws = torch.empty(gns.gram_workspace_bytes(torch.bfloat16, 4, 512, 1536), dtype=torch.uint8,
                             device="cuda")
            with torch.cuda.stream(s):
                for r in range(4):
                    got[i][r] = gns.gram_ns_batched(Xs[i], NS5, workspace=ws, stream=s)
                    got[i][r] = got[i][r].clone()
            s.synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    say("two threads")
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for r in range(4):
            assert torch.equal(got[i][r], want[i]), (i, r)


def _expspec(seed):
    # App. B.1.1's input: 128 x 512 with an exponentially decaying spectrum
    # (here 10^0 down to 10^-4), unit Frobenius norm, rounded to bf16
    return _bf16(1, 128, 512, seed=seed, dist="expspec")


@pytest.mark.parametrize("seed", [100, 101])
def test_naive_gram_bf16_diverges_without_restart(seed):
    """Dion3 App. B.1.1-B.1.2, Fig. 12: Algorithm 2 (naive algebra) in bfloat16
    with (15/8, -10/8, 3/8) for 10 steps drifts far from the fp64 result
    (spurious negative eigenvalues of R grow by at least (15/8)^2 per step);
    by a few steps more it returns Infs, which the debug checks report."""
    gns = need_gpu()
    X, X64 = _expspec(seed)
    co = [STAB] * 10
    say(f"stability naive no restart seed={seed}")
    out = gns.gram_ns_batched(X.cuda(), co, restarts=(), naive_algebra=True)
    torch.cuda.synchronize()
    got = synth.as_f64(out[0])
    ref = oracle.gram_ns(X64[0], co, restarts=(), algebra="naive")
    assert (not np.isfinite(got).all()) or rel_err(got, ref) > 1.0
    with pytest.raises(gns.GnsError) as e:
        gns.gram_ns_batched(X.cuda(), [STAB] * 16, restarts=(), naive_algebra=True, debug_checks=True)
    assert e.value.name == "GNS_E_NONFINITE"


@pytest.mark.parametrize("naive", [True, False])
@pytest.mark.parametrize("seed", [100, 101])
def test_restarts_keep_half_precision_stable(naive, seed):
    """Dion3 App. B.2, Fig. 16: the same run with a restart every five steps
    stays finite, its output's singular values stay near 1 (at most 1.2
    here), and it tracks the fp64 result; 16 steps with restarts after 5, 10
    and 15 pass the debug checks."""
    gns = need_gpu()
    X, X64 = _expspec(seed)
    co = [STAB] * 10
    say(f"stability restart every 5 naive={naive} seed={seed}")
    out = gns.gram_ns_batched(X.cuda(), co, restarts=(5,), naive_algebra=naive)
    torch.cuda.synchronize()
    got = synth.as_f64(out[0])
    assert np.isfinite(got).all()
    ref = oracle.gram_ns(X64[0], co, restarts=(5,), algebra="naive" if naive else "stabilized")
    assert rel_err(got, ref) <= 0.2
    assert np.linalg.svd(got, compute_uv=False).max() <= 1.2
    gns.gram_ns_batched(X.cuda(), [STAB] * 16, restarts=(5, 10, 15), naive_algebra=naive, debug_checks=True)
