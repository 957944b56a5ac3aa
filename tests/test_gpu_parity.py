"""HIP path (through the C ABI) against the fp64 oracle on seeded inputs at
sizes the oracle finishes in seconds: several tiles plus ragged tails, both
tile edges, every dtype combination, restart sets, both algebras, the row
subset, degenerate shapes, guard bands, determinism."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import (NS5, TOL_F32, TOL_HALF, need_gpu, per_matrix_rel, rel_err, say,
                        oracle_gram, oracle_standard)
from gram_newton_schulz_amd import synth

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "bf16x3": "bf16x3"}


def _inputs(B, n, m, io, seed, dist="normal"):
    X = synth.batch(B, n, m, seed=seed, dist=dist, dtype=DT[io])
    return X, synth.as_f64(X)


def _tol(cdt):
    return TOL_F32 if cdt == "f32" else TOL_HALF



def _run(gns, algo, Xd, cdt, **kw):
    if algo == "gram":
        return gns.gram_ns_batched(Xd, NS5, compute_dtype=DT[cdt], **kw)
    kw.pop("restarts", None)
    return gns.standard_ns_batched(Xd, NS5, compute_dtype=DT[cdt], **kw)


def test_config1_fp32():
    """64x256 fp32: Gram NS (restart after 2), standard NS and the SVD picture."""
    gns = need_gpu()
    X = synth.workload_batch(1)
    X64 = synth.as_f64(X)
    say("config1 fp32")
    g = gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,))
    s = gns.standard_ns_batched(X.cuda(), NS5)
    torch.cuda.synchronize()
    ref = oracle_gram(X64[0])
    assert rel_err(synth.as_f64(g)[0], ref) <= TOL_F32
    assert rel_err(synth.as_f64(s)[0], oracle_standard(X64[0])) <= TOL_F32
    assert rel_err(ref, oracle.spectral_map(X64[0], NS5)) <= 1e-10


@pytest.mark.parametrize("tile", [128, 256, "mixed"])
@pytest.mark.parametrize("algo", ["gram", "standard"])
@pytest.mark.parametrize("io,cdt", [("bf16", "bf16"), ("bf16", "f16"), ("f32", "f32"),
                                    ("f16", "f16"), ("f32", "bf16"), ("bf16", "bf16x3"),
                                    ("f32", "bf16x3")])
def test_ragged_parity(tile, algo, io, cdt):
    gns = need_gpu()
    B, n, m = 3, 300, 700          # 3 x 6 tiles of 128 with ragged tails
    X, X64 = _inputs(B, n, m, io, seed=11)
    say(f"ragged {algo} io={io} cdt={cdt} tile={tile} {B}x{n}x{m}")
    out = _run(gns, algo, X.cuda(), cdt, tile=tile)
    torch.cuda.synchronize()
    got = synth.as_f64(out)
    ref = np.stack([(oracle_gram if algo == "gram" else oracle_standard)(X64[b]) for b in range(B)])
    errs = per_matrix_rel(got, ref)
    say("  rel errs", errs)
    assert max(errs) <= _tol(cdt)
    assert out.dtype == X.dtype


@pytest.mark.parametrize("restarts", [(), (1,), (2,), (1, 3), (1, 2, 3, 4)])
def test_restart_sets_fp32(restarts):
    gns = need_gpu()
    X, X64 = _inputs(2, 200, 333, "f32", seed=12)
    say(f"restarts {restarts}")
    out = gns.gram_ns_batched(X.cuda(), NS5, restarts=restarts)
    torch.cuda.synchronize()
    ref = np.stack([oracle_gram(X64[b], restarts=restarts) for b in range(2)])
    assert max(per_matrix_rel(synth.as_f64(out), ref)) <= TOL_F32


@pytest.mark.parametrize("cdt", ["bf16", "f16"])
@pytest.mark.parametrize("restarts", [(1,), (2,), (3,), (4,), (1, 3)])
def test_restart_location_sweep_half(cdt, restarts):
    """Where the restart goes (Dion3 sweeps it in half precision): every
    location of a single restart, and two restarts, on 256-edge tiles, against
    the oracle with the same restart set."""
    gns = need_gpu()
    X, X64 = _inputs(2, 512, 1536, "bf16", seed=29)
    say(f"restart sweep {cdt} {restarts}")
    out = gns.gram_ns_batched(X.cuda(), NS5, restarts=restarts, compute_dtype=DT[cdt], tile=256)
    torch.cuda.synchronize()
    ref = np.stack([oracle_gram(X64[b], restarts=restarts) for b in range(2)])
    errs = per_matrix_rel(synth.as_f64(out), ref)
    say("  rel errs", errs)
    assert max(errs) <= TOL_HALF


@pytest.mark.parametrize("cdt,tile", [("f32", None), ("bf16", None), ("bf16", 256), ("f16", 256)])
def test_naive_algebra(cdt, tile):
    """Algorithm 2's algebra puts a_t on the diagonal of Z and, after an
    identity Q, writes Q = Z as a second output: with 256-edge tiles both go
    through the staged epilogue of the diagonal tiles (half-width waves)."""
    gns = need_gpu()
    X, X64 = _inputs(2, 260, 520, "f32", seed=13)
    say(f"naive algebra {cdt} tile {tile}")
    out = gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,), naive_algebra=True,
                              compute_dtype=DT[cdt], tile=tile)
    torch.cuda.synchronize()
    ref = np.stack([oracle_gram(X64[b], algebra="naive") for b in range(2)])
    assert max(per_matrix_rel(synth.as_f64(out), ref)) <= _tol(cdt)


@pytest.mark.parametrize("cdt,tile", [("f32", None), ("bf16", 256)])
def test_distinct_coefficients_per_iteration(cdt, tile):
    """A schedule whose iterations differ catches any mix-up of t or of (a,b,c)
    (with 256-edge tiles also in the diagonal-tile epilogue, where a_t enters
    the implicit Q = Z + aI and the Q update's second term)."""
    gns = need_gpu()
    co = [(3.0, -3.2, 1.2), (2.5, -2.0, 0.5), (15 / 8, -10 / 8, 3 / 8), (3.4445, -4.775, 2.0315),
          (1.9, -1.3, 0.4), (1.5, -0.5, 0.0)]
    X, X64 = _inputs(2, 150, 400, "f32", seed=14)
    say(f"distinct coefficients {cdt} tile {tile}")
    g = gns.gram_ns_batched(X.cuda(), co, restarts=(2, 4), compute_dtype=DT[cdt], tile=tile)
    s = gns.standard_ns_batched(X.cuda(), co, compute_dtype=DT[cdt], tile=tile)
    torch.cuda.synchronize()
    for b in range(2):
        ref = oracle.gram_ns(X64[b], co, restarts=(2, 4))
        assert rel_err(synth.as_f64(g)[b], ref) <= _tol(cdt)
        assert rel_err(synth.as_f64(s)[b], oracle.standard_ns(X64[b], co)) <= _tol(cdt)


@pytest.mark.parametrize("algo", ["gram", "standard"])
@pytest.mark.parametrize("cdt", ["bf16", "f32", "bf16x3"])
def test_row_subset(algo, cdt):
    """Dion3 rows: selected rows orthogonalised as one k x m matrix, the others
    left bit-exact."""
    gns = need_gpu()
    B, n, m, k = 2, 200, 520, 77
    io = "f32" if cdt == "f32" else "bf16"
    X, X64 = _inputs(B, n, m, io, seed=15)
    rows = np.stack([synth.row_subset(n, k, seed=15, index=b) for b in range(B)])
    init = torch.randn(B, n, m, generator=torch.Generator().manual_seed(3)).to(DT[io])
    out = init.clone().cuda()
    say(f"row subset {algo} {cdt}")
    _run(gns, algo, X.cuda(), cdt, row_idx=torch.from_numpy(rows).cuda(), out=out)
    torch.cuda.synchronize()
    got = synth.as_f64(out)
    init64 = synth.as_f64(init)
    for b in range(B):
        sel = rows[b]
        ref = (oracle_gram if algo == "gram" else oracle_standard)(X64[b][sel])
        assert rel_err(got[b][sel], ref) <= _tol(cdt)
        keep = np.setdiff1d(np.arange(n), sel)
        assert np.array_equal(got[b][keep], init64[b][keep])


@pytest.mark.parametrize("cdt", ["bf16", "f16"])
@pytest.mark.parametrize("restarts", [(2,), (1, 3), ()])
def test_row_subset_kmajor_products(cdt, restarts):
    """Row subset on 256-edge 16-bit tiles, where Q X reads X row-major
    (K-major B): ragged k and m, the restart's second row buffer, and the
    final product's row scatter; other rows bit-exact."""
    gns = need_gpu()
    B, n, m, k = 2, 600, 900, 301
    X, X64 = _inputs(B, n, m, "bf16", seed=37)
    rows = np.stack([synth.row_subset(n, k, seed=37, index=b) for b in range(B)])
    init = torch.randn(B, n, m, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    out = init.clone().cuda()
    say(f"row subset k-major {cdt} restarts={restarts}")
    gns.gram_ns_batched(X.cuda(), NS5, restarts=restarts, compute_dtype=DT[cdt], tile=256,
                        row_idx=torch.from_numpy(rows).cuda(), out=out)
    torch.cuda.synchronize()
    got = synth.as_f64(out)
    init64 = synth.as_f64(init)
    for b in range(B):
        sel = rows[b]
        assert rel_err(got[b][sel], oracle_gram(X64[b][sel], restarts=restarts)) <= TOL_HALF
        keep = np.setdiff1d(np.arange(n), sel)
        assert np.array_equal(got[b][keep], init64[b][keep])


@pytest.mark.parametrize("cdt", ["bf16", "f16"])
@pytest.mark.parametrize("m", [700, 702])
@pytest.mark.parametrize("subset", [False, True])
def test_f32_input_row_layout(cdt, m, subset):
    """fp32 input, 16-bit products on 256-edge tiles: the normalised copy is
    written in row layout only (one wave per row when m is a multiple of 4,
    the tiled kernel otherwise), with and without a row subset."""
    gns = need_gpu()
    B, n = 2, 300
    X, X64 = _inputs(B, n, m, "f32", seed=38)
    kw = {}
    rows = None
    if subset:
        rows = np.stack([synth.row_subset(n, 211, seed=38, index=b) for b in range(B)])
        kw = dict(row_idx=torch.from_numpy(rows).cuda(), out=torch.zeros(B, n, m, device="cuda"))
    say(f"f32 input row layout cdt={cdt} m={m} subset={subset}")
    out = gns.gram_ns_batched(X.cuda(), NS5, compute_dtype=DT[cdt], tile=256, **kw)
    torch.cuda.synchronize()
    got = synth.as_f64(out)
    for b in range(B):
        sel = rows[b] if subset else np.arange(n)
        assert rel_err(got[b][sel], oracle_gram(X64[b][sel])) <= TOL_HALF
        if subset:
            keep = np.setdiff1d(np.arange(n), sel)
            assert not np.any(got[b][keep])


@pytest.mark.parametrize("subset", [False, True])
@pytest.mark.parametrize("io,cdt", [("bf16", "f16"), ("bf16", "bf16"), ("f16", "f16")])
def test_final_staged_matches_element_path(io, cdt, subset):
    """The final product's staged row-piece stores (16-bit output, rows
    aligned) round exactly as its element-by-element stores (forced with an
    output 2 bytes off alignment): bit-identical, and within the oracle's
    tolerance; fp16 products with a bf16 output included."""
    gns = need_gpu()
    B, n, m = 2, 300, 1032
    X, X64 = _inputs(B, n, m, io, seed=42)
    kw = {}
    rows = None
    if subset:
        rows = np.stack([synth.row_subset(n, 173, seed=42, index=b) for b in range(B)])
        kw["row_idx"] = torch.from_numpy(rows).cuda()
    buf = torch.zeros(2 * B * n * m + 8, dtype=X.dtype, device="cuda")
    aligned = buf[:B * n * m].view(B, n, m)
    shifted = buf[B * n * m + 1:2 * B * n * m + 1].view(B, n, m)   # 2 bytes off 16-byte alignment
    say(f"final staged vs element io={io} cdt={cdt} subset={subset}")
    for out in (aligned, shifted):
        gns.gram_ns_batched(X.cuda(), NS5, compute_dtype=DT[cdt], tile=256, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.equal(aligned, shifted)
    got = synth.as_f64(aligned)
    for b in range(B):
        sel = rows[b] if subset else np.arange(n)
        assert rel_err(got[b][sel], oracle_gram(X64[b][sel])) <= TOL_HALF


def test_row_subset_full_permutation_matches_plain():
    gns = need_gpu()
    B, n, m = 2, 140, 300
    X, _ = _inputs(B, n, m, "f32", seed=16)
    perm = np.stack([np.random.default_rng(b).permutation(n) for b in range(B)])
    say("full permutation")
    a = gns.gram_ns_batched(X.cuda(), NS5, row_idx=torch.from_numpy(perm).cuda(),
                            out=torch.zeros(B, n, m, device="cuda"))
    b_ = gns.gram_ns_batched(X.cuda(), NS5)
    torch.cuda.synchronize()
    assert max(per_matrix_rel(synth.as_f64(a), synth.as_f64(b_))) <= 1e-5


@pytest.mark.parametrize("shape", [(1, 37), (1, 1), (130, 130), (256, 256), (5, 4099), (129, 129)])
@pytest.mark.parametrize("cdt", ["bf16", "f32"])
def test_edge_shapes(shape, cdt):
    gns = need_gpu()
    n, m = shape
    io = "f32" if cdt == "f32" else "bf16"
    X, X64 = _inputs(2, n, m, io, seed=17)
    say(f"edge {shape} {cdt}")
    g = gns.gram_ns_batched(X.cuda(), NS5, compute_dtype=DT[cdt])
    s = gns.standard_ns_batched(X.cuda(), NS5, compute_dtype=DT[cdt])
    torch.cuda.synchronize()
    for b in range(2):
        assert rel_err(synth.as_f64(g)[b], oracle_gram(X64[b])) <= _tol(cdt)
        assert rel_err(synth.as_f64(s)[b], oracle_standard(X64[b])) <= _tol(cdt)


@pytest.mark.parametrize("cdt,tol", [("f16", TOL_HALF), ("f32", TOL_F32), ("bf16", 0.15)])
def test_square_without_fallback(cdt, tol):
    """Gram NS forced on square matrices.  Forming X X^T squares the condition
    number of a square Gaussian, so bf16 products lose several percent (a CPU
    model of the same rounding points gives 0.06-0.08) while fp16 and fp32
    stay within their bounds; this is why square problems default to
    standard NS."""
    gns = need_gpu()
    io = "f32" if cdt == "f32" else "bf16"
    X, X64 = _inputs(2, 130, 130, io, seed=17)
    say(f"square no fallback {cdt}")
    g = gns.gram_ns_batched(X.cuda(), NS5, compute_dtype=DT[cdt], square_fallback=False)
    torch.cuda.synchronize()
    errs = [rel_err(synth.as_f64(g)[b], oracle_gram(X64[b])) for b in range(2)]
    say("  rel errs", errs)
    assert max(errs) <= tol


def test_single_selected_row():
    gns = need_gpu()
    X, X64 = _inputs(1, 50, 90, "f32", seed=18)
    ri = torch.tensor([[7]], dtype=torch.int64)
    say("k = 1")
    out = gns.gram_ns_batched(X.cuda(), NS5, row_idx=ri.cuda())
    torch.cuda.synchronize()
    assert rel_err(synth.as_f64(out)[0][[7]], oracle_gram(X64[0][[7]])) <= TOL_F32


def test_zero_matrix_gives_zero():
    gns = need_gpu()
    X = torch.zeros(2, 64, 200, dtype=torch.bfloat16, device="cuda")
    say("zero matrix")
    g = gns.gram_ns_batched(X, NS5)
    s = gns.standard_ns_batched(X, NS5)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g).item() == 0 and torch.count_nonzero(s).item() == 0


def test_batch_zero_is_noop():
    gns = need_gpu()
    X = torch.empty(0, 16, 32, dtype=torch.bfloat16, device="cuda")
    out = gns.gram_ns_batched(X, NS5)
    assert out.shape == (0, 16, 32)


def test_deterministic_and_inplace():
    gns = need_gpu()
    X, _ = _inputs(3, 300, 700, "bf16", seed=19)
    Xd = X.cuda()
    say("determinism")
    a = gns.gram_ns_batched(Xd, NS5)
    b = gns.gram_ns_batched(Xd, NS5)
    c = Xd.clone()
    gns.gram_ns_batched(c, NS5, out=c)          # out aliases X
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, c)


def test_output_guard_band():
    """Nothing is written outside out, and the workspace's leftovers from a
    bigger problem do not leak into a smaller one."""
    gns = need_gpu()
    B, n, m = 2, 200, 450
    X, X64 = _inputs(B, n, m, "bf16", seed=20)
    pad = 4096
    buf = torch.full((B * n * m + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + B * n * m].view(B, n, m)
    ws = torch.full((gns.gram_workspace_bytes(torch.bfloat16, 4, 400, 900),), 0x7f,
                    dtype=torch.uint8, device="cuda")
    say("guard band")
    gns.gram_ns_batched(X.cuda(), NS5, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:pad]).all() and torch.isnan(buf[-pad:]).all()
    assert not torch.isnan(out).any()
    ref = np.stack([oracle_gram(X64[b]) for b in range(B)])
    assert max(per_matrix_rel(synth.as_f64(out), ref)) <= TOL_HALF


def test_check_row_idx():
    gns = need_gpu()
    good = torch.tensor([[0, 5, 3], [9, 1, 2]], dtype=torch.int64, device="cuda")
    oob = torch.tensor([[0, 5, 3], [9, 10, 2]], dtype=torch.int64, device="cuda")
    dup = torch.tensor([[0, 5, 5], [9, 1, 2]], dtype=torch.int64, device="cuda")
    assert gns.check_row_idx(good, 10) == 0
    assert gns.check_row_idx(oob, 10) == 1
    assert gns.check_row_idx(dup, 10) == 2


def test_out_of_range_rows_touch_nothing():
    """A bad index reads as a zero row and is not written (no stray access)."""
    gns = need_gpu()
    X, _ = _inputs(1, 20, 40, "f32", seed=21)
    out = torch.zeros(1, 20, 40, device="cuda")
    ri = torch.tensor([[3, 25, 4]], dtype=torch.int64, device="cuda")
    gns.gram_ns_batched(X.cuda(), NS5, row_idx=ri, out=out)
    torch.cuda.synchronize()
    keep = [i for i in range(20) if i not in (3, 4)]
    assert torch.count_nonzero(out[0, keep]).item() == 0
    assert torch.isfinite(out).all()


def test_out_of_range_rows_on_direct_path():
    """The direct path's gather (bf16 rows that fill whole 256-edge tiles)
    also reads a bad index as a zero row and writes nothing for it: the other
    selected rows match the oracle on the gathered matrix with that row zero,
    and every unselected row keeps its value."""
    gns = need_gpu()
    B, n, m, k = 2, 512, 512, 256
    X, X64 = _inputs(B, n, m, "bf16", seed=23)
    rows = np.stack([np.sort(synth.row_subset(n, k, seed=23, index=b)) for b in range(B)])
    rows[0, 5] = n + 90                        # outside X_0
    rows[1, 0] = -1                            # outside X_1
    plan = gns.call_plan(False, 1 << 32, 2 << 32, B, n, m, torch.bfloat16, torch.bfloat16, NS5, (2,),
                         row_idx_ptr=3 << 32, k=k, opts=0x20)
    assert plan.direct_input == 1 and plan.input_copy == 1
    init = synth.batch(B, n, m, seed=24, dtype=torch.bfloat16)
    say("direct path, out-of-range rows")
    out = gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,), row_idx=torch.from_numpy(rows).cuda(),
                              out=init.clone().cuda(), tile=256).cpu()
    assert torch.isfinite(out.float()).all()
    for b in range(B):
        valid = (rows[b] >= 0) & (rows[b] < n)
        G = np.zeros((k, m))
        G[valid] = X64[b][rows[b][valid]]
        ref = oracle.gram_ns(G, NS5, restarts=(2,))
        assert rel_err(synth.as_f64(out[b])[rows[b][valid]], ref[valid]) <= TOL_HALF
        keep = np.setdiff1d(np.arange(n), rows[b][valid])
        assert torch.equal(out[b][keep], init[b][keep])


@pytest.mark.parametrize("algo", ["gram", "standard"])
def test_batch_split_matches_one_stream(algo):
    """Splitting a batch over the library's two streams gives bit-identical
    results to running every matrix on the caller's stream (odd batch)."""
    gns = need_gpu()
    X, X64 = _inputs(5, 300, 700, "bf16", seed=22)
    Xd = X.cuda()
    say(f"split vs one stream {algo}")
    a = _run(gns, algo, Xd, "bf16")
    b = _run(gns, algo, Xd, "bf16", split_batch=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = np.stack([(oracle_gram if algo == "gram" else oracle_standard)(X64[b_]) for b_ in range(5)])
    assert max(per_matrix_rel(synth.as_f64(a), ref)) <= TOL_HALF


def test_split_orders_against_caller_stream():
    """Work enqueued on the caller's stream before the call is seen by both
    halves, and work enqueued after it sees their results, with no device-wide
    synchronisation in between."""
    gns = need_gpu()
    X, _ = _inputs(4, 256, 1024, "bf16", seed=23)
    X2, _ = _inputs(4, 256, 1024, "bf16", seed=24)
    Xd = X.cuda()
    X2d = X2.cuda()
    ref = gns.gram_ns_batched(X2d, NS5, split_batch=False)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    say("split ordering on a side stream")
    with torch.cuda.stream(s):
        buf = Xd.clone()
        buf.copy_(X2d)                       # must be visible to both halves
        out = gns.gram_ns_batched(buf, NS5, stream=s)
        total = out.float().sum(dim=(1, 2))  # must see both halves' results
    s.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(total, ref.float().sum(dim=(1, 2)))


def test_split_planes_tighter_than_bf16():
    """The split-bf16 compute type keeps about 16 significant bits in every
    stored iterate: on a log-uniform spectrum it must beat plain bf16 by a
    wide margin and stay close to the fp32 path."""
    gns = need_gpu()
    B, n, m = 2, 256, 1024
    # fp32 input and output, so that no output rounding hides the difference
    X = synth.batch(B, n, m, seed=25, dist="logspec", dtype=torch.float32)
    X64 = synth.as_f64(X)
    say("split planes vs bf16 vs fp32, log spectrum 256x1024, fp32 I/O")
    outs = {c: gns.gram_ns_batched(X.cuda(), NS5, compute_dtype=DT[c]) for c in ("bf16", "bf16x3", "f32")}
    torch.cuda.synchronize()
    ref = np.stack([oracle_gram(X64[b]) for b in range(B)])
    err = {c: max(per_matrix_rel(synth.as_f64(o), ref)) for c, o in outs.items()}
    say("  errs", err)
    assert err["bf16x3"] <= 1e-3
    assert err["bf16x3"] < 0.25 * err["bf16"]
    assert err["f32"] <= TOL_F32


@pytest.mark.parametrize("algo", ["gram", "standard"])
@pytest.mark.parametrize("io,cdt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "bf16x3"), ("bf16", "f16")])
def test_tall_parity(algo, io, cdt):
    """n > m: the library orthogonalises X^T (its normalised copy is the
    transposed layout it writes anyway) and writes the result back in the
    caller's layout; several tiles and ragged tails on both sides."""
    gns = need_gpu()
    B, n, m = 3, 700, 300
    X, X64 = _inputs(B, n, m, io, seed=26)
    say(f"tall {algo} io={io} cdt={cdt} {B}x{n}x{m}")
    out = _run(gns, algo, X.cuda(), cdt)
    torch.cuda.synchronize()
    ref = np.stack([(oracle_gram if algo == "gram" else oracle_standard)(X64[b]) for b in range(B)])
    errs = per_matrix_rel(synth.as_f64(out), ref)
    say("  rel errs", errs)
    assert max(errs) <= _tol(cdt)
    assert out.shape == X.shape


@pytest.mark.parametrize("tile", [128, 256])
def test_tall_matches_transposed_problem(tile):
    """A tall batch and the wide batch of its transposes give the same
    results, transposed, up to the order of the norm's partial sums."""
    gns = need_gpu()
    X, _ = _inputs(2, 600, 260, "f32", seed=27)
    Xd = X.cuda()
    say(f"tall vs transposed, tile {tile}")
    a = gns.gram_ns_batched(Xd, NS5, tile=tile)
    b = gns.gram_ns_batched(Xd.transpose(1, 2).contiguous(), NS5, tile=tile)
    torch.cuda.synchronize()
    assert max(per_matrix_rel(synth.as_f64(a), synth.as_f64(b.transpose(1, 2)))) <= 1e-5


@pytest.mark.parametrize("tile", [256, "mixed"])
@pytest.mark.parametrize("algo", ["gram", "standard"])
def test_tall_16bit_tiles(algo, tile):
    """n > m in bf16 on forced 256-edge or mixed tiles: the transposed path
    of the rectangular products, and the final product's staged stores into
    the caller's layout (ragged on both sides)."""
    gns = need_gpu()
    B, n, m = 3, 700, 300
    X, X64 = _inputs(B, n, m, "bf16", seed=41)
    say(f"tall 16-bit {algo} tile={tile}")
    out = _run(gns, algo, X.cuda(), "bf16", tile=tile)
    torch.cuda.synchronize()
    ref = np.stack([(oracle_gram if algo == "gram" else oracle_standard)(X64[b]) for b in range(B)])
    assert max(per_matrix_rel(synth.as_f64(out), ref)) <= TOL_HALF


@pytest.mark.parametrize("tile", [None, 256, "mixed"])
def test_tall_row_subset(tile):
    """Dion3 rows with more selected rows than columns (k > m)."""
    gns = need_gpu()
    B, n, m, k = 2, 400, 150, 230
    X, X64 = _inputs(B, n, m, "bf16", seed=28)
    rows = np.stack([synth.row_subset(n, k, seed=28, index=b) for b in range(B)])
    init = torch.randn(B, n, m, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    out = init.clone().cuda()
    say(f"tall row subset tile={tile}")
    gns.gram_ns_batched(X.cuda(), NS5, row_idx=torch.from_numpy(rows).cuda(), out=out, tile=tile)
    torch.cuda.synchronize()
    got = synth.as_f64(out)
    init64 = synth.as_f64(init)
    for b in range(B):
        sel = rows[b]
        assert rel_err(got[b][sel], oracle_gram(X64[b][sel])) <= TOL_HALF
        keep = np.setdiff1d(np.arange(n), sel)
        assert np.array_equal(got[b][keep], init64[b][keep])


def test_tall_mlp_down_projection():
    """One 16384 x 4096 bf16 matrix (the shape of an MLP down-projection
    weight), against the oracle."""
    gns = need_gpu()
    X = synth.batch(1, 16384, 4096, seed=29, dtype=torch.bfloat16)
    say("tall 16384x4096")
    g = gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,))
    torch.cuda.synchronize()
    e = rel_err(synth.as_f64(g)[0], oracle_gram(synth.as_f64(X)[0]))
    say(f"  rel err {e:.4g}")
    assert e <= TOL_HALF


@pytest.mark.parametrize("split", [True, False])
def test_graph_capture_replays(split):
    """The whole call captured into a HIP graph and replayed several times,
    with eager work and synchronisations between replays: every replay
    equals the eager result bit for bit.  The library enqueues no memset and no allocation,
    and its two-stream fan-out is captured through its fork/join events."""
    gns = need_gpu()
    B, n, m = 4, 300, 700
    X, _ = _inputs(B, n, m, "bf16", seed=33)
    X2, _ = _inputs(B, n, m, "bf16", seed=34)
    Xd = X.cuda()
    static_in = Xd.clone()
    static_out = torch.empty_like(Xd)
    ws = torch.empty(gns.gram_workspace_bytes(torch.bfloat16, B, n, m), dtype=torch.uint8, device="cuda")
    eager = gns.gram_ns_batched(Xd, NS5, split_batch=split)
    eager2 = gns.gram_ns_batched(X2.cuda(), NS5, split_batch=split)
    torch.cuda.synchronize()
    say(f"graph capture split={split}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):      # warm up on the capture stream
        gns.gram_ns_batched(static_in, NS5, out=static_out, workspace=ws, split_batch=split)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gns.gram_ns_batched(static_in, NS5, out=static_out, workspace=ws, split_batch=split,
                            stream=torch.cuda.current_stream())
    for rep in range(4):
        static_in.copy_(Xd if rep % 2 == 0 else X2.cuda())
        static_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager if rep % 2 == 0 else eager2
        assert torch.equal(static_out, want), f"replay {rep}"
        _ = (static_out.float() * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("algo,restarts", [("gram", (2,)), ("gram", ()), ("gram", (1, 3)), ("standard", ())])
@pytest.mark.parametrize("io,tile", [("bf16", 128), ("bf16", 256), ("f16", 256), ("bf16", "mixed")])
def test_direct_input_path(algo, restarts, io, tile):
    """Whole-tile shapes with the input already in the compute type: the
    products read X itself and apply the normalisation in their epilogues
    (no normalised copy).  Against the oracle, T = 1 and T = 5."""
    gns = need_gpu()
    B, n, m = 3, 512, 1536
    X, X64 = _inputs(B, n, m, io, seed=35)
    say(f"direct {algo} restarts={restarts} io={io} tile={tile}")
    for co in (NS5, NS5[:1]):
        rs = tuple(r for r in restarts if r < len(co))
        if algo == "gram":
            out = gns.gram_ns_batched(X.cuda(), co, restarts=rs, tile=tile)
        else:
            out = gns.standard_ns_batched(X.cuda(), co, tile=tile)
        torch.cuda.synchronize()
        ref = np.stack([oracle.gram_ns(X64[b], co, restarts=rs) if algo == "gram"
                        else oracle.standard_ns(X64[b], co) for b in range(B)])
        errs = per_matrix_rel(synth.as_f64(out), ref)
        say("  T", len(co), "rel errs", errs)
        assert max(errs) <= TOL_HALF


@pytest.mark.parametrize("restarts", [(2,), ()])
@pytest.mark.parametrize("tile", [256, "mixed"])
def test_row_subset_on_direct_path(restarts, tile):
    """A row subset that fills whole tiles in the compute type: the input pass
    gathers the selected rows, unscaled, into the workspace and the products
    read that copy with the normalisation in their epilogues.  Bit-identical
    to the same call on the gathered rows as a dense batch, out of place and
    in place, with every other row untouched; against the oracle (Dion3 §6,
    Algorithm 4: only the selected rows are orthogonalised and written)."""
    gns = need_gpu()
    B, n, m, k = 3, 768, 1536, 512
    X, X64 = _inputs(B, n, m, "bf16", seed=37)
    rows = np.stack([synth.row_subset(n, k, seed=37, index=b) for b in range(B)])
    say(f"row subset direct restarts={restarts} tile={tile}")
    plan = gns.call_plan(False, 1 << 32, 2 << 32, B, n, m, torch.bfloat16, torch.bfloat16, NS5, restarts,
                         row_idx_ptr=3 << 32, k=k, opts=0x20 if tile == 256 else 0x80)
    assert plan.direct_input == 1 and plan.input_copy == 1
    ri = torch.from_numpy(rows).cuda()
    Xd = X.cuda()
    init = synth.batch(B, n, m, seed=38, dtype=torch.bfloat16).cuda()
    out = gns.gram_ns_batched(Xd, NS5, restarts=restarts, row_idx=ri, out=init.clone(), tile=tile)
    dense_in = torch.stack([Xd[b, ri[b]] for b in range(B)]).contiguous()
    dense = gns.gram_ns_batched(dense_in, NS5, restarts=restarts, tile=tile)
    inplace = Xd.clone()
    gns.gram_ns_batched(inplace, NS5, restarts=restarts, row_idx=ri, out=inplace, tile=tile)
    torch.cuda.synchronize()
    mask = torch.ones(B, n, dtype=torch.bool)
    for b in range(B):
        mask[b, rows[b]] = False
        assert torch.equal(out[b, ri[b]], dense[b]), b
        assert torch.equal(inplace[b, ri[b]], dense[b]), b
    assert torch.equal(out.cpu()[mask], init.cpu()[mask])
    assert torch.equal(inplace.cpu()[mask], X[mask])
    ref = np.stack([oracle.gram_ns(X64[b][rows[b]], NS5, restarts=restarts) for b in range(B)])
    errs = per_matrix_rel(synth.as_f64(dense), ref)
    say("  rel errs", errs)
    assert max(errs) <= TOL_HALF


@pytest.mark.parametrize("case", ["bf16", "f32", "rows", "standard"])
def test_gram_matrix_k_split(case):
    """Few 256-edge Gram tiles and a long contraction (8 x 1024x6144: 80 upper
    tiles over the batch): the size rule cuts the contraction into parts and a
    second pass sums them.  Against the oracle (matrices 0 and 7), with the
    direct input (bf16), the normalised copy (fp32 input), a row subset, and
    standard NS; the launch records show the two passes."""
    gns = need_gpu()
    B, n, m = 8, 1024, 6144
    io = "f32" if case == "f32" else "bf16"
    rows_n = 2048 if case == "rows" else n
    X, X64 = _inputs(B, rows_n, m, io, seed=43)
    kw = {}
    rows = None
    if case == "rows":
        rows = np.stack([np.sort(synth.row_subset(rows_n, n, seed=43, index=b)) for b in range(B)])
        init = torch.from_numpy(np.random.default_rng(43).standard_normal((B, rows_n, m), dtype=np.float32))
        init = init.to(X.dtype)
        kw = dict(row_idx=torch.from_numpy(rows).cuda(), out=init.cuda())
    say(f"k split {case}")
    gns.timing_reset()
    gns.timing_enable(True)
    if case == "standard":
        out = gns.standard_ns_batched(X.cuda(), NS5, compute_dtype=torch.bfloat16)
    else:
        out = gns.gram_ns_batched(X.cuda(), NS5, compute_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    recs = gns.timing_read()
    gns.timing_enable(False)
    grams = 5 if case == "standard" else 2          # Gram matrices formed per call
    parts_pass = [r for r in recs if r[0] == "syrk" and r[2] > 0]
    sum_pass = [r for r in recs if r[0] == "syrk" and r[2] == 0]
    # each stream of the batch fan-out forms its own Gram matrices, in two passes each
    assert len(parts_pass) == len(sum_pass) and len(parts_pass) in (grams, 2 * grams)
    got = synth.as_f64(out)
    if case == "rows":
        oc = out.cpu()
        for b in range(B):
            mask = torch.ones(rows_n, dtype=torch.bool)
            mask[torch.from_numpy(rows[b])] = False
            assert torch.equal(oc[b][mask], init[b][mask]), f"matrix {b}: an unselected row changed"
    for b in (0, B - 1):
        sel = rows[b] if case == "rows" else np.arange(n)
        ref = (oracle_standard if case == "standard" else oracle_gram)(X64[b][sel])
        assert rel_err(got[b][sel], ref) <= TOL_HALF


def test_gram_matrix_k_split_graph_replay():
    """The two passes of a K-split Gram matrix captured in a HIP graph: every
    replay equals the eager call bit for bit (8 x 1024x6144)."""
    gns = need_gpu()
    B, n, m = 8, 1024, 6144
    X, _ = _inputs(B, n, m, "bf16", seed=44)
    Xd = X.cuda()
    static_out = torch.empty_like(Xd)
    ws = torch.empty(gns.gram_workspace_bytes(torch.bfloat16, B, n, m), dtype=torch.uint8, device="cuda")
    eager = gns.gram_ns_batched(Xd, NS5)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                        # warm up on the capture stream
        gns.gram_ns_batched(Xd, NS5, out=static_out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    say("k split graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gns.gram_ns_batched(Xd, NS5, out=static_out, workspace=ws, stream=torch.cuda.current_stream())
    for rep in range(3):
        static_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(static_out, eager), f"replay {rep}"
        _ = (static_out.float() * 2).sum().item()    # eager work between replays
