"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol include/gns.h declares, sizes workspaces, and rejects bad arguments
with the documented status before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gns.h")

gns = pytest.importorskip("gram_newton_schulz_amd")

pytestmark = pytest.mark.skipif(not os.path.exists(gns.LIB_PATH),
                                reason="libgns.so not built (run __graft_entry__.build())")

FAKE = 0x10000000  # never dereferenced: every call below fails validation first
E = {"OK": 0, "NULL": 1, "SHAPE": 2, "DTYPE": 3, "COEFF": 4, "RESTART": 5, "ROWIDX": 6,
     "ALIAS": 7, "WORKSPACE": 8, "HIP": 9, "FLAGS": 10, "PARAM": 11, "NONFINITE": 12}


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gns_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = gns.lib()
    decl = declared_functions()
    assert decl, "no declarations parsed"
    for name in decl:
        assert hasattr(L, name), f"{name} declared in gns.h but not exported"
    assert sorted(gns.EXPORTS) == decl


def test_version_and_strings():
    L = gns.lib()
    assert L.gns_abi_version() == 2
    for code in range(0, 13):
        assert L.gns_status_str(code)
        assert L.gns_status_str(code) != b"unknown status"


def test_workspace_sizes():
    b = gns.gram_workspace_bytes(gns.GNS_BF16, 8, 4096, 16384)
    # X_hat, two transposed copies and five n x n iterates, bf16
    assert b >= 8 * 2 * (3 * 4096 * 16384 + 5 * 4096 * 4096)
    assert gns.gram_workspace_bytes(gns.GNS_BF16, 0, 4096, 16384) == 0
    assert gns.gram_workspace_bytes(gns.GNS_BF16, 1, 0, 5) == 0           # no rows
    assert gns.gram_workspace_bytes(gns.GNS_BF16, 1, 10, 0) == 0          # no columns
    # a tall problem needs what its transpose needs, up to the norm partials
    # (which follow the caller's rows)
    tall = gns.gram_workspace_bytes(gns.GNS_BF16, 2, 700, 300)
    wide = gns.gram_workspace_bytes(gns.GNS_BF16, 2, 300, 700)
    assert tall > 0 and abs(tall - wide) < 16384
    assert gns.gram_workspace_bytes(7, 1, 10, 20) == 0                     # bad dtype
    assert gns.standard_workspace_bytes(gns.GNS_F32, 1, 64, 256) > 0
    # split storage: two planes of every region, 128-edge tiles
    x3 = gns.gram_workspace_bytes(gns.GNS_BF16X3, 2, 300, 700)
    assert x3 >= 2 * 2 * 2 * (3 * 384 * 768 + 5 * 384 * 384)
    assert gns.standard_workspace_bytes(gns.GNS_BF16X3, 2, 300, 700) > 0
    # ragged shapes are padded to whole tiles
    small = gns.gram_workspace_bytes(gns.GNS_F32, 1, 1, 1)
    assert small >= 4 * (3 * 128 * 128 + 5 * 128 * 128)


def _gram(X=FAKE, out=FAKE + 1 << 20, batch=1, n=4, m=8, io=1, cdt=1, coeffs=None, T=None,
          restarts=(2,), row_idx=None, k=0, opts=0, ws=None, ws_bytes=None):
    L = gns.lib()
    if coeffs is None:
        coeffs = [(3.4445, -4.7750, 2.0315)] * 5
    flat = [float(v) for row in coeffs for v in row]
    carr = (ctypes.c_double * max(len(flat), 1))(*flat)
    T = len(coeffs) if T is None else T
    rs = list(restarts)
    rarr = (ctypes.c_int * max(len(rs), 1))(*rs) if rs else None
    rows = k if row_idx else n
    need = L.gns_gram_workspace_bytes(cdt, batch, rows, m)
    if ws is None:
        ws = 0x7f0000000000
    if ws_bytes is None:
        ws_bytes = need
    return L.gns_gram_batched(X, out, batch, n, m, io, cdt, carr, T, rarr, len(rs),
                              row_idx, k, opts, ws, ws_bytes, None)


def test_gram_argument_errors():
    assert _gram(io=5) == E["DTYPE"]
    assert _gram(cdt=9) == E["DTYPE"]
    assert _gram(io=gns.GNS_BF16X3) == E["DTYPE"]     # a compute type only
    assert _gram(n=0) == E["SHAPE"]
    assert _gram(m=0) == E["SHAPE"]
    assert _gram(n=9, m=8, ws_bytes=100) == E["WORKSPACE"]   # tall: accepted, checked further
    assert _gram(row_idx=FAKE, k=0) == E["SHAPE"]
    assert _gram(row_idx=FAKE, k=5, n=4) == E["SHAPE"]    # k > n
    assert _gram(coeffs=[], T=0, restarts=()) == E["COEFF"]
    assert _gram(coeffs=[(float("nan"), 1, 1)] * 3, restarts=(1,)) == E["COEFF"]
    assert _gram(coeffs=[(1, 1, 1)] * 65, restarts=()) == E["COEFF"]
    assert _gram(restarts=(0,)) == E["RESTART"]
    assert _gram(restarts=(5,)) == E["RESTART"]           # must be <= T-1
    assert _gram(restarts=(3, 2)) == E["RESTART"]
    assert _gram(restarts=(2, 2)) == E["RESTART"]
    assert _gram(opts=0x200) == E["FLAGS"]
    assert _gram(opts=0x30) == E["FLAGS"]                 # two tile bits
    assert _gram(opts=0x50) == E["FLAGS"]                 # autotune with a tile bit
    assert _gram(opts=0x60) == E["FLAGS"]
    assert _gram(opts=0x90) == E["FLAGS"] and _gram(opts=0xa0) == E["FLAGS"] and _gram(opts=0xc0) == E["FLAGS"]
    assert _gram(opts=0x80, ws_bytes=100) == E["WORKSPACE"]   # mixed tiles: a valid option
    # autotune validates every argument before it times anything
    assert _gram(opts=0x40, ws_bytes=100) == E["WORKSPACE"]
    assert _gram(opts=0x40, restarts=(5,)) == E["RESTART"]
    assert _gram(X=None) == E["NULL"]
    assert _gram(out=None) == E["NULL"]
    assert _gram(ws=None, ws_bytes=0) != E["OK"]
    assert _gram(ws_bytes=100) == E["WORKSPACE"]
    assert _gram(ws=0x7f0000000001) == E["WORKSPACE"]     # misaligned
    # workspace overlapping X
    assert _gram(X=0x7f0000000000 + 4096) == E["ALIAS"]


def test_gram_batch_zero_is_noop():
    assert _gram(batch=0, X=None, out=None, ws=None, ws_bytes=0) == E["OK"]


def test_standard_argument_errors():
    L = gns.lib()
    carr = (ctypes.c_double * 15)(*([3.4445, -4.775, 2.0315] * 5))
    ws = 0x7f0000000000
    need = L.gns_standard_workspace_bytes(1, 1, 4, 8)
    assert L.gns_standard_batched(FAKE, FAKE, 1, 4, 8, 1, 1, carr, 0, None, 0, 0, ws, need, None) == E["COEFF"]
    assert L.gns_standard_batched(FAKE, FAKE, 1, 9, 0, 1, 1, carr, 5, None, 0, 0, ws, need, None) == E["SHAPE"]
    assert L.gns_standard_batched(FAKE, FAKE, 1, 9, 8, 1, 1, carr, 5, None, 0, 0, ws, 16, None) == E["WORKSPACE"]
    assert L.gns_standard_batched(FAKE, FAKE, 1, 4, 8, 1, 1, carr, 5, None, 0, 0, ws, 16, None) == E["WORKSPACE"]
    assert L.gns_standard_batched(FAKE, FAKE, 1, 4, 8, 1, 1, carr, 5, None, 0, 1, ws, need, None) == E["FLAGS"]
    assert L.gns_standard_batched(FAKE, FAKE, 1, 4, 8, 1, 1, carr, 5, None, 0, 0xc0, ws, need, None) == E["FLAGS"]
    assert L.gns_standard_batched(None, None, 0, 4, 8, 1, 1, carr, 5, None, 0, 0, None, 0, None) == E["OK"]
    assert L.gns_standard_batched(FAKE, FAKE, 1, 4, 8, 1, 1, carr, 5, None, 0, 0x50, ws, need, None) == E["FLAGS"]
    assert L.gns_standard_batched(FAKE, FAKE, 1, 9, 8, 1, 1, carr, 5, None, 0, 0x40, ws, 16, None) == E["WORKSPACE"]
    assert L.gns_standard_batched(None, None, 0, 4, 8, 1, 1, carr, 5, None, 0, 0x40, None, 0, None) == E["OK"]


def test_check_row_idx_argument_errors():
    L = gns.lib()
    assert L.gns_check_row_idx(None, 1, 2, 4, FAKE, None) == E["NULL"]
    assert L.gns_check_row_idx(FAKE, 1, 5, 4, FAKE, None) == E["SHAPE"]
    assert L.gns_check_row_idx(FAKE, 1, 2, 70000, FAKE, None) == E["SHAPE"]


def test_binding_errors_are_raised():
    import torch
    X = torch.zeros(2, 3, 8)
    with pytest.raises(gns.GnsError):
        gns.gram_ns_batched(X, [(1, 0, 0)], restarts=(), compute_dtype=torch.int32)


def test_select_argument_errors():
    L = gns.lib()
    ws = 0x7f0000000000
    need = L.gns_select_workspace_bytes(2, 64)
    assert need >= 8 * 2 * 64 and L.gns_select_workspace_bytes(0, 64) == 0
    sel = lambda **kw: L.gns_select_rows_l1(kw.get("M", FAKE), kw.get("batch", 2), kw.get("n", 64),
                                            kw.get("m", 32), kw.get("dt", 1), kw.get("k", 16),
                                            kw.get("out", FAKE + (1 << 24)), kw.get("ws", ws),
                                            kw.get("ws_bytes", need), None)
    assert sel(dt=gns.GNS_BF16X3) == E["DTYPE"]
    assert sel(k=0) == E["SHAPE"] and sel(k=65) == E["SHAPE"] and sel(m=0) == E["SHAPE"]
    assert sel(batch=70000) == E["SHAPE"]
    assert sel(M=None) == E["NULL"] and sel(out=None) == E["NULL"]
    assert sel(ws_bytes=8) == E["WORKSPACE"] and sel(ws=ws + 8) == E["WORKSPACE"]
    assert sel(M=ws + 512) == E["ALIAS"]                  # input overlaps the workspace
    assert sel(batch=0, M=None, out=None, ws=None, ws_bytes=0) == E["OK"]


def test_gram_output_overlap():
    """out is X itself, or disjoint from it: a partial overlap would let one
    matrix's output overwrite input that another still reads."""
    nbytes = 1 * 4 * 8 * 2
    assert _gram(X=FAKE, out=FAKE, ws_bytes=100) == E["WORKSPACE"]      # in place: accepted so far
    assert _gram(X=FAKE, out=FAKE + 2) == E["ALIAS"]
    assert _gram(X=FAKE + 2, out=FAKE) == E["ALIAS"]
    assert _gram(X=FAKE, out=FAKE + nbytes, ws_bytes=100) == E["WORKSPACE"]   # adjacent: fine


def _plan(standard=0, X=0x100000000, out=0x200000000, batch=3, n=512, m=1536, io=1, cdt=1,
          coeffs=None, restarts=(), row_idx=None, k=0, opts=0x20):
    if coeffs is None:
        coeffs = [(3.4445, -4.7750, 2.0315)] * 5
    return gns.call_plan(bool(standard), X, out, batch, n, m, io, cdt, coeffs, restarts,
                         row_idx_ptr=row_idx or 0, k=k, opts=opts)


def test_plan_in_place_copies_input_only_where_needed():
    """The final product reads X itself only on the direct, K-major path with
    no restart; an in-place call there copies X first (Dion3 Algorithm 3:
    X <- Q_T X is the only write of the output)."""
    X = 0x100000000
    oop = _plan()                                   # whole 256-edge tiles, bf16 in bf16
    assert oop.direct_input == 1 and oop.kmajor_products == 1 and oop.input_copy == 0
    assert oop.tile == 256 and oop.standard == 0 and oop.split_streams == 1
    ip = _plan(out=X)
    assert ip.direct_input == 1 and ip.kmajor_products == 1 and ip.input_copy == 1
    ip1 = _plan(out=X, coeffs=[(3.4445, -4.7750, 2.0315)])          # T = 1
    assert ip1.input_copy == 1
    # the size rule picks 256-edge tiles on its own for larger batches
    big = _plan(out=X, batch=2, n=2048, m=4096, opts=0)
    assert big.tile == 256 and big.sym_tile == 128 and big.input_copy == 1
    # ... and 128-edge tiles (transposed form, X read only first) for small ones
    small = _plan(out=X, opts=0)
    assert small.tile == 128 and small.direct_input == 1 and small.input_copy == 0
    # a restart replaces X by a workspace buffer before the final product
    assert _plan(out=X, restarts=(2,)).input_copy == 0
    # no direct path: ragged tiles or another I/O type
    assert _plan(out=X, n=500).input_copy == 0 and _plan(out=X, n=500).direct_input == 0
    assert _plan(out=X, io=0).input_copy == 0
    # transposed form (128-edge tiles) and standard NS read X only first
    assert _plan(out=X, opts=0x10).input_copy == 0 and _plan(out=X, opts=0x10).direct_input == 1
    assert _plan(standard=1, out=X).input_copy == 0
    sq = _plan(out=X, n=1536)                        # square: standard NS fallback
    assert sq.standard == 1 and sq.input_copy == 0
    # the in-place copy lives in a region the quoted workspace already holds
    L = gns.lib()
    assert ip.workspace_bytes <= L.gns_gram_workspace_bytes(1, 3, 512, 1536)
    assert oop.workspace_bytes == ip.workspace_bytes


def test_plan_row_subset_reads_a_gathered_copy():
    """A row subset that fills whole tiles in the compute type takes the
    direct path in the K-major form: the input pass gathers the selected rows,
    unscaled, into the workspace, and the products read that copy (scaled in
    their epilogues) in place of a normalised copy.  Elsewhere a row subset
    keeps the normalised copy (Dion3 Algorithm 4: only the selected rows are
    orthogonalised)."""
    R = 0x300000000
    sub = _plan(row_idx=R, k=256)                   # 256 of 512 rows, 256-edge tiles
    assert sub.direct_input == 1 and sub.kmajor_products == 1 and sub.input_copy == 1
    assert _plan(out=0x100000000, row_idx=R, k=256).input_copy == 1      # in place too
    assert _plan(row_idx=R, k=256, restarts=(2,)).input_copy == 1
    # ragged subset, transposed form (128-edge tiles), another I/O type,
    # standard NS: the normalised copy
    for p in (_plan(row_idx=R, k=200), _plan(row_idx=R, k=256, opts=0x10),
              _plan(row_idx=R, k=256, io=0), _plan(standard=1, row_idx=R, k=256)):
        assert p.direct_input == 0 and p.input_copy == 0
    # the copy lives in a region the quoted workspace already holds
    assert sub.workspace_bytes <= gns.lib().gns_gram_workspace_bytes(1, 3, 256, 1536)


def test_plan_autotune_and_errors():
    L = gns.lib()
    L.gns_autotune_clear()
    X = 0x100000000
    assert _plan(opts=0x40).autotune_timed == 1
    assert _plan(out=X, opts=0x40).autotune_timed == 0       # in place: never timed
    assert _plan(cdt=0, io=0, opts=0x40).autotune_timed == 0  # fp32: one tile edge
    assert _plan(opts=0x40).tile == 128                       # untuned: the size rule
    assert _plan(batch=2, n=2048, m=4096, opts=0x40).tile == 256
    assert _plan(batch=0).tile == 0
    with pytest.raises(gns.GnsError):
        _plan(out=X + 2)                                      # partial overlap
    with pytest.raises(gns.GnsError):
        _plan(restarts=(5,))
    info = gns.PlanInfo()
    carr = (ctypes.c_double * 3)(1.0, 0.0, 0.0)
    assert L.gns_call_plan(0, X, X, 1, 4, 8, 1, 1, carr, 1, None, 0, None, 0, 0, None) == E["NULL"]
    assert L.gns_call_plan(0, X, X, 1, 4, 8, 1, 1, carr, 1, None, 0, None, 0, 0x200,
                           ctypes.byref(info)) == E["FLAGS"]
    # the K split of small Gram matrices and the mixed tiles of the size rule
    sub = _plan(batch=8, n=4096, m=16384, row_idx=0x300000000, k=1024, restarts=(2,), opts=0)
    assert sub.tile == 256 and sub.sym_tile == 128 and sub.gram_parts == 3 and sub.gram_tile == 256


def test_plan_gram_tile_edge():
    """Under the size rule the Gram matrix keeps 256-edge tiles where the n x n
    products take 128 but its 128-edge grid would overflow one round of two
    workgroups per compute unit (more than 512 upper tiles over the batch)."""
    w2 = _plan(batch=16, n=1024, m=4096, opts=0)               # 16 x 36 = 576 128-edge tiles
    assert (w2.tile, w2.sym_tile, w2.gram_tile, w2.gram_parts) == (256, 128, 256, 1)
    fits = _plan(batch=14, n=1024, m=4096, opts=0)             # 14 x 36 = 504: one round
    assert (fits.tile, fits.sym_tile, fits.gram_tile) == (256, 128, 128)
    assert _plan(batch=16, n=1024, m=4096, opts=0x80).gram_tile == 128   # forced mixed tiles
    assert _plan(batch=16, n=1024, m=4096, opts=0x10).gram_tile == 128   # forced 128
    big = _plan(batch=8, n=4096, m=16384, opts=0)
    assert (big.sym_tile, big.gram_tile) == (256, 256)
    assert _plan(batch=16, n=1024, m=4096, io=0, cdt=0, opts=0).gram_tile == 128   # fp32: 128 only


def test_plan_size_limits():
    """A 256-row panel must stay within the 32-bit offsets of the buffer
    loads, and a padded matrix within 2^31 elements: 256 x 4194048 bf16 (a
    panel of 2^31 - 2^17 bytes) is accepted, on 256-edge tiles with X read
    row-major as one operand; a row one tile longer is refused, tall or wide."""
    ok = _plan(batch=1, n=256, m=4194048, opts=0)
    assert ok.direct_input == 1 and ok.tile == 128
    ok256 = _plan(batch=1, n=256, m=4194048, opts=0x20)
    assert ok256.tile == 256 and ok256.kmajor_products == 1 and ok256.gram_parts == 1
    assert _plan(batch=1, n=4194048, m=256, opts=0x20).tile == 256          # tall: the same panels
    for n, m in ((256, 4194304), (4194304, 256), (32768, 65792)):
        with pytest.raises(gns.GnsError):
            _plan(batch=1, n=n, m=m, opts=0x20)
    assert _plan(batch=1, n=32768, m=65536, opts=0x10).tile == 128          # 2^31 elements


def test_debug_checks_option():
    """GNS_OPT_DEBUG_CHECKS is a valid option of the three compute entry
    points; validation still comes first."""
    assert _gram(opts=0x100, ws_bytes=100) == E["WORKSPACE"]
    assert _gram(opts=0x140, ws_bytes=100) == E["WORKSPACE"]    # with autotune
    assert _dion3(opts=0x100, ws_bytes=64) == E["WORKSPACE"]
    assert gns.binding.GNS_OPT_DEBUG_CHECKS == 0x100


def test_check_finite_argument_errors():
    L = gns.lib()
    assert L.gns_check_finite(FAKE, 3, 1, 4, 8, None, 0, FAKE, None) == E["DTYPE"]   # split type
    assert L.gns_check_finite(FAKE, 1, 1, 0, 8, None, 0, FAKE, None) == E["SHAPE"]
    assert L.gns_check_finite(FAKE, 1, 1, 4, 8, FAKE, 5, FAKE, None) == E["SHAPE"]   # k > rows
    assert L.gns_check_finite(FAKE, 1, 70000, 4, 8, None, 0, FAKE, None) == E["SHAPE"]
    assert L.gns_check_finite(None, 1, 1, 4, 8, None, 0, FAKE, None) == E["NULL"]
    assert L.gns_check_finite(FAKE, 1, 1, 4, 8, None, 0, None, None) == E["NULL"]


def test_select_count_and_safety_scale_in_library():
    """k = ceil(f n) (Dion3 Algorithm 4) and p_t(x / s) (Appendix B.2.2) are
    computed behind the C ABI; the binding only marshals them."""
    L = gns.lib()
    assert L.gns_select_count(4096, 0.25) == 1024
    assert L.gns_select_count(10, 0.01) == 1 and L.gns_select_count(10, 1.0) == 10
    assert L.gns_select_count(7, 0.5) == 4 and L.gns_select_count(3, 1e-12) == 1
    for bad in (0.0, -0.5, 1.5, float("nan")):
        assert L.gns_select_count(10, bad) == 0
    assert L.gns_select_count(0, 0.5) == 0
    co = (ctypes.c_double * 6)(3.4445, -4.7750, 2.0315, 1.875, -1.25, 0.375)
    out = (ctypes.c_double * 6)()
    assert L.gns_safety_scale(co, 2, 2.0, out) == E["OK"]
    assert list(out) == [3.4445 / 2, -4.7750 / 8, 2.0315 / 32, 1.875 / 2, -1.25 / 8, 0.375 / 32]
    assert L.gns_safety_scale(co, 2, 0.0, out) == E["PARAM"]
    assert L.gns_safety_scale(co, 2, float("inf"), out) == E["PARAM"]
    assert L.gns_safety_scale(co, 0, 1.05, out) == E["COEFF"]
    assert L.gns_safety_scale(None, 2, 1.05, out) == E["NULL"]
    with pytest.raises(ValueError):
        gns.select_count(10, 0.0)
    with pytest.raises(ValueError):
        gns.safety_scaled([(1, 0, 0)], -1.0)


def test_binding_rejects_bad_buffers_before_any_launch():
    """Every check runs on the host before the library is called: shapes,
    dtypes and layout first, then that the tensors live on the GPU."""
    import torch
    X = torch.zeros(2, 4, 8, dtype=torch.bfloat16)
    co = [(1.0, 0.0, 0.0)]
    bad_outs = [torch.zeros(2, 4, 9, dtype=torch.bfloat16),          # shape
                torch.zeros(2, 4, 8, dtype=torch.float32),           # dtype
                torch.zeros(2, 8, 4, dtype=torch.bfloat16).transpose(1, 2)]   # layout
    for fn in (gns.gram_ns_batched, gns.standard_ns_batched):
        for o in bad_outs:
            with pytest.raises(gns.GnsError) as e:
                fn(X, co, out=o) if fn is gns.standard_ns_batched else fn(X, co, restarts=(), out=o)
            assert e.value.code in (2, 3)
        with pytest.raises(gns.GnsError) as e:                        # host memory
            fn(X, co) if fn is gns.standard_ns_batched else fn(X, co, restarts=())
        assert e.value.code == 1 and "GPU" in str(e.value)
        with pytest.raises(gns.GnsError) as e:                        # row_idx dtype
            kw = dict(row_idx=torch.zeros(2, 2, dtype=torch.int32))
            fn(X, co, **kw) if fn is gns.standard_ns_batched else fn(X, co, restarts=(), **kw)
        assert e.value.code == 6
    W = torch.zeros(2, 4, 8)
    with pytest.raises(gns.GnsError) as e:                            # row_idx shape
        gns.dion3_step(W, W.clone(), W.clone(), None, 2, co, (), normuon=False,
                       row_idx=torch.zeros(2, 3, dtype=torch.int64))
    assert e.value.code == 6
    with pytest.raises(gns.GnsError) as e:                            # host memory
        gns.dion3_step(W, W.clone(), W.clone(), None, 2, co, (), normuon=False)
    assert e.value.code == 1
    with pytest.raises(gns.GnsError):
        gns.select_rows_l1(X, 2)
    with pytest.raises(gns.GnsError):
        gns.check_finite(X)


def test_safety_factor_helper():
    """p_t(x / s) has coefficients (a/s, b/s^3, c/s^5): one step of the scaled
    schedule at s*x equals one step of the original at x."""
    import numpy as np
    import oracle
    co = [(3.4445, -4.7750, 2.0315), (1.875, -1.25, 0.375)]
    sc = gns.safety_scaled(co, 1.05)
    xs = np.linspace(0.0, 1.0, 11)
    for t in range(2):
        assert np.allclose(oracle.composed_poly([sc[t]], 1.05 * xs), oracle.composed_poly([co[t]], xs),
                           rtol=1e-13, atol=1e-15)
    assert gns.select_count(4096, 0.25) == 1024 and gns.select_count(10, 0.01) == 1


def _dion3(W=FAKE, G=FAKE + (1 << 30), M=FAKE + (2 << 30), v=FAKE + (3 << 30), batch=2, n=64, m=96,
           gdt=1, cdt=1, k=16, coeffs=None, T=None, restarts=(2,), lr=0.02, wd=0.0, mu=0.95,
           beta2=0.95, eps=1e-8, normuon=1, rows=FAKE + (4 << 30), opts=0, ws=None, ws_bytes=None):
    L = gns.lib()
    if coeffs is None:
        coeffs = [(3.4445, -4.7750, 2.0315)] * 5
    flat = [float(x) for row in coeffs for x in row]
    carr = (ctypes.c_double * max(len(flat), 1))(*flat)
    T = len(coeffs) if T is None else T
    rs = list(restarts)
    rarr = (ctypes.c_int * max(len(rs), 1))(*rs) if rs else None
    if ws is None:
        ws = 0x7f0000000000
    if ws_bytes is None:
        ws_bytes = L.gns_dion3_workspace_bytes(cdt, batch, n, m, k)
    return L.gns_dion3_step(W, G, M, v, batch, n, m, gdt, cdt, k, carr, T, rarr, len(rs), lr, wd, mu,
                            beta2, eps, normuon, rows, opts, ws, ws_bytes, None)


def test_dion3_workspace_size():
    L = gns.lib()
    b, n, m, k = 2, 64, 96, 16
    need = L.gns_dion3_workspace_bytes(gns.GNS_BF16, b, n, m, k)
    gram = L.gns_gram_workspace_bytes(gns.GNS_BF16, b, k, m)
    # the orthogonalisation's workspace, then row keys, the fp32 update O and
    # two fp64 values per selected row
    assert need >= gram + 8 * b * n + 4 * b * k * m + 16 * b * k
    assert L.gns_dion3_workspace_bytes(gns.GNS_BF16, 0, n, m, k) == 0
    assert L.gns_dion3_workspace_bytes(gns.GNS_BF16, b, n, m, 0) == 0
    assert L.gns_dion3_workspace_bytes(gns.GNS_BF16, b, n, m, n + 1) == 0
    assert L.gns_dion3_workspace_bytes(9, b, n, m, k) == 0


def test_dion3_argument_errors():
    assert _dion3(gdt=gns.GNS_BF16X3) == E["DTYPE"]
    assert _dion3(cdt=7) == E["DTYPE"]
    assert _dion3(k=0) == E["SHAPE"] and _dion3(k=65) == E["SHAPE"] and _dion3(m=0) == E["SHAPE"]
    assert _dion3(batch=70000) == E["SHAPE"]
    assert _dion3(coeffs=[], T=0, restarts=()) == E["COEFF"]
    assert _dion3(restarts=(5,)) == E["RESTART"]
    assert _dion3(lr=float("nan")) == E["PARAM"]
    assert _dion3(mu=float("inf")) == E["PARAM"]
    assert _dion3(eps=0.0) == E["PARAM"]                   # NorMuon divides by sqrt(v) + eps
    assert _dion3(opts=0x200) == E["FLAGS"]
    assert _dion3(opts=0x40) == E["FLAGS"]                 # no autotune for the whole update
    assert _dion3(opts=0x90) == E["FLAGS"]                 # two tile bits
    assert _dion3(W=None) == E["NULL"] and _dion3(rows=None) == E["NULL"]
    assert _dion3(v=None) == E["NULL"]                     # NorMuon needs v
    assert _dion3(ws_bytes=64) == E["WORKSPACE"] and _dion3(ws=0x7f0000000008) == E["WORKSPACE"]
    assert _dion3(M=FAKE + 4096) == E["ALIAS"]             # momentum overlaps the weights
    assert _dion3(G=0x7f0000000000 + 256) == E["ALIAS"]    # gradient overlaps the workspace
    assert _dion3(batch=0, W=None, G=None, M=None, v=None, rows=None, ws=None, ws_bytes=0) == E["OK"]


def test_autotune_table_starts_empty_and_clears():
    L = gns.lib()
    L.gns_autotune_clear()
    assert gns.tuned_tile(gns.GNS_BF16, gns.GNS_BF16, 8, 4096, 16384) == 0
    assert gns.tuned_tile(gns.GNS_BF16, gns.GNS_BF16, 8, 4096, 16384, standard=True) == 0
    # a validation failure keeps nothing
    assert _gram(opts=0x40, ws_bytes=100) == E["WORKSPACE"]
    sym = ctypes.c_int(-1)
    assert L.gns_tuned_tile(0, 1, 1, 1, 4, 8, ctypes.byref(sym)) == 0 and sym.value == 0
    assert L.gns_tuned_tile(0, 1, 1, 1, 4, 8, None) == 0
    gns.autotune_clear()


def test_binding_tile_option():
    from gram_newton_schulz_amd import binding
    assert binding._tile_opts(None) == 0
    assert binding._tile_opts(128) == binding.GNS_OPT_TILE_128
    assert binding._tile_opts(256) == binding.GNS_OPT_TILE_256
    assert binding._tile_opts("auto") == binding.GNS_OPT_TILE_AUTOTUNE
    assert binding._tile_opts("mixed") == binding.GNS_OPT_TILE_MIXED
    with pytest.raises(gns.GnsError):
        binding._tile_opts(64)


def test_build_refuses_spilling_gemm_kernels():
    """The GEMM kernels' hand-counted DMA waits and m0 use assume no spills:
    the build parses the compiler's resource report and names any GEMM
    kernel that uses scratch."""
    from gram_newton_schulz_amd.build import scratch_users
    ok = ("remark: Function Name: _ZN3gns7gemm_ntINS_5EBF16ELi256E [-Rpass-analysis]\n"
          "remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis]\n"
          "remark:     VGPRs Spill: 0 [-Rpass-analysis]\n"
          "remark: Function Name: _ZN3gns9norm_partialI [-Rpass-analysis]\n"
          "remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis]\n")
    assert scratch_users(ok) == []
    bad = ok + ("remark: Function Name: _ZN3gns7gemm_ntINS_4EF32ELi256E [-Rpass-analysis]\n"
                "remark:     ScratchSize [bytes/lane]: 720 [-Rpass-analysis]\n"
                "remark:     VGPRs Spill: 180 [-Rpass-analysis]\n")
    assert scratch_users(bad) == ["_ZN3gns7gemm_ntINS_4EF32ELi256E"]
