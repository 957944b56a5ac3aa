"""ctypes binding of libgns.so (the C ABI in include/gns.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the stream.
The binding fails loudly when the library has not been built; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgns.so")

GNS_F32, GNS_BF16, GNS_F16, GNS_BF16X3 = 0, 1, 2, 3
GNS_OPT_NAIVE_ALGEBRA = 0x1
GNS_OPT_NO_SQUARE_FALLBACK = 0x2
GNS_OPT_ONE_STREAM = 0x4
GNS_OPT_TILE_128 = 0x10
GNS_OPT_TILE_256 = 0x20
GNS_OPT_TILE_AUTOTUNE = 0x40
GNS_OPT_TILE_MIXED = 0x80
GNS_OPT_DEBUG_CHECKS = 0x100
MAX_ITERS = 64

_DT = {torch.float32: GNS_F32, torch.bfloat16: GNS_BF16, torch.float16: GNS_F16}
_STATUS = {
    0: "GNS_OK", 1: "GNS_E_NULL", 2: "GNS_E_SHAPE", 3: "GNS_E_DTYPE", 4: "GNS_E_COEFF",
    5: "GNS_E_RESTART", 6: "GNS_E_ROWIDX", 7: "GNS_E_ALIAS", 8: "GNS_E_WORKSPACE",
    9: "GNS_E_HIP", 10: "GNS_E_FLAGS", 11: "GNS_E_PARAM", 12: "GNS_E_NONFINITE",
}

#: every symbol include/gns.h declares
EXPORTS = [
    "gns_abi_version", "gns_status_str", "gns_gram_workspace_bytes",
    "gns_standard_workspace_bytes", "gns_gram_batched", "gns_standard_batched",
    "gns_check_row_idx", "gns_timing_enable", "gns_timing_read", "gns_timing_reset",
    "gns_select_workspace_bytes", "gns_select_rows_l1",
    "gns_dion3_workspace_bytes", "gns_dion3_step", "gns_tuned_tile", "gns_autotune_clear",
    "gns_call_plan", "gns_check_finite", "gns_select_count", "gns_safety_scale",
    "gns_gram_batched_noalloc",
]


class GnsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code
        self.name = _STATUS.get(code, str(code))


class PlanInfo(ctypes.Structure):
    """gns_plan_info: what a call with given arguments would do (gns_call_plan)."""
    _fields_ = [("standard", ctypes.c_int), ("tile", ctypes.c_int), ("sym_tile", ctypes.c_int),
                ("gram_parts", ctypes.c_int), ("direct_input", ctypes.c_int),
                ("kmajor_products", ctypes.c_int), ("input_copy", ctypes.c_int),
                ("split_streams", ctypes.c_int), ("autotune_timed", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("gram_tile", ctypes.c_int)]


class LaunchRecord(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("kernel", ctypes.c_char_p), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double), ("ms", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgns.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m gram_newton_schulz_amd.build or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.gns_abi_version.restype = ctypes.c_int
    L.gns_status_str.restype = ctypes.c_char_p
    L.gns_status_str.argtypes = [ctypes.c_int]
    for f in (L.gns_gram_workspace_bytes, L.gns_standard_workspace_bytes):
        f.restype = sz
        f.argtypes = [ctypes.c_int, i64, i64, i64]
    L.gns_gram_batched.restype = ctypes.c_int
    L.gns_gram_batched.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                   vp, i64, ctypes.c_uint, vp, sz, vp]
    L.gns_standard_batched.restype = ctypes.c_int
    L.gns_standard_batched.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                       vp, i64, ctypes.c_uint, vp, sz, vp]
    L.gns_select_workspace_bytes.restype = sz
    L.gns_select_workspace_bytes.argtypes = [i64, i64]
    L.gns_select_rows_l1.restype = ctypes.c_int
    L.gns_select_rows_l1.argtypes = [vp, i64, i64, i64, ctypes.c_int, i64, vp, vp, sz, vp]
    L.gns_dion3_workspace_bytes.restype = sz
    L.gns_dion3_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, i64]
    dbl = ctypes.c_double
    L.gns_dion3_step.restype = ctypes.c_int
    L.gns_dion3_step.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, i64,
                                 ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                 dbl, dbl, dbl, dbl, dbl, ctypes.c_int, vp, ctypes.c_uint, vp, sz, vp]
    L.gns_tuned_tile.restype = ctypes.c_int
    L.gns_tuned_tile.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                 ctypes.POINTER(ctypes.c_int)]
    L.gns_autotune_clear.restype = None
    L.gns_autotune_clear.argtypes = []
    L.gns_check_row_idx.restype = ctypes.c_int
    L.gns_check_row_idx.argtypes = [vp, i64, i64, i64, vp, vp]
    L.gns_gram_batched_noalloc.restype = ctypes.c_int
    L.gns_gram_batched_noalloc.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_int), ctypes.c_int, vp, i64,
                                           ctypes.c_uint, vp]
    L.gns_call_plan.restype = ctypes.c_int
    L.gns_call_plan.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                ctypes.POINTER(ctypes.c_int), ctypes.c_int, vp, i64, ctypes.c_uint,
                                ctypes.POINTER(PlanInfo)]
    L.gns_check_finite.restype = ctypes.c_int
    L.gns_check_finite.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i64, vp, vp]
    L.gns_select_count.restype = i64
    L.gns_select_count.argtypes = [i64, ctypes.c_double]
    L.gns_safety_scale.restype = ctypes.c_int
    L.gns_safety_scale.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_double,
                                   ctypes.POINTER(ctypes.c_double)]
    L.gns_timing_enable.argtypes = [ctypes.c_int]
    L.gns_timing_enable.restype = None
    L.gns_timing_reset.restype = None
    L.gns_timing_read.restype = ctypes.c_int
    L.gns_timing_read.argtypes = [ctypes.POINTER(LaunchRecord), ctypes.c_int]
    _lib = L
    return L


def _check(code: int) -> None:
    if code != 0:
        raise GnsError(code, lib().gns_status_str(code).decode())


def _dtype_code(dt) -> int:
    """torch dtype -> gns_dtype code; also accepts a code, or "bf16x3" for the
    split-bf16 compute type (GNS_BF16X3)."""
    if isinstance(dt, int):
        return dt
    if dt == "bf16x3":
        return GNS_BF16X3
    if dt not in _DT:
        raise GnsError(3, f"unsupported dtype {dt}")
    return _DT[dt]


def _coeff_array(coeffs) -> "ctypes.Array":
    flat = []
    for row in coeffs:
        a, b, c = row
        flat += [float(a), float(b), float(c)]
    return (ctypes.c_double * max(len(flat), 1))(*flat), len(flat) // 3


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gram_workspace_bytes(compute_dtype, batch: int, rows: int, m: int) -> int:
    return int(lib().gns_gram_workspace_bytes(_dtype_code(compute_dtype), batch, rows, m))


def standard_workspace_bytes(compute_dtype, batch: int, rows: int, m: int) -> int:
    return int(lib().gns_standard_workspace_bytes(_dtype_code(compute_dtype), batch, rows, m))


def _tile_opts(tile) -> int:
    """None: size-based choice; 128 or 256: that edge for every product;
    "mixed": 256 for the rectangular and 128 for the symmetric products;
    "auto": measured per shape (GNS_OPT_TILE_AUTOTUNE)."""
    if tile is None:
        return 0
    if tile == "auto":
        return GNS_OPT_TILE_AUTOTUNE
    if tile == "mixed":
        return GNS_OPT_TILE_MIXED
    if tile == 128:
        return GNS_OPT_TILE_128
    if tile == 256:
        return GNS_OPT_TILE_256
    raise GnsError(10, f"tile must be None, 128, 256, 'mixed' or 'auto', got {tile}")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _device_tensor(name: str, t: torch.Tensor, device) -> None:
    """Raise unless t lives on the GPU (on `device` when given): the kernels
    take its address as a device pointer."""
    if t.device.type != "cuda":
        raise GnsError(1, f"{name} must be a GPU tensor, got device {t.device}")
    if device is not None and t.device != device:
        raise GnsError(1, f"{name} is on {t.device}, X on {device}")


def _prepare(X: torch.Tensor, row_idx: Optional[torch.Tensor], out: Optional[torch.Tensor]):
    """Shape, dtype, layout and device checks shared by the orthogonalisation
    calls (all before anything reaches the library).  Returns
    (Xb, row_idx, out, squeeze, k)."""
    squeeze = X.dim() == 2
    Xb = X.unsqueeze(0) if squeeze else X
    if Xb.dim() != 3 or not Xb.is_contiguous():
        raise GnsError(2, "X must be a contiguous [batch, n, m] tensor")
    B, n, m = Xb.shape
    if Xb.dtype not in _DT:
        raise GnsError(3, f"unsupported dtype {Xb.dtype}")
    k = 0
    if row_idx is not None:
        ri = row_idx.unsqueeze(0) if row_idx.dim() == 1 else row_idx
        if ri.dtype != torch.int64 or ri.dim() != 2 or not ri.is_contiguous() or ri.shape[0] != B:
            raise GnsError(6, "row_idx must be a contiguous int64 [batch, k] tensor")
        k = ri.shape[1]
        row_idx = ri
    if out is not None:
        ob = out.unsqueeze(0) if (squeeze and out.dim() == 2) else out
        if ob.shape != Xb.shape:
            raise GnsError(2, f"out has shape {tuple(out.shape)}, X has {tuple(X.shape)}")
        if ob.dtype != Xb.dtype:
            raise GnsError(3, f"out has dtype {out.dtype}, X has {X.dtype}")
        if not ob.is_contiguous():
            raise GnsError(2, "out must be contiguous")
        out = ob
    _device_tensor("X", Xb, None)
    if row_idx is not None:
        _device_tensor("row_idx", row_idx, Xb.device)
    if out is not None:
        _device_tensor("out", out, Xb.device)
    elif row_idx is not None:
        out = Xb.clone()
    else:
        out = torch.empty_like(Xb)
    return Xb, row_idx, out, squeeze, k


def gram_ns_batched(X: torch.Tensor, coeffs: Sequence, restarts: Sequence[int] = (2,), *,
                    row_idx: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    compute_dtype=None, naive_algebra: bool = False, square_fallback: bool = True,
                    tile=None, split_batch: bool = True, debug_checks: bool = False,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Gram Newton-Schulz of every matrix in X ([batch, n, m] or [n, m], on the
    GPU) via gns_gram_batched (``tile``: None, 128, 256, "mixed" or "auto").
    ``row_idx`` ([batch, k] int64, device) selects the rows to orthogonalise;
    the other rows of ``out`` are left as they are (``out`` defaults to a copy
    of X in that case).  ``out`` may be X itself.  ``debug_checks`` sets
    GNS_OPT_DEBUG_CHECKS (synchronous row-subset and Inf/NaN checks)."""
    Xb, row_idx, out, squeeze, k = _prepare(X, row_idx, out)
    B, n, m = Xb.shape
    cdt = _dtype_code(Xb.dtype if compute_dtype is None else compute_dtype)
    rows = k if row_idx is not None else n
    ws = _workspace(gram_workspace_bytes(cdt, B, rows, m), Xb.device, workspace)
    carr, T = _coeff_array(coeffs)
    rs = list(restarts)
    rarr = (ctypes.c_int * max(len(rs), 1))(*rs)
    _check(lib().gns_gram_batched(
        _ptr(Xb), _ptr(out), B, n, m, _dtype_code(Xb.dtype), cdt, carr, T, rarr, len(rs),
        _ptr(row_idx), k,
        (GNS_OPT_NAIVE_ALGEBRA if naive_algebra else 0)
        | (0 if square_fallback else GNS_OPT_NO_SQUARE_FALLBACK) | _tile_opts(tile)
        | (0 if split_batch else GNS_OPT_ONE_STREAM) | (GNS_OPT_DEBUG_CHECKS if debug_checks else 0),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out.squeeze(0) if squeeze else out


def standard_ns_batched(X: torch.Tensor, coeffs: Sequence, *,
                        row_idx: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, compute_dtype=None,
                        tile=None, split_batch: bool = True, debug_checks: bool = False,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Standard Newton-Schulz (Algorithm 1) via gns_standard_batched
    (``tile``: None, 128, 256, "mixed" or "auto")."""
    Xb, row_idx, out, squeeze, k = _prepare(X, row_idx, out)
    B, n, m = Xb.shape
    cdt = _dtype_code(Xb.dtype if compute_dtype is None else compute_dtype)
    rows = k if row_idx is not None else n
    ws = _workspace(standard_workspace_bytes(cdt, B, rows, m), Xb.device, workspace)
    carr, T = _coeff_array(coeffs)
    _check(lib().gns_standard_batched(
        _ptr(Xb), _ptr(out), B, n, m, _dtype_code(Xb.dtype), cdt, carr, T,
        _ptr(row_idx), k, _tile_opts(tile) | (0 if split_batch else GNS_OPT_ONE_STREAM)
        | (GNS_OPT_DEBUG_CHECKS if debug_checks else 0),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out.squeeze(0) if squeeze else out


NOALLOC_SCRATCH_BYTES = 128 << 20


def gram_ns_batched_noalloc(X: torch.Tensor, out: torch.Tensor, coeffs: Sequence,
                            restarts: Sequence[int] = (2,), *, row_idx: Optional[torch.Tensor] = None,
                            compute_dtype=None, naive_algebra: bool = False,
                            square_fallback: bool = True, tile=None, stream=None) -> torch.Tensor:
    """gns_gram_batched_noalloc: Gram Newton-Schulz with the library's own
    fixed device array (NOALLOC_SCRATCH_BYTES per GPU) as the workspace; the
    call itself allocates nothing.  ``out`` is required (allocate it
    beforehand); everything runs on ``stream``."""
    Xb, row_idx, outb, squeeze, k = _prepare(X, row_idx, out)
    B, n, m = Xb.shape
    cdt = _dtype_code(Xb.dtype if compute_dtype is None else compute_dtype)
    carr, T = _coeff_array(coeffs)
    rs = list(restarts)
    rarr = (ctypes.c_int * max(len(rs), 1))(*rs)
    _check(lib().gns_gram_batched_noalloc(
        _ptr(Xb), _ptr(outb), B, n, m, _dtype_code(Xb.dtype), cdt, carr, T, rarr, len(rs),
        _ptr(row_idx), k,
        (GNS_OPT_NAIVE_ALGEBRA if naive_algebra else 0)
        | (0 if square_fallback else GNS_OPT_NO_SQUARE_FALLBACK) | _tile_opts(tile),
        _stream(stream)))
    return out


def call_plan(standard: bool, X_ptr: int, out_ptr: int, batch: int, n: int, m: int, io_dtype,
              compute_dtype, coeffs: Sequence, restarts: Sequence[int] = (), *, row_idx_ptr: int = 0,
              k: int = 0, opts: int = 0) -> PlanInfo:
    """The host-side plan of a call (gns_call_plan).  Pointers are plain
    integers: they are compared and their alignment examined, never
    dereferenced, so this needs no GPU."""
    carr, T = _coeff_array(coeffs)
    rs = list(restarts)
    rarr = (ctypes.c_int * max(len(rs), 1))(*rs)
    info = PlanInfo()
    _check(lib().gns_call_plan(1 if standard else 0, X_ptr, out_ptr, batch, n, m, _dtype_code(io_dtype),
                               _dtype_code(compute_dtype), carr, T, rarr, len(rs), row_idx_ptr or None, k,
                               opts, ctypes.byref(info)))
    return info


def check_finite(A: torch.Tensor, row_idx: Optional[torch.Tensor] = None, stream=None) -> bool:
    """True when every element of A ([batch, rows, cols] or [rows, cols], on
    the GPU; only the rows in row_idx when given) is finite
    (gns_check_finite; synchronises)."""
    Ab = A.unsqueeze(0) if A.dim() == 2 else A
    if Ab.dim() != 3 or not Ab.is_contiguous():
        raise GnsError(2, "A must be a contiguous [batch, rows, cols] tensor")
    k = 0
    if row_idx is not None:
        row_idx = row_idx.unsqueeze(0) if row_idx.dim() == 1 else row_idx
        if row_idx.dtype != torch.int64 or not row_idx.is_contiguous() or row_idx.shape[0] != Ab.shape[0]:
            raise GnsError(6, "row_idx must be a contiguous int64 [batch, k] tensor")
        k = row_idx.shape[1]
        _device_tensor("row_idx", row_idx, Ab.device)
    _device_tensor("A", Ab, None)
    res = torch.empty(1, dtype=torch.int32, device=Ab.device)
    _check(lib().gns_check_finite(_ptr(Ab), _dtype_code(Ab.dtype), Ab.shape[0], Ab.shape[1], Ab.shape[2],
                                  _ptr(row_idx), k, _ptr(res), _stream(stream)))
    return int(res.item()) == 0


def tuned_tile(compute_dtype, io_dtype, batch: int, rows: int, m: int, standard: bool = False,
               symmetric: bool = False) -> int:
    """Tile edge kept by tile="auto" for this shape (rows = k with a row
    subset, else n) for the rectangular products, or with ``symmetric`` for
    the symmetric ones; 0 if the shape has not been tuned (gns_tuned_tile)."""
    sym = ctypes.c_int(0)
    rect = int(lib().gns_tuned_tile(1 if standard else 0, _dtype_code(compute_dtype),
                                    _dtype_code(io_dtype), batch, rows, m, ctypes.byref(sym)))
    return sym.value if symmetric else rect


def autotune_clear() -> None:
    """Forget every tuned shape (gns_autotune_clear)."""
    lib().gns_autotune_clear()


def check_row_idx(row_idx: torch.Tensor, n: int, stream=None) -> int:
    """0 = valid, 1 = index out of range, 2 = repeated index (synchronises)."""
    ri = row_idx.unsqueeze(0) if row_idx.dim() == 1 else row_idx
    res = torch.empty(1, dtype=torch.int32, device=ri.device)
    _check(lib().gns_check_row_idx(_ptr(ri), ri.shape[0], ri.shape[1], n, _ptr(res), _stream(stream)))
    return int(res.item())


def timing_enable(on: bool = True) -> None:
    lib().gns_timing_enable(1 if on else 0)


def timing_reset() -> None:
    lib().gns_timing_reset()


def timing_read():
    """List of (name, kernel, flops, bytes, ms) for every timed launch since the last reset."""
    L = lib()
    n = L.gns_timing_read(None, 0)
    recs = (LaunchRecord * max(n, 1))()
    n = L.gns_timing_read(recs, n)
    return [(r.name.decode(), r.kernel.decode(), r.flops, r.bytes, r.ms) for r in recs[:n]]


def select_rows_l1(M: torch.Tensor, k: int, *, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Indices of the k rows of largest l1 norm of every matrix in M
    ([batch, n, m] or [n, m]), ascending, via gns_select_rows_l1 (the Dion3
    selection step).  Returns an int64 [batch, k] (or [k]) device tensor."""
    squeeze = M.dim() == 2
    Mb = M.unsqueeze(0) if squeeze else M
    if Mb.dim() != 3 or not Mb.is_contiguous():
        raise GnsError(2, "M must be a contiguous [batch, n, m] tensor")
    B, n, m = Mb.shape
    if Mb.dtype not in _DT:
        raise GnsError(3, f"unsupported dtype {Mb.dtype}")
    _device_tensor("M", Mb, None)
    out = torch.empty(B, k, dtype=torch.int64, device=Mb.device)
    ws = _workspace(int(lib().gns_select_workspace_bytes(B, n)), Mb.device, workspace)
    _check(lib().gns_select_rows_l1(_ptr(Mb), B, n, m, _dtype_code(Mb.dtype), k, _ptr(out),
                                    _ptr(ws), ws.numel(), _stream(stream)))
    return out.squeeze(0) if squeeze else out


def select_count(n: int, fraction: float) -> int:
    """k = ceil(f n) rows for a fraction f in (0, 1] (Dion3 Algorithm 4), as
    the library computes it (gns_select_count)."""
    k = int(lib().gns_select_count(int(n), float(fraction)))
    if k == 0:
        raise ValueError("need n >= 1 and a fraction in (0, 1]")
    return k


def safety_scaled(coeffs: Sequence, s: float = 1.05) -> list:
    """Coefficients of p_t(x / s) for every step (gns_safety_scale; Dion3
    Appendix B.2.2: s = 1.02 usual, 1.05 conservative)."""
    carr, T = _coeff_array(coeffs)
    out = (ctypes.c_double * (3 * max(T, 1)))()
    code = lib().gns_safety_scale(carr, T, float(s), out)
    if code != 0:
        raise ValueError(f"safety_scaled: {_STATUS.get(code, code)}")
    return [(out[3 * t], out[3 * t + 1], out[3 * t + 2]) for t in range(T)]


def dion3_workspace_bytes(compute_dtype, batch: int, n: int, m: int, k: int) -> int:
    return int(lib().gns_dion3_workspace_bytes(_dtype_code(compute_dtype), batch, n, m, k))


def dion3_step(W: torch.Tensor, G: torch.Tensor, M: torch.Tensor, v: Optional[torch.Tensor],
               k: int, coeffs: Sequence, restarts: Sequence[int] = (2,), *, lr: float = 0.02,
               weight_decay: float = 0.0, mu: float = 0.95, beta2: float = 0.95, eps: float = 1e-8,
               normuon: bool = True, compute_dtype=torch.bfloat16, naive_algebra: bool = False,
               square_fallback: bool = True, tile=None, split_batch: bool = True,
               debug_checks: bool = False, row_idx: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One Dion3 update (Algorithm 4) of every matrix in W ([batch, n, m] or
    [n, m], fp32) via gns_dion3_step: W, M (fp32) and v (fp32 [batch, n], or
    None without NorMuon) are updated in place; G is fp32, bf16 or fp16.
    Returns the selected rows S (int64 [batch, k], ascending)."""
    squeeze = W.dim() == 2
    Wb, Gb, Mb = (t.unsqueeze(0) if squeeze else t for t in (W, G, M))
    vb = None if v is None else (v.unsqueeze(0) if v.dim() == 1 else v)
    for name, t in (("W", Wb), ("G", Gb), ("M", Mb)):
        if t.dim() != 3 or not t.is_contiguous():
            raise GnsError(2, f"{name} must be a contiguous [batch, n, m] tensor")
    if Wb.dtype != torch.float32 or Mb.dtype != torch.float32:
        raise GnsError(3, "W and M must be float32")
    B, n, m = Wb.shape
    if Gb.shape != Wb.shape or Mb.shape != Wb.shape:
        raise GnsError(2, "W, G and M must have the same shape")
    if vb is not None and (vb.dtype != torch.float32 or vb.shape != (B, n) or not vb.is_contiguous()):
        raise GnsError(2, "v must be a contiguous float32 [batch, n] tensor")
    if Gb.dtype not in _DT:
        raise GnsError(3, f"unsupported gradient dtype {Gb.dtype}")
    if row_idx is not None:
        row_idx = row_idx.unsqueeze(0) if row_idx.dim() == 1 else row_idx
        if row_idx.dtype != torch.int64 or tuple(row_idx.shape) != (B, k) or not row_idx.is_contiguous():
            raise GnsError(6, f"row_idx must be a contiguous int64 [{B}, {k}] tensor")
    for name, t in (("W", Wb), ("G", Gb), ("M", Mb), ("v", vb), ("row_idx", row_idx)):
        if t is not None:
            _device_tensor(name, t, Wb.device if name != "W" else None)
    cdt = _dtype_code(compute_dtype)
    if row_idx is None:
        row_idx = torch.empty(B, k, dtype=torch.int64, device=Wb.device)
    ws = _workspace(dion3_workspace_bytes(cdt, B, n, m, k), Wb.device, workspace)
    carr, T = _coeff_array(coeffs)
    rs = list(restarts)
    rarr = (ctypes.c_int * max(len(rs), 1))(*rs)
    _check(lib().gns_dion3_step(
        _ptr(Wb), _ptr(Gb), _ptr(Mb), _ptr(vb), B, n, m, _dtype_code(Gb.dtype), cdt, k, carr, T,
        rarr, len(rs), float(lr), float(weight_decay), float(mu), float(beta2), float(eps),
        1 if normuon else 0, _ptr(row_idx),
        (GNS_OPT_NAIVE_ALGEBRA if naive_algebra else 0)
        | (0 if square_fallback else GNS_OPT_NO_SQUARE_FALLBACK) | _tile_opts(tile)
        | (0 if split_batch else GNS_OPT_ONE_STREAM) | (GNS_OPT_DEBUG_CHECKS if debug_checks else 0),
        _ptr(ws), ws.numel(), _stream(stream)))
    return row_idx.squeeze(0) if squeeze else row_idx
