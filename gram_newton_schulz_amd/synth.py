"""Seeded synthetic inputs shared by the oracle-side and the GPU-side checks.

This module only draws random numbers and stores them in the workload's
dtype: it contains none of the orthogonalisation arithmetic.  Every matrix is
drawn in float64 from ``numpy.random.default_rng([seed, index])`` (so any
single batch member can be regenerated on its own), normalised in float64
where the workload says so, and rounded once to the storage dtype.  That
rounded tensor is *the* input: the oracle upcasts the same bits.

Workloads (dense-MLP and MoE-expert weight shapes):

1. 1 x 64x256 fp32, i.i.d. N(0,1), unit Frobenius norm.
2. 16 x 1024x4096 bf16, U diag(s) V^T with Haar U, V and s log-uniform in
   [1e-4, 1], unit Frobenius norm.
3. 8 x 4096x16384 bf16, i.i.d. N(0, 0.02^2), unit Frobenius norm
   (dense-LLM MLP momentum, aspect ratio 4).
4. 64 x 2048x7168 bf16, Student-t (nu = 3), unit norm per matrix
   (stack of MoE expert momenta, aspect ratio 3.5).
5. 8 x 4096x16384 bf16, i.i.d. N(0,1) (not normalised), plus per matrix a
   seeded random set of 1024 distinct rows (fraction 1/4).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

# Coefficient schedules printed in the sources.
#: Five iterations of the fixed Muon quintic (a, b, c) = (3.4445, -4.7750,
#: 2.0315), as used by "Scaling Muon for Diffusion Transformers" (App. D.3).
NS5_MUON = [(3.4445, -4.7750, 2.0315)] * 5
#: (15/8, -10/8, 3/8): the convergent quintic of the stability study in
#: Dion3 Appendix B.1.1 (h(y) = 15/8 - 10/8 y + 3/8 y^2, p(1) = 1).
CONVERGENT = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)


@dataclass(frozen=True)
class Workload:
    cfg: int
    batch: int
    n: int
    m: int
    dtype: torch.dtype
    dist: str
    normalize: bool
    k: Optional[int] = None     # selected rows per matrix (fractional-row mode)

    @property
    def seed(self) -> int:
        return 1000 + self.cfg


WORKLOADS = {
    1: Workload(1, 1, 64, 256, torch.float32, "normal", True),
    2: Workload(2, 16, 1024, 4096, torch.bfloat16, "logspec", True),
    3: Workload(3, 8, 4096, 16384, torch.bfloat16, "normal", True),
    4: Workload(4, 64, 2048, 7168, torch.bfloat16, "student_t3", True),
    5: Workload(5, 8, 4096, 16384, torch.bfloat16, "normal", False, k=1024),
}


def _rng(seed: int, index: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(index)])


def _haar(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """Orthonormal columns: QR of a Gaussian with the column signs fixed by
    sign(diag(R)), which makes the distribution Haar."""
    g = rng.standard_normal((rows, cols))
    q, r = np.linalg.qr(g)
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d


def draw_f64(dist: str, n: int, m: int, seed: int, index: int,
             spectrum=(-4.0, 0.0)) -> np.ndarray:
    """One n x m float64 matrix from the named distribution."""
    rng = _rng(seed, index)
    if dist == "normal":
        return rng.standard_normal((n, m))
    if dist == "normal002":
        return 0.02 * rng.standard_normal((n, m))
    if dist == "student_t3":
        return rng.standard_t(3.0, size=(n, m))
    if dist in ("logspec", "expspec"):
        r = min(n, m)
        U = _haar(rng, n, r)
        V = _haar(rng, m, r)
        lo, hi = spectrum
        if dist == "logspec":
            s = 10.0 ** rng.uniform(lo, hi, size=r)
        else:  # exponentially decaying, from 10^hi down to 10^lo
            s = 10.0 ** np.linspace(hi, lo, r)
        return (U * s) @ V.T
    raise ValueError(dist)


def to_storage(x64: np.ndarray, dtype: torch.dtype, normalize: bool) -> torch.Tensor:
    """Optionally scale to unit Frobenius norm (float64), then round once."""
    if normalize:
        flat = x64.ravel()
        x64 = x64 / np.sqrt(np.dot(flat, flat))
    return torch.from_numpy(np.ascontiguousarray(x64)).to(dtype)


def matrix(n: int, m: int, *, seed: int, index: int = 0, dist: str = "normal",
           dtype: torch.dtype = torch.bfloat16, normalize: bool = True,
           spectrum=(-4.0, 0.0)) -> torch.Tensor:
    return to_storage(draw_f64(dist, n, m, seed, index, spectrum), dtype, normalize)


def _workers(count: int) -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(count, cores, 16))


def _fill(out: torch.Tensor, make) -> torch.Tensor:
    """out[b] = make(b) for every b, on a thread pool (numpy's generators
    release the GIL); each member has its own seed, so the result does not
    depend on the pool size."""
    def one(b):
        out[b] = make(b)
    workers = _workers(out.shape[0])
    # one BLAS thread per worker: the pool already uses every core, and
    # nested BLAS threads oversubscribe them (16 Haar-spectrum matrices of
    # 1024 x 4096: 112 s with 8 x 8 threads, a few seconds with 8 x 1)
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas") if workers > 1 else None
    except ImportError:  # pragma: no cover
        limit = None
    try:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(out.shape[0])))
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return out


def batch(count: int, n: int, m: int, *, seed: int, dist: str = "normal",
          dtype: torch.dtype = torch.bfloat16, normalize: bool = True,
          spectrum=(-4.0, 0.0), first: int = 0) -> torch.Tensor:
    out = torch.empty((count, n, m), dtype=dtype)
    return _fill(out, lambda b: matrix(n, m, seed=seed, index=first + b, dist=dist, dtype=dtype,
                                       normalize=normalize, spectrum=spectrum))


def row_subset(n: int, k: int, *, seed: int, index: int) -> np.ndarray:
    """k distinct row indices in [0, n), in random order (int64)."""
    rng = _rng(seed + 500, index)
    return rng.choice(n, size=k, replace=False).astype(np.int64)


def workload_matrix(cfg: int, index: int) -> torch.Tensor:
    w = WORKLOADS[cfg]
    dist = {"normal": "normal002" if cfg == 3 else "normal"}.get(w.dist, w.dist)
    return matrix(w.n, w.m, seed=w.seed, index=index, dist=dist, dtype=w.dtype,
                  normalize=w.normalize)


def workload_batch(cfg: int, count: Optional[int] = None) -> torch.Tensor:
    w = WORKLOADS[cfg]
    count = w.batch if count is None else count
    out = torch.empty((count, w.n, w.m), dtype=w.dtype)
    return _fill(out, lambda b: workload_matrix(cfg, b))


def workload_rows(cfg: int, count: Optional[int] = None) -> Optional[torch.Tensor]:
    w = WORKLOADS[cfg]
    if w.k is None:
        return None
    count = w.batch if count is None else count
    return torch.from_numpy(np.stack([row_subset(w.n, w.k, seed=w.seed, index=b)
                                      for b in range(count)]))


def as_f64(t: torch.Tensor) -> np.ndarray:
    """The exact values of a stored tensor as float64 (bf16/fp16/fp32 all
    embed exactly in float64)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def dion3_state(count: int, n: int, m: int, *, seed: int, grad_dtype: torch.dtype = torch.bfloat16):
    """Optimizer state for one Dion3 update of `count` n x m weights:
    W ~ N(0, 0.02^2) fp32 weights, G ~ N(0, 1) gradient in grad_dtype,
    M ~ N(0, 0.5^2) fp32 momentum and v ~ U[0.5, 1.5] / m fp32 row second
    moments (the size of a mean square of an orthogonalised row).  Each
    member b is drawn from default_rng([seed, b]) in float64 and rounded once.
    Returns (W, G, M, v) on the CPU."""
    W = torch.empty((count, n, m), dtype=torch.float32)
    G = torch.empty((count, n, m), dtype=grad_dtype)
    M = torch.empty((count, n, m), dtype=torch.float32)
    v = torch.empty((count, n), dtype=torch.float32)

    def one(b):
        rng = _rng(seed, b)
        W[b] = torch.from_numpy(0.02 * rng.standard_normal((n, m)))
        G[b] = torch.from_numpy(rng.standard_normal((n, m))).to(grad_dtype)
        M[b] = torch.from_numpy(0.5 * rng.standard_normal((n, m)))
        v[b] = torch.from_numpy(rng.uniform(0.5, 1.5, size=n) / m)
    with ThreadPoolExecutor(_workers(count)) as ex:
        list(ex.map(one, range(count)))
    return W, G, M, v
