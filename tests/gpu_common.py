"""Shared helpers of the GPU tests: run the HIP path through the C ABI on
seeded inputs and compare with the fp64 oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle
from gram_newton_schulz_amd import synth

NS5 = synth.NS5_MUON
TOL_HALF = 3e-2   # relative Frobenius error, bf16 / fp16 paths
TOL_F32 = 1e-4    # fp32 path


def gpu_available() -> bool:
    return torch.cuda.is_available()


def need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")
    import gram_newton_schulz_amd as gns
    if not os.path.exists(gns.LIB_PATH):
        raise RuntimeError("libgns.so not built: the HIP path is required where a GPU is present")
    return gns


def say(*a):
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print(*a, file=sys.stderr, flush=True)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    d = np.linalg.norm(got - ref)
    r = np.linalg.norm(ref)
    return float(d / r) if r > 0 else float(d)


def per_matrix_rel(got: np.ndarray, ref: np.ndarray) -> list:
    return [rel_err(got[b], ref[b]) for b in range(got.shape[0])]


def oracle_gram(X64: np.ndarray, coeffs=NS5, restarts=(2,), algebra="stabilized"):
    return oracle.gram_ns(X64, coeffs, restarts=restarts, algebra=algebra)


def oracle_standard(X64: np.ndarray, coeffs=NS5):
    return oracle.standard_ns(X64, coeffs)
