"""fp64 CPU oracle for Gram / standard Newton-Schulz.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from .newton_schulz import (  # noqa: F401
    EPS, frobenius_normalize, standard_ns, gram_ns, gram_ns_trace, theorem2_q,
    composed_poly, spectral_map, polar, dion3_select, dion3_rows, dion3_step, normuon_rows,
    flops_standard, flops_gram, restart_model, restart_sweep,
)
