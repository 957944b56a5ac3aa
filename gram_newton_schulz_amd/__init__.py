"""MI355X-native (gfx950) Gram Newton-Schulz orthogonalisation.

The computation lives in the HIP library libgns.so behind the C ABI of
include/gns.h; this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    GnsError, gram_ns_batched, standard_ns_batched, gram_workspace_bytes,
    standard_workspace_bytes, check_row_idx, timing_enable, timing_reset, timing_read,
    select_rows_l1, select_count, safety_scaled, dion3_step, dion3_workspace_bytes,
    tuned_tile, autotune_clear, call_plan, check_finite, PlanInfo, lib, LIB_PATH, EXPORTS,
    GNS_F32, GNS_BF16, GNS_F16, GNS_BF16X3, GNS_OPT_DEBUG_CHECKS,
)
