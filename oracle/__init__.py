"""fp64 CPU oracle for K-interval attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, smoke() in
__graft_entry__.py and the benchmark's CPU-baseline leg, never by the HIP
library or its binding.  It shares no code with them.
"""
from .kia_oracle import (  # noqa: F401
    DETACH, EPS_SPAN, EXACT, EXP_BF16, EXP_FAMILY, EXP_FP8, FORMATS, FULL, FWM, FWM_UNTRUNC,
    GEOMETRY_FIELDS, LERP, MAX_ONLY, MIN_ONLY, MINMAX, NEAREST, P1, PROB_STE, WEIGHT_STE, Params,
    backward, calibrate, format_neighbours, forward, geometry, grid, head_backward, head_forward, head_geometry,
    reconstruct, round_to_format, row_backward, row_forward, row_geometry, row_scores,
)
