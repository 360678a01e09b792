"""CPU oracle for the fully-integer attention forward pass (test infrastructure only).

Importable only by the test suite, the smoke check and the benchmark's
CPU-baseline leg. It shares no code with the HIP path.
"""
from .intattn_oracle import (  # noqa: F401
    DEFAULT_CLIP, IDX_SHIFT, LUT_SIZE, OracleRangeError, Params, allowed_mask,
    build_lut, derive_params, forward, head_forward, normalise, reciprocal,
    requantise, slot_index,
)
