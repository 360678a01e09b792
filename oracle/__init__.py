"""CPU oracle for the fully-integer attention forward pass (test infrastructure only).

Importable only by the test suite, the smoke check and the benchmark's
CPU-baseline leg. It shares no code with the HIP path.
"""
from .intattn_oracle import (  # noqa: F401
    DEFAULT_CLIP, IDX_SHIFT, LUT_SIZE, OracleRangeError, Params, allowed_mask,
    build_lut, derive_params, forward, head_forward, index_softmax, normalise,
    pv_requant, qk_scores, reciprocal, requantise, slot_index,
)
from .fp_baseline import dequant_alpha, fp_softmax_codes  # noqa: F401
from .kv_cache import kv_append, quantise_f32  # noqa: F401
