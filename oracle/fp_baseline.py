"""CPU oracle of the floating-point softmax the integer pipeline replaces.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU leg
may use it; the product path never does). numpy only; shares no code with the
HIP path.

Source: the IntAttention digest pages (euno.news, arXiv 2511.21513v1),
section "Methodology", step 1 "Problem identification": in an INT8 Transformer
the products are integer, but the softmax runs in FP16/FP32; the integer
scores are converted to floating point, exponentiated, normalised and
converted back to integers. The pages fix none of the details. Readings
(stated, and matched by the comparator kernel):
  * dequantise a score with alpha = s_q * s_k / sqrt(D), rounded once to
    float32, so y = float32(s) * alpha in float32;
  * softmax over the allowed keys with the row max subtracted, in float32;
    the exponential is exp2((y - m) * log2(e)) as the device computes it;
  * requantise p to the uint8 code rint(255 * p) (ties to even) clamped to
    255, computed as rint(e * (255 / sum)); keys that are not allowed get 0.
A quantised code is decided by floating point here, so this oracle takes the
decision in the kernel's precision (float32). Its exponential and summation
order are numpy's, so a code can still differ by one from the device's where
255 * p lies within float32 rounding of a half-integer; the tests allow
exactly that (|difference| <= 1, rarely). Pinned in
tests/test_oracle_stages.py against scipy.special.softmax in float64.
"""
from __future__ import annotations

import math

import numpy as np

from .intattn_oracle import allowed_mask


def dequant_alpha(D: int, s_q: float, s_k: float) -> np.float32:
    """alpha = s_q * s_k / sqrt(D) in binary64 from the float32 scales, rounded to float32."""
    return np.float32(float(np.float32(s_q)) * float(np.float32(s_k)) / math.sqrt(D))


def fp_softmax_codes(S, alpha, causal: bool):
    """uint8 codes [Sq, Skv] of one head's int32 scores S (float32 steps)."""
    S = np.asarray(S)
    Sq, Skv = S.shape
    allow = allowed_mask(Sq, Skv, causal)
    a = np.float32(alpha)
    y = np.where(allow, S.astype(np.float32) * a, np.float32(-np.inf)).astype(np.float32)
    m = y.max(axis=1, keepdims=True)
    e = np.where(allow, np.exp2((y - m) * np.float32(math.log2(math.e))), np.float32(0)).astype(np.float32)
    total = e.sum(axis=1, keepdims=True, dtype=np.float32)
    scale = (np.float32(255.0) / total).astype(np.float32)
    codes = np.minimum(np.rint(e * scale), np.float32(255.0))
    return codes.astype(np.uint8)
