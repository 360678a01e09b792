"""CPU oracle of the decode-step K/V cache update.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU leg
may use it; the product path never does). numpy only; shares no code with the
HIP path.

The pages do not describe this step: it is the part of a decoder's decode
step that precedes the attention call, where the keys and values of the new
tokens join the int8 cache the attention reads (the pages' "Methodology"
step 3 keeps that data flow INT8 end to end). Readings, stated here and
matched by the device:
  * the cache has one per-tensor symmetric scale per tensor (s_k for K, s_v
    for V), fixed when the cache was filled, so earlier codes never change;
  * a new value x (float32) is coded as the inputs of the attention are:
    clip(rint(x / s), -127, 127), with x / s the IEEE float32 quotient
    (round to nearest, ties to even) and rint rounding ties to even; a NaN
    codes as 0 and +-inf as +-127;
  * T new tokens of each (batch, K/V head) go to cache rows pos .. pos+T-1;
    nothing else in the cache changes.
"""
from __future__ import annotations

import numpy as np


def quantise_f32(x, s: float) -> np.ndarray:
    """int8 codes of float32 x under scale s (float32): clip(rint(x / s), -127, 127)."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        y = np.rint(x / np.float32(s))            # float32 quotient, ties to even
    y = np.where(np.isnan(y), np.float32(0), np.clip(y, np.float32(-127), np.float32(127)))
    return y.astype(np.int8)


def kv_append(k_cache, v_cache, k_new, v_new, pos: int, s_k: float, s_v: float):
    """Caches int8 [B, Hkv, capacity, D] and new tokens float32 [B, Hkv, T, D]:
    returns copies of the caches with rows pos .. pos+T-1 replaced by the
    codes of the new tokens."""
    k_cache = np.array(k_cache, dtype=np.int8, copy=True)
    v_cache = np.array(v_cache, dtype=np.int8, copy=True)
    T = k_new.shape[2]
    if k_new.shape != v_new.shape or k_cache.shape != v_cache.shape:
        raise ValueError("shape mismatch")
    if k_new.shape[:2] != k_cache.shape[:2] or k_new.shape[3] != k_cache.shape[3]:
        raise ValueError("new tokens and cache disagree on B, heads or D")
    if pos < 0 or pos + T > k_cache.shape[2]:
        raise ValueError("rows pos .. pos+T-1 must lie inside the cache")
    k_cache[:, :, pos:pos + T] = quantise_f32(k_new, s_k)
    v_cache[:, :, pos:pos + T] = quantise_f32(v_new, s_v)
    return k_cache, v_cache
