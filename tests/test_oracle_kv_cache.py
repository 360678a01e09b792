"""Pins for the decode-step cache update oracle (oracle/kv_cache.py).

The quantisation rule is pinned against exact rational arithmetic: with a
power-of-two scale the float32 quotient x / s is exact, so the code must be
the round-half-even of the exact rational value, clipped; ties, saturation,
infinities and NaN are checked one by one; and the update must touch
exactly the rows it names.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import kv_cache as KV


def _round_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


@pytest.mark.parametrize("s", [2.0 ** -7, 2.0 ** -3, 0.5, 4.0])
def test_power_of_two_scale_equals_exact_rounding(s):
    rng = np.random.default_rng(int(1 / s) if s < 1 else 7)
    x = (rng.standard_normal(20000) * 60 * s).astype(np.float32)
    got = KV.quantise_f32(x, s)
    want = [max(-127, min(127, _round_half_even(Fraction(float(v)) / Fraction(s)))) for v in x]
    assert got.tolist() == want


def test_ties_go_to_even_and_saturation():
    s = 2.0 ** -4
    halves = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 125.5], dtype=np.float64)
    x = (halves * s).astype(np.float32)
    assert KV.quantise_f32(x, s).tolist() == [0, 2, 2, 0, -2, -2, 126, -126, 126]
    big = np.array([127.4999, 127.5, 128.0, 1e30, -127.5, -1e30], dtype=np.float64) * s
    assert KV.quantise_f32(big.astype(np.float32), s).tolist() == [127, 127, 127, 127, -127, -127]


def test_non_finite_values():
    x = np.array([np.inf, -np.inf, np.nan, -np.nan], dtype=np.float32)
    assert KV.quantise_f32(x, 0.1).tolist() == [127, -127, 0, 0]


def test_codes_match_the_inputs_rule_on_the_decode_draws():
    """Same rule as the inputs of the attention: codes of float32 N(0,1) draws
    with scale float32(absmax / 127) stay within [-127, 127] and hit both ends."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 8, 16)).astype(np.float32)
    s = float(np.float32(np.abs(x).max() / 127.0))
    q = KV.quantise_f32(x, s)
    assert q.min() >= -127 and q.max() <= 127
    assert np.abs(q).max() == 127                 # the absmax value codes to +-127
    # dequantised codes lie within half a step of the values
    assert (np.abs(q.astype(np.float64) * s - x) <= 0.5 * s * (1 + 1e-6)).all()


def test_append_touches_exactly_its_rows():
    rng = np.random.default_rng(4)
    kc = rng.integers(-127, 128, (2, 3, 20, 16)).astype(np.int8)
    vc = rng.integers(-127, 128, (2, 3, 20, 16)).astype(np.int8)
    kn = rng.standard_normal((2, 3, 5, 16)).astype(np.float32)
    vn = rng.standard_normal((2, 3, 5, 16)).astype(np.float32)
    k2, v2 = KV.kv_append(kc, vc, kn, vn, 7, 0.02, 0.03)
    assert np.array_equal(k2[:, :, :7], kc[:, :, :7]) and np.array_equal(k2[:, :, 12:], kc[:, :, 12:])
    assert np.array_equal(v2[:, :, :7], vc[:, :, :7]) and np.array_equal(v2[:, :, 12:], vc[:, :, 12:])
    assert np.array_equal(k2[:, :, 7:12], KV.quantise_f32(kn, 0.02))
    assert np.array_equal(v2[:, :, 7:12], KV.quantise_f32(vn, 0.03))
    with pytest.raises(ValueError):
        KV.kv_append(kc, vc, kn, vn, 16, 0.02, 0.03)
    with pytest.raises(ValueError):
        KV.kv_append(kc, vc, kn, vn, -1, 0.02, 0.03)
