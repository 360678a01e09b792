"""Pins for the oracle's host-side parameters: the exp table, the bin multiplier,
the clip point and the requantisation multiplier.

The pages (IntAttention digest, "Methodology" step 2) fix only that the table
has 32 entries and approximates exp over the clipped range. The values are
pinned here against mathematics, not against the oracle's own formula:
high-precision Decimal exponentials, exact rational bounds, and a parameter
set worked out by hand.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import intattn_oracle as O


CLIPS = [O.DEFAULT_CLIP, 1.0, 2.5, 4.0, 8.0, 12.0, 0.0605]


def _dec_exp(x: Decimal) -> Decimal:
    getcontext().prec = 50
    return x.exp()


@pytest.mark.parametrize("clip", CLIPS)
def test_lut_endpoints_and_monotone(clip):
    lut = O.build_lut(clip)
    assert len(lut) == 32
    assert lut[0] == 32768                       # exp(0) in Q15
    assert lut[31] == 0                          # the sparse tail slot
    assert all(0 <= e <= 65535 for e in lut)
    # non-increasing; strictly decreasing whenever adjacent exact values are
    # more than one unit apart (then rounding cannot merge them)
    for k in range(30):
        assert lut[k] >= lut[k + 1]
        gap = 32768 * (math.exp(-k * clip / 31) - math.exp(-(k + 1) * clip / 31))
        if gap > 1.0 + 1e-6:
            assert lut[k] > lut[k + 1]


@pytest.mark.parametrize("clip", CLIPS)
def test_lut_matches_high_precision_exp(clip):
    """|LUT[k] - 2^15 exp(-k*c/31)| <= 1/2 with c the float32 clip, in 50-digit decimal."""
    getcontext().prec = 50
    c = Decimal(float(np.float32(clip)))          # exact value of the float32
    lut = O.build_lut(clip)
    for k in range(31):
        ref = Decimal(32768) * _dec_exp(-(Decimal(k) * c / Decimal(31)))
        assert abs(Decimal(lut[k]) - ref) <= Decimal("0.5") + Decimal("1e-9"), (k, lut[k], ref)


def test_default_clip_makes_tail_provably_zero():
    """A key past the clip has softmax weight < e^-c <= 1/510 < half a uint8 step of 255."""
    c = O.DEFAULT_CLIP
    assert math.exp(-c) <= 1.0 / 510.0 * (1 + 1e-6)
    assert 255.0 * math.exp(-c) < 0.5 + 1e-6


def test_hand_worked_parameters():
    """A parameter set derived by hand.

    s_q = s_k = 2^-6, D = 64  ->  alpha = 2^-12 / 8 = 2^-15.
    clip = 31 * 2^-9 (exact in float32)  ->  delta = 2^-9, mu = 2^-6.
    M = 2^-6 * 2^24 = 2^18.  X_clip = ceil(61 * 2^23 / 2^18) = 61 * 32 = 1952.
    s_o = s_v / 255 is not exact in float32; with s_v = 255 * 2^-10 and
    s_o = 2^-10: mu_o = 1 = 0.5 * 2^1  ->  M_o = 2^30, sh_o = 31 - 1 = 30.
    """
    p = O.derive_params(64, 2 ** -6, 2 ** -6, 255 * 2 ** -10, 2 ** -10, 31 * 2 ** -9)
    assert p.alpha == 2 ** -15
    assert p.delta == 2 ** -9
    assert p.mu == 2 ** -6
    assert p.idx_mul == 2 ** 18
    assert p.idx_shift == 24
    assert p.x_clip == 1952
    assert p.req_mul == 2 ** 30
    assert p.req_shift == 30


def test_hand_worked_parameters_large_multiplier():
    """mu >= 1/2, derived by hand.

    s_q = s_k = 2^-2, D = 64 -> alpha = 2^-4 / 8 = 2^-7; clip = 31 * 2^-9
    -> delta = 2^-9, mu = 2^2 = 0.5 * 2^3 -> sh = 23 - 3 = 20,
    M = 2^2 * 2^20 = 2^22. X_clip = ceil(61 * 2^19 / 2^22) = ceil(7.625) = 8:
    x = 7 gives (7 * 2^22 + 2^19) >> 20 = 28, x = 8 gives 32 (slot 31).
    """
    p = O.derive_params(64, 2 ** -2, 2 ** -2, 255 * 2 ** -10, 2 ** -10, 31 * 2 ** -9)
    assert p.mu == 4.0
    assert (p.idx_mul, p.idx_shift, p.x_clip) == (2 ** 22, 20, 8)
    assert list(O.slot_index(np.arange(10), p)) == [0, 4, 8, 12, 16, 20, 24, 28, 31, 31]


def test_hand_worked_parameters_small_multiplier():
    """mu < 2^-16, derived by hand.

    s_q = s_k = 2^-13, D = 64 -> alpha = 2^-26 / 8 = 2^-29; clip = 31 * 2^-9
    -> mu = 2^-20 -> sh = 24, M = 2^4. X_clip = ceil(61 * 2^23 / 2^4) =
    61 * 2^19 = 31981568 (beyond any int8 score gap: no key is clipped);
    slot(x) = (16 x + 2^23) >> 24 = round(x / 2^20).
    """
    p = O.derive_params(64, 2 ** -13, 2 ** -13, 255 * 2 ** -10, 2 ** -10, 31 * 2 ** -9)
    assert p.mu == 2.0 ** -20
    assert (p.idx_mul, p.idx_shift, p.x_clip) == (16, 24, 61 * 2 ** 19)
    x = np.array([0, 2 ** 19 - 1, 2 ** 19, 3 * 2 ** 19, 2 * 64 * 127 * 127])
    assert list(O.slot_index(x, p)) == [0, 0, 1, 2, 2]


SCALE_SETS = [
    # (D, s_q, s_k, s_v, s_o, clip)
    (64, 0.0307, 0.0317, 0.0354, 0.0101, O.DEFAULT_CLIP),   # tiny-like
    (64, 0.3375, 0.2547, 0.2601, 0.1660, O.DEFAULT_CLIP),   # BERT with outliers
    (128, 0.8041, 0.6373, 0.4146, 0.0457, O.DEFAULT_CLIP),  # heavy-tailed prefill
    (128, 0.0326, 0.0471, 0.0473, 0.00073, O.DEFAULT_CLIP), # decode
    (64, 0.01, 0.01, 0.02, 0.02, 3.0),
    (128, 0.05, 0.02, 0.001, 0.5, 6.0),
    # from mu = 1/2 on (large scales: a gap of one score unit moves half a
    # bin or more) and below mu = 2^-16 (small scales)
    (64, 0.7, 0.9, 0.05, 0.05, O.DEFAULT_CLIP),             # mu ~ 0.39
    (64, 1.0, 1.0, 0.05, 0.05, O.DEFAULT_CLIP),              # mu ~ 0.62
    (128, 3.0, 2.5, 0.05, 0.05, O.DEFAULT_CLIP),             # mu ~ 3.3
    (64, 40.0, 50.0, 0.05, 0.05, O.DEFAULT_CLIP),            # mu ~ 1.2e3
    (64, 100.0, 150.0, 0.05, 0.05, O.DEFAULT_CLIP),          # mu ~ 9.3e3
    (64, 0.002, 0.003, 0.05, 0.05, O.DEFAULT_CLIP),          # mu ~ 3.7e-6 (below 2^-16)
    (128, 4e-4, 4e-4, 0.05, 0.05, O.DEFAULT_CLIP),           # mu ~ 7.0e-8 (near 2^-24)
]


@pytest.mark.parametrize("D,sq,sk,sv,so,clip", SCALE_SETS)
def test_multiplier_rounding_is_exact(D, sq, sk, sv, so, clip):
    p = O.derive_params(D, sq, sk, sv, so, clip)
    f = lambda x: Fraction(float(np.float32(x)))
    # mu to within a few ulp of the exact rational value
    exact_alpha_sq = (f(sq) * f(sk)) ** 2 / D          # alpha^2 exactly (sqrt irrational)
    assert abs(Fraction(p.alpha) ** 2 - exact_alpha_sq) <= exact_alpha_sq * Fraction(1, 2 ** 49)
    mu = Fraction(p.mu)
    sh = p.idx_shift
    # M is the nearest integer to mu * 2^sh: sh = 24 below mu = 1/2, and
    # from there the multiplier is kept at 22 or 23 significant bits
    assert abs(p.idx_mul - mu * 2 ** sh) <= Fraction(1, 2)
    if mu < Fraction(1, 2):
        assert sh == 24 and 1 <= p.idx_mul <= 2 ** 23
    else:
        assert 9 <= sh <= 23 and 2 ** 22 <= p.idx_mul <= 2 ** 23
    # clip point: smallest x with slot 31
    assert (p.x_clip * p.idx_mul + 2 ** (sh - 1)) >> sh >= 31
    assert p.x_clip >= 1 and ((p.x_clip - 1) * p.idx_mul + 2 ** (sh - 1)) >> sh <= 30
    if mu <= 1:     # a score unit moves at most one bin: every slot is reached
        assert ((p.x_clip - 1) * p.idx_mul + 2 ** (sh - 1)) >> sh == 30
    # requantisation multiplier normalised and nearest
    assert 2 ** 30 <= p.req_mul < 2 ** 31
    mu_o = Fraction(p.mu_o)
    assert abs(Fraction(p.req_mul, 2 ** p.req_shift) - mu_o) <= Fraction(1, 2 ** (p.req_shift + 1))
    exact_mu_o = f(sv) / (255 * f(so))
    assert abs(mu_o - exact_mu_o) <= exact_mu_o * Fraction(1, 2 ** 51)


def test_range_refusals():
    with pytest.raises(O.OracleRangeError):
        O.derive_params(64, 1e-4, 1e-4, 1.0, 1.0, 6.0)      # mu ~ 2^-27 < 2^-24
    with pytest.raises(O.OracleRangeError):
        O.derive_params(64, 200.0, 300.0, 1.0, 1.0, 6.0)    # mu ~ 3.9e4 >= 2^14
    # the edges of [2^-24, 2^14) themselves, exactly: s_q = s_k = s, D = 64,
    # clip = 31 * 2^-9 (delta = 2^-9), so mu = s^2 / 8 / 2^-9 = 64 s^2
    p = O.derive_params(64, 2.0 ** -15, 2.0 ** -15, 1.0, 1.0, 31 * 2 ** -9)
    assert p.mu == 2.0 ** -24 and p.idx_mul == 1 and p.idx_shift == 24
    with pytest.raises(O.OracleRangeError):
        O.derive_params(64, 2.0 ** 4, 2.0 ** 4, 1.0, 1.0, 31 * 2 ** -9)   # mu = 2^14
    p = O.derive_params(64, 15.9, 15.9, 1.0, 1.0, 31 * 2 ** -9)          # mu just below 2^14
    assert p.idx_shift == 9 and 2 ** 22 <= p.idx_mul <= 2 ** 23
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(O.OracleRangeError):
            O.derive_params(64, bad, 0.01, 0.01, 0.01, 6.0)
        with pytest.raises(O.OracleRangeError):
            O.derive_params(64, 0.01, 0.01, 0.01, 0.01, bad)
    with pytest.raises(O.OracleRangeError):
        O.derive_params(64, 0.05, 0.05, 1e-12, 1.0, 6.0)    # output shift > 63
    with pytest.raises(O.OracleRangeError):
        O.derive_params(0, 0.05, 0.05, 0.05, 0.05, 6.0)


@pytest.mark.parametrize("D,sq,sk,sv,so,clip", SCALE_SETS)
def test_slot_index_exhaustive(D, sq, sk, sv, so, clip):
    """Every relative score from 0 to past the clip point.

    * slot(0) = 0; slots are monotone and never skip a slot;
    * slot is the nearest bin under the encoded multiplier:
      |slot * 2^sh - x * M| <= 2^(sh-1) for x below the clip point;
    * the encoded multiplier tracks the exact one: the slot is within
      1/2 + x*|mu - M/2^sh| of x*mu;
    * everything from the clip point on is slot 31.
    Relative scores stop at 2*D*127^2 (no int8 product reaches further), so
    for tiny multipliers the sweep ends there instead of at the clip point.
    """
    p = O.derive_params(D, sq, sk, sv, so, clip)
    sh = p.idx_shift
    x = np.arange(0, min(p.x_clip + 3, 2 * D * 127 * 127 + 1), dtype=np.int64)
    s = O.slot_index(x, p)
    assert s[0] == 0
    d = np.diff(s)
    assert (d >= 0).all()
    if p.mu <= 1:   # at most one bin per score unit: no slot is skipped
        assert ((d == 0) | (d == 1)).all()
    assert (s[p.x_clip:] == 31).all()
    assert (s[:p.x_clip] <= 30).all()
    below = x[:p.x_clip]
    sb = s[:p.x_clip]
    assert (np.abs(sb * (1 << sh) - below * p.idx_mul) <= (1 << (sh - 1))).all()
    mu = Fraction(p.mu)
    err_m = abs(mu - Fraction(p.idx_mul, 1 << sh))
    worst = max(abs(Fraction(int(xx)) * mu - int(ss)) - int(xx) * err_m
                for xx, ss in zip(below[:: max(1, len(below) // 4000)], sb[:: max(1, len(below) // 4000)]))
    assert worst <= Fraction(1, 2)
