"""Pins for the oracle's variants: finer exp tables (64 and 128 entries),
uint8 table entries, grouped K/V heads and uint16 probabilities.

The pages' "Limitations & Future Work" (lookup-table granularity) say the
32-entry table trades accuracy for memory and that very large heads may need
finer tables; the variant keeps every step of the method and only refines the
bins (delta = clip/(N-1)). Pinned here against mathematics, not against the
oracle's own formulas: high-precision exponentials, a hand-worked parameter
set, exhaustive slot checks, the brute-force twin (nearest bin by exact
rationals), the float64 softmax error bound, and, for grouped heads,
numpy's repeat of the K/V heads.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import intattn_oracle as O
from oracle import scalar_twin as T
from integer_only_quantized_amd import workloads as W

FINE = [64, 128]
CLIPS = [O.DEFAULT_CLIP, 1.0, 4.0, 12.0]


@pytest.mark.parametrize("n", FINE)
@pytest.mark.parametrize("clip", CLIPS)
def test_fine_lut_matches_high_precision_exp(n, clip):
    """|LUT[k] - 2^15 exp(-k c/(N-1))| <= 1/2 in 50-digit decimal; endpoints; monotone."""
    getcontext().prec = 50
    lut = O.build_lut(clip, n)
    assert len(lut) == n and lut[0] == 32768 and lut[-1] == 0
    c = Decimal(float(np.float32(clip)))
    for k in range(n - 1):
        ref = Decimal(32768) * (-(Decimal(k) * c / Decimal(n - 1))).exp()
        assert abs(Decimal(lut[k]) - ref) <= Decimal("0.5") + Decimal("1e-9"), (n, k)
    assert all(lut[k] >= lut[k + 1] for k in range(n - 1))


def test_lut_size_refused_outside_the_variants():
    for bad in (0, 16, 31, 33, 96, 256):
        with pytest.raises(O.OracleRangeError):
            O.build_lut(O.DEFAULT_CLIP, bad)
        with pytest.raises(O.OracleRangeError):
            O.derive_params(64, 0.05, 0.05, 0.05, 0.05, O.DEFAULT_CLIP, bad)


@pytest.mark.parametrize("n,x_clip", [(64, 4000), (128, 8096)])
def test_hand_worked_fine_parameters(n, x_clip):
    """s_q = s_k = 2^-6, D = 64 -> alpha = 2^-15; clip = (N-1) * 2^-9 (exact in
    float32) -> delta = 2^-9, mu = 2^-6, M = 2^18; the clip point is the
    smallest x with x * 2^18 >= (2N - 3) * 2^23, i.e. (2N - 3) * 32."""
    p = O.derive_params(64, 2 ** -6, 2 ** -6, 255 * 2 ** -10, 2 ** -10, (n - 1) * 2 ** -9, n)
    assert p.lut_size == n
    assert p.delta == 2 ** -9 and p.mu == 2 ** -6 and p.idx_mul == 2 ** 18
    assert p.x_clip == x_clip == (2 * n - 3) * 32
    assert p.req_mul == 2 ** 30 and p.req_shift == 30


SCALE_SETS = [
    (64, 0.0307, 0.0317, 0.0354, 0.0101, O.DEFAULT_CLIP),
    (64, 0.3375, 0.2547, 0.2601, 0.1660, O.DEFAULT_CLIP),
    (128, 0.8041, 0.6373, 0.4146, 0.0457, O.DEFAULT_CLIP),
    (128, 0.05, 0.02, 0.001, 0.5, 6.0),
]


@pytest.mark.parametrize("n", FINE)
@pytest.mark.parametrize("D,sq,sk,sv,so,clip", SCALE_SETS)
def test_fine_slot_index_exhaustive(n, D, sq, sk, sv, so, clip):
    """slot(0) = 0, monotone (no skipped slot while mu <= 1), nearest bin
    under the encoded multiplier below the clip point, slot N-1 from the clip
    point on; the multiplier is the nearest integer to mu 2^sh with
    mu = alpha (N-1) / clip (sh = 24 below mu = 1/2; finer bins raise mu with
    N, and from 1/2 on the fraction narrows so that M <= 2^23)."""
    f = lambda x: Fraction(float(np.float32(x)))
    p = O.derive_params(D, sq, sk, sv, so, clip, n)
    sh = p.idx_shift
    assert abs(p.idx_mul - Fraction(p.mu) * 2 ** sh) <= Fraction(1, 2)
    assert (sh == 24) == (p.mu < 0.5) and p.idx_mul <= 2 ** 23
    # mu tracks alpha (N-1)/c: compare squares (sqrt(D) is irrational)
    mu_sq = (f(sq) * f(sk)) ** 2 / D * Fraction(n - 1) ** 2 / f(clip) ** 2
    assert abs(Fraction(p.mu) ** 2 - mu_sq) <= mu_sq * Fraction(1, 2 ** 48)
    x = np.arange(0, p.x_clip + 3, dtype=np.int64)
    s = O.slot_index(x, p)
    assert s[0] == 0
    d = np.diff(s)
    assert (d >= 0).all()
    if p.mu <= 1:
        assert ((d == 0) | (d == 1)).all()
    assert (s[p.x_clip:] == n - 1).all() and (s[:p.x_clip] <= n - 2).all()
    assert (np.abs(s[:p.x_clip] * (1 << sh) - x[:p.x_clip] * p.idx_mul) <= (1 << (sh - 1))).all()


@pytest.mark.parametrize("scale", [0.3, 1.1, 4.0])   # mu below 1/2, just above, several bins a unit
def test_fine_twin_slot_agrees_everywhere(scale):
    for n in FINE:
        prm = O.derive_params(64, scale, scale, 0.1, 0.1, O.DEFAULT_CLIP, n)
        xs = np.arange(0, prm.x_clip + 5)
        a = O.slot_index(xs, prm)
        b = [T.nearest_slot(int(xx), prm.idx_mul, prm.idx_shift, n) for xx in xs]
        assert a.tolist() == b


TWIN = [
    (3, 5, 4, False, 0, (0.02, 0.03, 0.05, 0.02)),
    (6, 6, 8, True, 1, (0.01, 0.02, 0.05, 0.01)),
    (4, 11, 16, True, 2, (0.005, 0.01, 0.05, 0.03)),
    (9, 16, 8, False, 3, (0.004, 0.004, 0.1, 0.07)),
]


@pytest.mark.parametrize("n", FINE)
@pytest.mark.parametrize("Sq,Skv,D,causal,seed,scales", TWIN)
def test_fine_twin_agrees_on_tiny_shapes(n, Sq, Skv, D, causal, seed, scales):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, (1, 1, Sq, D)).astype(np.int8)
    k = rng.integers(-127, 128, (1, 1, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 1, Skv, D)).astype(np.int8)
    prm = O.derive_params(D, *scales, O.DEFAULT_CLIP, n)
    out, m, E, P = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True, lut_size=n)
    tout, tm, tE, tP = T.head_forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), prm, causal)
    assert out[0, 0].tolist() == tout and m[0, 0].tolist() == tm
    assert E[0, 0].tolist() == tE and P[0, 0].tolist() == tP


LARGE_MU_TWIN = [
    # (Sq, Skv, D, causal, seed, scales): mu from just above 1/2 to several
    # bins per score unit; small integer inputs keep score gaps near the clip
    (5, 9, 16, False, 20, (0.8, 0.6, 0.05, 0.02)),     # mu 0.6 (32 entries) .. 2.4 (128)
    (7, 7, 8, True, 21, (1.2, 0.95, 0.05, 0.01)),      # mu 2 .. 8
    (4, 12, 4, False, 22, (2.0, 1.2, 0.05, 0.03)),     # mu 6 .. 24
]


@pytest.mark.parametrize("n", [32] + list(FINE))
@pytest.mark.parametrize("Sq,Skv,D,causal,seed,scales", LARGE_MU_TWIN)
def test_twin_agrees_at_large_multipliers(n, Sq, Skv, D, causal, seed, scales):
    rng = np.random.default_rng(seed)
    q = rng.integers(-3, 4, (1, 1, Sq, D)).astype(np.int8)
    k = rng.integers(-3, 4, (1, 1, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 1, Skv, D)).astype(np.int8)
    prm = O.derive_params(D, *scales, O.DEFAULT_CLIP, n)
    assert prm.mu >= 0.5 and prm.idx_shift < 24
    out, m, E, P = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True, lut_size=n)
    tout, tm, tE, tP = T.head_forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), prm, causal)
    assert out[0, 0].tolist() == tout and m[0, 0].tolist() == tm
    assert E[0, 0].tolist() == tE and P[0, 0].tolist() == tP
    # rows are not all one-hot: some key other than the max has p > 0
    assert (P[0, 0] > 0).sum() > Sq


def _ref_softmax(qh, kh, alpha, causal):
    S = qh.astype(np.float64) @ kh.astype(np.float64).T
    allow = O.allowed_mask(qh.shape[0], kh.shape[0], causal)
    L = np.where(allow, alpha * S, -np.inf)
    L -= L.max(axis=1, keepdims=True)
    Wt = np.exp(L)
    return Wt / Wt.sum(axis=1, keepdims=True)


def _beta(prm):
    """Per-key multiplicative error bound of e_j against exp(-alpha x_j), log units."""
    err_m = abs(prm.mu - prm.idx_mul / 2 ** prm.idx_shift)
    smallest = min(e for e in prm.lut[:-1] if e > 0)
    return prm.delta / 2 + prm.delta * prm.x_clip * err_m - math.log(1.0 - 0.5 / smallest)


CASES = [
    (1, 2, 64, 300, 64, False, 5, "channel_outliers"),
    (1, 2, 100, 100, 128, True, 6, "student_t_tail"),
    (1, 1, 1, 2048, 128, False, 8, "normal"),
]


@pytest.mark.parametrize("n", [32] + FINE)
@pytest.mark.parametrize("B,H,Sq,Skv,D,causal,seed,kind", CASES)
def test_fine_tables_against_float64_softmax(n, B, H, Sq, Skv, D, causal, seed, kind):
    """|p/255 - p_ref| <= tanh(beta/2) + tau_row + (1/2 + 2^-9)/255 per row
    (beta shrinks with the bin width); and with 128 entries the bound without
    the clipped mass is below the 0.02 tolerance a 32-entry table cannot
    guarantee."""
    w = W.make_random(B, H, Sq, Skv, D, causal, seed, kind)
    prm = O.derive_params(D, *w.scales, w.clip, n)
    _, m, _, P = O.forward(w.q, w.k, w.v, w.scales, w.clip, causal, stats=True, lut_size=n)
    tb = math.tanh(_beta(prm) / 2)
    if n == 128:
        assert tb + (0.5 + 2 ** -9) / 255 < 0.02
    if n == 32:
        assert tb > 0.02
    for b in range(B):
        for h in range(H):
            pref = _ref_softmax(w.q[b, h], w.k[b, h], prm.alpha, causal)
            S = w.q[b, h].astype(np.int64) @ w.k[b, h].astype(np.int64).T
            allow = O.allowed_mask(Sq, Skv, causal)
            clipped = allow & (m[b, h][:, None] - S >= prm.x_clip)
            tau = np.where(clipped, pref, 0.0).sum(axis=1)
            dp = np.abs(P[b, h] / 255.0 - pref).max(axis=1)
            assert (dp <= tb + tau + (0.5 + 2 ** -9) / 255 + 1e-12).all()


def test_finer_tables_track_softmax_more_closely():
    """On the same peaked rows the mean |p/255 - p_ref| falls as the table refines."""
    w = W.make_random(1, 4, 64, 256, 64, False, 11, "channel_outliers")
    errs = []
    for n in (32, 64, 128):
        prm = O.derive_params(64, *w.scales, w.clip, n)
        P = O.forward(w.q, w.k, w.v, w.scales, w.clip, False, stats=True, lut_size=n)[3]
        e = 0.0
        for h in range(4):
            e += np.abs(P[0, h] / 255.0 - _ref_softmax(w.q[0, h], w.k[0, h], prm.alpha, False)).mean()
        errs.append(e)
    assert errs[0] > errs[1] > errs[2]


@pytest.mark.parametrize("H,hkv", [(4, 4), (4, 2), (4, 1), (6, 3), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_kv_heads_equal_repeated_heads(H, hkv, causal):
    """kv_heads = Hkv equals multi-head attention on K/V repeated G = H/Hkv
    times along the head axis (numpy's repeat: head h gets K/V head h // G)."""
    rng = np.random.default_rng(H * 10 + hkv)
    q = rng.integers(-127, 128, (2, H, 9, 16)).astype(np.int8)
    k = rng.integers(-127, 128, (2, hkv, 13, 16)).astype(np.int8)
    v = rng.integers(-127, 128, (2, hkv, 13, 16)).astype(np.int8)
    sc = (0.01, 0.012, 0.05, 0.02)
    g = H // hkv
    got = O.forward(q, k, v, sc, causal=causal, kv_heads=hkv)
    want = O.forward(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), sc, causal=causal)
    assert np.array_equal(got, want)
    # and each query head's output depends on its own group's K/V only
    k2 = k.copy()
    k2[:, hkv - 1] = rng.integers(-127, 128, k2[:, hkv - 1].shape).astype(np.int8)
    got2 = O.forward(q, k2, v, sc, causal=causal, kv_heads=hkv)
    assert np.array_equal(got2[:, : H - g], got[:, : H - g])


def test_grouped_kv_heads_refusals():
    q = np.zeros((1, 4, 2, 8), np.int8)
    k = np.zeros((1, 3, 2, 8), np.int8)
    with pytest.raises(O.OracleRangeError):
        O.forward(q, k, k, (0.05, 0.05, 0.05, 0.05), kv_heads=3)      # 3 does not divide 4
    with pytest.raises(O.OracleRangeError):
        O.forward(q, k, k, (0.05, 0.05, 0.05, 0.05), kv_heads=2)      # shape says 3


# ---------------------------------------------------------------------------
# uint16 probabilities (the dynamic-range variant)
# ---------------------------------------------------------------------------
def test_p16_uniform_rows_never_underflow():
    """A uniform row of n keys (every e = 2^15, E = n 2^15): for every
    admissible n (1..65535) the uint16 p is the rounding of 65535/n within
    1/2 + 1/4, and never 0, where uint8 p is 0 for every n >= 513."""
    n = np.arange(1, 65536, dtype=np.int64)
    E = n << 15
    p16 = O.normalise16(np.int64(1 << 15), O.reciprocal16(E))
    p8 = O.normalise(np.int64(1 << 15), O.reciprocal(E))
    assert (p16 >= 1).all()
    assert (np.abs(p16 * n - 65535) <= n * 0.75).all()      # |p - 65535/n| <= 3/4, in integers
    assert p16[0] == 65535 and p16[1] == 32768 and p16[65534] == 1
    assert (p8[512:] == 0).all() and (p8[:512] >= 1).all()


def test_p16_normalisation_bound_exact():
    """|p - 65535 e / E| <= 1/2 + e / 2^17 with exact rationals, and e*R16 + 2^15 < 2^32."""
    rng = np.random.default_rng(21)
    E = rng.integers(1 << 15, 65535 << 15, 20000).astype(np.int64)
    e = np.minimum(rng.integers(0, 1 << 15, 20000).astype(np.int64), E)
    R = O.reciprocal16(E)
    assert int((e * R + (1 << 15)).max()) < (1 << 32)
    p = O.normalise16(e, R)
    for ei, Ei, pi in list(zip(e.tolist(), E.tolist(), p.tolist()))[::7]:
        assert abs(Fraction(pi) - Fraction(65535 * ei, Ei)) <= Fraction(1, 2) + Fraction(ei, 1 << 17)


def test_p16_single_key_returns_v():
    """One key: p = 65535, and with s_o = s_v the output is v for every int8 value."""
    vals = np.arange(-127, 128, dtype=np.int8)
    v1 = vals.reshape(1, 1, 1, 255)
    rng = np.random.default_rng(22)
    q1 = rng.integers(-127, 128, (1, 1, 3, 255)).astype(np.int8)
    k1 = rng.integers(-127, 128, (1, 1, 1, 255)).astype(np.int8)
    out, _, E, P = O.forward(q1, k1, v1, (0.05, 0.05, 0.01, 0.01), stats=True, prob_bits=16)
    assert (P == 65535).all() and (E == 1 << 15).all()
    assert (out[0, 0] == vals[None, :]).all()


@pytest.mark.parametrize("Sq,Skv,D,causal,seed,scales", TWIN)
def test_p16_twin_agrees_on_tiny_shapes(Sq, Skv, D, causal, seed, scales):
    rng = np.random.default_rng(seed + 50)
    q = rng.integers(-127, 128, (1, 1, Sq, D)).astype(np.int8)
    k = rng.integers(-127, 128, (1, 1, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 1, Skv, D)).astype(np.int8)
    prm = O.derive_params(D, *scales, O.DEFAULT_CLIP, 32, 16)
    out, m, E, P = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True, prob_bits=16)
    tout, tm, tE, tP = T.head_forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), prm, causal)
    assert out[0, 0].tolist() == tout and E[0, 0].tolist() == tE and P[0, 0].tolist() == tP


@pytest.mark.parametrize("B,H,Sq,Skv,D,causal,seed,kind", CASES)
def test_p16_against_float64_softmax(B, H, Sq, Skv, D, causal, seed, kind):
    """|p/65535 - p_ref| <= tanh(beta/2) + tau_row + (1/2 + 1/4)/65535 per row."""
    w = W.make_random(B, H, Sq, Skv, D, causal, seed, kind)
    prm = O.derive_params(D, *w.scales, w.clip, 32, 16)
    _, m, _, P = O.forward(w.q, w.k, w.v, w.scales, w.clip, causal, stats=True, prob_bits=16)
    tb = math.tanh(_beta(prm) / 2)
    for b in range(B):
        for h in range(H):
            pref = _ref_softmax(w.q[b, h], w.k[b, h], prm.alpha, causal)
            S = w.q[b, h].astype(np.int64) @ w.k[b, h].astype(np.int64).T
            allow = O.allowed_mask(Sq, Skv, causal)
            clipped = allow & (m[b, h][:, None] - S >= prm.x_clip)
            tau = np.where(clipped, pref, 0.0).sum(axis=1)
            dp = np.abs(P[b, h] / 65535.0 - pref).max(axis=1)
            assert (dp <= tb + tau + 0.75 / 65535 + 1e-12).all()


def test_p16_cures_long_flat_row_underflow():
    """A decode-like row of 8192 keys from N(0,1) data: with uint8 P most
    kept keys round to 0 and the output collapses towards 0; with uint16 P
    the output tracks float64 attention (mean error at least 4x smaller)."""
    w = W.make_random(1, 2, 1, 8192, 128, False, 23, "normal")
    sv = w.scales[2]
    so8 = w.scales[3]
    out8, _, _, P8 = O.forward(w.q, w.k, w.v, w.scales, w.clip, False, stats=True)
    out16, _, _, P16 = O.forward(w.q, w.k, w.v, w.scales, w.clip, False, stats=True, prob_bits=16)
    prm = O.derive_params(128, *w.scales, w.clip)
    errs = []
    for out in (out8, out16):
        e = 0.0
        for h in range(2):
            pref = _ref_softmax(w.q[0, h], w.k[0, h], prm.alpha, False)
            Oref = (pref @ w.v[0, h].astype(np.float64)) * sv / so8
            e += np.abs(out[0, h].astype(np.float64) - Oref).mean()
        errs.append(e)
    assert (P8 > 0).mean() < (P16 > 0).mean()
    assert errs[1] * 4 < errs[0]


def test_prob_bits_refused_outside_8_and_16():
    for bad in (0, 4, 12, 32):
        with pytest.raises(O.OracleRangeError):
            O.derive_params(64, 0.05, 0.05, 0.05, 0.05, O.DEFAULT_CLIP, 32, bad)
    p8 = O.derive_params(64, 0.05, 0.05, 0.05, 0.05, O.DEFAULT_CLIP, 32, 8)
    p16 = O.derive_params(64, 0.05, 0.05, 0.05, 0.05, O.DEFAULT_CLIP, 32, 16)
    # the output multiplier carries the probability scale: mu_o(16) = mu_o(8) * 255 / 65535
    assert abs(p16.mu_o * 65535 - p8.mu_o * 255) <= 1e-15 * p8.mu_o * 255
    assert (p16.idx_mul, p16.x_clip, p16.lut) == (p8.idx_mul, p8.x_clip, p8.lut)


# ---------------------------------------------------------------------------
# uint8 exp table (the narrow end of the table's accuracy/memory trade)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [32] + FINE)
@pytest.mark.parametrize("clip", CLIPS)
def test_lut8_matches_high_precision_exp(n, clip):
    """|e8[k] - 255 exp(-k c/(N-1))| <= 1/2 in 50-digit decimal; 255 at a
    zero relative score, 0 in the tail slot; non-increasing."""
    getcontext().prec = 50
    lut = O.build_lut(clip, n, 8)
    assert len(lut) == n and lut[0] == 255 and lut[-1] == 0
    c = Decimal(float(np.float32(clip)))
    for k in range(n - 1):
        ref = Decimal(255) * (-(Decimal(k) * c / Decimal(n - 1))).exp()
        assert abs(Decimal(lut[k]) - ref) <= Decimal("0.5") + Decimal("1e-9"), (n, k)
    assert all(lut[k] >= lut[k + 1] for k in range(n - 1))


@pytest.mark.parametrize("n", [32] + FINE)
def test_lut8_halving_table(n):
    """clip = (N-1) ln 2 makes the bin width ln 2, so slot k holds 255 / 2^k
    rounded: 64, 32, 16, 8, 4, 2, 1 for k = 2..8 and 0 from k = 9 on (slot 1,
    127.5, sits on a rounding tie that float32 clip decides either way)."""
    lut = O.build_lut((n - 1) * math.log(2.0), n, 8)
    assert lut[0] == 255 and lut[1] in (127, 128)
    assert list(lut[2:9]) == [64, 32, 16, 8, 4, 2, 1]
    assert not any(lut[9:])


def test_lut8_uniform_rows():
    """A uniform row of n keys (every e8 = 255, E8 = 255 n): uint8 p is
    floor(255/n + 1/2) for every admissible n, hence 0 from n = 511 on; the
    uint16 p stays within 3/4 of 65535/n and never reaches 0."""
    n = np.arange(1, 65536, dtype=np.int64)
    E8 = 255 * n
    p8 = O.normalise8(np.int64(255), O.reciprocal8(E8))
    want = np.array([(Fraction(255, int(k)) + Fraction(1, 2)).__floor__() for k in n[:4000]])
    assert np.array_equal(p8[:4000], want)
    assert (p8[510:] == 0).all() and (p8[:510] >= 1).all()
    p16 = O.normalise8_16(np.int64(255), O.reciprocal8_16(E8))
    assert (p16 >= 1).all() and p16[0] == 65535 and p16[1] == 32768
    assert (np.abs(p16 * n - 65535) <= n * 0.75).all()


def test_lut8_normalisation_bound_exact():
    """|p - 255 e8/E8| <= 1/2 + e8/2^17 (uint8 p) and |p - 65535 e8/E8| <=
    1/2 + e8/2^10 (uint16 p) with exact rationals: the reciprocal is within
    1/2 of its real value. p never exceeds 255 (65535)."""
    rng = np.random.default_rng(31)
    E8 = rng.integers(255, 65535 * 255, 20000).astype(np.int64)
    e8 = np.minimum(rng.integers(0, 256, 20000).astype(np.int64), E8)
    p8 = O.normalise8(e8, O.reciprocal8(E8))
    p16 = O.normalise8_16(e8, O.reciprocal8_16(E8))
    assert int(p8.max()) <= 255 and int(p16.max()) <= 65535
    for ei, Ei, a, b in list(zip(e8.tolist(), E8.tolist(), p8.tolist(), p16.tolist()))[::7]:
        assert abs(Fraction(a) - Fraction(255 * ei, Ei)) <= Fraction(1, 2) + Fraction(ei, 1 << 17)
        assert abs(Fraction(b) - Fraction(65535 * ei, Ei)) <= Fraction(1, 2) + Fraction(ei, 1 << 10)
    # a row whose keys all sit at the max: p = 255 (65535)
    assert int(O.normalise8(255, O.reciprocal8(255))) == 255
    assert int(O.normalise8_16(255, O.reciprocal8_16(255))) == 65535


def test_lut8_equals_the_q15_normaliser_on_entries_times_128():
    """128 e8 in a Q15 slot leaves every probability unchanged: with E = 128 E8
    the Q15 reciprocal floor((255*2^23 + E/2)/E) equals floor((255*2^17 + E8)/(2 E8))
    and (128 e8 R + 2^22) >> 23 equals (e8 R + 2^15) >> 16 (and likewise for
    uint16 p), exhaustively over e8 and over row sums from one key up."""
    rng = np.random.default_rng(32)
    E8 = np.concatenate([np.arange(255, 5000), rng.integers(5000, 65535 * 255, 20000)]).astype(np.int64)
    assert np.array_equal(O.reciprocal8(E8), O.reciprocal(128 * E8))
    assert np.array_equal(O.reciprocal8_16(E8), O.reciprocal16(128 * E8))
    for e in range(256):
        ee = np.minimum(np.int64(e), E8)
        assert np.array_equal(O.normalise8(ee, O.reciprocal8(E8)), O.normalise(128 * ee, O.reciprocal(128 * E8)))
        assert np.array_equal(O.normalise8_16(ee, O.reciprocal8_16(E8)),
                              O.normalise16(128 * ee, O.reciprocal16(128 * E8)))


def test_lut_bits_refused_outside_the_variants():
    for bad in (0, 4, 12, 32):
        with pytest.raises(O.OracleRangeError):
            O.build_lut(O.DEFAULT_CLIP, 32, bad)
        with pytest.raises(O.OracleRangeError):
            O.derive_params(64, 0.05, 0.05, 0.05, 0.05, O.DEFAULT_CLIP, 32, 8, bad)


@pytest.mark.parametrize("n", [32, 128])
@pytest.mark.parametrize("prob_bits", [8, 16])
@pytest.mark.parametrize("Sq,Skv,D,causal,seed,scales", TWIN)
def test_lut8_twin_agrees_on_tiny_shapes(n, prob_bits, Sq, Skv, D, causal, seed, scales):
    rng = np.random.default_rng(seed + 40)
    q = rng.integers(-127, 128, (1, 1, Sq, D)).astype(np.int8)
    k = rng.integers(-127, 128, (1, 1, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 1, Skv, D)).astype(np.int8)
    prm = O.derive_params(D, *scales, O.DEFAULT_CLIP, n, prob_bits, 8)
    out, m, E, P = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True, lut_size=n,
                             prob_bits=prob_bits, lut_bits=8)
    tout, tm, tE, tP = T.head_forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), prm, causal)
    assert out[0, 0].tolist() == tout and m[0, 0].tolist() == tm
    assert E[0, 0].tolist() == tE and P[0, 0].tolist() == tP


def test_lut8_single_key_returns_v():
    """One key: e8 = 255, p = 255, and with s_o = s_v the output is v."""
    vals = np.arange(-127, 128, dtype=np.int8)
    v1 = vals.reshape(1, 1, 1, 255)
    rng = np.random.default_rng(33)
    q1 = rng.integers(-127, 128, (1, 1, 3, 255)).astype(np.int8)
    k1 = rng.integers(-127, 128, (1, 1, 1, 255)).astype(np.int8)
    out, _, E, P = O.forward(q1, k1, v1, (0.05, 0.05, 0.01, 0.01), stats=True, lut_bits=8)
    assert (P == 255).all() and (E == 255).all()
    assert (out[0, 0] == vals[None, :]).all()


@pytest.mark.parametrize("B,H,Sq,Skv,D,causal,seed,kind", CASES)
def test_lut8_against_float64_softmax(B, H, Sq, Skv, D, causal, seed, kind):
    """The float64 bound of the Q15 tables holds for the uint8 table with its
    own per-key error (beta from its smallest nonzero entry), and on these
    rows the mean |p/255 - p_ref| stays within 2% of the Q15 table's."""
    w = W.make_random(B, H, Sq, Skv, D, causal, seed, kind)
    prm = O.derive_params(D, *w.scales, w.clip, 32, 8, 8)
    _, m, _, P = O.forward(w.q, w.k, w.v, w.scales, w.clip, causal, stats=True, lut_bits=8)
    P16 = O.forward(w.q, w.k, w.v, w.scales, w.clip, causal, stats=True)[3]
    tb = math.tanh(_beta(prm) / 2)
    e8 = e16 = 0.0
    for b in range(B):
        for h in range(H):
            pref = _ref_softmax(w.q[b, h], w.k[b, h], prm.alpha, causal)
            S = w.q[b, h].astype(np.int64) @ w.k[b, h].astype(np.int64).T
            allow = O.allowed_mask(Sq, Skv, causal)
            clipped = allow & (m[b, h][:, None] - S >= prm.x_clip)
            tau = np.where(clipped, pref, 0.0).sum(axis=1)
            dp = np.abs(P[b, h] / 255.0 - pref).max(axis=1)
            assert (dp <= tb + tau + (0.5 + 2 ** -9) / 255 + 1e-12).all()
            e8 += np.abs(P[b, h] / 255.0 - pref).mean()
            e16 += np.abs(P16[b, h] / 255.0 - pref).mean()
    assert e8 <= 1.02 * e16
