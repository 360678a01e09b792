"""Pins for the oracle's IndexSoftmax and value contraction against mathematics.

IntAttention digest, "Methodology" step 2: the integer pseudo-exponents,
normalised by an integer reciprocal multiply and right shift, form a
softmax-like distribution. Pinned here by:
  * the rounding bound of the reciprocal normalisation (exact rationals);
  * closed forms: uniform rows (softmax 1/n), a dominant key (one-hot),
    a single key (attention returns the value itself);
  * the row-sum and monotonicity invariants;
  * a derived tolerance against float64 softmax of the dequantised logits,
    and the corresponding bound on the int8 output against float64 attention.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import intattn_oracle as O
from integer_only_quantized_amd import workloads as W


def test_normalisation_rounding_bound():
    """|p - 255 e / E| <= 1/2 + 2^-9 for every e <= E (exact rationals)."""
    rng = np.random.default_rng(11)
    E = np.concatenate([rng.integers(32768, 2 ** 31 - 1, 4000),
                        np.array([32768, 32769, 65536, 98304, 2 ** 31 - 1])])
    for Ei in E[:600]:
        Ei = int(Ei)
        R = int(O.reciprocal(Ei))
        assert R < 2 ** 16
        es = set(int(x) for x in rng.integers(0, min(Ei, 32768) + 1, 40)) | {0, min(Ei, 32768)}
        for e in es:
            p = int(O.normalise(e, R))
            assert 0 <= p <= 255
            assert abs(Fraction(p) - Fraction(255 * e, Ei)) <= Fraction(1, 2) + Fraction(1, 512)
    # the largest product stays inside int32 (device arithmetic relies on it)
    assert 32768 * int(O.reciprocal(32768)) + (1 << 22) < 2 ** 31


def _uniform_p(n):
    E = 32768 * n
    return int(O.normalise(32768, O.reciprocal(E)))


def test_uniform_rows_closed_form():
    """All n scores equal: softmax is 1/n, so p must be within 1/2 + 2^-9 of 255/n."""
    for n in list(range(1, 1100)) + [4096, 8192, 65535]:
        p = _uniform_p(n)
        assert abs(Fraction(p) - Fraction(255, n)) <= Fraction(1, 2) + Fraction(1, 512), n
    assert _uniform_p(1) == 255
    # 255/n < 1/2 - 2^-9 forces 0: every n >= 513 underflows to p = 0
    assert all(_uniform_p(n) == 0 for n in range(513, 1100))


def _uniform_row_case(n, D=16, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, (1, 1, 3, D)).astype(np.int8)
    krow = rng.integers(-127, 128, D).astype(np.int8)
    k = np.broadcast_to(krow, (1, 1, n, D)).copy()
    v = rng.integers(-127, 128, (1, 1, n, D)).astype(np.int8)
    return q, k, v


@pytest.mark.parametrize("n", [1, 2, 3, 5, 16, 100, 513, 700])
def test_uniform_rows_through_forward(n):
    q, k, v = _uniform_row_case(n)
    sv = 0.01
    out, m, E, P = O.forward(q, k, v, (0.02, 0.02, sv, sv), causal=False, stats=True)
    p = _uniform_p(n)
    assert (P == p).all()
    assert (E == 32768 * n).all()
    # out = requant(p * sum_j v_j) with s_o = s_v: round(p * colsum / 255)
    colsum = v[0, 0].astype(np.int64).sum(axis=0)
    expect = np.array([int(math.copysign(min(127, int(Fraction(abs(int(a)) * p, 255) + Fraction(1, 2))), a))
                       for a in colsum], dtype=np.int64)
    # s_o = s_v gives mu_o = 1/255 up to a 2^-31 relative multiplier error;
    # p * colsum / 255 is never closer than 1/510 to a rounding tie, so the
    # encoded result equals the exact rounding
    assert (out[0, 0].astype(np.int64) == expect[None, :]).all()


def test_one_hot_and_single_key():
    """A key leading all others by at least the clip gap takes p = 255; with
    s_o = s_v the output is that key's value row, exactly."""
    D, n = 8, 40
    rng = np.random.default_rng(3)
    v = rng.integers(-127, 128, (1, 1, n, D)).astype(np.int8)
    q = np.zeros((1, 1, 1, D), dtype=np.int8)
    q[..., 0] = 127
    k = rng.integers(-20, 21, (1, 1, n, D)).astype(np.int8)
    k[..., 0] = rng.integers(-20, 21, n)
    j_star = 17
    k[0, 0, j_star, 0] = 127                    # score 127*127 vs <= 127*20 + others
    scales = (0.05, 0.05, 0.01, 0.01)
    prm = O.derive_params(D, *scales, O.DEFAULT_CLIP)
    s = q[0, 0].astype(np.int64) @ k[0, 0].astype(np.int64).T
    assert (s.max() - np.sort(s[0])[-2]) >= prm.x_clip
    out, m, E, P = O.forward(q, k, v, scales, stats=True)
    assert P[0, 0, 0, j_star] == 255 and P[0, 0, 0].sum() == 255
    assert (out[0, 0, 0] == v[0, 0, j_star]).all()
    # a single key (Skv = 1): every int8 value comes back unchanged
    vals = np.arange(-127, 128, dtype=np.int8)
    v1 = vals.reshape(1, 1, 1, 255)
    q1 = rng.integers(-127, 128, (1, 1, 4, 255)).astype(np.int8)
    k1 = rng.integers(-127, 128, (1, 1, 1, 255)).astype(np.int8)
    out1 = O.forward(q1, k1, v1, (0.05, 0.05, 0.01, 0.01))
    assert (out1[0, 0] == vals[None, :]).all()


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
    lut30 = min(e for e in prm.lut[:31] if e > 0)
    return (prm.delta / 2 + prm.delta * prm.x_clip * err_m
            - math.log(1.0 - 0.5 / lut30))


CASES = [
    # (B, H, Sq, Skv, D, causal, seed, kind)
    (1, 1, 128, 128, 64, False, 0, "normal"),
    (1, 2, 64, 300, 64, False, 5, "channel_outliers"),
    (1, 2, 100, 100, 128, True, 6, "student_t_tail"),
    (2, 1, 33, 65, 64, True, 7, "normal"),
    (1, 1, 1, 2048, 128, False, 8, "normal"),
]


@pytest.mark.parametrize("B,H,Sq,Skv,D,causal,seed,kind", CASES)
def test_against_float64_softmax_and_attention(B, H, Sq, Skv, D, causal, seed, kind):
    """|p/255 - p_ref| <= tanh(beta/2) + tau_row + (1/2 + 2^-9)/255 per row, where
    tau_row is the reference mass of the keys clipped into the zero slot; and
    |out - O_ref/s_o| <= 1/2 + |a| |mu_o - M_o 2^-sh_o| + (s_v/s_o) max|v| sum_j |dp_j|."""
    w = W.make_random(B, H, Sq, Skv, D, causal, seed, kind)
    prm = O.derive_params(D, *w.scales, w.clip)
    out, m, E, P = O.forward(w.q, w.k, w.v, w.scales, w.clip, causal, stats=True)
    tb = math.tanh(_beta(prm) / 2)
    round_term = (0.5 + 2 ** -9) / 255
    sv, so = w.scales[2], w.scales[3]
    worst_dp = 0.0
    for b in range(B):
        for h in range(H):
            pref = _ref_softmax(w.q[b, h], w.k[b, h], prm.alpha, causal)
            S = w.q[b, h].astype(np.int64) @ w.k[b, h].astype(np.int64).T
            x = m[b, h][:, None] - S
            allow = O.allowed_mask(Sq, Skv, causal)
            clipped = allow & (x >= prm.x_clip)
            tau = np.where(clipped, pref, 0.0).sum(axis=1)
            dp = np.abs(P[b, h] / 255.0 - pref)
            bound = tb + tau + round_term + 1e-12
            assert (dp.max(axis=1) <= bound).all()
            worst_dp = max(worst_dp, float(dp.max()))
            # output against float64 attention
            Oref = (pref @ w.v[b, h].astype(np.float64)) * sv / so
            a = P[b, h].astype(np.int64) @ w.v[b, h].astype(np.int64)
            mu_o_err = abs(prm.mu_o - prm.req_mul / 2 ** prm.req_shift)
            vmax = np.abs(w.v[b, h]).max(axis=0).astype(np.float64)
            l1 = dp.sum(axis=1)
            obound = 0.5 + np.abs(a) * mu_o_err + (sv / so) * l1[:, None] * vmax[None, :] + 1e-9
            assert (np.abs(out[b, h] - Oref) <= obound).all()
    # the invariants the row must satisfy whatever the data
    nnz = (P > 0).sum(axis=-1)
    rowsum = P.astype(np.int64).sum(axis=-1)
    n_kept = np.zeros_like(rowsum)
    for b in range(B):
        for h in range(H):
            S = w.q[b, h].astype(np.int64) @ w.k[b, h].astype(np.int64).T
            allow = O.allowed_mask(Sq, Skv, causal)
            n_kept[b, h] = (allow & (m[b, h][:, None] - S < prm.x_clip)).sum(axis=1)
    assert (np.abs(rowsum - 255) <= n_kept * (0.5 + 2 ** -9)).all()
    assert (nnz <= n_kept).all()


def test_probabilities_monotone_in_score():
    w = W.make_random(1, 2, 40, 90, 64, True, 12, "channel_outliers")
    out, m, E, P = O.forward(w.q, w.k, w.v, w.scales, w.clip, True, stats=True)
    for h in range(2):
        S = w.q[0, h].astype(np.int64) @ w.k[0, h].astype(np.int64).T
        allow = O.allowed_mask(40, 90, True)
        for i in range(40):
            js = np.nonzero(allow[i])[0]
            order = np.argsort(S[i, js], kind="stable")
            ps = P[0, h, i, js][order].astype(np.int64)
            assert (np.diff(ps) >= 0).all()
            assert (P[0, h, i, ~allow[i]] == 0).all()


@pytest.mark.parametrize("scale", [0.3, 1.5, 6.0, 40.0])   # mu 0.06, 1.4, 22, 995
def test_two_key_rows_exhaustive(scale):
    """Two keys with score gap x, for every x up to past the clip point:
    p0 >= p1, p0 + p1 within one of 255, and p1/255 within the derived
    tolerance of the logistic 1 / (1 + e^(alpha x)); from mu = 1/2 on, with
    the narrower multiplier fraction, as below it."""
    prm = O.derive_params(64, scale, scale, 0.1, 0.1, O.DEFAULT_CLIP)
    tb = math.tanh(_beta(prm) / 2)
    lut = np.asarray(prm.lut, dtype=np.int64)
    x = np.arange(0, prm.x_clip + 2, dtype=np.int64)
    e1 = lut[O.slot_index(x, prm)]
    E = lut[0] + e1
    R = O.reciprocal(E)
    p0 = O.normalise(lut[0], R)
    p1 = O.normalise(e1, R)
    assert (p0 >= p1).all()
    assert (np.abs(p0 + p1 - 255) <= 1).all()
    ref1 = 1.0 / (1.0 + np.exp(prm.alpha * x))
    tau = np.where(x >= prm.x_clip, ref1, 0.0)
    assert (np.abs(p1 / 255.0 - ref1) <= tb + tau + (0.5 + 2 ** -9) / 255).all()


def test_requantise_bound_and_symmetry():
    prm = O.derive_params(64, 0.05, 0.05, 0.02, 0.013, O.DEFAULT_CLIP)
    a = np.concatenate([np.arange(-70000, 70001, 7), [2 ** 31 - 1, -(2 ** 31 - 1), 0]]).astype(np.int64)
    out = O.requantise(a, prm).astype(np.int64)
    assert (out == -O.requantise(-a, prm).astype(np.int64)).all()
    mu_o = Fraction(prm.mu_o)
    Mq = Fraction(prm.req_mul, 2 ** prm.req_shift)
    for ai, oi in zip(a[::97], out[::97]):
        exact = Fraction(int(ai)) * mu_o
        if abs(exact) < 126:
            assert abs(oi - exact) <= Fraction(1, 2) + abs(int(ai)) * abs(mu_o - Mq)
        # the encoded multiplier rounds half away from zero
        r = Fraction(abs(int(ai))) * Mq
        mag = min(127, int(r + Fraction(1, 2)))
        assert oi == (mag if ai >= 0 else -mag)
