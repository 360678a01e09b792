"""Pins of the oracle's pipeline stages (Q.K^T, IndexSoftmax, P.V) and of the
floating-point comparator, against library routines, closed forms and
properties the pages fix (methodology steps 1-3)."""
import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

from oracle import fp_baseline as F
from oracle import intattn_oracle as O

RNG = np.random.default_rng(20261203)


def _rand(shape):
    return RNG.integers(-127, 128, shape).astype(np.int8)


def test_qk_scores_is_integer_matmul():
    q, k = _rand((37, 64)), _rand((53, 64))
    ref = q.astype(np.int64) @ k.astype(np.int64).T         # numpy integer matmul
    assert np.array_equal(O.qk_scores(q, k), ref)


@pytest.mark.parametrize("causal", [False, True])
def test_stages_compose_to_forward(causal):
    q, k, v = _rand((1, 2, 40, 64)), _rand((1, 2, 70, 64)), _rand((1, 2, 70, 64))
    scales = (0.02, 0.02, 0.03, 0.01)
    out, m, E, P = O.forward(q, k, v, scales, causal=causal, stats=True)
    prm = O.derive_params(64, *scales, O.DEFAULT_CLIP)
    for h in range(2):
        S = O.qk_scores(q[0, h], k[0, h])
        P2, m2, E2 = O.index_softmax(S, prm, causal)
        assert np.array_equal(P2, P[0, h]) and np.array_equal(m2, m[0, h]) and np.array_equal(E2, E[0, h])
        assert np.array_equal(O.pv_requant(P2, v[0, h], prm), out[0, h])


def test_index_softmax_single_allowed_key_is_255():
    # causal, Sq = Skv: row 0 attends key 0 only, so E = LUT[0] and p = 255
    prm = O.derive_params(64, 0.02, 0.02, 0.03, 0.01, O.DEFAULT_CLIP)
    S = RNG.integers(-2 ** 20, 2 ** 20, (5, 5))
    P, m, E = O.index_softmax(S, prm, causal=True)
    assert P[0, 0] == 255 and not P[0, 1:].any()
    assert E[0] == 1 << 15 and m[0] == S[0, 0]


def test_index_softmax_row_sums_and_order():
    prm = O.derive_params(64, 0.05, 0.05, 0.03, 0.01, O.DEFAULT_CLIP)
    S = RNG.integers(-30000, 30000, (64, 300))
    P, m, E = O.index_softmax(S, prm, causal=False)
    P = P.astype(np.int64)
    nz = (P > 0).sum(axis=1)
    # each p is rounded to nearest from e*R/2^23 with sum(e)*R = 255*2^23 up to R's rounding
    assert (np.abs(P.sum(axis=1) - 255) <= nz // 2 + 1).all()
    # a higher score never gets a smaller probability
    for i in range(64):
        o = np.argsort(S[i], kind="stable")
        assert (np.diff(P[i][o]) >= 0).all()


def test_fp_codes_match_float64_softmax_within_one():
    for causal in (False, True):
        for n, scale in ((8, 0.05), (300, 0.02), (512, 0.2)):
            S = RNG.integers(-20000, 20000, (n if causal else 33, n))
            alpha = F.dequant_alpha(64, scale, scale)
            codes = F.fp_softmax_codes(S, alpha, causal).astype(np.int64)
            allow = O.allowed_mask(*S.shape, causal)
            y = np.where(allow, S.astype(np.float64) * float(alpha), -np.inf)
            p = scipy_softmax(y, axis=1)                          # library routine, float64
            ref = np.minimum(np.rint(255.0 * p), 255).astype(np.int64)
            assert np.abs(codes - ref).max() <= 1
            assert (codes[~allow] == 0).all()
            assert (codes != ref).mean() < 0.01


def test_fp_codes_single_key_and_uniform_rows():
    alpha = F.dequant_alpha(64, 0.05, 0.05)
    S = RNG.integers(-1000, 1000, (4, 4))
    codes = F.fp_softmax_codes(S, alpha, causal=True)
    assert codes[0, 0] == 255 and not codes[0, 1:].any()
    for n in (1, 2, 3, 5, 7, 200):
        U = np.full((2, n), 1234, dtype=np.int64)
        c = F.fp_softmax_codes(U, alpha, causal=False)
        assert (c == np.rint(255.0 / n)).all()
