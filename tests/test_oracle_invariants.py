"""Structural invariants and brute-force agreement of the CPU oracle.

Exact identities that any correct implementation of the integer attention
(IntAttention digest, "Methodology" steps 2-3) must satisfy, independent of
the table values: key permutation, value negation, causal/decode consistency,
per-head independence; plus equality with the loop-and-Fraction twin on tiny
shapes.
"""
import numpy as np
import pytest

from oracle import intattn_oracle as O
from oracle import scalar_twin as T
from integer_only_quantized_amd import workloads as W


def _w(B=1, H=2, Sq=24, Skv=40, D=64, causal=False, seed=21, kind="normal"):
    return W.make_random(B, H, Sq, Skv, D, causal, seed, kind)


def test_key_permutation_invariance():
    w = _w()
    perm = np.random.default_rng(1).permutation(w.Skv)
    a = O.forward(w.q, w.k, w.v, w.scales, w.clip)
    b = O.forward(w.q, w.k[:, :, perm], w.v[:, :, perm], w.scales, w.clip)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_value_negation_is_odd(causal):
    w = _w(causal=causal, Sq=40)
    a = O.forward(w.q, w.k, w.v, w.scales, w.clip, causal)
    b = O.forward(w.q, w.k, -w.v, w.scales, w.clip, causal)
    assert np.array_equal(a.astype(np.int16), -b.astype(np.int16))


def test_causal_last_row_equals_decode():
    w = _w(causal=True, Sq=32, Skv=32, D=128, seed=4, kind="student_t_tail")
    full, m, E, P = O.forward(w.q, w.k, w.v, w.scales, w.clip, True, stats=True)
    dec, m1, E1, P1 = O.forward(w.q[:, :, -1:], w.k, w.v, w.scales, w.clip, False, stats=True)
    assert np.array_equal(full[:, :, -1:], dec)
    assert np.array_equal(m[:, :, -1:], m1) and np.array_equal(E[:, :, -1:], E1)


@pytest.mark.parametrize("Sq,Skv", [(5, 19), (12, 12), (1, 7)])
def test_bottom_right_causal_rows(Sq, Skv):
    """Row i of a causal call sees keys 0 .. i + Skv - Sq: it equals a
    non-causal single-query call on that key prefix."""
    w = _w(causal=True, Sq=Sq, Skv=Skv, seed=9)
    full = O.forward(w.q, w.k, w.v, w.scales, w.clip, True)
    for i in range(Sq):
        n = i + Skv - Sq + 1
        one = O.forward(w.q[:, :, i:i + 1], w.k[:, :, :n], w.v[:, :, :n], w.scales, w.clip, False)
        assert np.array_equal(full[:, :, i:i + 1], one)


def test_causal_single_query_equals_noncausal():
    w = _w(Sq=1, Skv=50, seed=5)
    a = O.forward(w.q, w.k, w.v, w.scales, w.clip, True)
    b = O.forward(w.q, w.k, w.v, w.scales, w.clip, False)
    assert np.array_equal(a, b)


def test_heads_are_independent():
    w = _w(B=2, H=3, seed=8, kind="channel_outliers")
    full = O.forward(w.q, w.k, w.v, w.scales, w.clip)
    for b in range(2):
        for h in range(3):
            one = O.forward(w.q[b:b + 1, h:h + 1], w.k[b:b + 1, h:h + 1], w.v[b:b + 1, h:h + 1],
                            w.scales, w.clip)
            assert np.array_equal(full[b, h], one[0, 0])


def test_argument_refusals():
    w = _w(Sq=24, Skv=40)
    with pytest.raises(O.OracleRangeError):                      # causal needs Sq <= Skv
        O.forward(w.k, w.q, w.q, w.scales, w.clip, True)
    with pytest.raises(O.OracleRangeError):                      # empty key set
        O.forward(w.q, w.k[:, :, :0], w.v[:, :, :0], w.scales, w.clip)
    bad = w.v.copy()
    bad[0, 0, 0, 0] = -128                                       # outside the symmetric range
    with pytest.raises(O.OracleRangeError):
        O.forward(w.q, w.k, bad, w.scales, w.clip)
    with pytest.raises(O.OracleRangeError):
        O.forward(w.q.astype(np.int16), w.k, w.v, w.scales, w.clip)
    # empty batch is a valid no-op
    e = O.forward(w.q[:0], w.k[:0], w.v[:0], w.scales, w.clip)
    assert e.shape == (0,) + w.q.shape[1:]


def _twin_case(Sq, Skv, D, causal, seed, scales, lo=-127, hi=128):
    rng = np.random.default_rng(seed)
    q = rng.integers(lo, hi, (1, 1, Sq, D)).astype(np.int8)
    k = rng.integers(lo, hi, (1, 1, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 1, Skv, D)).astype(np.int8)
    return q, k, v


TWIN = [
    # (Sq, Skv, D, causal, seed, scales)
    (3, 5, 4, False, 0, (0.02, 0.03, 0.05, 0.02)),
    (6, 6, 8, True, 1, (0.01, 0.02, 0.05, 0.01)),
    (4, 11, 16, True, 2, (0.005, 0.01, 0.05, 0.03)),
    (9, 16, 8, False, 3, (0.004, 0.004, 0.1, 0.07)),
    (1, 13, 32, False, 4, (0.003, 0.02, 0.02, 0.004)),
    (12, 12, 2, True, 5, (0.2, 0.1, 0.05, 0.05)),
]


@pytest.mark.parametrize("Sq,Skv,D,causal,seed,scales", TWIN)
def test_twin_agrees_on_tiny_shapes(Sq, Skv, D, causal, seed, scales):
    q, k, v = _twin_case(Sq, Skv, D, causal, seed, scales)
    prm = O.derive_params(D, *scales, O.DEFAULT_CLIP)
    out, m, E, P = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True)
    tout, tm, tE, tP = T.head_forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), prm, causal)
    assert out[0, 0].tolist() == tout
    assert m[0, 0].tolist() == tm
    assert E[0, 0].tolist() == tE
    assert P[0, 0].tolist() == tP
    # the case must exercise more than one slot (not a degenerate all-equal row)
    assert len(set(int(x) for x in P[0, 0].ravel())) >= 2


def test_twin_slot_agrees_everywhere_on_a_small_clip():
    prm = O.derive_params(64, 0.3, 0.3, 0.1, 0.1, O.DEFAULT_CLIP)
    xs = np.arange(0, prm.x_clip + 5)
    a = O.slot_index(xs, prm)
    b = [T.nearest_slot(int(x), prm.idx_mul, prm.idx_shift) for x in xs]
    assert a.tolist() == b
