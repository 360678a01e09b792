"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bar: bit-exact on every output byte and on the IndexSoftmax row state (row
max m_i, row sum E_i, and the uint8 probabilities where the oracle can hold
them), on the same seeded inputs. Covers the five workloads (full size,
sampled heads where the oracle would be slow), ragged and tile-edge sizes,
causal with Sq < Skv, both head sizes, adversarial rows and repeatability.
"""
import numpy as np
import pytest
import torch

from oracle import intattn_oracle as O
from integer_only_quantized_amd import workloads as W

pytestmark = pytest.mark.gpu

IA = pytest.importorskip("integer_only_quantized_amd._binding")


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _say(msg):
    print(msg, flush=True)


def _run(w, debug=False, probs=False):
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    if debug:
        out, rm, rs, pr = IA.forward_debug(q, k, v, w.scales, w.clip, w.causal, with_probs=probs)
        torch.cuda.synchronize()
        return (out.cpu().numpy(), rm.cpu().numpy().astype(np.int64),
                rs.cpu().numpy().view(np.uint32).astype(np.int64),
                pr.cpu().numpy() if pr is not None else None)
    out = IA.forward(q, k, v, w.scales, w.clip, w.causal)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _assert_equal(name, got, ref):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{name}: {len(bad)} of {ref.size} differ; first at {bad[0].tolist()}: "
                             f"got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}")


def _check_full(w, probs=True):
    _say(f"case {w.name} shape={w.shape} causal={w.causal} seed={w.meta.get('seed')}")
    ref, m, E, P = O.forward(w.q, w.k, w.v, w.scales, w.clip, w.causal, stats=True)
    out, rm, rs, pr = _run(w, debug=True, probs=probs)
    _assert_equal("row_max", rm, m)
    _assert_equal("row_sum", rs, E)
    if probs:
        _assert_equal("probs", pr, P)
    _assert_equal("out(debug)", out, ref)
    out2 = _run(w)
    _assert_equal("out", out2, ref)


def test_tiny_config_bit_exact():
    _check_full(W.make_config("tiny"))


EDGE = [
    # (B, H, Sq, Skv, D, causal, seed, kind)
    (1, 1, 1, 1, 64, False, 100, "normal"),
    (1, 1, 1, 1, 128, True, 101, "normal"),
    (1, 2, 15, 15, 64, True, 102, "normal"),
    (2, 1, 16, 16, 128, False, 103, "normal"),
    (1, 2, 17, 17, 64, True, 104, "channel_outliers"),
    (1, 3, 197, 197, 64, False, 105, "normal"),
    (1, 1, 257, 257, 128, True, 106, "student_t_tail"),
    (1, 2, 1000, 1000, 64, False, 107, "normal"),
    (1, 1, 1000, 1000, 128, True, 108, "normal"),
    (1, 2, 5, 300, 128, True, 109, "normal"),        # causal, Sq < Skv, bottom-right
    (2, 2, 130, 129, 64, False, 110, "normal"),       # Sq > Skv, non-causal
    (1, 1, 63, 200, 64, True, 111, "channel_outliers"),
    (1, 1, 129, 65, 128, False, 112, "normal"),
    (3, 1, 1, 777, 64, False, 113, "normal"),         # single query, ragged keys
    (2, 3, 1, 16384, 128, False, 114, "normal"),      # decode kernel, largest key count
    (1, 2, 1, 16385, 64, True, 115, "normal"),        # one key past it: general kernel
    (4, 2, 1, 255, 128, False, 116, "channel_outliers"),
    (1, 1, 1, 5, 64, False, 117, "student_t_tail"),
    # short-row block skipping: causal blocks past a query group's last row,
    # empty trailing query groups, key blocks past Skv
    (2, 2, 512, 512, 64, True, 118, "channel_outliers"),
    (1, 2, 100, 300, 64, True, 119, "normal"),
    (1, 2, 33, 40, 128, True, 120, "normal"),
    (2, 1, 70, 197, 64, False, 121, "normal"),
    (1, 1, 250, 250, 128, True, 122, "student_t_tail"),
]


@pytest.mark.parametrize("B,H,Sq,Skv,D,causal,seed,kind", EDGE)
def test_edge_shapes_bit_exact(B, H, Sq, Skv, D, causal, seed, kind):
    w = W.make_random(B, H, Sq, Skv, D, causal, seed, kind, name="edge")
    _check_full(w)


def _custom(q, k, v, scales, causal=False, name="custom"):
    B, H, Sq, D = q.shape
    return W.Workload(name, B, H, Sq, k.shape[2], D, causal, q, k, v, scales)


def test_constant_keys_uniform_rows():
    rng = np.random.default_rng(7)
    for n in (1, 2, 3, 64, 65, 512, 513, 700):
        q = rng.integers(-127, 128, (1, 1, 40, 64)).astype(np.int8)
        k = np.broadcast_to(rng.integers(-127, 128, 64).astype(np.int8), (1, 1, n, 64)).copy()
        v = rng.integers(-127, 128, (1, 1, n, 64)).astype(np.int8)
        _check_full(_custom(q, k, v, (0.02, 0.02, 0.01, 0.01), name=f"uniform{n}"))


def test_one_hot_rows():
    rng = np.random.default_rng(8)
    D, n = 128, 300
    q = np.zeros((1, 2, 20, D), dtype=np.int8)
    q[..., 0] = 127
    k = rng.integers(-10, 11, (1, 2, n, D)).astype(np.int8)
    k[..., 0] = rng.integers(-10, 11, (1, 2, n))
    k[0, 0, 123, 0] = 127
    k[0, 1, 7, 0] = 127
    v = rng.integers(-127, 128, (1, 2, n, D)).astype(np.int8)
    scales = (0.2, 0.2, 0.01, 0.01)
    prm = O.derive_params(D, *scales, O.DEFAULT_CLIP)
    assert 127 * 127 - 127 * 10 >= prm.x_clip          # the lead exceeds the clip gap
    w = _custom(q, k, v, scales, name="one_hot")
    _check_full(w)
    out = _run(w)
    assert (out[0, 0] == v[0, 0, 123][None, :]).all()
    assert (out[0, 1] == v[0, 1, 7][None, :]).all()


def test_scores_on_bin_edges():
    """M = 2^18 (mu = 2^-6) puts bin edges at relative scores 64k - 32 exactly."""
    rng = np.random.default_rng(9)
    D = 64
    q = np.zeros((1, 1, 3, D), dtype=np.int8)
    q[0, 0, :, 0] = [1, 2, -1]
    k = np.zeros((1, 1, 255, D), dtype=np.int8)
    k[0, 0, :, 0] = np.arange(-127, 128)
    v = rng.integers(-127, 128, (1, 1, 255, D)).astype(np.int8)
    scales = (2 ** -6, 2 ** -6, 0.01, 0.005)
    prm = O.derive_params(D, *scales, 31 * 2 ** -9)
    assert prm.idx_mul == 2 ** 18
    w = W.Workload("bin_edges", 1, 1, 3, 255, D, False, q, k, v, scales, 31 * 2 ** -9)
    _check_full(w)


LARGE_M_CASES = [
    # (Sq, Skv, D, causal, scale): every kernel family with M >= 2^21, where
    # the slot is computed from the clipped score instead of the saturating
    # multiply-add
    (40, 200, 64, False, 0.5),     # short-row kernel
    (130, 700, 64, True, 0.5),     # long-row kernel
    (70, 400, 128, False, 0.6),    # long-row kernel, d = 128
    (1, 1000, 64, False, 0.5),     # decode kernel
]


@pytest.mark.parametrize("Sq,Skv,D,causal,scale", LARGE_M_CASES)
def test_large_index_multiplier(Sq, Skv, D, causal, scale):
    rng = np.random.default_rng(1000 + Skv)
    q = rng.integers(-8, 9, (1, 2, Sq, D)).astype(np.int8)
    k = rng.integers(-8, 9, (1, 2, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 2, Skv, D)).astype(np.int8)
    scales = (scale, scale, 0.01, 0.01)
    prm = O.derive_params(D, *scales, float(O.DEFAULT_CLIP))
    assert prm.idx_mul >= 2 ** 21
    _check_full(_custom(q, k, v, scales, causal, name=f"largeM{Skv}"))


def test_repeat_launches_identical():
    w = W.make_random(2, 4, 300, 300, 64, False, 31, "channel_outliers", name="repeat")
    _say(f"case repeat shape={w.shape}")
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    outs = []
    for _ in range(10):
        outs.append(IA.forward(q, k, v, w.scales, w.clip, w.causal).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    _assert_equal("out", outs[0].cpu().numpy(), O.forward(w.q, w.k, w.v, w.scales, w.clip))


@pytest.mark.parametrize("name", ["bert", "vit"])
def test_config_full_bit_exact(name):
    _check_full(W.make_config(name), probs=False)


def test_llama_prefill_full_size_all_heads():
    """Full-size causal prefill (B=1, H=32, S=4096, d=128) on the GPU, every
    head compared with the oracle: the output of the plain launch, and the
    output and row state (m_i, E_i) of one debug launch over the same
    full-size workload (the launch configuration the benchmark times)."""
    w = W.make_config("llama_prefill")
    _say(f"case llama_prefill shape={w.shape}")
    out = _run(w)
    o2, rm, rs, _ = _run(w, debug=True)
    prm = O.derive_params(w.D, *w.scales, w.clip)
    for h in range(w.H):
        ref, m, E, _P = O.head_forward(w.q[0, h], w.k[0, h], w.v[0, h], prm, True)
        _assert_equal(f"out head {h}", out[0, h], ref)
        _assert_equal(f"out(debug) head {h}", o2[0, h], ref)
        _assert_equal(f"row_max head {h}", rm[0, h], m)
        _assert_equal(f"row_sum head {h}", rs[0, h], E)
    _say(f"llama_prefill: {w.H} of {w.H} heads bit-exact")


def test_decode_full_size_bit_exact():
    w = W.make_config("decode")
    _say(f"case decode shape={w.shape}")
    out = _run(w)
    ref, m, E, P = O.forward(w.q, w.k, w.v, w.scales, w.clip, False, stats=True)
    _assert_equal("out", out, ref)
    o2, rm, rs, _ = _run(w, debug=True)
    _assert_equal("row_max", rm, m)
    _assert_equal("row_sum", rs, E)
    # causal with Sq = 1 attends the whole cache: same result
    w2 = W.Workload("decode_causal", w.B, w.H, 1, w.Skv, w.D, True, w.q, w.k, w.v, w.scales, w.clip)
    _assert_equal("out(causal)", _run(w2), ref)
