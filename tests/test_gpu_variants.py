"""GPU parity of the variants through intattn_forward_ex: finer exp tables (64
and 128 entries), grouped K/V heads (grouped-query / multi-query) and uint16
probabilities.

Bar: bit-exact against the oracle (out, row max, row sum) on every kernel
family: short rows (K/V of a head in LDS), long rows (tiled, three passes),
decode (one query row), each with the slot-word scale k the host picks
(4, 2 or 1 as the multiplier grows).
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


def _eq(name, got, ref):
    got, ref = np.asarray(got), np.asarray(ref)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{name}: {len(bad)} of {ref.size} differ; first at {bad[0].tolist()}: "
                             f"got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}")


def _run(q, k, v, scales, causal, lut_size, label):
    H, Hkv = q.shape[1], k.shape[1]
    _say(f"case {label} q={q.shape} kv={k.shape} causal={causal} lut={lut_size}")
    out, rm, rs = IA.forward_ex(_dev(q), _dev(k), _dev(v), scales, O.DEFAULT_CLIP, causal, lut_size, stats=True)
    torch.cuda.synchronize()
    ref, m, E, _ = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True, lut_size=lut_size,
                             kv_heads=Hkv)
    _eq(f"{label} out", out.cpu().numpy(), ref)
    _eq(f"{label} row_max", rm.cpu().numpy(), m)
    _eq(f"{label} row_sum", rs.cpu().numpy().view(np.uint32), E)
    return ref


FINE_CASES = [
    # (B, H, Sq, Skv, D, causal, seed, kind): short, long, decode; ragged tails
    (2, 2, 128, 128, 64, False, 400, "normal"),
    (1, 2, 197, 197, 64, False, 401, "channel_outliers"),
    (1, 2, 100, 256, 128, True, 402, "student_t_tail"),
    (1, 2, 300, 700, 64, True, 403, "normal"),
    (1, 2, 257, 600, 128, False, 404, "channel_outliers"),
    (4, 2, 1, 3000, 128, False, 405, "normal"),
    (2, 2, 1, 513, 64, False, 406, "student_t_tail"),
]


@pytest.mark.parametrize("n", [64, 128])
@pytest.mark.parametrize("B,H,Sq,Skv,D,causal,seed,kind", FINE_CASES)
def test_fine_table_bit_exact(n, B, H, Sq, Skv, D, causal, seed, kind):
    w = W.make_random(B, H, Sq, Skv, D, causal, seed, kind, name="fine")
    _run(w.q, w.k, w.v, w.scales, causal, n, f"fine{n}")


def test_table_32_through_forward_ex_equals_forward():
    w = W.make_random(2, 2, 150, 300, 64, True, 407, "normal", name="ex32")
    out = _run(w.q, w.k, w.v, w.scales, True, 32, "ex32")
    got = IA.forward(_dev(w.q), _dev(w.k), _dev(w.v), w.scales, w.clip, True).cpu().numpy()
    _eq("forward == forward_ex", got, out)


SCALE_K_CASES = [
    # (lut_size, scale, k the host picks): the saturating slot word scaled by
    # the largest k with k*M < 2^23 (4 -> 2 -> 1 as mu grows)
    (32, 0.5, 2), (32, 0.7, 1), (64, 0.35, 2), (64, 0.5, 1), (128, 0.3, 1),
]


@pytest.mark.parametrize("n,scale,kexp", SCALE_K_CASES)
@pytest.mark.parametrize("Sq,Skv,D,causal", [(40, 200, 64, False), (130, 700, 64, True), (1, 900, 64, False)])
def test_slot_scale_choices(n, scale, kexp, Sq, Skv, D, causal):
    rng = np.random.default_rng(int(scale * 100) + n + Skv)
    q = rng.integers(-8, 9, (1, 2, Sq, D)).astype(np.int8)
    k = rng.integers(-8, 9, (1, 2, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 2, Skv, D)).astype(np.int8)
    scales = (scale, scale, 0.01, 0.01)
    prm = O.derive_params(D, *scales, O.DEFAULT_CLIP, n)
    kk = 128 // n
    while kk > 1 and kk * prm.idx_mul >= 2 ** 23:
        kk //= 2
    assert kk == kexp
    _run(q, k, v, scales, causal, n, f"k{kexp}_n{n}")


GQA_CASES = [
    # (B, H, Hkv, Sq, Skv, D, causal, lut): grouped-query and multi-query
    (2, 8, 2, 128, 128, 64, False, 32),
    (1, 8, 1, 200, 256, 128, True, 32),
    (1, 4, 2, 300, 1000, 128, True, 64),
    (1, 6, 3, 257, 600, 64, False, 128),
    (4, 32, 8, 1, 2048, 128, False, 32),
    (2, 8, 1, 1, 777, 64, False, 128),
    # decode with at least 512 query heads in pairs: two query heads of one
    # K/V head a workgroup (K and V read once for both)
    (16, 32, 8, 1, 3000, 128, False, 32),
    (32, 16, 2, 1, 8192, 64, False, 64),
    (16, 32, 1, 1, 1001, 128, False, 128),
]


@pytest.mark.parametrize("B,H,Hkv,Sq,Skv,D,causal,lut", GQA_CASES)
def test_grouped_kv_heads_bit_exact(B, H, Hkv, Sq, Skv, D, causal, lut):
    w = W.make_random(B, H, Sq, Skv, D, causal, 500 + H + Hkv + Skv, "normal", name="gqa")
    # K/V with Hkv heads (the first Hkv of the generated ones)
    k = np.ascontiguousarray(w.k[:, :Hkv])
    v = np.ascontiguousarray(w.v[:, :Hkv])
    _run(w.q, k, v, w.scales, causal, lut, f"gqa{H}x{Hkv}")


def test_bert_size_fine_table_all_heads():
    """BERT shape (8 x 12 x 512 x 64) with 128 entries: the launch the
    variant benchmark times, every row of every head compared."""
    w = W.make_config("bert")
    _say("case bert lut=128")
    out, rm, rs = IA.forward_ex(_dev(w.q), _dev(w.k), _dev(w.v), w.scales, w.clip, False, 128, stats=True)
    torch.cuda.synchronize()
    out, rm, rs = out.cpu().numpy(), rm.cpu().numpy(), rs.cpu().numpy().view(np.uint32)
    prm = O.derive_params(w.D, *w.scales, w.clip, 128)
    for b, h in [(b, h) for b in range(w.B) for h in range(w.H)]:
        ref, m, E, _ = O.head_forward(w.q[b, h], w.k[b, h], w.v[b, h], prm, False)
        _eq(f"bert128 out {b},{h}", out[b, h], ref)
        _eq(f"bert128 m {b},{h}", rm[b, h], m)
        _eq(f"bert128 E {b},{h}", rs[b, h], E)


P16_CASES = [
    # (B, H, Hkv, Sq, Skv, D, causal, lut, seed, kind): uint16 probabilities on
    # the long-row kernel (longer rows), the decode kernel (Sq = 1) and, below,
    # the short-row kernel
    (2, 2, 2, 128, 128, 64, False, 32, 600, "normal"),
    (1, 2, 2, 197, 197, 64, False, 64, 601, "channel_outliers"),
    (1, 2, 2, 300, 1100, 128, True, 32, 602, "student_t_tail"),
    (1, 4, 2, 257, 700, 64, True, 32, 603, "normal"),
    (4, 8, 2, 1, 8192, 128, False, 32, 604, "normal"),
    (2, 2, 2, 1, 3001, 64, False, 64, 605, "channel_outliers"),
    (1, 2, 1, 1, 777, 128, True, 128, 606, "normal"),
    # the decode kernel's largest key count (96 KB of LDS with uint16 P), and
    # one key past it (without a workspace: the three-pass decode kernel)
    (1, 2, 2, 1, 16384, 128, False, 32, 608, "normal"),
    (1, 2, 1, 1, 16385, 64, False, 32, 609, "student_t_tail"),
    # the short-row kernel (Skv <= 512 at d = 64, <= 256 at d = 128): full
    # rows, ragged tails, causal block skipping, grouped K/V heads, every
    # table size
    (2, 3, 3, 512, 512, 64, False, 32, 610, "channel_outliers"),
    (1, 4, 2, 197, 197, 64, False, 32, 611, "normal"),
    (2, 2, 2, 300, 300, 64, True, 128, 612, "student_t_tail"),
    (1, 2, 2, 33, 40, 128, True, 64, 613, "normal"),
    (2, 2, 1, 256, 256, 128, False, 32, 614, "channel_outliers"),
    (1, 2, 2, 70, 197, 64, False, 32, 615, "normal"),
    (1, 1, 1, 1000, 480, 64, False, 32, 616, "normal"),
]


@pytest.mark.parametrize("B,H,Hkv,Sq,Skv,D,causal,lut,seed,kind", P16_CASES)
def test_uint16_probabilities_bit_exact(B, H, Hkv, Sq, Skv, D, causal, lut, seed, kind):
    w = W.make_random(B, H, Sq, Skv, D, causal, seed, kind, name="p16")
    k = np.ascontiguousarray(w.k[:, :Hkv])
    v = np.ascontiguousarray(w.v[:, :Hkv])
    _say(f"case p16 q={w.q.shape} kv={k.shape} causal={causal} lut={lut}")
    out, rm, rs = IA.forward_ex(_dev(w.q), _dev(k), _dev(v), w.scales, O.DEFAULT_CLIP, causal, lut, stats=True,
                                prob_bits=16)
    torch.cuda.synchronize()
    ref, m, E, _ = O.forward(w.q, k, v, w.scales, O.DEFAULT_CLIP, causal, stats=True, lut_size=lut, kv_heads=Hkv,
                             prob_bits=16)
    _eq("p16 out", out.cpu().numpy(), ref)
    _eq("p16 row_max", rm.cpu().numpy(), m)
    _eq("p16 row_sum", rs.cpu().numpy().view(np.uint32), E)


def test_uint16_probabilities_bert_size_all_heads():
    """BERT shape (8 x 12 x 512 x 64) with uint16 probabilities on the
    short-row kernel, every head against the oracle."""
    w = W.make_config("bert")
    _say("case bert prob_bits=16")
    s16 = w.scales
    out, rm, rs = IA.forward_ex(_dev(w.q), _dev(w.k), _dev(w.v), s16, w.clip, False, 32, stats=True, prob_bits=16)
    torch.cuda.synchronize()
    out, rm, rs = out.cpu().numpy(), rm.cpu().numpy(), rs.cpu().numpy().view(np.uint32)
    prm = O.derive_params(w.D, *s16, w.clip, 32, 16)
    for b, h in [(b, h) for b in range(w.B) for h in range(w.H)]:
        ref, m, E, _ = O.head_forward(w.q[b, h], w.k[b, h], w.v[b, h], prm, False)
        _eq(f"bert p16 out {b},{h}", out[b, h], ref)
        _eq(f"bert p16 m {b},{h}", rm[b, h], m)
        _eq(f"bert p16 E {b},{h}", rs[b, h], E)


def test_uint16_probabilities_single_key_returns_v():
    """One key (Skv = 1, the decode kernel): p = 65535 and, with s_o = s_v,
    out = v exactly on the device as in the oracle."""
    rng = np.random.default_rng(607)
    q = rng.integers(-127, 128, (1, 2, 1, 128)).astype(np.int8)
    k = rng.integers(-127, 128, (1, 2, 1, 128)).astype(np.int8)
    v = np.tile(np.arange(-64, 64, dtype=np.int8), (1, 2, 1, 1))
    out = IA.forward_ex(_dev(q), _dev(k), _dev(v), (0.02, 0.02, 0.01, 0.01), O.DEFAULT_CLIP, False, 32, prob_bits=16)
    torch.cuda.synchronize()
    _eq("single key", out.cpu().numpy(), v)


# ---------------------------------------------------------------------------
# uint8 table entries (reach the kernels as 128 e8 in the Q15 slots)
# ---------------------------------------------------------------------------
LUT8_CASES = [
    # (B, H, Hkv, Sq, Skv, D, causal, lut, prob_bits, seed, kind): short rows,
    # long rows and decode (one and two query heads a workgroup), uint8 and
    # uint16 probabilities
    (2, 2, 2, 128, 128, 64, False, 32, 8, 700, "normal"),
    (1, 2, 2, 197, 197, 64, False, 32, 8, 701, "channel_outliers"),
    (1, 2, 2, 100, 256, 128, True, 64, 8, 702, "student_t_tail"),
    (1, 2, 2, 300, 1100, 128, True, 32, 8, 703, "normal"),
    (1, 4, 2, 257, 700, 64, False, 128, 8, 704, "channel_outliers"),
    (4, 2, 2, 1, 3000, 128, False, 32, 8, 705, "normal"),
    (16, 32, 8, 1, 3000, 128, False, 32, 8, 706, "student_t_tail"),
    (1, 2, 2, 300, 1100, 128, True, 32, 16, 707, "normal"),
    (4, 8, 2, 1, 4096, 128, False, 64, 16, 708, "channel_outliers"),
    (2, 2, 2, 200, 512, 64, False, 32, 16, 709, "channel_outliers"),
    (1, 2, 2, 130, 130, 128, True, 128, 16, 710, "student_t_tail"),
]


def _run8(q, k, v, scales, causal, lut, prob_bits, label):
    Hkv = k.shape[1]
    _say(f"case {label} q={q.shape} kv={k.shape} causal={causal} lut={lut} prob_bits={prob_bits} lut_bits=8")
    out, rm, rs = IA.forward_ex(_dev(q), _dev(k), _dev(v), scales, O.DEFAULT_CLIP, causal, lut, stats=True,
                                prob_bits=prob_bits, lut_bits=8)
    torch.cuda.synchronize()
    ref, m, E8, _ = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True, lut_size=lut, kv_heads=Hkv,
                              prob_bits=prob_bits, lut_bits=8)
    rs = rs.cpu().numpy().view(np.uint32)
    _eq(f"{label} out", out.cpu().numpy(), ref)
    _eq(f"{label} row_max", rm.cpu().numpy(), m)
    _eq(f"{label} row_sum", rs, 128 * E8)        # the row sum in Q15 units
    return rs


@pytest.mark.parametrize("B,H,Hkv,Sq,Skv,D,causal,lut,prob_bits,seed,kind", LUT8_CASES)
def test_uint8_table_bit_exact(B, H, Hkv, Sq, Skv, D, causal, lut, prob_bits, seed, kind):
    w = W.make_random(B, H, Sq, Skv, D, causal, seed, kind, name="lut8")
    k = np.ascontiguousarray(w.k[:, :Hkv])
    v = np.ascontiguousarray(w.v[:, :Hkv])
    _run8(w.q, k, v, w.scales, causal, lut, prob_bits, "lut8")


@pytest.mark.parametrize("B,H,Sq,Skv,D,prob_bits", [
    (2, 2, 64, 300, 64, 8), (1, 2, 100, 256, 128, 8), (1, 2, 300, 1100, 128, 8),
    (4, 4, 1, 1000, 128, 8), (1, 2, 300, 1100, 128, 16), (4, 4, 1, 1000, 64, 16)])
def test_uint8_table_one_hot_rows(B, H, Sq, Skv, D, prob_bits):
    """Every row has one key far above the rest (a key equal to 127 times the
    signs of its query, every other key within +-2), so every other key is
    clipped and E8 = 255: the smallest row sum, where the short-row kernel's
    reciprocal reaches 2^16 and is clamped. Bit-exact, and every row sum is
    128 * 255."""
    rng = np.random.default_rng(710 + Skv + D)
    q = rng.integers(-127, 128, (B, H, Sq, D)).astype(np.int8)
    q[q == 0] = 1
    k = rng.integers(-2, 3, (B, H, Skv, D)).astype(np.int8)
    hot = rng.permutation(Skv)[:Sq]
    for i in range(Sq):
        k[:, :, hot[i]] = (127 * np.sign(q[:, :, i])).astype(np.int8)
    v = rng.integers(-127, 128, (B, H, Skv, D)).astype(np.int8)
    rs = _run8(q, k, v, (0.02, 0.02, 0.05, 0.05), False, 32, prob_bits, "lut8 one-hot")
    assert (rs == 128 * 255).all()


# ---------------------------------------------------------------------------
# Decode over long caches: keys split over several workgroups per head
# ---------------------------------------------------------------------------
SPLIT_CASES = [
    # (B, H, Hkv, Skv, D, lut, prob_bits, lut_bits, cap_extra, seed, kind): one key past the
    # decode kernel's limit, ragged last chunks, the largest cache, grouped
    # heads, cache prefixes, every table and probability width
    (2, 4, 4, 16385, 128, 32, 8, 16, 0, 900, "normal"),
    (1, 2, 2, 65535, 128, 32, 8, 16, 0, 901, "channel_outliers"),
    (2, 8, 2, 20000, 64, 64, 8, 16, 37, 902, "student_t_tail"),
    (1, 4, 1, 33000, 128, 128, 16, 16, 0, 903, "normal"),
    (2, 4, 2, 24577, 64, 32, 16, 8, 100, 904, "channel_outliers"),
    (1, 2, 2, 40960, 128, 32, 8, 8, 0, 905, "student_t_tail"),
    # few heads over shorter caches: the decode kernel would run one
    # workgroup per head, so the keys are split (chunks down to 512 keys)
    (1, 32, 8, 8192, 128, 32, 8, 16, 0, 906, "normal"),
    (1, 4, 4, 5000, 128, 64, 16, 16, 0, 907, "channel_outliers"),
    (1, 2, 1, 4100, 64, 32, 8, 8, 7, 908, "student_t_tail"),
]


@pytest.mark.parametrize("B,H,Hkv,Skv,D,lut,prob_bits,lut_bits,cap_extra,seed,kind", SPLIT_CASES)
def test_split_decode_bit_exact(B, H, Hkv, Skv, D, lut, prob_bits, lut_bits, cap_extra, seed, kind):
    w = W.make_random(B, H, 1, Skv + cap_extra, D, False, seed, kind, name="split")
    k = np.ascontiguousarray(w.k[:, :Hkv])
    v = np.ascontiguousarray(w.v[:, :Hkv])
    _say(f"case split B={B} H={H} Hkv={Hkv} Skv={Skv} cap={Skv + cap_extra} D={D} lut={lut} "
         f"prob_bits={prob_bits} lut_bits={lut_bits}")
    assert IA.workspace_bytes(B, H, 1, Skv, D) > 0
    out, rm, rs = IA.forward_ex(_dev(w.q), _dev(k), _dev(v), w.scales, O.DEFAULT_CLIP, False, lut, stats=True,
                                skv=Skv, prob_bits=prob_bits, lut_bits=lut_bits)
    torch.cuda.synchronize()
    ref, m, E, _ = O.forward(w.q, k[:, :, :Skv], v[:, :, :Skv], w.scales, O.DEFAULT_CLIP, False, stats=True,
                             lut_size=lut, kv_heads=Hkv, prob_bits=prob_bits, lut_bits=lut_bits)
    _eq("split out", out.cpu().numpy(), ref)
    _eq("split row_max", rm.cpu().numpy(), m)
    _eq("split row_sum", rs.cpu().numpy().view(np.uint32), E * (128 if lut_bits == 8 else 1))
    # the same call without a workspace (one workgroup per head) agrees, and a second
    # call through the same workspace gives the same result (accumulators cleared)
    ws = torch.empty(IA.workspace_bytes(B, H, 1, Skv, D), dtype=torch.uint8, device="cuda")
    qd, kd, vd = _dev(w.q), _dev(k), _dev(v)
    a = IA.forward_ex(qd, kd, vd, w.scales, O.DEFAULT_CLIP, False, lut, skv=Skv, prob_bits=prob_bits,
                      lut_bits=lut_bits, workspace=ws)
    b = IA.forward_ex(qd, kd, vd, w.scales, O.DEFAULT_CLIP, False, lut, skv=Skv, prob_bits=prob_bits,
                      lut_bits=lut_bits, workspace=ws)
    c = IA.forward_ex(qd, kd, vd, w.scales, O.DEFAULT_CLIP, False, lut, skv=Skv, prob_bits=prob_bits,
                      lut_bits=lut_bits, workspace=False)
    torch.cuda.synchronize()
    _eq("split repeat", b.cpu().numpy(), a.cpu().numpy())
    _eq("split vs the call without a workspace", c.cpu().numpy(), ref)
    _eq("split through a given workspace", a.cpu().numpy(), ref)


# Decode past 16384 keys without a workspace: one workgroup per head, K
# streamed three times, P formed chunk by chunk (8192 keys) in LDS.
LONG_DECODE_CASES = [
    # (B, H, Hkv, Skv, D, lut, prob_bits, lut_bits, cap_extra, seed, kind): one key past the
    # decode kernel's limit, a ragged last chunk, exactly two chunks, the largest cache,
    # grouped heads, cache prefixes, every table and probability width
    (2, 3, 3, 16385, 128, 32, 8, 16, 0, 950, "normal"),
    (1, 4, 2, 16384 + 255, 64, 32, 8, 16, 33, 951, "channel_outliers"),
    (1, 2, 1, 3 * 8192, 128, 64, 8, 8, 0, 952, "student_t_tail"),
    (1, 2, 2, 65535, 128, 32, 8, 16, 0, 953, "normal"),
    (2, 4, 1, 30001, 64, 128, 16, 16, 5, 954, "channel_outliers"),
    (1, 3, 3, 40961, 128, 32, 16, 8, 0, 955, "student_t_tail"),
]


@pytest.mark.parametrize("B,H,Hkv,Skv,D,lut,prob_bits,lut_bits,cap_extra,seed,kind", LONG_DECODE_CASES)
def test_long_decode_without_workspace_bit_exact(B, H, Hkv, Skv, D, lut, prob_bits, lut_bits, cap_extra, seed,
                                                 kind):
    w = W.make_random(B, H, 1, Skv + cap_extra, D, False, seed, kind, name="longdec")
    k = np.ascontiguousarray(w.k[:, :Hkv])
    v = np.ascontiguousarray(w.v[:, :Hkv])
    _say(f"case long decode B={B} H={H} Hkv={Hkv} Skv={Skv} cap={Skv + cap_extra} D={D} lut={lut} "
         f"prob_bits={prob_bits} lut_bits={lut_bits}")
    out, rm, rs = IA.forward_ex(_dev(w.q), _dev(k), _dev(v), w.scales, O.DEFAULT_CLIP, False, lut, stats=True,
                                skv=Skv, prob_bits=prob_bits, lut_bits=lut_bits, workspace=False)
    torch.cuda.synchronize()
    ref, m, E, _ = O.forward(w.q, k[:, :, :Skv], v[:, :, :Skv], w.scales, O.DEFAULT_CLIP, False, stats=True,
                             lut_size=lut, kv_heads=Hkv, prob_bits=prob_bits, lut_bits=lut_bits)
    _eq("long decode out", out.cpu().numpy(), ref)
    _eq("long decode row_max", rm.cpu().numpy(), m)
    _eq("long decode row_sum", rs.cpu().numpy().view(np.uint32), E * (128 if lut_bits == 8 else 1))


def test_long_decode_plain_entry_point_and_debug():
    """intattn_forward and intattn_forward_debug (no workspace argument) on
    a 20000-key decode: the same bits as the oracle, row statistics too."""
    w = W.make_random(2, 4, 1, 20000, 128, False, 960, "normal", name="longdec")
    _say("case long decode plain/debug B=2 H=4 Skv=20000 D=128")
    ref, m, E, _ = O.forward(w.q, w.k, w.v, w.scales, O.DEFAULT_CLIP, False, stats=True)
    out = IA.forward(_dev(w.q), _dev(w.k), _dev(w.v), w.scales, O.DEFAULT_CLIP, False)
    o2, rm, rs, pr = IA.forward_debug(_dev(w.q), _dev(w.k), _dev(w.v), w.scales, O.DEFAULT_CLIP, False)
    torch.cuda.synchronize()
    assert pr is None
    _eq("plain out", out.cpu().numpy(), ref)
    _eq("debug out", o2.cpu().numpy(), ref)
    _eq("debug row_max", rm.cpu().numpy(), m)
    _eq("debug row_sum", rs.cpu().numpy().view(np.uint32), E)
