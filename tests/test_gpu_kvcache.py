"""GPU parity of the decode step around the attention: the K/V cache update
(intattn_kv_append) and attention over a cache prefix with grouped K/V heads
(intattn_forward_ex with kv_capacity > Skv).

Bar: bit-exact. The cache update against oracle/kv_cache.py byte for byte
over the whole cache (rows outside the update must not change), including
ties, saturation, infinities and NaN; attention against the oracle on the
attended prefix.
"""
import numpy as np
import pytest
import torch

from oracle import intattn_oracle as O
from oracle import kv_cache as KV

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


APPEND_CASES = [
    # (B, Hkv, T, D, capacity, pos)
    (16, 8, 1, 128, 64, 37),        # one decode token
    (2, 4, 33, 64, 100, 0),         # a chunk at the start
    (1, 8, 100, 128, 100, 0),       # fills the cache
    (3, 2, 7, 64, 50, 43),          # ends at the last row
    (1, 32, 512, 128, 1024, 300),   # a prefill-sized chunk
]


@pytest.mark.parametrize("B,Hkv,T,D,cap,pos", APPEND_CASES)
def test_kv_append_bit_exact(B, Hkv, T, D, cap, pos):
    _say(f"case append B={B} Hkv={Hkv} T={T} D={D} cap={cap} pos={pos}")
    rng = np.random.default_rng(B * 1000 + T + pos)
    kc = rng.integers(-127, 128, (B, Hkv, cap, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (B, Hkv, cap, D)).astype(np.int8)
    kn = (rng.standard_normal((B, Hkv, T, D)) * 1.7).astype(np.float32)
    vn = (rng.standard_normal((B, Hkv, T, D)) * 0.9).astype(np.float32)
    s_k, s_v = 0.021, 0.0093
    # exact ties under a power-of-two scale, saturation and non-finite values
    kn.reshape(-1)[:8] = np.array([0.5, 1.5, 2.5, -2.5, 126.5, -127.5, 300.0, -1e9], np.float32) * np.float32(s_k)
    vn.reshape(-1)[:4] = np.array([np.inf, -np.inf, np.nan, 1e38], np.float32)
    kd, vd = _dev(kc), _dev(vc)
    IA.kv_append(_dev(kn), _dev(vn), kd, vd, pos, s_k, s_v)
    torch.cuda.synchronize()
    kr, vr = KV.kv_append(kc, vc, kn, vn, pos, s_k, s_v)
    _eq("k cache", kd.cpu().numpy(), kr)
    _eq("v cache", vd.cpu().numpy(), vr)


def test_kv_append_power_of_two_ties():
    """Every half-integer multiple of a power-of-two scale: ties to even."""
    s = 2.0 ** -5
    vals = (np.arange(-260, 261) / 2.0).astype(np.float32) * np.float32(s)      # -130 .. 130 step 1/2
    n = vals.size
    D = 64
    T = (n + D - 1) // D
    kn = np.zeros((1, 1, T, D), np.float32)
    kn.reshape(-1)[:n] = vals
    kc = np.zeros((1, 1, T, D), np.int8)
    kd, vd = _dev(kc), _dev(kc.copy())
    IA.kv_append(_dev(kn), _dev(kn), kd, vd, 0, s, s)
    torch.cuda.synchronize()
    kr, _ = KV.kv_append(kc, kc, kn, kn, 0, s, s)
    _eq("ties", kd.cpu().numpy(), kr)


PREFIX_CASES = [
    # (B, H, Hkv, Sq, Skv, capacity, D, causal): decode, short and long rows
    (16, 32, 8, 1, 4097, 8192, 128, False),
    (4, 8, 1, 1, 300, 512, 64, False),
    (2, 8, 2, 64, 200, 256, 64, True),
    (1, 4, 2, 130, 900, 1024, 128, True),
]


@pytest.mark.parametrize("B,H,Hkv,Sq,Skv,cap,D,causal", PREFIX_CASES)
def test_attention_over_cache_prefix(B, H, Hkv, Sq, Skv, cap, D, causal):
    _say(f"case prefix B={B} H={H} Hkv={Hkv} Sq={Sq} Skv={Skv} cap={cap} D={D}")
    rng = np.random.default_rng(Skv + cap + H)
    q = rng.integers(-100, 101, (B, H, Sq, D)).astype(np.int8)
    kc = rng.integers(-100, 101, (B, Hkv, cap, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (B, Hkv, cap, D)).astype(np.int8)
    scales = (0.02, 0.02, 0.01, 0.003)
    out, rm, rs = IA.forward_ex(_dev(q), _dev(kc), _dev(vc), scales, O.DEFAULT_CLIP, causal, 32, stats=True,
                                skv=Skv)
    torch.cuda.synchronize()
    ref, m, E, _ = O.forward(q, kc[:, :, :Skv], vc[:, :, :Skv], scales, O.DEFAULT_CLIP, causal, stats=True,
                             kv_heads=Hkv)
    _eq("out", out.cpu().numpy(), ref)
    _eq("row_max", rm.cpu().numpy(), m)
    _eq("row_sum", rs.cpu().numpy().view(np.uint32), E)


def test_decode_steps_append_then_attend():
    """Three decode steps of a grouped-query decoder: append each new token's
    K/V to the cache, then attend over the filled prefix; each step equals the
    oracle on the oracle-updated cache."""
    B, H, Hkv, D, cap, filled = 4, 16, 4, 128, 256, 200
    rng = np.random.default_rng(77)
    kc = np.zeros((B, Hkv, cap, D), np.int8)
    vc = np.zeros((B, Hkv, cap, D), np.int8)
    kc[:, :, :filled] = rng.integers(-127, 128, (B, Hkv, filled, D))
    vc[:, :, :filled] = rng.integers(-127, 128, (B, Hkv, filled, D))
    s_q, s_k, s_v, s_o = 0.02, 0.02, 0.015, 0.004
    kd, vd = _dev(kc), _dev(vc)
    for step in range(3):
        pos = filled + step
        _say(f"case decode step {step} pos={pos}")
        kn = rng.standard_normal((B, Hkv, 1, D)).astype(np.float32)
        vn = rng.standard_normal((B, Hkv, 1, D)).astype(np.float32)
        q = rng.integers(-127, 128, (B, H, 1, D)).astype(np.int8)
        IA.kv_append(_dev(kn), _dev(vn), kd, vd, pos, s_k, s_v)
        out = IA.forward_ex(_dev(q), kd, vd, (s_q, s_k, s_v, s_o), O.DEFAULT_CLIP, False, 32, skv=pos + 1)
        torch.cuda.synchronize()
        kc, vc = KV.kv_append(kc, vc, kn, vn, pos, s_k, s_v)
        ref = O.forward(q, kc[:, :, :pos + 1], vc[:, :, :pos + 1], (s_q, s_k, s_v, s_o), O.DEFAULT_CLIP,
                        False, kv_heads=Hkv)
        _eq(f"step {step} cache", kd.cpu().numpy(), kc)
        _eq(f"step {step} out", out.cpu().numpy(), ref)
