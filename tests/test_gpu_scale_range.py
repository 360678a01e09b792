"""GPU parity across the whole accepted range of the bin multiplier
mu = alpha / delta in [2^-24, 2^14).

Below mu = 1/2 every kernel takes the table slot from the saturating slot
word (or the row-constant form); from 1/2 on a score unit moves half a bin or
more, the clip point is at most 2N - 3 units from the row max, and the
kernels index a table by the clipped score gap itself. Bar: bit-exact against
the oracle (out, row max, row sum; P where a path writes it) on every kernel
family: short rows, long rows (causal), decode, decode with keys split over
workgroups, the debug path that writes P, and the separate IndexSoftmax stage;
table sizes 32, 64 and 128, uint8 table entries and uint16 probabilities; and
the causal-prefill workload with a 128-entry table (mu ~ 0.9 there), every
head at full size.
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


def _scale_for(mu, D, n):
    """s (= s_q = s_k) giving bin multiplier mu for head size D and n entries."""
    delta = O.DEFAULT_CLIP / (n - 1)
    return float(np.float32(np.sqrt(mu * delta * np.sqrt(D))))


def _inputs(B, H, Sq, Skv, D, seed, amp):
    rng = np.random.default_rng(seed)
    q = rng.integers(-amp, amp + 1, (B, H, Sq, D)).astype(np.int8)
    k = rng.integers(-amp, amp + 1, (B, H, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (B, H, Skv, D)).astype(np.int8)
    return q, k, v


def _check(q, k, v, scales, causal, n, label, prob_bits=8, lut_bits=16, workspace=None):
    prm = O.derive_params(q.shape[3], *scales, O.DEFAULT_CLIP, n, prob_bits, lut_bits)
    _say(f"case {label} q={q.shape} kv={k.shape} causal={causal} lut={n} mu={prm.mu:.4g} sh={prm.idx_shift} "
         f"x_clip={prm.x_clip} prob_bits={prob_bits} lut_bits={lut_bits}")
    kw = {} if workspace is None else {"workspace": workspace}
    out, rm, rs = IA.forward_ex(_dev(q), _dev(k), _dev(v), scales, O.DEFAULT_CLIP, causal, n, stats=True,
                                prob_bits=prob_bits, lut_bits=lut_bits, **kw)
    torch.cuda.synchronize()
    ref, m, E, _ = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True, lut_size=n,
                             prob_bits=prob_bits, lut_bits=lut_bits)
    _eq(f"{label} out", out.cpu().numpy(), ref)
    _eq(f"{label} row_max", rm.cpu().numpy(), m)
    E_dev = rs.cpu().numpy().view(np.uint32).astype(np.int64)
    _eq(f"{label} row_sum", E_dev, E * 128 if lut_bits == 8 else E)
    return prm


# (B, H, Sq, Skv, D, causal): short rows, long rows, decode
SHAPES = [
    (2, 2, 128, 197, 64, False),
    (1, 2, 100, 256, 128, True),
    (1, 2, 300, 700, 64, True),
    (1, 1, 257, 600, 128, False),
    (4, 2, 1, 3000, 128, False),
    (2, 3, 1, 513, 64, False),
]
# both sides of mu = 1/2, then up to the top of the range
MUS = [0.4999, 0.5001, 0.62, 3.3, 47.0, 2500.0, 16000.0]


@pytest.mark.parametrize("mu", MUS)
@pytest.mark.parametrize("n", [32, 64, 128])
def test_large_multiplier_every_kernel(n, mu):
    for i, (B, H, Sq, Skv, D, causal) in enumerate(SHAPES):
        s = _scale_for(mu, D, n)
        # small integers keep score gaps near the clip point, so rows are not one-hot
        q, k, v = _inputs(B, H, Sq, Skv, D, 1000 + 7 * i, 3)
        prm = _check(q, k, v, (s, s, 0.05, 0.02), causal, n, f"mu~{mu}")
        assert (prm.idx_shift < 24) == (prm.mu >= 0.5)


@pytest.mark.parametrize("mu", [2.0 ** -24 * 1.01, 2.0 ** -23, 3e-7, 2.0 ** -20, 2.0 ** -17, 2.0 ** -16 * 0.99])
@pytest.mark.parametrize("n", [32, 64, 128])
def test_small_multiplier_every_kernel(n, mu):
    """Multipliers below 2^-16 (M below 256): masked and padded keys (causal
    rows, key blocks past Skv) no longer saturate the slot word and land on
    a slot no allowed key reaches, whose entry is 0."""
    for i, (B, H, Sq, Skv, D, causal) in enumerate(SHAPES):
        s = _scale_for(mu, D, n)
        q, k, v = _inputs(B, H, Sq, Skv, D, 2000 + 7 * i, 127)
        prm = _check(q, k, v, (s, s, 0.05, 0.02), causal, n, f"mu~{mu:.3g}")
        assert prm.idx_shift == 24 and prm.idx_mul <= 256


@pytest.mark.parametrize("prob_bits,lut_bits", [(16, 16), (8, 8), (16, 8)])
def test_large_multiplier_variants(prob_bits, lut_bits):
    for i, (B, H, Sq, Skv, D, causal) in enumerate(SHAPES):
        for n, mu in ((32, 0.7), (128, 5.0)):
            s = _scale_for(mu, D, n)
            q, k, v = _inputs(B, H, Sq, Skv, D, 3000 + 7 * i, 3)
            _check(q, k, v, (s, s, 0.05, 0.0002 if prob_bits == 16 else 0.02), causal, n,
                   f"mu~{mu} variant", prob_bits, lut_bits)


def test_large_multiplier_split_decode():
    """Keys split over workgroups (caller workspace): past 16384 keys, and
    few heads for the cache length (Skv >= 4096 and Skv > 128 B H)."""
    for (B, H, Skv, D), n, mu in (((1, 4, 20000, 128), 32, 0.9), ((1, 2, 5000, 64), 128, 12.0)):
        s = _scale_for(mu, D, n)
        q, k, v = _inputs(B, H, 1, Skv, D, 4000 + Skv, 3)
        ws = torch.empty(IA.workspace_bytes(B, H, 1, Skv, D), dtype=torch.uint8, device="cuda")
        assert ws.numel() > 0
        _check(q, k, v, (s, s, 0.05, 0.02), False, n, "split decode", workspace=ws)


def test_large_multiplier_debug_probs_and_stage():
    """The path that writes P (debug) and the separate IndexSoftmax stage
    (32-entry table), P compared element by element."""
    for i, (B, H, Sq, Skv, D, causal) in enumerate([(1, 2, 70, 300, 64, True), (2, 1, 33, 129, 128, False)]):
        for mu in (0.55, 9.0, 2.0 ** -24 * 1.01, 2.0 ** -20):
            s = _scale_for(mu, D, 32)
            scales = (s, s, 0.05, 0.02)
            q, k, v = _inputs(B, H, Sq, Skv, D, 5000 + 7 * i, 3 if mu > 0.1 else 127)
            w = W.Workload("largeM", B, H, Sq, Skv, D, causal, q, k, v, scales)
            _say(f"case debug/stage mu~{mu} q={q.shape} Skv={Skv} causal={causal}")
            ref, m, E, P = O.forward(q, k, v, scales, O.DEFAULT_CLIP, causal, stats=True)
            out, rm, rs, pr = IA.forward_debug(_dev(q), _dev(k), _dev(v), scales, O.DEFAULT_CLIP, causal,
                                               with_probs=True)
            torch.cuda.synchronize()
            _eq("debug out", out.cpu().numpy(), ref)
            _eq("debug P", pr.cpu().numpy(), P)
            _eq("debug row_sum", rs.cpu().numpy().view(np.uint32).astype(np.int64), E)
            S = IA.qk_scores(_dev(q), _dev(k))
            P2, rm2, rs2 = IA.index_softmax(S, D, scales, O.DEFAULT_CLIP, causal, stats=True)
            torch.cuda.synchronize()
            _eq("stage P", P2.cpu().numpy(), P)
            _eq("stage row_max", rm2.cpu().numpy(), m)
            _eq("stage row_sum", rs2.cpu().numpy().view(np.uint32).astype(np.int64), E)
            assert w.shape == (B, H, Sq, Skv, D)


def test_prefill_workload_128_entry_table_all_heads():
    """The causal-prefill workload (B=1, H=32, S=4096, d=128) with a 128-entry
    table: mu ~ 0.9 on its scales, the direct table, every head compared."""
    w = W.make_config("llama_prefill")
    prm = O.derive_params(w.D, *w.scales, w.clip, 128)
    _say(f"case llama_prefill lut=128 mu={prm.mu:.4g} sh={prm.idx_shift} x_clip={prm.x_clip}")
    assert prm.mu >= 0.5
    out, rm, rs = IA.forward_ex(_dev(w.q), _dev(w.k), _dev(w.v), w.scales, w.clip, True, 128, stats=True)
    torch.cuda.synchronize()
    out, rm, rs = out.cpu().numpy(), rm.cpu().numpy(), rs.cpu().numpy().view(np.uint32).astype(np.int64)
    for h in range(w.H):
        ref, m, E, _ = O.head_forward(w.q[0, h], w.k[0, h], w.v[0, h], prm, True)
        _eq(f"out head {h}", out[0, h], ref)
        _eq(f"row_max head {h}", rm[0, h], m)
        _eq(f"row_sum head {h}", rs[0, h], E)
