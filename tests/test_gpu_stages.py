"""GPU parity of the separate pipeline stages (scores and P in device memory).

Bar: Q.K^T scores, IndexSoftmax probabilities and row state, and P.V outputs
bit-exact against the oracle; the integer stages chained equal
intattn_forward. The floating-point comparator's uint8 codes within one code
of the oracle's float32 steps (exponential and summation order differ), with
P.V on those codes again bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import fp_baseline as F
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


def _check(w, heads=None):
    _say(f"case {w.name} shape={w.shape} causal={w.causal}")
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    S = IA.qk_scores(q, k)
    P, rm, rs = IA.index_softmax(S, w.D, w.scales, w.clip, w.causal, stats=True)
    out = IA.pv(P, v, w.scales, w.clip, w.causal)
    C = IA.fp_softmax(S, w.D, w.scales, w.causal)
    outc = IA.pv(C, v, w.scales, w.clip, w.causal)
    fused = IA.forward(q, k, v, w.scales, w.clip, w.causal)
    torch.cuda.synchronize()
    _eq("chain == forward", out.cpu().numpy(), fused.cpu().numpy())
    S, P, rm, rs = S.cpu().numpy(), P.cpu().numpy(), rm.cpu().numpy(), rs.cpu().numpy().view(np.uint32)
    C, out, outc = C.cpu().numpy(), out.cpu().numpy(), outc.cpu().numpy()
    prm = O.derive_params(w.D, *w.scales, w.clip)
    alpha = F.dequant_alpha(w.D, w.scales[0], w.scales[1])
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    worst, mism, total = 0, 0, 0
    for b, h in heads:
        Sr = O.qk_scores(w.q[b, h], w.k[b, h])
        _eq(f"scores {b},{h}", S[b, h], Sr)
        Pr, mr, Er = O.index_softmax(Sr, prm, w.causal)
        _eq(f"probs {b},{h}", P[b, h], Pr)
        _eq(f"row_max {b},{h}", rm[b, h], mr)
        _eq(f"row_sum {b},{h}", rs[b, h], Er)
        _eq(f"out {b},{h}", out[b, h], O.pv_requant(Pr, w.v[b, h], prm))
        Cr = F.fp_softmax_codes(Sr, alpha, w.causal).astype(np.int64)
        d = np.abs(C[b, h].astype(np.int64) - Cr)
        worst = max(worst, int(d.max()))
        mism += int((d != 0).sum())
        total += d.size
        _eq(f"out(fp codes) {b},{h}", outc[b, h], O.pv_requant(C[b, h], w.v[b, h], prm))
    assert worst <= 1, f"fp codes differ by {worst}"
    assert mism <= max(4, total // 100), f"{mism} of {total} fp codes differ"
    _say(f"  fp codes differing by one: {mism} of {total}")


def test_tiny_stages():
    _check(W.make_config("tiny"))


def test_bert_stages_all_heads():
    _check(W.make_config("bert"))


STAGE_CASES = [
    # (B, H, Sq, Skv, D, causal, seed, kind)
    (1, 2, 40, 197, 64, False, 300, "normal"),           # unaligned P rows (byte path)
    (2, 1, 130, 300, 128, True, 301, "channel_outliers"),  # causal, Sq < Skv, d = 128
    (1, 1, 1, 77, 64, False, 302, "normal"),             # one query row
    (1, 1, 257, 257, 128, True, 303, "student_t_tail"),
    (1, 1, 64, 4096, 64, True, 304, "normal"),           # longest row the stages hold
]


@pytest.mark.parametrize("B,H,Sq,Skv,D,causal,seed,kind", STAGE_CASES)
def test_stage_edge_shapes(B, H, Sq, Skv, D, causal, seed, kind):
    _check(W.make_random(B, H, Sq, Skv, D, causal, seed, kind, name="stage"))


def test_stages_large_index_multiplier():
    rng = np.random.default_rng(305)
    q = rng.integers(-8, 9, (1, 2, 50, 64)).astype(np.int8)
    k = rng.integers(-8, 9, (1, 2, 260, 64)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 2, 260, 64)).astype(np.int8)
    scales = (0.5, 0.5, 0.01, 0.01)
    assert O.derive_params(64, *scales, O.DEFAULT_CLIP).idx_mul >= 2 ** 21
    _check(W.Workload("stage_largeM", 1, 2, 50, 260, 64, False, q, k, v, scales))
