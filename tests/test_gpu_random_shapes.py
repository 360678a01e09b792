"""Seeded random sweep over shapes and variants, GPU against the oracle.

Each case draws B, H, a K/V head count dividing H, Sq, Skv (and a cache
capacity at least Skv), d, causal, the table size, the probability width and
the table's entry width (Q15 or uint8),
so that every kernel (short rows, long rows, decode, with one or two query
heads a workgroup) and the edges between them are met: ragged query groups
and key blocks, a single key, a single query row, keys just past a block or
tile, caches larger than the attended prefix. Inputs come from the seeded
workload generator (normal, channel outliers, Student-t tails).

Bar: bit-exact out, row max and row sum on every element. Where the oracle
refuses the parameters (the table's index multiplier out of range for its
size), the library must refuse the same call.
"""
import numpy as np
import pytest
import torch

from oracle import intattn_oracle as O
from integer_only_quantized_amd import workloads as W

pytestmark = pytest.mark.gpu

IA = pytest.importorskip("integer_only_quantized_amd._binding")

KINDS = ["normal", "channel_outliers", "student_t_tail"]


def _case(i):
    rng = np.random.default_rng(9000 + i)
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    H = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.choice([h for h in (1, 2, 4) if H % h == 0]))
    form = i % 4
    if form == 0:                       # decode
        Sq = 1
        Skv = int(rng.integers(1, 3000))
    elif form == 1:                     # short rows
        Skv = int(rng.integers(1, (512 if D == 64 else 256) + 1))
        Sq = int(rng.integers(2, 300))
    else:                               # long rows (and anything in between)
        Skv = int(rng.integers(200, 1400))
        Sq = int(rng.integers(2, 400))
    causal = bool(rng.integers(0, 2)) and Sq <= Skv
    cap = Skv + int(rng.choice([0, 0, int(rng.integers(1, 200))]))
    lut = int(rng.choice([32, 32, 64, 128]))
    prob_bits = int(rng.choice([8, 8, 16]))
    kind = KINDS[i % 3]
    lut_bits = int(rng.choice([16, 16, 8]))
    return B, H, Hkv, Sq, Skv, cap, D, causal, lut, prob_bits, kind, lut_bits


CASES = [_case(i) for i in range(40)]


def _eq(name, got, ref):
    got, ref = np.asarray(got), np.asarray(ref)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{name}: {len(bad)} of {ref.size} differ; first at {bad[0].tolist()}: "
                             f"got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}")


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_shape_bit_exact(i):
    B, H, Hkv, Sq, Skv, cap, D, causal, lut, prob_bits, kind, lut_bits = CASES[i]
    print(f"case {i}: B={B} H={H} Hkv={Hkv} Sq={Sq} Skv={Skv} cap={cap} D={D} causal={causal} "
          f"lut={lut} prob_bits={prob_bits} kind={kind} lut_bits={lut_bits}", flush=True)
    w = W.make_random(B, H, Sq, cap, D, False, 9100 + i, kind, name="sweep")
    k = np.ascontiguousarray(w.k[:, :Hkv])
    v = np.ascontiguousarray(w.v[:, :Hkv])
    try:
        ref, m, E, _ = O.forward(w.q, k[:, :, :Skv], v[:, :, :Skv], w.scales, O.DEFAULT_CLIP, causal,
                                 stats=True, lut_size=lut, kv_heads=Hkv, prob_bits=prob_bits, lut_bits=lut_bits)
    except O.OracleRangeError:
        with pytest.raises(IA.IntAttnError):
            IA.forward_ex(torch.from_numpy(w.q).cuda(), torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                          w.scales, O.DEFAULT_CLIP, causal, lut, skv=Skv, prob_bits=prob_bits, lut_bits=lut_bits)
        return
    out, rm, rs = IA.forward_ex(torch.from_numpy(w.q).cuda(), torch.from_numpy(k).cuda(),
                                torch.from_numpy(v).cuda(), w.scales, O.DEFAULT_CLIP, causal, lut, stats=True,
                                skv=Skv, prob_bits=prob_bits, lut_bits=lut_bits)
    torch.cuda.synchronize()
    _eq("out", out.cpu().numpy(), ref)
    _eq("row_max", rm.cpu().numpy(), m)
    _eq("row_sum", rs.cpu().numpy().view(np.uint32), E * (128 if lut_bits == 8 else 1))   # Q15 units
