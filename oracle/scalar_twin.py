"""Brute-force twin of the oracle: explicit loops, Python ints and Fractions.

TEST INFRASTRUCTURE ONLY (same rules as intattn_oracle: only tests, the
smoke check and the benchmark's CPU-baseline leg may import it).

It restates each IndexSoftmax step of the IntAttention digest pages
(section "Methodology", step 2: clip, table lookup (32 entries, or a finer
table of 64 or 128, with Q15 or uint8 entries), int32 sum,
reciprocal multiply + shift; step 3: integer Q.K^T and P.V) in a different
form from the vectorised oracle, so that a slip in either (a transposed
operand, a wrong axis, an off-by-one in a rounding) shows up as a mismatch:

  * the slot of a relative score x is found as the nearest bin centre by
    exact rational comparison (|x*mu_q - k| minimal, ties to the upper bin),
    where mu_q = M / 2^sh is the encoded multiplier, not by a shift formula;
  * probabilities (uint8, or the uint16 variant) and the requantised output
    are rounded with Fractions (floor(v + 1/2)), not with add-and-shift.

Meant for tiny shapes only (Sq, Skv <= ~32).
"""
from __future__ import annotations

from fractions import Fraction


def nearest_slot(x: int, idx_mul: int, idx_shift: int, nslots: int = 32) -> int:
    """Nearest bin index for x >= 0 under multiplier M/2^sh, clipped to the last slot."""
    pos = Fraction(x * idx_mul, 1 << idx_shift)      # exact position in bin units
    best = None
    for k in range(nslots):
        d = abs(pos - k)
        # ties (d equal) resolve to the larger k: round half up
        if best is None or d < best[0] or (d == best[0] and k > best[1]):
            best = (d, k)
    k = best[1]
    # positions beyond the last slot also clip to it
    if pos > nslots - 1:
        k = nslots - 1
    return k


def round_half_up(v: Fraction) -> int:
    return (v + Fraction(1, 2)).__floor__()


def head_forward(q, k, v, prm, causal: bool):
    """q: [Sq][D], k/v: [Skv][D] nested lists of ints. Returns (out, m, E, P)."""
    Sq, D, Skv = len(q), len(q[0]), len(k)
    out, ms, Es, Ps = [], [], [], []
    for i in range(Sq):
        scores = []
        for j in range(Skv):
            s = 0
            for d in range(D):
                s += q[i][d] * k[j][d]
            ok = (not causal) or (j <= i + Skv - Sq)
            scores.append((s, ok))
        m = max(s for s, ok in scores if ok)
        e = []
        for s, ok in scores:
            if not ok:
                e.append(0)
            else:
                e.append(prm.lut[nearest_slot(m - s, prm.idx_mul, prm.idx_shift, len(prm.lut))])
        E = sum(e)
        if getattr(prm, "lut_bits", 16) == 8:
            # uint8 table: R nearest to 255*2^16/E (uint8 p) or 65535*2^9/E (uint16 p)
            one, frac = (65535, 9) if getattr(prm, "prob_bits", 8) == 16 else (255, 16)
            R = round_half_up(Fraction(one << frac, E))
            p = [round_half_up(Fraction(ej * R, 1 << frac)) for ej in e]
        elif getattr(prm, "prob_bits", 8) == 16:
            R = round_half_up(Fraction(65535 << 16, E))  # R16 = floor(65535*2^16/E + 1/2)
            p = [round_half_up(Fraction(ej * R, 1 << 16)) for ej in e]
        else:
            R = round_half_up(Fraction(255 << 23, E))  # R = floor(255*2^23/E + 1/2)
            p = [round_half_up(Fraction(ej * R, 1 << 23)) for ej in e]
        row = []
        for d in range(D):
            a = 0
            for j in range(Skv):
                a += p[j] * v[j][d]
            mag = round_half_up(Fraction(abs(a) * prm.req_mul, 1 << prm.req_shift))
            mag = min(127, mag)
            row.append(mag if a >= 0 else -mag)
        out.append(row)
        ms.append(m)
        Es.append(E)
        Ps.append(p)
    return out, ms, Es, Ps
