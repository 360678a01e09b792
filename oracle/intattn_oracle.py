"""Plain CPU oracle for the IntAttention fully-integer attention forward pass.

TEST INFRASTRUCTURE ONLY. This module is the slow, obviously-correct statement
of what the GPU path must compute. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does, and
this module imports nothing from the product package (numpy and the standard
library only).

Source: the IntAttention digest pages (euno.news, arXiv 2511.21513v1, Chinese
and Korean editions), section "Methodology":
  * step 2 "Integer-only softmax (IndexSoftmax)": raw int32 scores are clipped
    with a sparsity-aware threshold into a small range; a precomputed
    32-entry table holds exp approximations over that range and is indexed
    directly by the integer score; the pseudo-exponents are summed in int32
    and scaled by an integer reciprocal (multiply + right shift) into a
    softmax-like distribution, with no floating point;
  * step 3 "Integration": Q.K^T and the value product stay in the integer
    domain, keeping the data flow INT8 end to end.
The pages fix none of the integer widths, roundings, the table contents or the
threshold value. Every such choice below is a stated reading of the pages,
described where it is made, and is the specification the GPU path must
reproduce bit for bit.

Arithmetic conventions
  * Host parameters: IEEE-754 binary64 from float32 inputs, correctly rounded
    operations only (*, /, sqrt), round-half-even (Python round == C rint),
    math.frexp (exact), math.exp (the platform libm) for the table.
  * Device-side steps: exact integers. Python ints or numpy int64. The two
    contractions use float64 BLAS, which is exact here because every partial
    sum is an integer of magnitude below 2**53 (|Q.K| <= D*127**2 and
    |P.V| <= Skv*255*127), so any summation order gives the exact integer.

Variants (the pages' "Limitations & Future Work" name them; each is a
stated reading beside the 32-entry specification above, which stays the
default):
  * finer tables: the section on lookup-table granularity calls the 32-entry
    table a trade-off between accuracy and memory and says very large
    attention heads may need finer tables. lut_size N in {32, 64, 128}: bin
    width delta = clip/(N-1), entries for slots 0..N-2 as for N = 32, the
    last slot N-1 the sparse tail (entry 0), idx = min(N-1, (x*M + 2^(sh-1)) >> sh)
    with (M, sh) from mu = alpha/delta; everything after the table is unchanged.
  * grouped K/V heads: kv_heads K/V heads shared by the H query heads in
    consecutive groups of G = H/kv_heads (query head h reads K/V head h//G);
    kv_heads = H is ordinary multi-head attention, 1 is multi-query.
  * uint16 probabilities: the dynamic-range item of the same section warns
    of underflow on skewed or long score rows (a uint8 row of n >= 513
    uniform keys is all zeros). prob_bits = 16: target row sum 65535,
    R16 = floor((65535*2^16 + floor(E/2)) / E) and p = (e*R16 + 2^15) >> 16
    (uint16; e*R16 + 2^15 < 2^32), and the output multiplier
    mu_o = s_v / (65535 * s_o); every other step is unchanged.
  * uint8 table: the lookup-table granularity item frames the table as a
    trade-off between accuracy and memory; lut_bits = 8 is the narrow end
    of that trade (entry width, independent of N). Entries
    e8[k] = rint(255 exp(-k delta)) for k < N-1 (255 for a key at the row
    max), e8[N-1] = 0; E8 = sum of the e8; the reciprocal is the nearest
    integer to 255*2^16 / E8, halves rounded up:
    R8 = floor((255*2^17 + E8) / (2*E8)), p = (e8*R8 + 2^15) >> 16 (uint8);
    with uint16 probabilities R8 = floor((65535*2^10 + E8) / (2*E8))
    (nearest to 65535*2^9 / E8) and p = (e8*R8 + 2^8) >> 9. The row sum
    reported is E8.

Parity pins: see tests/test_oracle_*.py. Every function here is pinned by a
property, closed form, brute-force twin or exact-rational bound; none is
"parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------
# Fixed widths of the integer encoding.
# ---------------------------------------------------------------------------
LUT_SIZE = 32                 # the pages: a 32-entry exp table
LUT_SIZES = (32, 64, 128)     # the finer-table variants
LUT_ONE = 1 << 15             # Q15: table entry for a zero relative score
IDX_SHIFT = 24                # fraction bits of the bin multiplier for mu < 1/2
IDX_MUL_BITS = 23             # above: the widest multiplier, M <= 2^23
P_ONE = 255                   # uint8 probabilities, target row sum 255
R_SHIFT = 23                  # reciprocal fixed point: R = round(255*2^23 / E)
P16_ONE = 65535               # uint16 probabilities (variant), target row sum 65535
R16_SHIFT = 16                # R16 = round(65535*2^16 / E)
PROB_BITS = (8, 16)
LUT8_ONE = 255                # uint8 table variant: entry for a zero relative score
LUT_BITS = (16, 8)            # table entry width: Q15 (the specification) or uint8
REQ_FRAC = 31                 # requantisation multiplier normalised to [2^30, 2^31)
SKV_MAX = 65535               # keeps E < 2^31 and every int32 accumulator exact
MU_MIN = 2.0 ** -24           # bin multiplier range (index units per score unit)
MU_MAX = 2.0 ** 14
REQ_SHIFT_MIN = 1
REQ_SHIFT_MAX = 63

# Default sparsity-aware threshold, in logit units: a key whose
# logit trails the row max by more than ln(510) has exact softmax weight
# below 1/510 of the max key's, i.e. below half a uint8 step, so it is a
# provable zero of the 8-bit probability and may be dropped.
DEFAULT_CLIP = float(np.float32(math.log(510.0)))


class OracleRangeError(ValueError):
    """Arguments outside the ranges the integer encoding is defined for."""


@dataclass(frozen=True)
class Params:
    """Integers frozen on the host before any score is computed."""
    lut: tuple            # lut_size table entries (Q15, or uint8 when lut_bits = 8), the last one 0
    idx_mul: int          # M: bin multiplier, idx = (x*M + 2^(sh-1)) >> sh
    idx_shift: int        # sh: 24 for mu < 1/2, else 23 - e with mu = m 2^e, m in [1/2, 1)
    x_clip: int           # smallest relative score x that lands in slot 31
    req_mul: int          # M_o in [2^30, 2^31)
    req_shift: int        # sh_o
    alpha: float          # logit units per integer score unit
    delta: float          # table bin width in logit units
    mu: float             # alpha / delta
    mu_o: float           # s_v / (P_one * s_o), P_one = 255 or 65535
    lut_size: int = LUT_SIZE  # N: table entries (slots 0..N-1)
    prob_bits: int = 8        # probability width: 8 (uint8) or 16 (uint16 variant)
    lut_bits: int = 16        # table entry width: 16 (Q15) or 8 (uint8 variant)


def _f32(x) -> float:
    """Round to float32 and widen to binary64 (the C ABI takes float32)."""
    return float(np.float32(x))


def _check_lut_size(lut_size: int) -> int:
    if lut_size not in LUT_SIZES:
        raise OracleRangeError("lut_size must be 32, 64 or 128")
    return int(lut_size)


def _check_lut_bits(lut_bits: int) -> int:
    if lut_bits not in LUT_BITS:
        raise OracleRangeError("lut_bits must be 16 or 8")
    return int(lut_bits)


def build_lut(clip: float, lut_size: int = LUT_SIZE, lut_bits: int = 16) -> tuple:
    """The N-entry exp table (N = 32: the pages' table).

    Slot k approximates exp(-k * delta) with delta = clip / (N-1), stored as
    round-half-even(one * exp(-k*delta)) for k < N-1, one = 2^15 (Q15) or
    255 (uint8 variant). Slot N-1 is the sparse tail and holds 0: every key
    clipped there drops out of the sum.
    """
    n = _check_lut_size(lut_size)
    one = LUT_ONE if _check_lut_bits(lut_bits) == 16 else LUT8_ONE
    c = _f32(clip)
    if not (math.isfinite(c) and c > 0.0):
        raise OracleRangeError("clip must be finite and > 0")
    delta = c / float(n - 1)
    lut = [int(round(one * math.exp(-(float(k) * delta)))) for k in range(n - 1)]
    lut.append(0)
    return tuple(lut)


def index_multiplier(mu: float):
    """(M, sh) with M * 2^-sh the encoded bin multiplier mu (slots per score unit).

    For mu < 1/2: a fixed 24-bit fraction, M = round(mu * 2^24), sh = 24
    (M from 1 at mu = 2^-24 up to 2^23). From mu = 1/2 on a 24-bit fraction
    would need M >= 2^23, so the fraction narrows instead: with
    mu = m * 2^e (m in [1/2, 1), frexp), sh = 23 - e and
    M = round(mu * 2^sh) = round(m * 2^23) in [2^22, 2^23], i.e. the widest
    multiplier of at most 2^23, 22 significant bits or more. The two rules
    meet at mu = 1/2 (2^23 / 2^24 = 2^22 / 2^23). At the top of the range,
    mu < 2^14, sh >= 9.
    """
    if mu < 0.5:
        sh = IDX_SHIFT
    else:
        _m, e = math.frexp(mu)
        sh = IDX_MUL_BITS - e
    return int(round(math.ldexp(mu, sh))), sh


def derive_params(D: int, s_q: float, s_k: float, s_v: float, s_o: float,
                  clip: float, lut_size: int = LUT_SIZE, prob_bits: int = 8,
                  lut_bits: int = 16) -> Params:
    """Host parameter derivation.

    alpha = s_q*s_k/sqrt(D) folds the 1/sqrt(d) attention scale into the
    index multiplier; mu = alpha/delta converts an integer score gap into
    table slots; M = round(mu * 2^sh) (index_multiplier).
    """
    n = _check_lut_size(lut_size)
    lut_bits = _check_lut_bits(lut_bits)
    if prob_bits not in PROB_BITS:
        raise OracleRangeError("prob_bits must be 8 or 16")
    if D < 1:
        raise OracleRangeError("D must be >= 1")
    sq, sk, sv, so, c = (_f32(s) for s in (s_q, s_k, s_v, s_o, clip))
    for s in (sq, sk, sv, so):
        if not (math.isfinite(s) and s > 0.0):
            raise OracleRangeError("scales must be finite and > 0")
    lut = build_lut(c, n, lut_bits)
    alpha = (sq * sk) / math.sqrt(float(D))
    delta = c / float(n - 1)
    mu = alpha / delta
    if not (MU_MIN <= mu < MU_MAX):
        raise OracleRangeError("index multiplier outside [2^-24, 2^14)")
    idx_mul, idx_shift = index_multiplier(mu)
    # smallest x with (x*M + 2^(sh-1)) >> sh >= N-1, i.e. x*M >= (2N-3) * 2^(sh-1)
    num = (2 * n - 3) << (idx_shift - 1)
    x_clip = -(-num // idx_mul)
    mu_o = sv / ((255.0 if prob_bits == 8 else 65535.0) * so)
    m_o, e_o = math.frexp(mu_o)
    req_mul = int(round(math.ldexp(m_o, REQ_FRAC)))
    if req_mul == (1 << REQ_FRAC):
        req_mul = 1 << (REQ_FRAC - 1)
        e_o += 1
    req_shift = REQ_FRAC - e_o
    if not (REQ_SHIFT_MIN <= req_shift <= REQ_SHIFT_MAX):
        raise OracleRangeError("output multiplier outside the encodable range")
    return Params(lut=lut, idx_mul=idx_mul, idx_shift=idx_shift, x_clip=x_clip,
                  req_mul=req_mul, req_shift=req_shift, alpha=alpha, delta=delta,
                  mu=mu, mu_o=mu_o, lut_size=n, prob_bits=prob_bits, lut_bits=lut_bits)


# ---------------------------------------------------------------------------
# Elementwise steps (numpy int64, exact)
# ---------------------------------------------------------------------------
def slot_index(x, prm: Params):
    """Table slot of a relative score x = m - s >= 0.

    Uniform bins of width delta, nearest bin: idx = (x*M + 2^(sh-1)) >> sh,
    clipped to the last slot N-1 (the sparsity-aware clip).
    """
    x = np.asarray(x, dtype=np.int64)
    half = np.int64(1 << (prm.idx_shift - 1))
    idx = (x * np.int64(prm.idx_mul) + half) >> np.int64(prm.idx_shift)
    return np.minimum(idx, prm.lut_size - 1)


def reciprocal(E):
    """Integer reciprocal of the row sum: R = floor((255*2^23 + floor(E/2)) / E)."""
    E = np.asarray(E, dtype=np.int64)
    return (np.int64(P_ONE << R_SHIFT) + E // 2) // E


def reciprocal16(E):
    """uint16 variant: R16 = floor((65535*2^16 + floor(E/2)) / E)."""
    E = np.asarray(E, dtype=np.int64)
    return (np.int64(P16_ONE << R16_SHIFT) + E // 2) // E


def normalise16(e, R):
    """uint16 variant: p = (e*R16 + 2^15) >> 16 (round half up)."""
    e = np.asarray(e, dtype=np.int64)
    return (e * R + np.int64(1 << (R16_SHIFT - 1))) >> np.int64(R16_SHIFT)


def normalise(e, R):
    """uint8 probability p = (e*R + 2^22) >> 23 (round half up)."""
    e = np.asarray(e, dtype=np.int64)
    return (e * R + np.int64(1 << (R_SHIFT - 1))) >> np.int64(R_SHIFT)


def reciprocal8(E8):
    """uint8 table: R8 = floor((255*2^17 + E8) / (2*E8)), the nearest integer
    to 255*2^16 / E8 (halves up)."""
    E8 = np.asarray(E8, dtype=np.int64)
    return (np.int64(P_ONE << 17) + E8) // (2 * E8)


def normalise8(e8, R8):
    """uint8 table, uint8 p = (e8*R8 + 2^15) >> 16."""
    e8 = np.asarray(e8, dtype=np.int64)
    return (e8 * R8 + np.int64(1 << 15)) >> np.int64(16)


def reciprocal8_16(E8):
    """uint8 table, uint16 p: R = floor((65535*2^10 + E8) / (2*E8)), the
    nearest integer to 65535*2^9 / E8 (halves up)."""
    E8 = np.asarray(E8, dtype=np.int64)
    return (np.int64(P16_ONE << 10) + E8) // (2 * E8)


def normalise8_16(e8, R):
    """uint8 table, uint16 p = (e8*R + 2^8) >> 9."""
    e8 = np.asarray(e8, dtype=np.int64)
    return (e8 * R + np.int64(1 << 8)) >> np.int64(9)


def requantise(a, prm: Params):
    """int32 accumulator -> int8 output, symmetric round half away from zero.

    out = sign(a) * min(127, (|a|*M_o + 2^(sh_o-1)) >> sh_o). With
    |a| < 2^31 and M_o < 2^31 the product and the rounding term stay below
    2^63, so uint64 holds them exactly.
    """
    a = np.asarray(a, dtype=np.int64)
    mag = np.abs(a)
    if mag.size and int(mag.max()) >= (1 << 31):
        raise OracleRangeError("accumulator outside int32")
    mag = mag.astype(np.uint64)
    q = (mag * np.uint64(prm.req_mul) + np.uint64(1 << (prm.req_shift - 1))) >> np.uint64(prm.req_shift)
    q = np.minimum(q, np.uint64(127)).astype(np.int64)
    return (np.sign(a) * q).astype(np.int8)


# ---------------------------------------------------------------------------
# One attention head
# ---------------------------------------------------------------------------
def allowed_mask(Sq: int, Skv: int, causal: bool):
    """allowed(i, j): j < Skv and, when causal, j <= i + Skv - Sq (bottom-right)."""
    j = np.arange(Skv)[None, :]
    if not causal:
        return np.ones((Sq, Skv), dtype=bool)
    i = np.arange(Sq)[:, None]
    return j <= i + (Skv - Sq)


def qk_scores(qh, kh):
    """int32 scores S = Q.K^T of one head, [Sq, Skv] (methodology step 3:
    the score product stays integer). Exact: float64 BLAS below 2^53."""
    return np.rint(qh.astype(np.float64) @ kh.astype(np.float64).T).astype(np.int64)


def index_softmax(S, prm: Params, causal: bool):
    """IndexSoftmax of one head's int32 scores (methodology step 2).

    Row max over the allowed keys, relative scores x = m - s, table slots with
    the sparsity-aware clip, int32 row sum E of the table entries, integer
    reciprocal R and uint8 probabilities p = (e*R + 2^22) >> 23 (uint16
    variant: p = (e*R16 + 2^15) >> 16; uint8 table: reciprocal8 and
    normalise8, or their uint16 forms). Keys that are not allowed take the
    last slot (entry 0, p = 0). Returns P uint8 (or uint16) [Sq, Skv],
    m int64 [Sq], E int64 [Sq].
    """
    S = np.asarray(S, dtype=np.int64)
    Sq, Skv = S.shape
    allow = allowed_mask(Sq, Skv, causal)
    lo = np.iinfo(np.int64).min
    m = np.where(allow, S, lo).max(axis=1)
    x = m[:, None] - S
    idx = np.where(allow, slot_index(np.where(allow, x, 0), prm), prm.lut_size - 1)
    lut = np.asarray(prm.lut, dtype=np.int64)
    e = lut[idx]
    E = e.sum(axis=1)
    if prm.lut_bits == 8:
        if prm.prob_bits == 16:
            P = normalise8_16(e, reciprocal8_16(E)[:, None])
            return P.astype(np.uint16), m, E
        P = normalise8(e, reciprocal8(E)[:, None])
        return P.astype(np.uint8), m, E
    if prm.prob_bits == 16:
        P = normalise16(e, reciprocal16(E)[:, None])
        return P.astype(np.uint16), m, E
    R = reciprocal(E)
    P = normalise(e, R[:, None])
    return P.astype(np.uint8), m, E


def pv_requant(P, vh, prm: Params):
    """out int8 [Sq, D] = requantise(P.V) (methodology step 3: the value
    product stays integer; the int32 accumulator returns to int8)."""
    A = np.rint(np.asarray(P).astype(np.float64) @ vh.astype(np.float64)).astype(np.int64)
    return requantise(A, prm)


def head_forward(qh, kh, vh, prm: Params, causal: bool):
    """One (b, h) slice. Returns out int8 [Sq, D], m int64 [Sq], E int64 [Sq],
    P uint8 [Sq, Skv]."""
    S = qk_scores(qh, kh)
    P, m, E = index_softmax(S, prm, causal)
    out = pv_requant(P, vh, prm)
    return out, m, E, P


def check_args(q, k, v, causal, kv_heads=None):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise OracleRangeError("tensors must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    hkv = H if kv_heads is None else int(kv_heads)
    if hkv < 1 or H % hkv != 0:
        raise OracleRangeError("kv_heads must divide H")
    if k.shape[:2] != (B, hkv) or v.shape != k.shape or k.shape[3] != D:
        raise OracleRangeError("shape mismatch")
    Skv = k.shape[2]
    if Skv < 1 or Skv > SKV_MAX:
        raise OracleRangeError("Skv must be in [1, 65535]")
    if causal and Sq > Skv:
        raise OracleRangeError("causal attention needs Sq <= Skv")
    for t in (q, k, v):
        if t.dtype != np.int8:
            raise OracleRangeError("inputs must be int8")
        if t.size and int(t.min()) < -127:
            raise OracleRangeError("inputs must lie in [-127, 127]")
    return B, H, Sq, Skv, D


def forward(q, k, v, scales, clip=DEFAULT_CLIP, causal=False, stats=False,
            lut_size=LUT_SIZE, kv_heads=None, prob_bits=8, lut_bits=16):
    """Full forward over int8 tensors q [B, H, Sq, D], k and v [B, Hkv, Skv, D].

    scales = (s_q, s_k, s_v, s_o); lut_size: table entries (32 is the pages'
    table); kv_heads = Hkv (None: H), query head h reading K/V head
    h // (H // Hkv); prob_bits: 8 (uint8 P) or 16 (uint16 variant);
    lut_bits: 16 (Q15 table) or 8 (uint8 table variant). Returns
    out int8 [B, H, Sq, D]; with stats=True also (m int64 [B,H,Sq],
    E int64 [B,H,Sq], P uint8/uint16 [B,H,Sq,Skv]).
    """
    q, k, v = (np.ascontiguousarray(t) for t in (q, k, v))
    B, H, Sq, Skv, D = check_args(q, k, v, causal, kv_heads)
    group = H // k.shape[1]
    prm = derive_params(D, *scales, clip, lut_size, prob_bits, lut_bits)
    out = np.zeros((B, H, Sq, D), dtype=np.int8)
    if stats:
        M = np.zeros((B, H, Sq), dtype=np.int64)
        Es = np.zeros((B, H, Sq), dtype=np.int64)
        Ps = np.zeros((B, H, Sq, Skv), dtype=np.uint8 if prob_bits == 8 else np.uint16)
    for b in range(B):
        for h in range(H):
            o, m, E, P = head_forward(q[b, h], k[b, h // group], v[b, h // group], prm, causal)
            out[b, h] = o
            if stats:
                M[b, h], Es[b, h], Ps[b, h] = m, E, P
    if stats:
        return out, M, Es, Ps
    return out
