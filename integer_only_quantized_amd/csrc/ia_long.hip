// Long-row integer attention kernel (gfx950 / CDNA4): key/value tiles
// streamed through LDS, three exact passes per query block. Used for rows
// longer than the short-row kernel holds (e.g. causal prefill at S = 4096).
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology",
// steps 2-3; integer widths and roundings as stated in include/intattn.h.
//
// Structure:
//   * one workgroup = 4 waves = 128 query rows of one (b, h); each wave owns
//     32 rows, holds their Q fragments, and produces S^T blocks (32 keys x
//     32 queries) on v_mfma_i32_32x32x32_i8, so each lane holds one row;
//   * keys arrive in tiles of 64 rows, double-buffered in LDS: the next
//     tile's global loads are issued into registers before the current
//     tile is computed and written to the other buffer afterwards (one
//     barrier per tile);
//   * the row max must be known before any slot and the row sum before any
//     probability, so there are three passes over the tiles with Q.K^T
//     recomputed in each: (1) row max; (2) the MFMA accumulator is seeded
//     with -m, so it yields s - m directly, from which the slot and the
//     table entry follow, summed into E; (3) the same slot indexes a per-row
//     table of the 32 probabilities (stored as p - 128), which is the P
//     operand of P.V; V^T tiles are column-summed on the side for the
//     +128 * colsum(V) correction;
//   * causal workgroups are dispatched heaviest first (the last query
//     blocks have the most keys), and when the head count allows, every XCD
//     owns a fixed subset of heads so their K/V stay in its L2.
// Slot forms: with y = s - m <= 0, if 4M < 2^23 the slot comes from a
// saturating multiply-add (the clip is free, slot bits 26..30, byte 3 =
// 4*slot + fraction); otherwise y is first clipped at -x_clip and the slot
// lands in byte 3 directly. The per-row table layout follows the form.
#include "ia_device.h"

namespace ia {
namespace {

constexpr int kLongWaves = 4;
constexpr int kLongRows = 32 * kLongWaves;   // query rows per workgroup
constexpr int kLongTile = 64;                // keys per tile

template <int D>
struct LongLds {
    static constexpr int KStride = D + 16;          // padded K row (conflict-free 16-byte reads)
    static constexpr int VStride = kLongTile + 16;  // padded V^T row
    static constexpr int PTRow = 132;               // per-row table: up to 128 entries + pad
    uint32_t lut[32];                               // first member: LDS byte address 0
    int32_t colsum[D];
    int8_t k[2][kLongTile * KStride];
    int8_t vt[2][D * VStride];
    uint8_t ptab[kLongWaves * 32 * PTRow];
};

template <int D, bool FAST>
__global__ __launch_bounds__(256) void ia_long_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int nqb, int32_t* __restrict__ row_max,
    uint32_t* __restrict__ row_sum) {
    using L = LongLds<D>;
    constexpr int KS = D / 32;
    constexpr int DB = D / 32;
    constexpr int KStride = L::KStride;
    constexpr int VStride = L::VStride;
    constexpr int KCH = kLongTile * D / 16 / 256;           // 16-byte K chunks per thread per tile
    constexpr int VITEMS = (kLongTile / 4) * (D / 16);      // V items (4 keys x 16 columns) per tile
    constexpr int CS_PARTS = 256 / D;                       // threads per column sum
    constexpr int CS_DW = kLongTile / 4 / CS_PARTS;         // dwords of a V^T row per thread

    __shared__ __attribute__((aligned(16))) L lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // ---- workgroup -> (head, query block) ---------------------------------
    const int nheads = P.B * P.H;
    const int bid = blockIdx.x;
    int head_i, qb;
    if (P.causal && (nheads & 7) == 0) {
        const int hpx = nheads >> 3, j = bid >> 3;
        head_i = (bid & 7) + 8 * (j % hpx);
        qb = nqb - 1 - j / hpx;
    } else if (P.causal) {
        head_i = bid % nheads;
        qb = nqb - 1 - bid / nheads;
    } else {
        const int lb = xcd_local_block(bid, static_cast<int>(gridDim.x));
        qb = lb % nqb;
        head_i = lb / nqb;
    }
    const size_t head = static_cast<size_t>(head_i);
    const int8_t* qh = q + head * P.Sq * D;
    const int8_t* kh = k + head * P.Skv * D;
    const int8_t* vh = v + head * P.Skv * D;

    const int shift = P.Skv - P.Sq;
    const int q0 = qb * kLongRows;
    const int qw0 = q0 + wave * 32;
    const int qrow = qw0 + l32;
    const int kend_row = P.causal ? min(P.Skv, qrow + shift + 1) : P.Skv;
    const int kend_wave = P.causal ? min(P.Skv, qw0 + shift + 1) : P.Skv;
    const int qlast = min(q0 + kLongRows, P.Sq) - 1;
    const int kend_wg = P.causal ? min(P.Skv, qlast + shift + 1) : P.Skv;
    const int ntiles = (kend_wg + kLongTile - 1) / kLongTile;

    if (tid < 32) lds.lut[tid] = lut_entry(P, tid);

    v4i qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (qrow < P.Sq)
            qf[ks] = *reinterpret_cast<const v4i*>(qh + static_cast<size_t>(qrow) * D + 32 * ks + 16 * hh);
        else
            qf[ks] = v4i{0, 0, 0, 0};
    }

    // ---- tile staging ----------------------------------------------------------
    auto load_k = [&](int t, v4i (&kr)[KCH]) {
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int c = u * 256 + tid;
            const int row = c / (D / 16), ch = c % (D / 16);
            const int key = t * kLongTile + row;
            kr[u] = v4i{0, 0, 0, 0};
            if (key < P.Skv) kr[u] = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(key) * D + 16 * ch);
        }
    };
    auto store_k = [&](int buf, const v4i (&kr)[KCH]) {
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int c = u * 256 + tid;
            const int row = c / (D / 16), ch = c % (D / 16);
            *reinterpret_cast<v4i*>(&lds.k[buf][row * KStride + 16 * ch]) = kr[u];
        }
    };
    auto load_v = [&](int t, v4i (&vr)[4]) {
        const int dc = tid % (D / 16), key0 = t * kLongTile + 4 * (tid / (D / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vr[i] = v4i{0, 0, 0, 0};
            if (tid < VITEMS && key0 + i < P.Skv)
                vr[i] = *reinterpret_cast<const v4i*>(vh + static_cast<size_t>(key0 + i) * D + 16 * dc);
        }
    };
    auto store_vt = [&](int buf, const v4i (&vr)[4]) {
        if (tid >= VITEMS) return;
        const int dc = tid % (D / 16), kt = 4 * (tid / (D / 16));   // key within the tile
        const int pos = 32 * (kt >> 5) + vt_pos(kt & 31);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // 4x4 byte transpose: keys kt..kt+3, value columns 16dc+4w..+3
            const uint32_t r0 = vr[0][w], r1 = vr[1][w], r2 = vr[2][w], r3 = vr[3][w];
            const uint32_t u0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
            const uint32_t u1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
            const uint32_t u2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
            const uint32_t u3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
            const int d0 = 16 * dc + 4 * w;
            int8_t* vt = lds.vt[buf];
            *reinterpret_cast<uint32_t*>(&vt[(d0 + 0) * VStride + pos]) = __builtin_amdgcn_perm(u2, u0, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&vt[(d0 + 1) * VStride + pos]) = __builtin_amdgcn_perm(u2, u0, 0x07060302u);
            *reinterpret_cast<uint32_t*>(&vt[(d0 + 2) * VStride + pos]) = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&vt[(d0 + 3) * VStride + pos]) = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
        }
    };

    // S^T block kb (0 or 1) of the tile in LDS buffer buf, from accumulator c0
    auto scores = [&](int buf, int kb, const v16i& c0) {
        v16i s = c0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v4i a = *reinterpret_cast<const v4i*>(&lds.k[buf][(32 * kb + l32) * KStride + 32 * ks + 16 * hh]);
            s = mfma_i8_32x32x32(a, qf[ks], s);
        }
        return s;
    };
    // key j0 + acc_row(r, hh) is allowed iff 8(r/4) + (r%4) < kend_row - j0 - 4hh
    auto mask = [&](v16i& s, int j0, int32_t fill) {
        if (j0 + 32 > kend_wave) {
            const int lim = kend_row - j0 - 4 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) >= lim) s[r] = fill;
        }
    };

    // ---- pass 1: row max ---------------------------------------------------
    const v16i zero16 = v16i{};
    int32_t mrow = INT_MIN;
    {
        v4i kr[KCH];
        load_k(0, kr);
        store_k(0, kr);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            const int buf = t & 1;
            if (t + 1 < ntiles) load_k(t + 1, kr);
            v16i s0 = scores(buf, 0, zero16);
            v16i s1 = scores(buf, 1, zero16);
            mask(s0, t * kLongTile, INT_MIN);
            mask(s1, t * kLongTile + 32, INT_MIN);
#pragma unroll
            for (int r = 0; r < 16; r += 2) mrow = max(mrow, max(max(s0[r], s0[r + 1]), max(s1[r], s1[r + 1])));
            if (t + 1 < ntiles) store_k(buf ^ 1, kr);
            __syncthreads();
        }
    }
    mrow = max(mrow, __shfl_xor(mrow, 32));

    // row constants of the slot arithmetic
    v16i cinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = -mrow;
    const int32_t negMs = FAST ? -4 * P.idx_mul : -P.idx_mul;
    const int32_t halfs = FAST ? (1 << 25) : (1 << 23);
    const int32_t ylo = -P.x_clip;
    // byte 3 of the slot word: 4*slot + fraction (FAST) or slot
    auto slot_word = [&](int32_t y) -> uint32_t {
        if constexpr (FAST) {
            return slot_word_sat(y, negMs, halfs);
        } else {
            return static_cast<uint32_t>(__mul24(max(y, ylo), negMs) + halfs);
        }
    };
    // byte address of the table entry of the slot (32 u32 entries at LDS 0)
    auto lut_addr = [&](uint32_t t) -> uint32_t {
        if constexpr (FAST) return (t >> 24) & 0x7cu;
        else return (t >> 24) << 2;
    };
    const int32_t ymask = FAST ? -(1 << 23) : INT_MIN / 2;

    // ---- pass 2: row sum of the table entries ------------------------------
    uint32_t E = 0;
    {
        v4i kr[KCH];
        load_k(0, kr);
        store_k(0, kr);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            const int buf = t & 1;
            if (t + 1 < ntiles) load_k(t + 1, kr);
            v16i s0 = scores(buf, 0, cinit);
            v16i s1 = scores(buf, 1, cinit);
            mask(s0, t * kLongTile, ymask);
            mask(s1, t * kLongTile + 32, ymask);
            const uint8_t* lb = reinterpret_cast<const uint8_t*>(&lds);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const uint32_t e0 = *reinterpret_cast<const uint32_t*>(lb + lut_addr(slot_word(s0[r])));
                const uint32_t e1 = *reinterpret_cast<const uint32_t*>(lb + lut_addr(slot_word(s0[r + 1])));
                const uint32_t e2 = *reinterpret_cast<const uint32_t*>(lb + lut_addr(slot_word(s1[r])));
                const uint32_t e3 = *reinterpret_cast<const uint32_t*>(lb + lut_addr(slot_word(s1[r + 1])));
                E += (e0 + e1) + (e2 + e3);
            }
            if (t + 1 < ntiles) store_k(buf ^ 1, kr);
            __syncthreads();
        }
    }
    E += __shfl_xor(E, 32);
    const uint32_t R = ((255u << 23) + (E >> 1)) / E;
    if (row_max != nullptr && hh == 0 && qrow < P.Sq) {
        row_max[head * P.Sq + qrow] = mrow;
        row_sum[head * P.Sq + qrow] = E;
    }

    // ---- per-row probability table (wave-private) ---------------------------
    // FAST: entries 4s..4s+3 hold p_s (indexed by 4*slot + fraction);
    // otherwise entry s holds p_s. Stored as p ^ 0x80 (p - 128 as int8).
    uint32_t pbase = static_cast<uint32_t>(offsetof(L, ptab)) + (wave * 32 + l32) * L::PTRow;
    asm volatile("" : "+v"(pbase));
    uint8_t* const ldsb = reinterpret_cast<uint8_t*>(&lds);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int s = 16 * hh + j;
        const uint32_t p = ((lds.lut[s] * R + (1u << 22)) >> 23) ^ 0x80u;
        if constexpr (FAST) {
            // row bases are multiples of 4 (132-byte rows)
            *reinterpret_cast<uint32_t*>(ldsb + pbase + 4 * s) = p * 0x01010101u;
        } else {
            ldsb[pbase + s] = static_cast<uint8_t>(p);
        }
    }
    if (tid < D) lds.colsum[tid] = 0;
    __syncthreads();

    // ---- pass 3: P from the tables, P.V on the MFMA --------------------------
    v16i o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = v16i{};
    int32_t csacc = 0;                      // this thread's part of a column sum
    const int cs_d = tid / CS_PARTS, cs_part = tid % CS_PARTS;
    auto pword = [&](const v16i& s, int w4) -> uint32_t {
        uint32_t b[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t t = slot_word(s[4 * w4 + c]);
            b[c] = ldsb[pbase + (t >> 24)];
        }
        const uint32_t lo2 = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
        const uint32_t hi2 = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
        return __builtin_amdgcn_perm(hi2, lo2, 0x05040100u);
    };
    {
        v4i kr[KCH], vr[4];
        load_k(0, kr);
        load_v(0, vr);
        store_k(0, kr);
        store_vt(0, vr);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            const int buf = t & 1;
            if (t + 1 < ntiles) {
                load_k(t + 1, kr);
                load_v(t + 1, vr);
            }
            // column sums of this V^T tile (every key of the tile is fed)
            {
                const int8_t* row = &lds.vt[buf][cs_d * VStride + 4 * CS_DW * cs_part];
#pragma unroll
                for (int j = 0; j < CS_DW; ++j)
                    csacc = __builtin_amdgcn_sdot4(*reinterpret_cast<const int*>(row + 4 * j), 0x01010101, csacc, false);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                v16i s = scores(buf, kb, cinit);
                mask(s, t * kLongTile + 32 * kb, ymask);
                const v4i pa = v4i{static_cast<int>(pword(s, 0)), static_cast<int>(pword(s, 1)),
                                   static_cast<int>(pword(s, 2)), static_cast<int>(pword(s, 3))};
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const v4i vb = *reinterpret_cast<const v4i*>(&lds.vt[buf][(32 * db + l32) * VStride + 32 * kb + 16 * hh]);
                    o[db] = mfma_i8_32x32x32(pa, vb, o[db]);
                }
            }
            if (t + 1 < ntiles) {
                store_k(buf ^ 1, kr);
                store_vt(buf ^ 1, vr);
            }
            __syncthreads();
        }
    }
    // combine the partial column sums of each value column
#pragma unroll
    for (int off = 1; off < CS_PARTS; off <<= 1) csacc += __shfl_xor(csacc, off);
    if (cs_part == 0) lds.colsum[cs_d] = csacc;
    __syncthreads();

    // ---- requantise and store -----------------------------------------------
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + l32;
        const int32_t cs = lds.colsum[d];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qi = qw0 + acc_row(r, hh);
            if (qi >= P.Sq) continue;
            out[(head * P.Sq + qi) * D + d] = requantise(o[db][r] + 128 * cs, P);
        }
    }
}

}  // namespace

int launch_long(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum) {
    const int nqb = (kp.Sq + kLongRows - 1) / kLongRows;
    const long long blocks = static_cast<long long>(nqb) * kp.H * kp.B;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool fast = kp.idx_mul < (1 << 21);
    if (D == 64) {
        if (fast)
            hipLaunchKernelGGL((ia_long_kernel<64, true>), grid, block, 0, s, q, k, v, out, kp, nqb, row_max, row_sum);
        else
            hipLaunchKernelGGL((ia_long_kernel<64, false>), grid, block, 0, s, q, k, v, out, kp, nqb, row_max, row_sum);
    } else {
        if (fast)
            hipLaunchKernelGGL((ia_long_kernel<128, true>), grid, block, 0, s, q, k, v, out, kp, nqb, row_max, row_sum);
        else
            hipLaunchKernelGGL((ia_long_kernel<128, false>), grid, block, 0, s, q, k, v, out, kp, nqb, row_max, row_sum);
    }
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

}  // namespace ia
