// HIP kernels (gfx950 / CDNA4) and the C-ABI entry points of the integer
// attention forward pass.
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology":
// step 2 (IndexSoftmax: clip, 32-entry exp table, int32 sum, reciprocal
// multiply + shift) and step 3 (integer Q.K^T and P.V, INT8 end to end).
// The integer widths and roundings are those stated in include/intattn.h.
//
// General kernel (any Sq, Skv <= 65535, D = 64/128, causal or not):
//   * one workgroup = 4 waves = 128 query rows of one (b, h); each wave owns
//     32 query rows and keeps their Q fragments in registers;
//   * keys stream through LDS in tiles of 64 rows; scores are produced as
//     S^T tiles (keys x queries) by v_mfma_i32_32x32x32_i8 with K as the A
//     operand and Q^T as the B operand, so every lane holds scores of a
//     single query row: the row statistics (max, sum, reciprocal) are
//     per-lane scalars and the lane's 16 scores of a 32-key block are
//     exactly the A operand (16 uint8) of the P.V product for that block;
//   * an exact result needs the full row max before any table index and
//     the full row sum before any probability, so the kernel makes three
//     passes over the key tiles and recomputes Q.K^T in each (MFMA work is
//     cheap next to the per-score integer work): (1) row max, (2) slot
//     index, table lookup and row sum, (3) probabilities and P.V;
//   * the MFMA is signed x signed, so P.V runs on p - 128 (one XOR per four
//     bytes) and adds 128 * (column sum of the V rows fed), which covers
//     masked keys (p = 0) exactly; padded keys are zero rows;
//   * V tiles are stored transposed in LDS so that a lane's 16 keys of one
//     value column are one 16-byte LDS read in the order of the P operand.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include "intattn.h"
#include "intattn_internal.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kQRowsPerWave = 32;
constexpr int kQBlock = kWaves * kQRowsPerWave;  // 128 query rows per workgroup
constexpr int kKeyTile = 64;                      // keys per LDS tile
constexpr int kVtStride = kKeyTile + 16;          // bytes per transposed V row (padded)

__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Key (relative to its 32-key block) held by accumulator register r of a
// 32x32 MFMA result in lane half hh (lanes 0-31: hh = 0, lanes 32-63: 1).
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

// Byte position of a key of a 32-key block inside a transposed V row, such
// that lane half hh reads its 16 keys (acc_row(0..15, hh)) contiguously.
__device__ __forceinline__ int vt_pos(int key_in_block) {
    const int a = key_in_block >> 3, h = (key_in_block >> 2) & 1, c = key_in_block & 3;
    return 16 * h + 4 * a + c;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Renumber them so that consecutive logical blocks (the query blocks of
// one head, which read the same K and V) run on the same XCD. Bijective on
// [0, n): the first 8*floor(n/8) ids are regrouped, the remainder is kept.
__device__ __forceinline__ int xcd_local_block(int bid, int n) {
    const int full = n & ~7;
    if (bid >= full) return bid;
    const int per = full >> 3;
    return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; }

// Slot index of a score under the row constants: the clip is s' = max(s, lo)
// with lo = m - x_clip; then idx = ((m - s')*M + 2^23) >> 24, computed as
// (C - s'*M) mod 2^32 with C = m*M + 2^23 mod 2^32 (the true value is below
// 2^30, and every operand fits the 24-bit signed multiplier).
__device__ __forceinline__ uint32_t slot_of(int32_t s, int32_t lo, uint32_t C, int32_t negM) {
    const int32_t sp = max(s, lo);
    return (C + static_cast<uint32_t>(__mul24(sp, negM))) >> 24;
}

template <int D, bool kDebug>
__global__ __launch_bounds__(256) void ia_general_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int nqb,
    int32_t* __restrict__ row_max, uint32_t* __restrict__ row_sum, uint8_t* __restrict__ probs) {
    constexpr int KS = D / 32;       // 32-deep k-steps of the Q.K^T contraction
    constexpr int DB = D / 32;       // 32-wide value-column blocks of the output
    constexpr int KStride = D + 16;  // padded K row in LDS (conflict-free 16-byte reads)

    __shared__ __attribute__((aligned(16))) int8_t sk[kKeyTile * KStride];
    __shared__ __attribute__((aligned(16))) int8_t svt[D * kVtStride];
    __shared__ uint16_t slut[32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    int bid = blockIdx.x;
    const int qb = bid % nqb;
    bid /= nqb;
    const int h = bid % P.H;
    const int b = bid / P.H;
    const size_t head = static_cast<size_t>(b) * P.H + h;
    const int8_t* qh = q + head * P.Sq * D;
    const int8_t* kh = k + head * P.Skv * D;
    const int8_t* vh = v + head * P.Skv * D;

    if (tid < 32) slut[tid] = static_cast<uint16_t>(P.lut2[tid >> 1] >> (16 * (tid & 1)));

    const int shift = P.Skv - P.Sq;                  // bottom-right causal alignment
    const int q0 = qb * kQBlock;
    const int qw0 = q0 + wave * kQRowsPerWave;       // first query row of this wave
    const int qrow = qw0 + l32;                      // this lane's query row
    const int kend_row = P.causal ? min(P.Skv, qrow + shift + 1) : P.Skv;
    const int kend_wave = P.causal ? min(P.Skv, qw0 + shift + 1) : P.Skv;  // smallest in wave
    const int qlast = min(q0 + kQBlock, P.Sq) - 1;
    const int kend_wg = P.causal ? min(P.Skv, qlast + shift + 1) : P.Skv;
    const int ntiles = (kend_wg + kKeyTile - 1) / kKeyTile;

    v4i qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (qrow < P.Sq)
            qf[ks] = *reinterpret_cast<const v4i*>(qh + static_cast<size_t>(qrow) * D + 32 * ks + 16 * hh);
        else
            qf[ks] = v4i{0, 0, 0, 0};
    }

    auto stage_k = [&](int t) {
        constexpr int chunks = kKeyTile * D / 16;
        for (int c = tid; c < chunks; c += 256) {
            const int row = c / (D / 16), ch = c % (D / 16);
            const int key = t * kKeyTile + row;
            v4i val = v4i{0, 0, 0, 0};
            if (key < P.Skv) val = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(key) * D + 16 * ch);
            *reinterpret_cast<v4i*>(&sk[row * KStride + 16 * ch]) = val;
        }
    };
    auto stage_vt = [&](int t) {
        constexpr int items = (kKeyTile / 4) * (D / 4);
        for (int c = tid; c < items; c += 256) {
            const int kq = c % (kKeyTile / 4), dq = c / (kKeyTile / 4);
            const int key0 = t * kKeyTile + 4 * kq;
            uint32_t r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = key0 + i;
                r[i] = key < P.Skv ? *reinterpret_cast<const uint32_t*>(vh + static_cast<size_t>(key) * D + 4 * dq) : 0u;
            }
            const int kt = 4 * kq;                       // key within tile
            const int pos = 32 * (kt >> 5) + vt_pos(kt & 31);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t w = byte_of(r[0], d) | (byte_of(r[1], d) << 8) |
                                   (byte_of(r[2], d) << 16) | (byte_of(r[3], d) << 24);
                *reinterpret_cast<uint32_t*>(&svt[(4 * dq + d) * kVtStride + pos]) = w;
            }
        }
    };
    // S^T for the tile's two 32-key blocks; masked keys become INT_MIN.
    auto scores = [&](int t, v16i& s0, v16i& s1) {
        s0 = v16i{};
        s1 = v16i{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v4i a0 = *reinterpret_cast<const v4i*>(&sk[l32 * KStride + 32 * ks + 16 * hh]);
            const v4i a1 = *reinterpret_cast<const v4i*>(&sk[(32 + l32) * KStride + 32 * ks + 16 * hh]);
            s0 = mfma_i8_32x32x32(a0, qf[ks], s0);
            s1 = mfma_i8_32x32x32(a1, qf[ks], s1);
        }
        if ((t + 1) * kKeyTile > kend_wave) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j0 = t * kKeyTile + acc_row(r, hh);
                if (j0 >= kend_row) s0[r] = INT_MIN;
                if (j0 + 32 >= kend_row) s1[r] = INT_MIN;
            }
        }
    };

    // ---- pass 1: row max -------------------------------------------------
    int32_t mrow = INT_MIN;
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
        stage_k(t);
        __syncthreads();
        v16i s0, s1;
        scores(t, s0, s1);
#pragma unroll
        for (int r = 0; r < 16; ++r) mrow = max(mrow, max(s0[r], s1[r]));
    }
    mrow = max(mrow, __shfl_xor(mrow, 32));
    const int32_t lo = mrow - P.x_clip;
    const uint32_t C = static_cast<uint32_t>(mrow) * static_cast<uint32_t>(P.idx_mul) + (1u << 23);
    const int32_t negM = -P.idx_mul;

    // ---- pass 2: slot index, table lookup, row sum ----------------------
    uint32_t E = 0;
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
        stage_k(t);
        __syncthreads();
        v16i s0, s1;
        scores(t, s0, s1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            E += slut[slot_of(s0[r], lo, C, negM)];
            E += slut[slot_of(s1[r], lo, C, negM)];
        }
    }
    E += __shfl_xor(E, 32);
    const uint32_t R = ((255u << 23) + (E >> 1)) / E;

    if (kDebug && hh == 0 && qrow < P.Sq) {
        row_max[head * P.Sq + qrow] = mrow;
        row_sum[head * P.Sq + qrow] = E;
    }

    // ---- pass 3: probabilities and P.V ----------------------------------
    v16i o[DB];
    int32_t csum[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        o[db] = v16i{};
        csum[db] = 0;
    }
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
        stage_k(t);
        stage_vt(t);
        __syncthreads();
        v16i s[2];
        scores(t, s[0], s[1]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            uint32_t pw[4];
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                uint32_t word = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 4 * w4 + c;
                    const uint32_t e = slut[slot_of(s[kb][r], lo, C, negM)];
                    const uint32_t p = (e * R + (1u << 22)) >> 23;
                    word |= p << (8 * c);
                    if (kDebug && probs != nullptr) {
                        const int j = t * kKeyTile + 32 * kb + acc_row(r, hh);
                        if (qrow < P.Sq && j < P.Skv)
                            probs[(head * P.Sq + qrow) * static_cast<size_t>(P.Skv) + j] = static_cast<uint8_t>(p);
                    }
                }
                pw[w4] = word ^ 0x80808080u;             // p - 128 as int8
            }
            const v4i pa = v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]),
                               static_cast<int>(pw[2]), static_cast<int>(pw[3])};
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const v4i vb = *reinterpret_cast<const v4i*>(&svt[(32 * db + l32) * kVtStride + 32 * kb + 16 * hh]);
                o[db] = mfma_i8_32x32x32(pa, vb, o[db]);
                csum[db] = __builtin_amdgcn_sdot4(vb[0], 0x01010101, csum[db], false);
                csum[db] = __builtin_amdgcn_sdot4(vb[1], 0x01010101, csum[db], false);
                csum[db] = __builtin_amdgcn_sdot4(vb[2], 0x01010101, csum[db], false);
                csum[db] = __builtin_amdgcn_sdot4(vb[3], 0x01010101, csum[db], false);
            }
        }
    }

    // keys past the workgroup's last tile are masked for all its rows: p = 0
    if (kDebug && probs != nullptr && qrow < P.Sq) {
        for (int j = ntiles * kKeyTile + hh; j < P.Skv; j += 2)
            probs[(head * P.Sq + qrow) * static_cast<size_t>(P.Skv) + j] = 0;
    }

    // ---- requantise and store ---------------------------------------------
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int32_t cs = csum[db] + __shfl_xor(csum[db], 32);
        const int d = 32 * db + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qi = qw0 + acc_row(r, hh);
            if (qi >= P.Sq) continue;
            const int32_t a = o[db][r] + 128 * cs;
            const uint32_t mag = static_cast<uint32_t>(a < 0 ? -a : a);
            const uint64_t prod = static_cast<uint64_t>(mag) * P.req_mul + (uint64_t(1) << (P.req_shift - 1));
            uint64_t qv = prod >> P.req_shift;
            if (qv > 127) qv = 127;
            const int32_t res = a < 0 ? -static_cast<int32_t>(qv) : static_cast<int32_t>(qv);
            out[(head * P.Sq + qi) * D + d] = static_cast<int8_t>(res);
        }
    }
}

// Short-row kernel: the whole key range of a head (NKB blocks of 32 keys, a
// compile-time count) stays resident in LDS for the whole workgroup: K
// row-major (padded rows) and V transposed in the P-operand key order. Each
// wave owns 32 query rows.
//   pass 1: S^T blocks from K in LDS -> per-lane row max;
//   pass 2: S^T - m (the MFMA accumulator starts from -m) -> slot -> table
//           lookup -> row sum; each score's slot is kept in registers as one
//           byte (4 * slot);
//   tables: each row's 32 probabilities (p ^ 0x80, i.e. p - 128 as int8) in
//           LDS, reusing the K area;
//   pass 3: P operand = per-row table indexed by the stored slot bytes, then
//           P.V on the MFMA with V^T from LDS, plus one MFMA against an
//           all-ones operand that yields the column sums of the V rows fed.
// V is prefetched into registers before pass 1 and written to LDS after
// pass 2, so its load latency hides behind passes 1 and 2.
//
// Slot arithmetic (FAST, used when M < 2^21): with y = s - m <= 0,
//   t = sat_int32(y * (-4M) + 2^25),  slot = t >> 26.
// Scaling the spec's (x*M + 2^23) >> 24 by 4 gives the same quotient; the
// value is below 2^31 whenever slot < 31, and saturation to 2^31 - 1 lands
// exactly in slot 31, so the clip costs nothing. Masked keys use y = -2^23.
// Otherwise the explicit clip s' = max(s, m - x_clip) is used and the slot is
// moved to the same bit position with one shift.
template <int D, int NKB>
struct ShortLds {
    static constexpr int KPAD = 32 * NKB;
    static constexpr int KStride = D + 16;     // padded K row: conflict-free 16-byte reads
    static constexpr int VStride = KPAD + 16;  // padded V^T row
    static constexpr int PTBlock = 132;        // 4 interleaved row tables (bank spread)
    static constexpr int KBytes = KPAD * KStride > 8 * 8 * PTBlock ? KPAD * KStride : 8 * 8 * PTBlock;
    uint32_t lut[32];                          // first member: LDS byte address 0
    int8_t k[KBytes];                          // K, later the probability tables
    int8_t vt[D * VStride];
};

template <int D, int NKB, bool FAST>
__global__ __launch_bounds__(512) void ia_short_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int nqb) {
    using L = ShortLds<D, NKB>;
    constexpr int KPAD = L::KPAD;
    constexpr int KS = D / 32;
    constexpr int DB = D / 32;
    constexpr int KStride = L::KStride;
    constexpr int VStride = L::VStride;

    __shared__ __attribute__((aligned(16))) L lds;

    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nw = nthreads >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    int bid = xcd_local_block(blockIdx.x, gridDim.x);
    const int qb = bid % nqb;
    bid /= nqb;
    const int h = bid % P.H;
    const int b = bid / P.H;
    const size_t head = static_cast<size_t>(b) * P.H + h;
    const int8_t* qh = q + head * P.Sq * D;
    const int8_t* kh = k + head * P.Skv * D;
    const int8_t* vh = v + head * P.Skv * D;

    // ---- stage K (rounds of eight 16-byte loads in flight per thread) -------
    constexpr int KCH = KPAD * (D / 16);
    for (int base = 0; base < KCH; base += 8 * nthreads) {
        v4i val[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = base + u * nthreads + tid;
            const int row = c / (D / 16), ch = c % (D / 16);
            val[u] = v4i{0, 0, 0, 0};
            if (c < KCH && row < P.Skv)
                val[u] = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(row) * D + 16 * ch);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = base + u * nthreads + tid;
            const int row = c / (D / 16), ch = c % (D / 16);
            if (c < KCH) *reinterpret_cast<v4i*>(&lds.k[row * KStride + 16 * ch]) = val[u];
        }
    }
    // ---- prefetch V (4 keys x 16 value columns per item, two items/thread) --
    constexpr int VIT = (KPAD / 4) * (D / 16);
    auto load_v = [&](int c, v4i (&r)[4]) {
        const int dc = c % (D / 16), key0 = 4 * (c / (D / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[i] = v4i{0, 0, 0, 0};
            if (c < VIT && key0 + i < P.Skv)
                r[i] = *reinterpret_cast<const v4i*>(vh + static_cast<size_t>(key0 + i) * D + 16 * dc);
        }
    };
    auto store_vt = [&](int c, const v4i (&r)[4]) {
        if (c >= VIT) return;
        const int dc = c % (D / 16), key0 = 4 * (c / (D / 16));
        const int pos = 32 * (key0 >> 5) + vt_pos(key0 & 31);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // 4x4 byte transpose: keys key0..key0+3, value columns 16dc+4w..+3
            const uint32_t r0 = r[0][w], r1 = r[1][w], r2 = r[2][w], r3 = r[3][w];
            const uint32_t u0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
            const uint32_t u1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
            const uint32_t u2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
            const uint32_t u3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
            const int d0 = 16 * dc + 4 * w;
            *reinterpret_cast<uint32_t*>(&lds.vt[(d0 + 0) * VStride + pos]) = __builtin_amdgcn_perm(u2, u0, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&lds.vt[(d0 + 1) * VStride + pos]) = __builtin_amdgcn_perm(u2, u0, 0x07060302u);
            *reinterpret_cast<uint32_t*>(&lds.vt[(d0 + 2) * VStride + pos]) = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&lds.vt[(d0 + 3) * VStride + pos]) = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
        }
    };
    v4i vpre[2][4];
    load_v(tid, vpre[0]);
    load_v(tid + nthreads, vpre[1]);

    if (tid < 32) lds.lut[tid] = (P.lut2[tid >> 1] >> (16 * (tid & 1))) & 0xffffu;
    __syncthreads();

    const int shift = P.Skv - P.Sq;
    const int qw0 = qb * 32 * nw + wave * 32;
    const int qrow = qw0 + l32;
    const int kend_row = P.causal ? min(P.Skv, qrow + shift + 1) : P.Skv;
    const int kend_wave = P.causal ? min(P.Skv, qw0 + shift + 1) : P.Skv;

    v4i qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (qrow < P.Sq)
            qf[ks] = *reinterpret_cast<const v4i*>(qh + static_cast<size_t>(qrow) * D + 32 * ks + 16 * hh);
        else
            qf[ks] = v4i{0, 0, 0, 0};
    }

    // S^T block (MFMA only) starting from accumulator c0
    auto scores = [&](int kb, const v16i& c0) {
        v16i s = c0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v4i a = *reinterpret_cast<const v4i*>(&lds.k[(32 * kb + l32) * KStride + 32 * ks + 16 * hh]);
            s = mfma_i8_32x32x32(a, qf[ks], s);
        }
        return s;
    };
    // key 32kb + acc_row(r, hh) is allowed iff 8(r/4) + (r%4) < kend_row - 32kb - 4hh
    auto mask = [&](v16i& s, int kb, int32_t fill) {
        if (32 * kb + 32 > kend_wave) {
            const int lim = kend_row - 32 * kb - 4 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) >= lim) s[r] = fill;
        }
    };

    // Each pass is software-pipelined by hand (MFMAs of block kb+1 issued
    // before the integer work on block kb) and fenced per block with a
    // scheduling barrier; empty asm statements pin per-block reductions so
    // the compiler cannot defer them into one cross-block tree.

    // ---- pass 1: row max ---------------------------------------------------
    const v16i zero16 = v16i{};
    int32_t mrow = INT_MIN;
    {
        v16i cur = scores(0, zero16);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            v16i nxt;
            if (kb + 1 < NKB) nxt = scores(kb + 1, zero16);
            mask(cur, kb, INT_MIN);
#pragma unroll
            for (int r = 0; r < 16; r += 2) mrow = max(mrow, max(cur[r], cur[r + 1]));
            asm volatile("" : "+v"(mrow));
            if (kb + 1 < NKB) cur = nxt;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    mrow = max(mrow, __shfl_xor(mrow, 32));
    asm volatile("" ::: "memory");   // re-read K fragments in pass 2

    // ---- pass 2: slots, table lookups, row sum; slot bytes kept ------------
    const uint8_t* const ldsb_c = reinterpret_cast<const uint8_t*>(&lds);
    uint32_t idxw[NKB][4];
    uint32_t E = 0;
    {
        v16i cinit;
        int32_t negM4 = 0, half4 = 1 << 25, lo = 0, negM = 0;
        uint32_t C = 0;
        if constexpr (FAST) {
#pragma unroll
            for (int r = 0; r < 16; ++r) cinit[r] = -mrow;
            negM4 = -4 * P.idx_mul;
        } else {
            cinit = zero16;
            lo = mrow - P.x_clip;
            C = static_cast<uint32_t>(mrow) * static_cast<uint32_t>(P.idx_mul) + (1u << 23);
            negM = -P.idx_mul;
        }
        // 4 * slot of each score, in bits 26..30 of t (byte 3 = 4 * slot + fraction)
        auto slot_word = [&](int32_t y) -> uint32_t {
            if constexpr (FAST) {
                int32_t t;
                asm("v_mad_i32_i24 %0, %1, %2, %3 clamp" : "=v"(t) : "v"(y), "v"(negM4), "v"(half4));
                return static_cast<uint32_t>(t);
            } else {
                const int32_t sp = max(y, lo);
                return (C + static_cast<uint32_t>(__mul24(sp, negM))) << 2;
            }
        };
        v16i cur = scores(0, cinit);
        uint32_t ep[16];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            v16i nxt;
            if (kb + 1 < NKB) nxt = scores(kb + 1, cinit);
            mask(cur, kb, FAST ? -(1 << 23) : INT_MIN);
            uint32_t en[16];
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                uint32_t t[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    t[c] = slot_word(cur[4 * w4 + c]);
                    // table entry at byte 4 * slot = (t >> 24) & 0x7c
                    en[4 * w4 + c] = *reinterpret_cast<const uint32_t*>(ldsb_c + ((t[c] >> 24) & 0x7cu));
                }
                const uint32_t w01 = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0703u);
                const uint32_t w23 = __builtin_amdgcn_perm(t[3], t[2], 0x0c0c0703u);
                idxw[kb][w4] = __builtin_amdgcn_perm(w23, w01, 0x05040100u) & 0x7c7c7c7cu;
                // keep the packed word (not the four values it came from)
                // live until pass 3
                asm volatile("" : "+v"(idxw[kb][w4]));
            }
            // lookups of the previous block are summed one block later
            if (kb > 0) {
#pragma unroll
                for (int i = 0; i < 16; i += 2) E += ep[i] + ep[i + 1];
                asm volatile("" : "+v"(E));
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) ep[i] = en[i];
            if (kb + 1 < NKB) cur = nxt;
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) E += ep[i] + ep[i + 1];
    }
    E += __shfl_xor(E, 32);
    const uint32_t R = ((255u << 23) + (E >> 1)) / E;

    // ---- V^T into LDS (prefetched items, then any remaining ones) -----------
    store_vt(tid, vpre[0]);
    store_vt(tid + nthreads, vpre[1]);
    for (int c = tid + 2 * nthreads; c < VIT; c += nthreads) {
        v4i r[4];
        load_v(c, r);
        store_vt(c, r);
    }
    __syncthreads();   // V^T complete; every wave is done with K

    // ---- per-row probability tables (wave-private, in the K area) -----------
    // Rows are interleaved four to a 132-byte block: entry (row, slot) at
    // byte block*132 + 4*slot + (row & 3), so equal slots of different
    // blocks fall in different banks.
    uint32_t pbase = static_cast<uint32_t>(offsetof(L, k)) + (wave * 8 + (l32 >> 2)) * L::PTBlock + (l32 & 3);
    asm volatile("" : "+v"(pbase));
    uint8_t* const ldsb = reinterpret_cast<uint8_t*>(&lds);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int kslot = 16 * hh + j;
        const uint32_t p = (lds.lut[kslot] * R + (1u << 22)) >> 23;
        ldsb[pbase + 4 * kslot] = static_cast<uint8_t>(p ^ 0x80u);
    }
    // the tables are read only by the wave that wrote them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- pass 3: P from the tables, P.V and column sums on the MFMA ---------
    // Three stages in flight: table lookups for block kb+2, byte packing of
    // block kb+1, MFMAs of block kb.
    auto plookup = [&](int kb, uint32_t (&pl)[16]) {
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            const uint32_t x = idxw[kb][w4];
            pl[4 * w4 + 0] = ldsb[pbase + (x & 0xffu)];
            pl[4 * w4 + 1] = ldsb[pbase + ((x >> 8) & 0xffu)];
            pl[4 * w4 + 2] = ldsb[pbase + ((x >> 16) & 0xffu)];
            pl[4 * w4 + 3] = ldsb[pbase + (x >> 24)];
        }
    };
    auto ppack = [&](const uint32_t (&pl)[16]) {
        uint32_t pw[4];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            const uint32_t lo2 = __builtin_amdgcn_perm(pl[4 * w4 + 1], pl[4 * w4 + 0], 0x0c0c0400u);
            const uint32_t hi2 = __builtin_amdgcn_perm(pl[4 * w4 + 3], pl[4 * w4 + 2], 0x0c0c0400u);
            pw[w4] = __builtin_amdgcn_perm(hi2, lo2, 0x05040100u);
        }
        return v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]), static_cast<int>(pw[2]),
                   static_cast<int>(pw[3])};
    };
    const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
    v16i o[DB], oc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        o[db] = v16i{};
        oc[db] = v16i{};
    }
    {
        uint32_t pl[16];
        plookup(0, pl);
        v4i pa = ppack(pl);
        if (NKB > 1) plookup(1, pl);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            v4i pnext;
            if (kb + 1 < NKB) pnext = ppack(pl);
            if (kb + 2 < NKB) plookup(kb + 2, pl);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const v4i vb = *reinterpret_cast<const v4i*>(&lds.vt[(32 * db + l32) * VStride + 32 * kb + 16 * hh]);
                o[db] = mfma_i8_32x32x32(pa, vb, o[db]);
                oc[db] = mfma_i8_32x32x32(ones, vb, oc[db]);
            }
            if (kb + 1 < NKB) pa = pnext;
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- requantise and store -----------------------------------------------
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + l32;
        const int32_t cs = oc[db][0];   // every row of ones x V^T is the column sum
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qi = qw0 + acc_row(r, hh);
            if (qi >= P.Sq) continue;
            const int32_t a = o[db][r] + 128 * cs;
            const uint32_t mag = static_cast<uint32_t>(a < 0 ? -a : a);
            const uint64_t prod = static_cast<uint64_t>(mag) * P.req_mul + (uint64_t(1) << (P.req_shift - 1));
            uint64_t qv = prod >> P.req_shift;
            if (qv > 127) qv = 127;
            const int32_t res = a < 0 ? -static_cast<int32_t>(qv) : static_cast<int32_t>(qv);
            out[(head * P.Sq + qi) * D + d] = static_cast<int8_t>(res);
        }
    }
}

// Decode kernel: one query row per head (Sq = 1), keys streamed from HBM.
// One workgroup (4 waves) per (b, h). D/16 consecutive lanes cover one key
// row with 16-byte loads (fully coalesced); each lane handles 4 keys.
//   A: scores s_j = q . k_j: four sdot4 per 16 bytes, then a butterfly over
//      the D/16 lanes of a row (DPP), scores kept in LDS (int32 per key);
//   B: row max (wave reduction + LDS);
//   C: slots, table lookups and row sum; the scores' LDS words are reused
//      for the slots; then p_j for every key (one 32-entry table per row);
//   D: P.V: each lane transposes its 4 keys x 16 value columns (v_perm) and
//      accumulates udot4(p, v + 128) (adding 128 to a signed byte = XOR 0x80),
//      so a_d = sum_j p_j v_jd = acc_d - 128 * sum_j p_j; lanes and waves are
//      then reduced and the result requantised.
// HBM traffic is one read of K and V; the LDS holds 5 bytes per key.
constexpr int kDecodeThreads = 256;

__device__ __forceinline__ int32_t dpp_xor1(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true); }
__device__ __forceinline__ int32_t dpp_xor2(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true); }
__device__ __forceinline__ int32_t dpp_half_mirror(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true); }

template <int D>
__global__ __launch_bounds__(kDecodeThreads) void ia_decode_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int skv_pad) {
    constexpr int CPR = D / 16;                 // lanes per key row
    constexpr int GPW = 64 / CPR;               // key groups (of 4 keys) per wave
    constexpr int KEYS_IT = 4 * GPW * (kDecodeThreads / 64);   // keys per iteration
    extern __shared__ __attribute__((aligned(16))) int32_t dsm[];
    int32_t* s_score = dsm;                                     // skv_pad ints (scores, then slots)
    uint8_t* s_p = reinterpret_cast<uint8_t*>(dsm + skv_pad);   // skv_pad bytes
    __shared__ uint32_t s_lut[32];
    __shared__ int32_t s_red[4][D];
    __shared__ int32_t s_scal[8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane % CPR;                   // 16-byte column chunk
    const int g = lane / CPR;                   // key group within the wave
    const size_t head = blockIdx.x;
    const int8_t* kh = k + head * P.Skv * D;
    const int8_t* vh = v + head * P.Skv * D;
    const v4i qv = *reinterpret_cast<const v4i*>(q + head * D + 16 * c);
    if (tid < 32) s_lut[tid] = (P.lut2[tid >> 1] >> (16 * (tid & 1))) & 0xffffu;

    // ---- A: scores ---------------------------------------------------------
    int32_t tmax = INT_MIN;
    for (int base = 0; base < P.Skv; base += 2 * KEYS_IT) {
        v4i kr[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = base + u * KEYS_IT + wave * 4 * GPW + 4 * g + i;
                kr[u][i] = v4i{0, 0, 0, 0};
                if (key < P.Skv) kr[u][i] = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(key) * D + 16 * c);
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int32_t sc = __builtin_amdgcn_sdot4(kr[u][i][0], qv[0], 0, false);
                sc = __builtin_amdgcn_sdot4(kr[u][i][1], qv[1], sc, false);
                sc = __builtin_amdgcn_sdot4(kr[u][i][2], qv[2], sc, false);
                sc = __builtin_amdgcn_sdot4(kr[u][i][3], qv[3], sc, false);
                sc += dpp_xor1(sc);
                sc += dpp_xor2(sc);
                if (CPR == 8) sc += dpp_half_mirror(sc);
                const int key = base + u * KEYS_IT + wave * 4 * GPW + 4 * g + i;
                if (key < P.Skv) {
                    tmax = max(tmax, sc);
                    if (c == i) s_score[key] = sc;
                }
            }
    }
    // ---- B: row max ----------------------------------------------------------
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tmax = max(tmax, __shfl_xor(tmax, off));
    if (lane == 0) s_scal[wave] = tmax;
    __syncthreads();
    const int32_t m = max(max(s_scal[0], s_scal[1]), max(s_scal[2], s_scal[3]));
    const int32_t lo = m - P.x_clip;
    const uint32_t Cm = static_cast<uint32_t>(m) * static_cast<uint32_t>(P.idx_mul) + (1u << 23);
    const int32_t negM = -P.idx_mul;

    // ---- C: slots and row sum, then probabilities ------------------------------
    uint32_t E = 0;
    for (int j = tid; j < P.Skv; j += kDecodeThreads) {
        const int32_t sp = max(s_score[j], lo);
        const uint32_t slot = (Cm + static_cast<uint32_t>(__mul24(sp, negM))) >> 24;
        E += s_lut[slot];
        s_score[j] = static_cast<int32_t>(slot);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) E += __shfl_xor(E, off);
    __syncthreads();
    if (lane == 0) s_scal[4 + wave] = static_cast<int32_t>(E);
    __syncthreads();
    E = static_cast<uint32_t>(s_scal[4]) + static_cast<uint32_t>(s_scal[5]) +
        static_cast<uint32_t>(s_scal[6]) + static_cast<uint32_t>(s_scal[7]);
    const uint32_t R = ((255u << 23) + (E >> 1)) / E;
    uint32_t psum = 0;
    for (int j = tid; j < skv_pad; j += kDecodeThreads) {
        uint32_t p = 0;
        if (j < P.Skv) p = (s_lut[s_score[j]] * R + (1u << 22)) >> 23;
        s_p[j] = static_cast<uint8_t>(p);
        psum += p;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) psum += __shfl_xor(psum, off);
    __syncthreads();
    if (lane == 0) s_scal[wave] = static_cast<int32_t>(psum);
    __syncthreads();
    psum = static_cast<uint32_t>(s_scal[0]) + static_cast<uint32_t>(s_scal[1]) +
           static_cast<uint32_t>(s_scal[2]) + static_cast<uint32_t>(s_scal[3]);

    // ---- D: P.V ----------------------------------------------------------------
    uint32_t acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0;
    for (int base = 0; base < P.Skv; base += 2 * KEYS_IT) {
        v4i vr[2][4];
        uint32_t pk[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int key0 = base + u * KEYS_IT + wave * 4 * GPW + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vr[u][i] = v4i{0, 0, 0, 0};
                if (key0 + i < P.Skv)
                    vr[u][i] = *reinterpret_cast<const v4i*>(vh + static_cast<size_t>(key0 + i) * D + 16 * c);
            }
            pk[u] = key0 < skv_pad ? *reinterpret_cast<const uint32_t*>(s_p + key0) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t r0 = static_cast<uint32_t>(vr[u][0][w]) ^ 0x80808080u;
                const uint32_t r1 = static_cast<uint32_t>(vr[u][1][w]) ^ 0x80808080u;
                const uint32_t r2 = static_cast<uint32_t>(vr[u][2][w]) ^ 0x80808080u;
                const uint32_t r3 = static_cast<uint32_t>(vr[u][3][w]) ^ 0x80808080u;
                const uint32_t u0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
                const uint32_t u1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
                const uint32_t u2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
                const uint32_t u3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
                acc[4 * w + 0] = __builtin_amdgcn_udot4(__builtin_amdgcn_perm(u2, u0, 0x05040100u), pk[u], acc[4 * w + 0], false);
                acc[4 * w + 1] = __builtin_amdgcn_udot4(__builtin_amdgcn_perm(u2, u0, 0x07060302u), pk[u], acc[4 * w + 1], false);
                acc[4 * w + 2] = __builtin_amdgcn_udot4(__builtin_amdgcn_perm(u3, u1, 0x05040100u), pk[u], acc[4 * w + 2], false);
                acc[4 * w + 3] = __builtin_amdgcn_udot4(__builtin_amdgcn_perm(u3, u1, 0x07060302u), pk[u], acc[4 * w + 3], false);
            }
    }
    // lanes with the same column chunk (stride CPR) hold partial sums
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int off = CPR; off < 64; off <<= 1) acc[i] += __shfl_xor(acc[i], off);
    }
    if (g == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s_red[wave][16 * c + i] = static_cast<int32_t>(acc[i]);
    }
    __syncthreads();
    for (int d = tid; d < D; d += kDecodeThreads) {
        const uint32_t tot = static_cast<uint32_t>(s_red[0][d]) + static_cast<uint32_t>(s_red[1][d]) +
                             static_cast<uint32_t>(s_red[2][d]) + static_cast<uint32_t>(s_red[3][d]);
        const int32_t a = static_cast<int32_t>(tot - 128u * psum);
        const uint32_t mag = static_cast<uint32_t>(a < 0 ? -a : a);
        const uint64_t prod = static_cast<uint64_t>(mag) * P.req_mul + (uint64_t(1) << (P.req_shift - 1));
        uint64_t qv2 = prod >> P.req_shift;
        if (qv2 > 127) qv2 = 127;
        out[head * D + d] = static_cast<int8_t>(a < 0 ? -static_cast<int32_t>(qv2) : static_cast<int32_t>(qv2));
    }
}

// Largest key count served by the decode kernel (5 bytes of LDS per key).
constexpr int kDecodeMaxKeys = 16384;

int launch_decode(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                  const IaKernelParams& kp, hipStream_t stream) {
    const long long blocks = static_cast<long long>(kp.B) * kp.H;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    const int skv_pad = (kp.Skv + 255) / 256 * 256;
    const size_t shm = static_cast<size_t>(skv_pad) * 5;
    if (D == 64) {
        static bool attr64 = false;
        if (!attr64) {
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(&ia_decode_kernel<64>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 5 * kDecodeMaxKeys) != hipSuccess)
                return INTATTN_E_HIP;
            attr64 = true;
        }
        hipLaunchKernelGGL((ia_decode_kernel<64>), dim3(static_cast<unsigned>(blocks)), dim3(kDecodeThreads), shm,
                           stream, q, k, v, out, kp, skv_pad);
    } else {
        static bool attr128 = false;
        if (!attr128) {
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(&ia_decode_kernel<128>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 5 * kDecodeMaxKeys) != hipSuccess)
                return INTATTN_E_HIP;
            attr128 = true;
        }
        hipLaunchKernelGGL((ia_decode_kernel<128>), dim3(static_cast<unsigned>(blocks)), dim3(kDecodeThreads), shm,
                           stream, q, k, v, out, kp, skv_pad);
    }
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int prepare(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
            const intattn_shape* shape, const intattn_scales* scales, float clip, int causal,
            IaKernelParams* kp) {
    if (!q || !k || !v || !out || !shape || !scales) return INTATTN_E_NULL;
    int st = intattn_validate_shape(shape, causal);
    if (st != INTATTN_OK) return st;
    if (shape->D != 64 && shape->D != 128) return INTATTN_E_DIM;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return INTATTN_E_ALIGN;
    intattn_params prm;
    st = intattn_derive_params(shape, scales, clip, &prm);
    if (st != INTATTN_OK) return st;
    kp->B = shape->B;
    kp->H = shape->H;
    kp->Sq = shape->Sq;
    kp->Skv = shape->Skv;
    kp->causal = causal ? 1 : 0;
    kp->idx_mul = prm.idx_mul;
    kp->x_clip = prm.x_clip;
    kp->req_shift = prm.req_shift;
    kp->req_mul = static_cast<uint32_t>(prm.req_mul);
    for (int i = 0; i < 16; ++i)
        kp->lut2[i] = static_cast<uint32_t>(prm.lut[2 * i]) | (static_cast<uint32_t>(prm.lut[2 * i + 1]) << 16);
    return INTATTN_OK;
}

template <bool kDebug>
int launch_general(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                   const IaKernelParams& kp, hipStream_t stream, int32_t* row_max,
                   uint32_t* row_sum, uint8_t* probs) {
    const int nqb = (kp.Sq + kQBlock - 1) / kQBlock;
    const long long blocks = static_cast<long long>(nqb) * kp.H * kp.B;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (D == 64)
        hipLaunchKernelGGL((ia_general_kernel<64, kDebug>), grid, block, 0, stream, q, k, v, out, kp, nqb,
                           row_max, row_sum, probs);
    else
        hipLaunchKernelGGL((ia_general_kernel<128, kDebug>), grid, block, 0, stream, q, k, v, out, kp, nqb,
                           row_max, row_sum, probs);
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

template <int D, int NKB>
int launch_short_t(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                   const IaKernelParams& kp, hipStream_t stream) {
    // the saturating slot form needs 4*M to fit the 24-bit multiplier operand
    const bool fast = kp.idx_mul < (1 << 21);
    const int nqb32 = (kp.Sq + 31) / 32;
    const long long heads = static_cast<long long>(kp.B) * kp.H;
    // waves per workgroup: as many as there are 32-row query blocks (<= 8),
    // halved while the grid would leave compute units idle
    int nw = nqb32 < 8 ? nqb32 : 8;
    while (nw > 1 && heads * ((nqb32 + nw - 1) / nw) < 256) nw = (nw + 1) / 2;
    const int nqb = (nqb32 + nw - 1) / nw;
    const long long blocks = heads * nqb;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    if (fast)
        hipLaunchKernelGGL((ia_short_kernel<D, NKB, true>), dim3(static_cast<unsigned>(blocks)), dim3(64 * nw),
                           0, stream, q, k, v, out, kp, nqb);
    else
        hipLaunchKernelGGL((ia_short_kernel<D, NKB, false>), dim3(static_cast<unsigned>(blocks)), dim3(64 * nw),
                           0, stream, q, k, v, out, kp, nqb);
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

// Largest number of 32-key blocks served by the short-row kernel, per head
// size (K, V^T and the tables stay under 80 KB of LDS: two workgroups per CU).
constexpr int short_max_blocks(int D) { return D == 64 ? 16 : 8; }

template <int D, int NKB>
int launch_short_n(int nkb, const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                   const IaKernelParams& kp, hipStream_t stream) {
    if constexpr (NKB > short_max_blocks(D)) {
        return INTATTN_E_SHAPE;
    } else {
        if (nkb == NKB) return launch_short_t<D, NKB>(q, k, v, out, kp, stream);
        return launch_short_n<D, NKB + 1>(nkb, q, k, v, out, kp, stream);
    }
}

int launch_short(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                 const IaKernelParams& kp, hipStream_t stream) {
    const int nkb = (kp.Skv + 31) / 32;
    if (D == 64) return launch_short_n<64, 1>(nkb, q, k, v, out, kp, stream);
    return launch_short_n<128, 1>(nkb, q, k, v, out, kp, stream);
}

}  // namespace

extern "C" int intattn_forward(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                               const intattn_shape* shape, const intattn_scales* scales, float clip,
                               int causal, void* stream) {
    IaKernelParams kp;
    const int st = prepare(q, k, v, out, shape, scales, clip, causal, &kp);
    if (st != INTATTN_OK) return st;
    if (static_cast<long long>(kp.B) * kp.H * kp.Sq == 0) return INTATTN_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (kp.Sq == 1 && kp.Skv <= kDecodeMaxKeys) return launch_decode(q, k, v, out, shape->D, kp, s);
    if ((kp.Skv + 31) / 32 <= short_max_blocks(shape->D)) return launch_short(q, k, v, out, shape->D, kp, s);
    return launch_general<false>(q, k, v, out, shape->D, kp, s, nullptr, nullptr, nullptr);
}

extern "C" int intattn_forward_debug(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                                     const intattn_shape* shape, const intattn_scales* scales, float clip,
                                     int causal, void* stream, int32_t* row_max, uint32_t* row_sum,
                                     uint8_t* probs) {
    if (!row_max || !row_sum) return INTATTN_E_NULL;
    IaKernelParams kp;
    const int st = prepare(q, k, v, out, shape, scales, clip, causal, &kp);
    if (st != INTATTN_OK) return st;
    if (static_cast<long long>(kp.B) * kp.H * kp.Sq == 0) return INTATTN_OK;
    return launch_general<true>(q, k, v, out, shape->D, kp, static_cast<hipStream_t>(stream), row_max,
                                row_sum, probs);
}
