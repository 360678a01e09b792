// General integer attention kernel (gfx950 / CDNA4): any Sq, Skv and mask;
// also the kernel behind the full-probability debug output.
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
#include "ia_device.h"

namespace ia {
namespace {

constexpr int kWaves = 4;
constexpr int kQRowsPerWave = 32;
constexpr int kQBlock = kWaves * kQRowsPerWave;  // 128 query rows per workgroup
constexpr int kKeyTile = 64;                      // keys per LDS tile
constexpr int kVtStride = kKeyTile + 16;          // bytes per transposed V row (padded)

template <int D, bool kDebug>
__global__ __launch_bounds__(256) void ia_general_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, InvariantDiv nqb_div,
    int32_t* __restrict__ row_max, uint32_t* __restrict__ row_sum, uint8_t* __restrict__ probs) {
    constexpr int KS = D / 32;       // 32-deep k-steps of the Q.K^T contraction
    constexpr int DB = D / 32;       // 32-wide value-column blocks of the output
    constexpr int KStride = D + 16;  // padded K row in LDS (conflict-free 16-byte reads)

    __shared__ __attribute__((aligned(16))) int8_t sk[kKeyTile * KStride];
    __shared__ __attribute__((aligned(16))) int8_t svt[D * kVtStride];
    __shared__ uint16_t slut[kIaTabEntries];  // exp table by slot, or the direct table by gap (rest 0)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const UDivMod bq = divmod_invariant(blockIdx.x, nqb_div);
    const int qb = static_cast<int>(bq.r);
    const UDivMod bh = divmod_invariant(bq.q, P.h_div);
    const int h = static_cast<int>(bh.r);
    const int b = static_cast<int>(bh.q);
    const size_t head = static_cast<size_t>(b) * P.H + h;
    const int8_t* qh = q + head * P.Sq * D;
    // grouped K/V heads: query head h reads K/V head h / kv_group of its batch
    const uint32_t hkv = divmod_invariant(static_cast<uint32_t>(P.H), P.kvg_div).q;
    const size_t kvhead = static_cast<size_t>(b) * hkv + divmod_invariant(static_cast<uint32_t>(h), P.kvg_div).q;
    const int8_t* kh = k + kvhead * P.kv_rows * D;
    const int8_t* vh = v + kvhead * P.kv_rows * D;

    if (wave == 0) fill_lut_u16(P, slut, lane);

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
    const uint32_t C = static_cast<uint32_t>(mrow) * static_cast<uint32_t>(P.tab_mul) + P.tab_half;
    const int32_t negM = -P.tab_mul;
    const uint32_t tsh = static_cast<uint32_t>(P.tab_shift);
    // table entry of a score; a masked key (INT_MIN, never an int8 product)
    // has entry 0 outright: with a very small bin multiplier the clip point
    // lies beyond any score gap, and lo need not fit the 24-bit multiply
    auto entry = [&](int32_t sc) -> uint32_t { return sc == INT_MIN ? 0u : slut[slot_of(sc, lo, C, negM, tsh)]; };

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
            E += entry(s0[r]);
            E += entry(s1[r]);
        }
    }
    E += __shfl_xor(E, 32);
    const uint32_t R = reciprocal8(E);

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
                    const uint32_t e = entry(s[kb][r]);
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
            out[(head * P.Sq + qi) * D + d] = requantise(o[db][r] + 128 * cs, P);
        }
    }
}

}  // namespace

void clear_pending_hip_error() { (void)hipGetLastError(); }

int launch_general(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                   const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum,
                   uint8_t* probs) {
    const int nqb = (kp.Sq + kQBlock - 1) / kQBlock;
    const long long blocks = static_cast<long long>(nqb) * kp.H * kp.B;
    const InvariantDiv nqb_div = invariant_div(static_cast<uint32_t>(nqb));
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool debug = row_max != nullptr;
    if (D == 64) {
        if (debug)
            hipLaunchKernelGGL((ia_general_kernel<64, true>), grid, block, 0, s, q, k, v, out, kp, nqb_div, row_max, row_sum, probs);
        else
            hipLaunchKernelGGL((ia_general_kernel<64, false>), grid, block, 0, s, q, k, v, out, kp, nqb_div, row_max, row_sum, probs);
    } else {
        if (debug)
            hipLaunchKernelGGL((ia_general_kernel<128, true>), grid, block, 0, s, q, k, v, out, kp, nqb_div, row_max, row_sum, probs);
        else
            hipLaunchKernelGGL((ia_general_kernel<128, false>), grid, block, 0, s, q, k, v, out, kp, nqb_div, row_max, row_sum, probs);
    }
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

}  // namespace ia
