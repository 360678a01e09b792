// The attention pipeline as separate kernels with HBM between the stages:
// Q.K^T -> softmax -> P.V. The fused kernels never write scores or
// probabilities; these stages do, so the time of each stage (and the share
// of the softmax) can be measured on its own, and the integer softmax can be
// compared with the floating-point one it replaces.
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology":
// step 1 (an INT8 pipeline converts the integer scores to floating point,
// exponentiates, normalises and converts back: the comparator stage here),
// step 2 (IndexSoftmax), step 3 (integer Q.K^T and P.V). Integer widths and
// roundings as stated in include/intattn.h.
#include <cmath>

#include "ia_device.h"

namespace ia {
namespace {

// rows of the softmax stages are held in registers: up to 64 chunks of 64
constexpr int kStageMaxChunks = 64;

// ---------------------------------------------------------------------------
// Stage 1: scores = Q.K^T (int32, every (i, j); masks are applied later)
// ---------------------------------------------------------------------------
// One workgroup = 4 waves = 128 queries x 64 keys of one head. S tiles
// (queries x keys) on v_mfma_i32_32x32x32_i8 with Q as the A operand: lane
// (l32, hh) holds key column l32 of 16 query rows, so every store writes 32
// consecutive int32 of a row per lane half.
// Query row within its head of stage row 4 * block + w (w < 4), i.e.
// (4 * block + w) mod Sq, from a 32-bit division of the block index: the
// remainder r of block by Sq gives 4r + w < 4 Sq, three subtractions at most.
__device__ __forceinline__ int row_in_head(uint32_t block, int w, int Sq, const InvariantDiv& sq_div) {
    uint64_t t = 4ull * divmod_invariant(block, sq_div).r + static_cast<uint64_t>(w);
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if (t >= static_cast<uint64_t>(Sq)) t -= static_cast<uint64_t>(Sq);
    return static_cast<int>(t);
}

template <int D>
__global__ __launch_bounds__(256) void ia_qk_kernel(const int8_t* __restrict__ q, const int8_t* __restrict__ k,
                                                    int32_t* __restrict__ scores, int Sq, int Skv,
                                                    InvariantDiv nqb_div, InvariantDiv nkt_div) {
    constexpr int KS = D / 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const UDivMod bk = divmod_invariant(blockIdx.x, nkt_div);
    const UDivMod bq = divmod_invariant(bk.q, nqb_div);
    const int kt = static_cast<int>(bk.r);
    const int qb = static_cast<int>(bq.r);
    const size_t head = bq.q;
    const int8_t* qh = q + head * Sq * D;
    const int8_t* kh = k + head * Skv * D;
    const int q0 = qb * 128 + 32 * wave;

    v4i qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = (q0 + l32 < Sq) ? *reinterpret_cast<const v4i*>(qh + static_cast<size_t>(q0 + l32) * D + 32 * ks + 16 * hh)
                                 : v4i{0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int key = kt * 64 + 32 * kb + l32;
        const int kr = min(key, Skv - 1);
        v4i kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[ks] = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(kr) * D + 32 * ks + 16 * hh);
        v16i s = v16i{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma_i8_32x32x32(qf[ks], kf[ks], s);
        if (key < Skv) {
            int32_t* const col = scores + (head * Sq + q0 + 4 * hh) * Skv + key;
            if (q0 + 32 <= Sq) {
#pragma unroll
                for (int r = 0; r < 16; ++r) col[static_cast<size_t>(acc_row(r, 0)) * Skv] = s[r];
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (q0 + 4 * hh + acc_row(r, 0) < Sq) col[static_cast<size_t>(acc_row(r, 0)) * Skv] = s[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Stage 2: softmax rows (one wave per row, the row held in registers)
// ---------------------------------------------------------------------------
// Lane l holds elements j = 64c + l, c = 0..NCH-1 (coalesced dword loads);
// NCH*64 >= Skv. Keys j >= kend (causal) or j >= Skv are not allowed.
__device__ __forceinline__ int32_t wave_max(int32_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ float wave_maxf(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sumf(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// IndexSoftmax of one row: row max, slot words (clamped 24-bit multiply-add
// as in the fused kernels; y = s - m is first clamped at -2^23, which every
// allowed key below -x_clip reaches in the last slot anyway), table entries,
// row sum E, R = floor((255*2^23 + floor(E/2)) / E), p = top byte of
// e*2R + 2^23. Scores must satisfy |s| < 2^30 (true for Q.K^T of int8).
template <int NCH, int KM>
__global__ __launch_bounds__(256) void ia_index_softmax_kernel(const int32_t* __restrict__ scores,
                                                               uint8_t* __restrict__ probs,
                                                               int32_t* __restrict__ row_max,
                                                               uint32_t* __restrict__ row_sum,
                                                               const IaKernelParams P, long long rows,
                                                               InvariantDiv sq_div) {
    __shared__ uint32_t lut[kIaTabEntries / 2];   // exp table, layout KM
    const int tid = threadIdx.x;
    if (tid < 64) fill_lut_table<KM>(P, lut, tid);   // wave 0, whole
    __syncthreads();
    const int lane = tid & 63;
    const long long row = static_cast<long long>(blockIdx.x) * 4 + (tid >> 6);
    if (row >= rows) return;
    const int Skv = P.Skv;
    const int i = row_in_head(blockIdx.x, tid >> 6, P.Sq, sq_div);
    const int kend = P.causal ? min(Skv, i + (Skv - P.Sq) + 1) : Skv;
    const int32_t* src = scores + row * Skv;

    int32_t s[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j = 64 * c + lane;
        s[c] = j < Skv ? src[j] : 0;
    }
    int32_t m = INT_MIN;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (64 * c + lane < kend) m = max(m, s[c]);
    m = wave_max(m);

    uint32_t e[NCH];
    uint32_t E = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int32_t y = 64 * c + lane < kend ? max(s[c] - m, -(1 << 23)) : -(1 << 23);
        e[c] = lut_load<KM>(lds_addr(lut) + entry_addr<KM>(y, P.ent_a, P.ent_b));
        E += e[c];
    }
    E = wave_sum(E);
    const uint32_t R2 = 2 * reciprocal8(E);
    uint8_t* dst = probs + row * Skv;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j = 64 * c + lane;
        if (j < Skv) dst[j] = static_cast<uint8_t>((__umul24(e[c], R2) + (1u << 23)) >> 24);
    }
    if (lane == 0 && row_max != nullptr) {
        row_max[row] = m;
        row_sum[row] = E;
    }
}

// Floating-point comparator of the same row: dequantise (y = alpha * s in
// float32), softmax with the row max subtracted (exp2 of (y - m) * log2 e on
// the hardware exp unit, float32 sum), requantise p to a uint8 code
// rint(255 * p) (ties to even), clamped to 255. Keys that are not allowed
// get code 0.
template <int NCH>
__global__ __launch_bounds__(256) void ia_fp_softmax_kernel(const int32_t* __restrict__ scores,
                                                            uint8_t* __restrict__ probs, float alpha, int Sq,
                                                            int Skv, int causal, long long rows) {
    const int lane = threadIdx.x & 63;
    const long long row = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int i = static_cast<int>(row % Sq);
    const int kend = causal ? min(Skv, i + (Skv - Sq) + 1) : Skv;
    const int32_t* src = scores + row * Skv;
    constexpr float kLog2e = 1.4426950408889634f;
    float y[NCH];
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j = 64 * c + lane;
        y[c] = j < kend ? static_cast<float>(src[j]) * alpha : -INFINITY;
        m = fmaxf(m, y[c]);
    }
    m = wave_maxf(m);
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        y[c] = 64 * c + lane < kend ? __builtin_amdgcn_exp2f((y[c] - m) * kLog2e) : 0.0f;
        sum += y[c];
    }
    sum = wave_sumf(sum);
    const float scale = 255.0f / sum;
    uint8_t* dst = probs + row * Skv;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j = 64 * c + lane;
        if (j < Skv) dst[j] = static_cast<uint8_t>(fminf(__builtin_rintf(y[c] * scale), 255.0f));
    }
}

// ---------------------------------------------------------------------------
// Stage 3: out = requantise(P.V)
// ---------------------------------------------------------------------------
// One workgroup = 4 waves = 128 query rows of one head; V tiles of 64 keys
// are staged row-major by global_load_lds (double buffered), chunks swizzled
// so that the transpose reads of 8 consecutive keys are conflict free; P
// comes from HBM in key order (16 consecutive keys per lane and block). The
// MFMA is signed, so P enters as p - 128 and the column sums of the V rows
// fed are added back (tail keys past Skv enter with p = 0).
template <int D>
__device__ __forceinline__ int vc_swz(int key) {
    return D == 128 ? (key & 6) : ((key >> 1) & 2);
}

template <int D, bool ALIGNED>
__global__ __launch_bounds__(256) void ia_pv_kernel(const uint8_t* __restrict__ probs, const int8_t* __restrict__ v,
                                                    int8_t* __restrict__ out, const IaKernelParams P,
                                                    InvariantDiv nqb_div) {
    constexpr int DB = D / 32;
    constexpr int TB = 64 * D;                   // bytes per V tile
    constexpr int CPR = D / 16;
    constexpr int LOADS = TB / 1024 / 4;         // 1 KB loads per wave per tile
    __shared__ __attribute__((aligned(16))) int8_t vt[2][TB];
    __shared__ int32_t colsum[4][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const UDivMod bq = divmod_invariant(blockIdx.x, nqb_div);
    const int qb = static_cast<int>(bq.r);
    const size_t head = bq.q;
    const int Sq = P.Sq, Skv = P.Skv;
    const uint8_t* ph = probs + head * Sq * Skv;
    const int8_t* vh = v + head * Skv * D;
    const int qw0 = qb * 128 + 32 * wave;
    const int qrow = qw0 + l32;
    const int qlast = min(qb * 128 + 128, Sq) - 1;
    // keys past the causal limit of the workgroup's last row have p = 0 for
    // every row of it: their tiles contribute nothing and are skipped
    const int kend_wg = P.causal ? min(Skv, qlast + (Skv - Sq) + 1) : Skv;
    const int ntiles = (kend_wg + 63) / 64;

    auto issue = [&](int t, int st) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int blk = wave * LOADS + i;
            const int row = blk * (1024 / D) + lane / CPR;
            const int chunk = (lane % CPR) ^ vc_swz<D>(row);
            const int key = min(t * 64 + row, Skv - 1);
            __builtin_amdgcn_global_load_lds(vh + static_cast<size_t>(key) * D + 16 * chunk,
                                             (lds_void_t*)(&vt[st][blk * 1024]), 16, 0, 0);
        }
    };
    // transpose-read addresses (stage 0, key block 0): read rd of column
    // block db, lane pair (2i, 2i+1) supplies key 16hh + 8rd + i
    uint32_t va[2 * DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int key = 16 * hh + 8 * rd + ((lane & 15) >> 1);
            const int col = 32 * db + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
            va[2 * db + rd] = lds_addr(&vt[0][0]) +
                              static_cast<uint32_t>(key * D + 16 * ((col >> 4) ^ vc_swz<D>(key)) + (col & 15));
        }

    v16i o[DB];
    int32_t cs[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        o[db] = v16i{};
        cs[db] = 0;
    }
    if (ntiles > 0) {
        issue(0, 0);
        wait_vmcnt(0);
    }
    lds_barrier();
    for (int t = 0; t < ntiles; ++t) {
        const int st = t & 1;
        if (t + 1 < ntiles) issue(t + 1, st ^ 1);
        uint32_t vs[2 * DB];
#pragma unroll
        for (int i2 = 0; i2 < 2 * DB; ++i2) vs[i2] = va[i2] + static_cast<uint32_t>(st * TB);
        const bool turn = (t & 3) == wave;
        static_for<2>([&](auto kbc) {
            constexpr int kb = decltype(kbc)::value;
            const int key0 = t * 64 + 32 * kb + 16 * hh;      // this lane's 16 keys
            v4i pa;
            if (qrow < Sq && key0 < Skv) {
                const uint8_t* pp = ph + static_cast<size_t>(qrow) * Skv + key0;
                if (ALIGNED) {
                    pa = *reinterpret_cast<const v4i*>(pp);
                } else {
                    uint32_t w[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        w[x] = 0;
#pragma unroll
                        for (int y = 0; y < 4; ++y)
                            if (key0 + 4 * x + y < Skv) w[x] |= static_cast<uint32_t>(pp[4 * x + y]) << (8 * y);
                    }
                    pa = v4i{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]),
                             static_cast<int>(w[3])};
                }
            } else {
                pa = v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) pa[x] ^= static_cast<int>(0x80808080u);   // p - 128
            v4i vb[DB];
            tr8_operands<DB, kb * 32 * D>(vs, vb);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma_i8_32x32x32(pa, vb[db], o[db]);
            if (turn) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    asm volatile("" : "+v"(cs[db]));
#pragma unroll
                    for (int w = 0; w < 4; ++w) cs[db] = __builtin_amdgcn_sdot4(vb[db][w], 0x01010101, cs[db], false);
                }
            }
        });
        wait_vmcnt(0);
        lds_barrier();
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int32_t tot = cs[db] + __shfl_xor(cs[db], 32);
        if (hh == 0) colsum[wave][32 * db + l32] = tot;
    }
    __syncthreads();
    int8_t* const obase = out + (head * Sq + qw0 + 4 * hh) * D;
    const bool full = qw0 + 32 <= Sq;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + l32;
        const int32_t c128 = 128 * (colsum[0][d] + colsum[1][d] + colsum[2][d] + colsum[3][d]);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (full || qw0 + 4 * hh + acc_row(r, 0) < Sq)
                obase[acc_row(r, 0) * D + d] = requantise(o[db][r] + c128, P);
    }
}

// number of 64-element register chunks for a row, rounded up to a power of 2
int row_chunks(int Skv) {
    int n = 1;
    while (64 * n < Skv) n *= 2;
    return n;
}

template <int NCH>
int launch_isoftmax_n(int nch, const int32_t* scores, uint8_t* probs, int32_t* row_max, uint32_t* row_sum,
                      const IaKernelParams& kp, hipStream_t s, long long rows, unsigned blocks) {
    if constexpr (NCH > kStageMaxChunks) {
        return INTATTN_E_SHAPE;
    } else {
        if (nch != NCH)
            return launch_isoftmax_n<NCH * 2>(nch, scores, probs, row_max, row_sum, kp, s, rows, blocks);
        if (kp.slot_k == 4)
            hipLaunchKernelGGL((ia_index_softmax_kernel<NCH, 4>), dim3(blocks), dim3(256), 0, s, scores, probs,
                               row_max, row_sum, kp, rows, invariant_div(static_cast<uint32_t>(kp.Sq)));
        else if (kp.slot_k == 2)
            hipLaunchKernelGGL((ia_index_softmax_kernel<NCH, 2>), dim3(blocks), dim3(256), 0, s, scores, probs,
                               row_max, row_sum, kp, rows, invariant_div(static_cast<uint32_t>(kp.Sq)));
        else if (kp.slot_k == 1)
            hipLaunchKernelGGL((ia_index_softmax_kernel<NCH, 1>), dim3(blocks), dim3(256), 0, s, scores, probs,
                               row_max, row_sum, kp, rows, invariant_div(static_cast<uint32_t>(kp.Sq)));
        else
            hipLaunchKernelGGL((ia_index_softmax_kernel<NCH, 0>), dim3(blocks), dim3(256), 0, s, scores, probs,
                               row_max, row_sum, kp, rows, invariant_div(static_cast<uint32_t>(kp.Sq)));
        return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
    }
}

template <int NCH>
int launch_fpsoftmax_n(int nch, const int32_t* scores, uint8_t* probs, float alpha, const IaKernelParams& kp,
                       hipStream_t s, long long rows, unsigned blocks) {
    if constexpr (NCH > kStageMaxChunks) {
        return INTATTN_E_SHAPE;
    } else {
        if (nch != NCH) return launch_fpsoftmax_n<NCH * 2>(nch, scores, probs, alpha, kp, s, rows, blocks);
        hipLaunchKernelGGL((ia_fp_softmax_kernel<NCH>), dim3(blocks), dim3(256), 0, s, scores, probs, alpha, kp.Sq,
                           kp.Skv, kp.causal, rows);
        return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
    }
}

}  // namespace

int stage_max_keys() { return 64 * kStageMaxChunks; }

int launch_qk_scores(const int8_t* q, const int8_t* k, int32_t* scores, int D, const IaKernelParams& kp,
                     void* stream) {
    const int nqb = (kp.Sq + 127) / 128;
    const int nkt = (kp.Skv + 63) / 64;
    const long long blocks = static_cast<long long>(kp.B) * kp.H * nqb * nkt;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (D == 64)
        hipLaunchKernelGGL((ia_qk_kernel<64>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, q, k, scores,
                           kp.Sq, kp.Skv, invariant_div(nqb), invariant_div(nkt));
    else
        hipLaunchKernelGGL((ia_qk_kernel<128>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, q, k, scores,
                           kp.Sq, kp.Skv, invariant_div(nqb), invariant_div(nkt));
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

int launch_index_softmax(const int32_t* scores, uint8_t* probs, int32_t* row_max, uint32_t* row_sum,
                         const IaKernelParams& kp, void* stream) {
    const long long rows = static_cast<long long>(kp.B) * kp.H * kp.Sq;
    const long long blocks = (rows + 3) / 4;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    return launch_isoftmax_n<1>(row_chunks(kp.Skv), scores, probs, row_max, row_sum, kp,
                                static_cast<hipStream_t>(stream), rows, static_cast<unsigned>(blocks));
}

int launch_fp_softmax(const int32_t* scores, uint8_t* probs, float alpha, const IaKernelParams& kp, void* stream) {
    const long long rows = static_cast<long long>(kp.B) * kp.H * kp.Sq;
    const long long blocks = (rows + 3) / 4;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    return launch_fpsoftmax_n<1>(row_chunks(kp.Skv), scores, probs, alpha, kp, static_cast<hipStream_t>(stream),
                                 rows, static_cast<unsigned>(blocks));
}

int launch_pv(const uint8_t* probs, const int8_t* v, int8_t* out, int D, const IaKernelParams& kp, void* stream) {
    const int nqb = (kp.Sq + 127) / 128;
    const long long blocks = static_cast<long long>(kp.B) * kp.H * nqb;
    const InvariantDiv nqb_div = invariant_div(static_cast<uint32_t>(nqb));
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool aligned = (kp.Skv % 16) == 0 && (reinterpret_cast<uintptr_t>(probs) & 15u) == 0;
    const dim3 g(static_cast<unsigned>(blocks));
    if (D == 64) {
        if (aligned) hipLaunchKernelGGL((ia_pv_kernel<64, true>), g, dim3(256), 0, s, probs, v, out, kp, nqb_div);
        else hipLaunchKernelGGL((ia_pv_kernel<64, false>), g, dim3(256), 0, s, probs, v, out, kp, nqb_div);
    } else {
        if (aligned) hipLaunchKernelGGL((ia_pv_kernel<128, true>), g, dim3(256), 0, s, probs, v, out, kp, nqb_div);
        else hipLaunchKernelGGL((ia_pv_kernel<128, false>), g, dim3(256), 0, s, probs, v, out, kp, nqb_div);
    }
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

}  // namespace ia
