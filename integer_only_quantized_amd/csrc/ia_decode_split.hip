// Decode (Sq = 1) with each head's keys split into chunks of 512 to 4096 keys
// (split_chunk: halved while the grid has fewer than 1024 workgroups), one
// workgroup per (head, chunk), so that a few heads still fill the GPU and the
// key count is not bounded by the LDS.
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology",
// steps 2-3; integer widths and roundings as stated in include/intattn.h.
// Splitting is exact: the row max and the row sum E are combined from the
// chunks before any probability is formed (the table slot depends on the
// global max), and the P.V partials are integers, added in any order.
//   1 scores:  s_j = q . k_j for the chunk (K streamed once), stored in the
//              workspace as int32; chunk max; chunk 0 clears the head's
//              accumulator;
//   2 sums:    m = max of the chunk maxima; table entries and their sum over
//              the chunk (the stored scores are read back);
//   3 P.V:     E = sum of the chunk sums, R; p for the chunk's keys, then
//              sum_j p_j v_j over the chunk (V streamed once), atomically
//              added to the head's int32 accumulator;
//   4 output:  requantisation of the accumulators.
// HBM traffic beyond one read of K and V: 12 bytes per key and head.
#include "ia_device.h"
#include "ia_launch.h"

namespace ia {
namespace {

constexpr int kSplitChunk = 4096;     // most keys per workgroup (LDS holds their P)
constexpr int kSplitChunkMin = 512;   // a multiple of every key step below
constexpr int kSplitThreads = 256;    // 4 waves
constexpr int kSplitNW = kSplitThreads / 64;
constexpr int kSplitUnroll = 2;       // key groups a lane loads before using them

// Workspace layout (device memory the caller provides).
struct SplitWs {
    int32_t* scores;   // [heads][Skv]
    int32_t* cmax;     // [heads][nchunks]
    uint32_t* csum;    // [heads][nchunks]
    int32_t* acc;      // [heads][D]
};

// (head, chunk) of a workgroup and the chunk's key range [k0, k1).
struct SplitBlock {
    uint32_t head, chunk;
    int k0, k1;
};

__device__ __forceinline__ SplitBlock split_block(const InvariantDiv& nchunks_div, int Skv, int chunk) {
    const UDivMod hc = divmod_invariant(blockIdx.x, nchunks_div);
    const int k0 = static_cast<int>(hc.r) * chunk;
    return SplitBlock{hc.q, hc.r, k0, min(Skv, k0 + chunk)};
}

// Workgroup max / sum of a per-thread value (every thread gets the result).
__device__ __forceinline__ int32_t block_max(int32_t x, int32_t* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    int32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kSplitNW; ++w) r = max(r, red[w]);
    return r;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t x, int32_t* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = static_cast<int32_t>(x);
    __syncthreads();
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kSplitNW; ++w) r += static_cast<uint32_t>(red[w]);
    return r;
}

// Global row max of a head: max of its chunk maxima.
__device__ __forceinline__ int32_t split_row_max(const SplitWs& ws, uint32_t head, int nchunks) {
    int32_t m = INT_MIN;
    for (int c = 0; c < nchunks; ++c) m = max(m, ws.cmax[static_cast<size_t>(head) * nchunks + c]);
    return m;
}

// ---- 1: scores ---------------------------------------------------------------
// D/16 consecutive lanes cover one key row with 16-byte loads; each lane
// handles 4 keys, as in the single-workgroup decode kernel.
template <int D>
__global__ __launch_bounds__(kSplitThreads) void ia_dsplit_scores_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const IaKernelParams P, InvariantDiv nchunks_div,
    int nchunks, int chunk, SplitWs ws) {
    constexpr int CPR = D / 16;
    constexpr int GPW = 64 / CPR;
    constexpr int KEYS_IT = 4 * GPW * kSplitNW;
    __shared__ int32_t red[kSplitNW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % CPR, g = lane / CPR;
    const SplitBlock sb = split_block(nchunks_div, P.Skv, chunk);
    const size_t kvhead = divmod_invariant(sb.head, P.kvg_div).q;
    const int8_t* kh = k + kvhead * P.kv_rows * D;
    const v4i qv = *reinterpret_cast<const v4i*>(q + static_cast<size_t>(sb.head) * D + 16 * c);
    int32_t* const srow = ws.scores + static_cast<size_t>(sb.head) * P.Skv;
    if (sb.chunk == 0)
        for (int d = tid; d < D; d += kSplitThreads) ws.acc[static_cast<size_t>(sb.head) * D + d] = 0;
    int32_t tmax = INT_MIN;
    for (int base = sb.k0; base < sb.k1; base += kSplitUnroll * KEYS_IT) {
        v4i kr[kSplitUnroll][4];
#pragma unroll
        for (int u = 0; u < kSplitUnroll; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = base + u * KEYS_IT + wave * 4 * GPW + 4 * g + i;
                kr[u][i] = v4i{0, 0, 0, 0};
                if (key < sb.k1) kr[u][i] = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(key) * D + 16 * c);
            }
#pragma unroll
        for (int u = 0; u < kSplitUnroll; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = base + u * KEYS_IT + wave * 4 * GPW + 4 * g + i;
                int32_t sc = __builtin_amdgcn_sdot4(kr[u][i][0], qv[0], 0, false);
                sc = __builtin_amdgcn_sdot4(kr[u][i][1], qv[1], sc, false);
                sc = __builtin_amdgcn_sdot4(kr[u][i][2], qv[2], sc, false);
                sc = __builtin_amdgcn_sdot4(kr[u][i][3], qv[3], sc, false);
                sc += dpp_xor1(sc);
                sc += dpp_xor2(sc);
                if (CPR == 8) sc += dpp_half_mirror(sc);
                if (key < sb.k1) {
                    tmax = max(tmax, sc);
                    if (c == i) srow[key] = sc;
                }
            }
    }
    tmax = block_max(tmax, red);
    if (tid == 0) ws.cmax[static_cast<size_t>(sb.head) * nchunks + sb.chunk] = tmax;
}

// ---- 2: table entries and their sum over a chunk ---------------------------------
__global__ __launch_bounds__(kSplitThreads) void ia_dsplit_sums_kernel(const IaKernelParams P,
                                                                       InvariantDiv nchunks_div, int nchunks,
                                                                       int chunk, SplitWs ws) {
    __shared__ uint16_t s_lut[kIaTabEntries];
    __shared__ int32_t red[kSplitNW];
    const int tid = threadIdx.x;
    if (tid < 64) fill_lut_u16(P, s_lut, tid);
    const SplitBlock sb = split_block(nchunks_div, P.Skv, chunk);
    const int32_t m = split_row_max(ws, sb.head, nchunks);
    const int32_t lo = m - P.x_clip;
    const uint32_t Cm = static_cast<uint32_t>(m) * static_cast<uint32_t>(P.tab_mul) + P.tab_half;
    const int32_t negM = -P.tab_mul;
    __syncthreads();
    const int32_t* srow = ws.scores + static_cast<size_t>(sb.head) * P.Skv;
    uint32_t E = 0;
    for (int j = sb.k0 + tid; j < sb.k1; j += kSplitThreads) {
        const int32_t sp = max(srow[j], lo);
        E += s_lut[(Cm + static_cast<uint32_t>(__mul24(sp, negM))) >> P.tab_shift];
    }
    E = block_sum(E, red);
    if (tid == 0) ws.csum[static_cast<size_t>(sb.head) * nchunks + sb.chunk] = E;
}

// ---- 3: probabilities and P.V over a chunk ------------------------------------------
template <int D, bool P16>
__global__ __launch_bounds__(kSplitThreads) void ia_dsplit_pv_kernel(
    const int8_t* __restrict__ v, const IaKernelParams P, InvariantDiv nchunks_div, int nchunks, int chunk,
    SplitWs ws, int32_t* __restrict__ row_max, uint32_t* __restrict__ row_sum) {
    constexpr int CPR = D / 16;
    constexpr int GPW = 64 / CPR;
    constexpr int KEYS_IT = 4 * GPW * kSplitNW;
    constexpr int STEP = kSplitUnroll * KEYS_IT;
    static_assert(kSplitChunkMin % STEP == 0, "chunks hold whole key steps");
    __shared__ uint16_t s_lut[kIaTabEntries];
    __shared__ __attribute__((aligned(16))) uint8_t s_p[kSplitChunk * (P16 ? 2 : 1)];
    __shared__ int32_t s_red[P16 ? 2 : 1][kSplitNW][D];
    __shared__ int32_t red[kSplitNW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % CPR, g = lane / CPR;
    if (tid < 64) fill_lut_u16(P, s_lut, tid);
    const SplitBlock sb = split_block(nchunks_div, P.Skv, chunk);
    const size_t kvhead = divmod_invariant(sb.head, P.kvg_div).q;
    const int8_t* vh = v + kvhead * P.kv_rows * D;
    const int32_t m = split_row_max(ws, sb.head, nchunks);
    uint32_t E = 0;
    for (int ch = 0; ch < nchunks; ++ch) E += ws.csum[static_cast<size_t>(sb.head) * nchunks + ch];
    const uint32_t R = P16 ? reciprocal16(E) : reciprocal8(E);
    if (row_max != nullptr && sb.chunk == 0 && tid == 0) {
        row_max[sb.head] = m;
        row_sum[sb.head] = E;
    }
    const int32_t lo = m - P.x_clip;
    const uint32_t Cm = static_cast<uint32_t>(m) * static_cast<uint32_t>(P.tab_mul) + P.tab_half;
    const int32_t negM = -P.tab_mul;
    __syncthreads();
    // p of the chunk's keys into LDS (0 past the last key, up to whole steps)
    const int n = sb.k1 - sb.k0;
    const int npad = (n + STEP - 1) / STEP * STEP;
    const int32_t* srow = ws.scores + static_cast<size_t>(sb.head) * P.Skv + sb.k0;
    uint32_t psum = 0, psum_lo = 0;
    for (int j = tid; j < npad; j += kSplitThreads) {
        uint32_t p = 0;
        if (j < n) {
            const int32_t sp = max(srow[j], lo);
            const uint32_t e = s_lut[(Cm + static_cast<uint32_t>(__mul24(sp, negM))) >> P.tab_shift];
            p = P16 ? (e * R + (1u << 15)) >> 16 : (e * R + (1u << 22)) >> 23;
        }
        if constexpr (P16) {
            reinterpret_cast<uint16_t*>(s_p)[j] = static_cast<uint16_t>(p);
            psum += p >> 8;
            psum_lo += p & 0xffu;
        } else {
            s_p[j] = static_cast<uint8_t>(p);
            psum += p;
        }
    }
    psum = block_sum(psum, red);
    if constexpr (P16) psum_lo = block_sum(psum_lo, red);
    // P.V as in the decode kernel: each lane transposes its 4 keys x 16 value
    // columns and accumulates udot4(p, v + 128); a_d = acc_d - 128 sum p
    uint32_t acc[16], acc_lo[P16 ? 16 : 1];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0;
#pragma unroll
    for (int i = 0; i < (P16 ? 16 : 1); ++i) acc_lo[i] = 0;
    for (int base = 0; base < npad; base += STEP) {
        v4i vr[kSplitUnroll][4];
        uint32_t pk[kSplitUnroll], pk_lo[kSplitUnroll];
#pragma unroll
        for (int u = 0; u < kSplitUnroll; ++u) {
            const int j0 = base + u * KEYS_IT + wave * 4 * GPW + 4 * g;   // chunk-relative, multiple of 4
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vr[u][i] = v4i{0, 0, 0, 0};
                if (j0 + i < n)
                    vr[u][i] = *reinterpret_cast<const v4i*>(vh + static_cast<size_t>(sb.k0 + j0 + i) * D + 16 * c);
            }
            if constexpr (P16) {
                const uint2 w = *reinterpret_cast<const uint2*>(s_p + 2 * j0);
                pk[u] = __builtin_amdgcn_perm(w.y, w.x, 0x07050301u);
                pk_lo[u] = __builtin_amdgcn_perm(w.y, w.x, 0x06040200u);
            } else {
                pk[u] = *reinterpret_cast<const uint32_t*>(s_p + j0);
                pk_lo[u] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kSplitUnroll; ++u)
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
                const uint32_t c0 = __builtin_amdgcn_perm(u2, u0, 0x05040100u);
                const uint32_t c1 = __builtin_amdgcn_perm(u2, u0, 0x07060302u);
                const uint32_t c2 = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
                const uint32_t c3 = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
                acc[4 * w + 0] = __builtin_amdgcn_udot4(c0, pk[u], acc[4 * w + 0], false);
                acc[4 * w + 1] = __builtin_amdgcn_udot4(c1, pk[u], acc[4 * w + 1], false);
                acc[4 * w + 2] = __builtin_amdgcn_udot4(c2, pk[u], acc[4 * w + 2], false);
                acc[4 * w + 3] = __builtin_amdgcn_udot4(c3, pk[u], acc[4 * w + 3], false);
                if constexpr (P16) {
                    acc_lo[4 * w + 0] = __builtin_amdgcn_udot4(c0, pk_lo[u], acc_lo[4 * w + 0], false);
                    acc_lo[4 * w + 1] = __builtin_amdgcn_udot4(c1, pk_lo[u], acc_lo[4 * w + 1], false);
                    acc_lo[4 * w + 2] = __builtin_amdgcn_udot4(c2, pk_lo[u], acc_lo[4 * w + 2], false);
                    acc_lo[4 * w + 3] = __builtin_amdgcn_udot4(c3, pk_lo[u], acc_lo[4 * w + 3], false);
                }
            }
    }
    // lanes with the same column chunk (stride CPR) hold partial sums
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int off = CPR; off < 64; off <<= 1) acc[i] += __shfl_xor(acc[i], off);
    }
    if constexpr (P16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
            for (int off = CPR; off < 64; off <<= 1) acc_lo[i] += __shfl_xor(acc_lo[i], off);
        }
    }
    if (g == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s_red[0][wave][16 * c + i] = static_cast<int32_t>(acc[i]);
        if constexpr (P16) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s_red[P16 ? 1 : 0][wave][16 * c + i] = static_cast<int32_t>(acc_lo[i]);
        }
    }
    __syncthreads();
    for (int d = tid; d < D; d += kSplitThreads) {
        uint32_t tot = 0;
#pragma unroll
        for (int w = 0; w < kSplitNW; ++w) tot += static_cast<uint32_t>(s_red[0][w][d]);
        // sum p v over the chunk = sum p (v + 128) - 128 sum p; uint16 P:
        // 256 (high bytes) + low bytes
        uint32_t a = tot - 128u * psum;
        if constexpr (P16) {
            uint32_t lo16 = 0;
#pragma unroll
            for (int w = 0; w < kSplitNW; ++w) lo16 += static_cast<uint32_t>(s_red[P16 ? 1 : 0][w][d]);
            a = 256u * a + (lo16 - 128u * psum_lo);
        }
        atomicAdd(ws.acc + static_cast<size_t>(sb.head) * D + d, static_cast<int32_t>(a));
    }
}

// ---- 4: requantisation ------------------------------------------------------------------
__global__ __launch_bounds__(kSplitThreads) void ia_dsplit_out_kernel(int8_t* __restrict__ out, const IaKernelParams P,
                                                                      SplitWs ws, int total) {
    const int i = static_cast<int>(blockIdx.x) * kSplitThreads + static_cast<int>(threadIdx.x);
    if (i < total) out[i] = requantise(ws.acc[i], P);
}

// 256-byte aligned regions of the workspace.
inline size_t split_align(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

}  // namespace

// Keys per chunk for B*H heads: 4096, halved (down to 512) while the grid
// would have fewer than 1024 workgroups.
int split_chunk(long long heads, int Skv) {
    int chunk = kSplitChunk;
    while (chunk > kSplitChunkMin && heads * ((Skv + chunk - 1) / chunk) < 1024) chunk /= 2;
    return chunk;
}

size_t decode_split_workspace_bytes(long long heads, int Skv, int D) {
    const int chunk = split_chunk(heads, Skv);
    const int nchunks = (Skv + chunk - 1) / chunk;
    return split_align(static_cast<size_t>(heads) * Skv * 4) + 2 * split_align(static_cast<size_t>(heads) * nchunks * 4) +
           split_align(static_cast<size_t>(heads) * D * 4);
}

int launch_decode_split(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D, const IaKernelParams& kp,
                        void* stream, void* workspace, int32_t* row_max, uint32_t* row_sum) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const long long heads = static_cast<long long>(kp.B) * kp.H;
    const int chunk = split_chunk(heads, kp.Skv);
    const int nchunks = (kp.Skv + chunk - 1) / chunk;
    const long long blocks = heads * nchunks;
    if (blocks > INT_MAX || heads * D > INT_MAX) return INTATTN_E_SHAPE;
    char* base = static_cast<char*>(workspace);
    SplitWs ws;
    ws.scores = reinterpret_cast<int32_t*>(base);
    base += split_align(static_cast<size_t>(heads) * kp.Skv * 4);
    ws.cmax = reinterpret_cast<int32_t*>(base);
    base += split_align(static_cast<size_t>(heads) * nchunks * 4);
    ws.csum = reinterpret_cast<uint32_t*>(base);
    base += split_align(static_cast<size_t>(heads) * nchunks * 4);
    ws.acc = reinterpret_cast<int32_t*>(base);
    const InvariantDiv ndiv = invariant_div(static_cast<uint32_t>(nchunks));
    const dim3 grid(static_cast<unsigned>(blocks)), block(kSplitThreads);
    if (D == 64) hipLaunchKernelGGL((ia_dsplit_scores_kernel<64>), grid, block, 0, s, q, k, kp, ndiv, nchunks, chunk, ws);
    else hipLaunchKernelGGL((ia_dsplit_scores_kernel<128>), grid, block, 0, s, q, k, kp, ndiv, nchunks, chunk, ws);
    hipLaunchKernelGGL(ia_dsplit_sums_kernel, grid, block, 0, s, kp, ndiv, nchunks, chunk, ws);
    const bool p16 = kp.prob_bits == 16;
    if (D == 64) {
        if (p16) hipLaunchKernelGGL((ia_dsplit_pv_kernel<64, true>), grid, block, 0, s, v, kp, ndiv, nchunks, chunk, ws, row_max, row_sum);
        else hipLaunchKernelGGL((ia_dsplit_pv_kernel<64, false>), grid, block, 0, s, v, kp, ndiv, nchunks, chunk, ws, row_max, row_sum);
    } else {
        if (p16) hipLaunchKernelGGL((ia_dsplit_pv_kernel<128, true>), grid, block, 0, s, v, kp, ndiv, nchunks, chunk, ws, row_max, row_sum);
        else hipLaunchKernelGGL((ia_dsplit_pv_kernel<128, false>), grid, block, 0, s, v, kp, ndiv, nchunks, chunk, ws, row_max, row_sum);
    }
    const int total = static_cast<int>(heads * D);
    hipLaunchKernelGGL(ia_dsplit_out_kernel, dim3(static_cast<unsigned>((total + kSplitThreads - 1) / kSplitThreads)),
                       block, 0, s, out, kp, ws, total);
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

}  // namespace ia
