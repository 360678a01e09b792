// Decode integer attention kernel (gfx950 / CDNA4): one query row per head,
// keys and values streamed once from HBM.
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology",
// steps 2-3; integer widths and roundings as stated in include/intattn.h.
#include "ia_device.h"
#include "ia_launch.h"

namespace ia {
namespace {

// Largest key count served by the decode kernel (5 bytes of LDS per key).
constexpr int kDecodeMaxKeys = 16384;

// Decode kernel: one query row per head (Sq = 1), keys streamed from HBM.
// One workgroup (NWQ = 4 waves, or 16 with fewer heads than compute units)
// per (b, h). D/16 consecutive lanes cover one key
// row with 16-byte loads (fully coalesced); each lane handles 4 keys.
//   A: scores s_j = q . k_j: four sdot4 per 16 bytes, then a butterfly over
//      the D/16 lanes of a row (DPP), scores kept in LDS (int32 per key);
//   B: row max (wave reduction + LDS);
//   C: slots, table lookups and row sum; the scores' LDS words are reused
//      for the slots; then p_j for every key (one table per row, N <= 128);
//   D: P.V: each lane transposes its 4 keys x 16 value columns (v_perm) and
//      accumulates udot4(p, v + 128) (adding 128 to a signed byte = XOR 0x80),
//      so a_d = sum_j p_j v_jd = acc_d - 128 * sum_j p_j; lanes and waves are
//      then reduced and the result requantised.
// HBM traffic is one read of K and V; the LDS holds 5 bytes per key.
constexpr int kDecodeThreads = 256;
// Key groups a lane loads before using any of them (its loads in flight).
constexpr int kDecodeUnroll = 2;


template <int D, bool P16, int QH, int NWQ>
__global__ __launch_bounds__(64 * NWQ * QH) void ia_decode_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int skv_pad, int32_t* __restrict__ row_max,
    uint32_t* __restrict__ row_sum) {
    static_assert(QH == 1 || (QH == 2 && !P16), "two query heads a workgroup with uint8 P only");
    constexpr int NT = 64 * NWQ * QH;           // threads: NWQ waves per query head
    constexpr int NW = NT / 64;                 // waves
    constexpr int CPR = D / 16;                 // lanes per key row
    constexpr int GPW = 64 / CPR;               // key groups (of 4 keys) per wave
    constexpr int KEYS_IT = 4 * GPW * NW;       // keys per iteration
    extern __shared__ __attribute__((aligned(16))) int32_t dsm[];
    // per query head h: skv_pad ints (scores, then slots) at dsm + h * skv_pad,
    // then skv_pad bytes of P (uint16 P: 2 per key)
    int32_t* const s_score = dsm;
    uint8_t* const s_p = reinterpret_cast<uint8_t*>(dsm + QH * skv_pad);
    __shared__ uint16_t s_lut[kIaTabEntries];  // exp table by slot, or the direct table by gap (rest 0)
    __shared__ int32_t s_red[P16 ? 2 : QH][NW][D];
    __shared__ int32_t s_scal[QH][3 * NW];     // per wave: row max, row sum, sum of p (uint16 P: low bytes)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane % CPR;                   // 16-byte column chunk
    const int g = lane / CPR;                   // key group within the wave
    // grouped K/V heads: the query heads of one K/V head run on the same XCD
    // (consecutive logical blocks), so its K and V stream once into that L2;
    // with QH = 2 a workgroup takes two query heads of one K/V head and reads
    // each K and V chunk once for both
    const int bid = P.kv_group > QH ? xcd_local_block(blockIdx.x, gridDim.x) : static_cast<int>(blockIdx.x);
    const size_t head0 = static_cast<size_t>(bid) * QH;
    const size_t kvhead = divmod_invariant(static_cast<uint32_t>(head0), P.kvg_div).q;
    const int8_t* kh = k + kvhead * P.kv_rows * D;
    const int8_t* vh = v + kvhead * P.kv_rows * D;
    v4i qv[QH];
#pragma unroll
    for (int h = 0; h < QH; ++h) qv[h] = *reinterpret_cast<const v4i*>(q + (head0 + h) * D + 16 * c);
    if (wave == 0) fill_lut_u16(P, s_lut, lane);

    // ---- A: scores ---------------------------------------------------------
    int32_t tmax[QH];
#pragma unroll
    for (int h = 0; h < QH; ++h) tmax[h] = INT_MIN;
    for (int base = 0; base < P.Skv; base += kDecodeUnroll * KEYS_IT) {
        v4i kr[kDecodeUnroll][4];
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = base + u * KEYS_IT + wave * 4 * GPW + 4 * g + i;
                kr[u][i] = v4i{0, 0, 0, 0};
                if (key < P.Skv) kr[u][i] = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(key) * D + 16 * c);
            }
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = base + u * KEYS_IT + wave * 4 * GPW + 4 * g + i;
#pragma unroll
                for (int h = 0; h < QH; ++h) {
                    int32_t sc = __builtin_amdgcn_sdot4(kr[u][i][0], qv[h][0], 0, false);
                    sc = __builtin_amdgcn_sdot4(kr[u][i][1], qv[h][1], sc, false);
                    sc = __builtin_amdgcn_sdot4(kr[u][i][2], qv[h][2], sc, false);
                    sc = __builtin_amdgcn_sdot4(kr[u][i][3], qv[h][3], sc, false);
                    sc += dpp_xor1(sc);
                    sc += dpp_xor2(sc);
                    if (CPR == 8) sc += dpp_half_mirror(sc);
                    if (key < P.Skv) {
                        tmax[h] = max(tmax[h], sc);
                        if (c == i) s_score[h * skv_pad + key] = sc;
                    }
                }
            }
    }
    // ---- B: row max ----------------------------------------------------------
#pragma unroll
    for (int h = 0; h < QH; ++h) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) tmax[h] = max(tmax[h], __shfl_xor(tmax[h], off));
        if (lane == 0) s_scal[h][wave] = tmax[h];
    }
    __syncthreads();
    int32_t m[QH], lo[QH], negM = -P.tab_mul;
    uint32_t Cm[QH];
#pragma unroll
    for (int h = 0; h < QH; ++h) {
        m[h] = s_scal[h][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) m[h] = max(m[h], s_scal[h][w]);
        lo[h] = m[h] - P.x_clip;
        Cm[h] = static_cast<uint32_t>(m[h]) * static_cast<uint32_t>(P.tab_mul) + P.tab_half;
    }

    // ---- C: slots and row sum, then probabilities ------------------------------
    uint32_t E[QH];
#pragma unroll
    for (int h = 0; h < QH; ++h) E[h] = 0;
    for (int j = tid; j < P.Skv; j += NT) {
#pragma unroll
        for (int h = 0; h < QH; ++h) {
            const uint32_t slot = slot_of(s_score[h * skv_pad + j], lo[h], Cm[h], negM, P.tab_shift);
            E[h] += s_lut[slot];
            s_score[h * skv_pad + j] = static_cast<int32_t>(slot);
        }
    }
#pragma unroll
    for (int h = 0; h < QH; ++h) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) E[h] += __shfl_xor(E[h], off);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < QH; ++h)
        if (lane == 0) s_scal[h][NW + wave] = static_cast<int32_t>(E[h]);
    __syncthreads();
    uint32_t R[QH];
#pragma unroll
    for (int h = 0; h < QH; ++h) {
        E[h] = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) E[h] += static_cast<uint32_t>(s_scal[h][NW + w]);
        R[h] = P16 ? reciprocal16(E[h]) : reciprocal8(E[h]);
        if (row_max != nullptr && tid == 0) {
            row_max[head0 + h] = m[h];
            row_sum[head0 + h] = E[h];
        }
    }
    // psum: sum of p (uint16 P: of the high bytes; psum_lo of the low bytes)
    uint32_t psum[QH], psum_lo = 0;
#pragma unroll
    for (int h = 0; h < QH; ++h) psum[h] = 0;
    for (int j = tid; j < skv_pad; j += NT) {
#pragma unroll
        for (int h = 0; h < QH; ++h) {
            uint32_t p = 0;
            if constexpr (P16) {
                if (j < P.Skv) p = (s_lut[s_score[j]] * R[0] + (1u << 15)) >> 16;
                reinterpret_cast<uint16_t*>(s_p)[j] = static_cast<uint16_t>(p);
                psum[0] += p >> 8;
                psum_lo += p & 0xffu;
            } else {
                if (j < P.Skv) p = (s_lut[s_score[h * skv_pad + j]] * R[h] + (1u << 22)) >> 23;
                s_p[h * skv_pad + j] = static_cast<uint8_t>(p);
                psum[h] += p;
            }
        }
    }
#pragma unroll
    for (int h = 0; h < QH; ++h) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) psum[h] += __shfl_xor(psum[h], off);
    }
    if constexpr (P16) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) psum_lo += __shfl_xor(psum_lo, off);
    }
    __syncthreads();
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < QH; ++h) s_scal[h][wave] = static_cast<int32_t>(psum[h]);
        s_scal[0][2 * NW + wave] = static_cast<int32_t>(psum_lo);
    }
    __syncthreads();
    psum_lo = 0;
#pragma unroll
    for (int h = 0; h < QH; ++h) {
        psum[h] = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) psum[h] += static_cast<uint32_t>(s_scal[h][w]);
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) psum_lo += static_cast<uint32_t>(s_scal[0][2 * NW + w]);

    // ---- D: P.V ----------------------------------------------------------------
    // uint16 P: acc takes the high probability bytes, acc_lo the low ones
    uint32_t acc[QH][16], acc_lo[P16 ? 16 : 1];
#pragma unroll
    for (int h = 0; h < QH; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] = 0;
#pragma unroll
    for (int i = 0; i < (P16 ? 16 : 1); ++i) acc_lo[i] = 0;
    for (int base = 0; base < P.Skv; base += kDecodeUnroll * KEYS_IT) {
        v4i vr[kDecodeUnroll][4];
        uint32_t pk[kDecodeUnroll][QH], pk_lo[kDecodeUnroll];
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            const int key0 = base + u * KEYS_IT + wave * 4 * GPW + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vr[u][i] = v4i{0, 0, 0, 0};
                if (key0 + i < P.Skv)
                    vr[u][i] = *reinterpret_cast<const v4i*>(vh + static_cast<size_t>(key0 + i) * D + 16 * c);
            }
            if constexpr (P16) {
                // four uint16 p: high bytes into pk, low bytes into pk_lo (key order kept)
                uint2 w = make_uint2(0u, 0u);
                if (key0 < skv_pad) w = *reinterpret_cast<const uint2*>(s_p + 2 * key0);
                pk[u][0] = __builtin_amdgcn_perm(w.y, w.x, 0x07050301u);
                pk_lo[u] = __builtin_amdgcn_perm(w.y, w.x, 0x06040200u);
            } else {
#pragma unroll
                for (int h = 0; h < QH; ++h)
                    pk[u][h] = key0 < skv_pad ? *reinterpret_cast<const uint32_t*>(s_p + h * skv_pad + key0) : 0u;
            }
        }
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u)
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
#pragma unroll
                for (int h = 0; h < QH; ++h) {
                    acc[h][4 * w + 0] = __builtin_amdgcn_udot4(c0, pk[u][h], acc[h][4 * w + 0], false);
                    acc[h][4 * w + 1] = __builtin_amdgcn_udot4(c1, pk[u][h], acc[h][4 * w + 1], false);
                    acc[h][4 * w + 2] = __builtin_amdgcn_udot4(c2, pk[u][h], acc[h][4 * w + 2], false);
                    acc[h][4 * w + 3] = __builtin_amdgcn_udot4(c3, pk[u][h], acc[h][4 * w + 3], false);
                }
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
    for (int h = 0; h < QH; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
            for (int off = CPR; off < 64; off <<= 1) acc[h][i] += __shfl_xor(acc[h][i], off);
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
        for (int h = 0; h < QH; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) s_red[h][wave][16 * c + i] = static_cast<int32_t>(acc[h][i]);
        if constexpr (P16) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s_red[P16 ? 1 : 0][wave][16 * c + i] = static_cast<int32_t>(acc_lo[i]);
        }
    }
    __syncthreads();
    for (int e = tid; e < QH * D; e += NT) {
        const int h = e / D, d = e % D;
        uint32_t tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += static_cast<uint32_t>(s_red[h][w][d]);
        // sum p v = sum p (v + 128) - 128 sum p; uint16 P: 256 (high bytes) + low bytes
        uint32_t a = tot - 128u * psum[QH == 1 ? 0 : (h & (QH - 1))];
        if constexpr (P16) {
            uint32_t lo16 = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) lo16 += static_cast<uint32_t>(s_red[P16 ? 1 : 0][w][d]);
            a = 256u * a + (lo16 - 128u * psum_lo);
        }
        out[(head0 + h) * D + d] = requantise(static_cast<int32_t>(a), P);
    }
}

// Decode past kDecodeMaxKeys keys without a workspace: one workgroup per
// head as above, but the scores are not kept. Three passes stream K from HBM
// (1: row max; 2: slots, table entries, row sum; 3: per chunk of
// kDecodeChunk keys, the probabilities into LDS, then P.V over the chunk's
// values), so the traffic is K three times and V once, and the LDS holds one
// chunk of P. Exact: the row max and the row sum are complete before any
// probability is formed, and every partial is an integer.
// Each head's workgroup has 16 waves: with one workgroup per head (64
// heads fill a quarter of the compute units), more loads in flight per
// compute unit raise the rate each one streams K and V at.
constexpr int kDecodeChunk = 8192;
constexpr int kDecodeLongWaves = 16;

template <int D, bool P16>
__global__ __launch_bounds__(64 * kDecodeLongWaves) void ia_decode_long_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int32_t* __restrict__ row_max,
    uint32_t* __restrict__ row_sum) {
    constexpr int NT = 64 * kDecodeLongWaves;
    constexpr int NW = NT / 64;
    constexpr int CPR = D / 16;                 // lanes per key row
    constexpr int GPW = 64 / CPR;               // key groups (of 4 keys) per wave
    constexpr int KEYS_IT = 4 * GPW * NW;       // keys per iteration
    constexpr int STEP = kDecodeUnroll * KEYS_IT;
    static_assert(kDecodeChunk % STEP == 0, "chunks hold whole iterations");
    extern __shared__ __attribute__((aligned(16))) uint8_t s_p[];   // one chunk of P (uint16 P: 2 bytes a key)
    __shared__ uint16_t s_lut[kIaTabEntries];
    __shared__ int32_t s_red[P16 ? 2 : 1][NW][D];
    __shared__ int32_t s_scal[3 * NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane % CPR;                   // 16-byte column chunk
    const int g = lane / CPR;                   // key group within the wave
    const int bid = P.kv_group > 1 ? xcd_local_block(blockIdx.x, gridDim.x) : static_cast<int>(blockIdx.x);
    const size_t head = static_cast<size_t>(bid);
    const size_t kvhead = divmod_invariant(static_cast<uint32_t>(head), P.kvg_div).q;
    const int8_t* kh = k + kvhead * P.kv_rows * D;
    const int8_t* vh = v + kvhead * P.kv_rows * D;
    const v4i qv = *reinterpret_cast<const v4i*>(q + head * D + 16 * c);
    if (wave == 0) fill_lut_u16(P, s_lut, lane);

    // f(key, score) for every key in [b0, b1) (b1 - b0 a multiple of STEP),
    // on the one lane of the key's row group whose column chunk c equals
    // the key's index i within its group of 4; keys past Skv score 0
    auto for_scores = [&](int b0, int b1, auto&& f) {
        for (int base = b0; base < b1; base += STEP) {
            v4i kr[kDecodeUnroll][4];
#pragma unroll
            for (int u = 0; u < kDecodeUnroll; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = base + u * KEYS_IT + wave * 4 * GPW + 4 * g + i;
                    kr[u][i] = v4i{0, 0, 0, 0};
                    if (key < P.Skv) kr[u][i] = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(key) * D + 16 * c);
                }
#pragma unroll
            for (int u = 0; u < kDecodeUnroll; ++u)
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
                    if (c == i) f(key, sc);
                }
        }
    };
    const int kend = (P.Skv + STEP - 1) / STEP * STEP;

    // ---- pass 1: row max -----------------------------------------------------
    int32_t tmax = INT_MIN;
    for_scores(0, kend, [&](int key, int32_t sc) {
        if (key < P.Skv) tmax = max(tmax, sc);
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tmax = max(tmax, __shfl_xor(tmax, off));
    if (lane == 0) s_scal[wave] = tmax;
    __syncthreads();
    int32_t m = s_scal[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = max(m, s_scal[w]);
    const int32_t lo = m - P.x_clip, negM = -P.tab_mul;
    const uint32_t Cm = static_cast<uint32_t>(m) * static_cast<uint32_t>(P.tab_mul) + P.tab_half;

    // ---- pass 2: slots and row sum ---------------------------------------------
    uint32_t E = 0;
    for_scores(0, kend, [&](int key, int32_t sc) {
        if (key < P.Skv) E += s_lut[slot_of(sc, lo, Cm, negM, P.tab_shift)];
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) E += __shfl_xor(E, off);
    if (lane == 0) s_scal[NW + wave] = static_cast<int32_t>(E);
    __syncthreads();
    E = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) E += static_cast<uint32_t>(s_scal[NW + w]);
    const uint32_t R = P16 ? reciprocal16(E) : reciprocal8(E);
    if (row_max != nullptr && tid == 0) {
        row_max[head] = m;
        row_sum[head] = E;
    }

    // ---- pass 3: per chunk, P into LDS, then P.V ----------------------------------
    uint32_t psum = 0, psum_lo = 0;
    uint32_t acc[16], acc_lo[P16 ? 16 : 1];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0;
#pragma unroll
    for (int i = 0; i < (P16 ? 16 : 1); ++i) acc_lo[i] = 0;
    for (int c0 = 0; c0 < kend; c0 += kDecodeChunk) {
        const int c1 = min(kend, c0 + kDecodeChunk);
        for_scores(c0, c1, [&](int key, int32_t sc) {
            uint32_t p = 0;
            if (key < P.Skv) {
                const uint32_t e = s_lut[slot_of(sc, lo, Cm, negM, P.tab_shift)];
                p = P16 ? (e * R + (1u << 15)) >> 16 : (e * R + (1u << 22)) >> 23;
            }
            if constexpr (P16) {
                reinterpret_cast<uint16_t*>(s_p)[key - c0] = static_cast<uint16_t>(p);
                psum += p >> 8;
                psum_lo += p & 0xffu;
            } else {
                s_p[key - c0] = static_cast<uint8_t>(p);
                psum += p;
            }
        });
        __syncthreads();
        for (int base = c0; base < c1; base += STEP) {
            v4i vr[kDecodeUnroll][4];
            uint32_t pk[kDecodeUnroll], pk_lo[kDecodeUnroll];
#pragma unroll
            for (int u = 0; u < kDecodeUnroll; ++u) {
                const int key0 = base + u * KEYS_IT + wave * 4 * GPW + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vr[u][i] = v4i{0, 0, 0, 0};
                    if (key0 + i < P.Skv)
                        vr[u][i] = *reinterpret_cast<const v4i*>(vh + static_cast<size_t>(key0 + i) * D + 16 * c);
                }
                if constexpr (P16) {
                    const uint2 w = *reinterpret_cast<const uint2*>(s_p + 2 * (key0 - c0));
                    pk[u] = __builtin_amdgcn_perm(w.y, w.x, 0x07050301u);
                    pk_lo[u] = __builtin_amdgcn_perm(w.y, w.x, 0x06040200u);
                } else {
                    pk[u] = *reinterpret_cast<const uint32_t*>(s_p + (key0 - c0));
                    pk_lo[u] = 0;
                }
            }
#pragma unroll
            for (int u = 0; u < kDecodeUnroll; ++u)
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
                    const uint32_t w0 = __builtin_amdgcn_perm(u2, u0, 0x05040100u);
                    const uint32_t w1 = __builtin_amdgcn_perm(u2, u0, 0x07060302u);
                    const uint32_t w2 = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
                    const uint32_t w3 = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
                    acc[4 * w + 0] = __builtin_amdgcn_udot4(w0, pk[u], acc[4 * w + 0], false);
                    acc[4 * w + 1] = __builtin_amdgcn_udot4(w1, pk[u], acc[4 * w + 1], false);
                    acc[4 * w + 2] = __builtin_amdgcn_udot4(w2, pk[u], acc[4 * w + 2], false);
                    acc[4 * w + 3] = __builtin_amdgcn_udot4(w3, pk[u], acc[4 * w + 3], false);
                    if constexpr (P16) {
                        acc_lo[4 * w + 0] = __builtin_amdgcn_udot4(w0, pk_lo[u], acc_lo[4 * w + 0], false);
                        acc_lo[4 * w + 1] = __builtin_amdgcn_udot4(w1, pk_lo[u], acc_lo[4 * w + 1], false);
                        acc_lo[4 * w + 2] = __builtin_amdgcn_udot4(w2, pk_lo[u], acc_lo[4 * w + 2], false);
                        acc_lo[4 * w + 3] = __builtin_amdgcn_udot4(w3, pk_lo[u], acc_lo[4 * w + 3], false);
                    }
                }
        }
        __syncthreads();                     // before the next chunk's P overwrites this one
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        psum += __shfl_xor(psum, off);
        if constexpr (P16) psum_lo += __shfl_xor(psum_lo, off);
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
    if (lane == 0) {
        s_scal[wave] = static_cast<int32_t>(psum);
        s_scal[2 * NW + wave] = static_cast<int32_t>(psum_lo);
    }
    __syncthreads();
    psum = 0;
    psum_lo = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        psum += static_cast<uint32_t>(s_scal[w]);
        psum_lo += static_cast<uint32_t>(s_scal[2 * NW + w]);
    }
    for (int d = tid; d < D; d += NT) {
        uint32_t tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += static_cast<uint32_t>(s_red[0][w][d]);
        // sum p v = sum p (v + 128) - 128 sum p; uint16 P: 256 (high bytes) + low bytes
        uint32_t a = tot - 128u * psum;
        if constexpr (P16) {
            uint32_t lo16 = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) lo16 += static_cast<uint32_t>(s_red[P16 ? 1 : 0][w][d]);
            a = 256u * a + (lo16 - 128u * psum_lo);
        }
        out[head * D + d] = requantise(static_cast<int32_t>(a), P);
    }
}

template <int D, bool P16>
int launch_decode_long_t(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, const IaKernelParams& kp,
                         hipStream_t stream, unsigned blocks, int32_t* row_max, uint32_t* row_sum) {
    const size_t shm = static_cast<size_t>(kDecodeChunk) * (P16 ? 2 : 1);
    hipLaunchKernelGGL((ia_decode_long_kernel<D, P16>), dim3(blocks), dim3(64 * kDecodeLongWaves), shm, stream, q,
                       k, v, out, kp, row_max, row_sum);
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

}  // namespace

int decode_max_keys() { return kDecodeMaxKeys; }

template <int D, bool P16, int QH, int NWQ = kDecodeThreads / 64>
int launch_decode_t(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, const IaKernelParams& kp,
                    hipStream_t stream, unsigned blocks, int skv_pad, int32_t* row_max, uint32_t* row_sum) {
    constexpr int kBytesPerKey = P16 ? 6 : 5 * QH;     // int32 score/slot + uint8 or uint16 p, per query head
    constexpr int kMaxKeys = QH == 1 ? kDecodeMaxKeys : kDecodeMaxKeys / 2;
    static std::atomic<uint64_t> lds_set{0};
    const int st = ensure_dynamic_lds(reinterpret_cast<const void*>(&ia_decode_kernel<D, P16, QH, NWQ>),
                                      kBytesPerKey * kMaxKeys, lds_set);
    if (st != INTATTN_OK) return st;
    const size_t shm = static_cast<size_t>(skv_pad) * kBytesPerKey;
    hipLaunchKernelGGL((ia_decode_kernel<D, P16, QH, NWQ>), dim3(blocks), dim3(64 * NWQ * QH), shm, stream, q, k, v, out,
                       kp, skv_pad, row_max, row_sum);
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

int launch_decode(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                  const IaKernelParams& kp, void* stream_v, int32_t* row_max, uint32_t* row_sum) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_v);
    const long long heads = static_cast<long long>(kp.B) * kp.H;
    if (heads > INT_MAX) return INTATTN_E_SHAPE;
    const unsigned nb = static_cast<unsigned>(heads);
    if (kp.Skv > kDecodeMaxKeys) {
        if (kp.prob_bits == 16)
            return D == 64 ? launch_decode_long_t<64, true>(q, k, v, out, kp, stream, nb, row_max, row_sum)
                           : launch_decode_long_t<128, true>(q, k, v, out, kp, stream, nb, row_max, row_sum);
        return D == 64 ? launch_decode_long_t<64, false>(q, k, v, out, kp, stream, nb, row_max, row_sum)
                       : launch_decode_long_t<128, false>(q, k, v, out, kp, stream, nb, row_max, row_sum);
    }
    const int skv_pad = (kp.Skv + 255) / 256 * 256;
    // fewer heads than compute units: 16 waves a head (more loads in flight
    // per compute unit), as for the three-pass form
    if (heads < 256) {
        if (kp.prob_bits == 16)
            return D == 64 ? launch_decode_t<64, true, 1, 16>(q, k, v, out, kp, stream, nb, skv_pad, row_max, row_sum)
                           : launch_decode_t<128, true, 1, 16>(q, k, v, out, kp, stream, nb, skv_pad, row_max, row_sum);
        return D == 64 ? launch_decode_t<64, false, 1, 16>(q, k, v, out, kp, stream, nb, skv_pad, row_max, row_sum)
                       : launch_decode_t<128, false, 1, 16>(q, k, v, out, kp, stream, nb, skv_pad, row_max, row_sum);
    }
    if (kp.prob_bits == 16)
        return D == 64 ? launch_decode_t<64, true, 1>(q, k, v, out, kp, stream, nb, skv_pad, row_max, row_sum)
                       : launch_decode_t<128, true, 1>(q, k, v, out, kp, stream, nb, skv_pad, row_max, row_sum);
    // two query heads of one K/V head a workgroup when heads share K/V in
    // pairs, the rows fit its LDS (10 bytes a key) and the halved grid still
    // gives every compute unit a workgroup
    if (kp.kv_group % 2 == 0 && skv_pad <= kDecodeMaxKeys / 2 && heads / 2 >= 256) {
        const unsigned nb2 = static_cast<unsigned>(heads / 2);
        return D == 64 ? launch_decode_t<64, false, 2>(q, k, v, out, kp, stream, nb2, skv_pad, row_max, row_sum)
                       : launch_decode_t<128, false, 2>(q, k, v, out, kp, stream, nb2, skv_pad, row_max, row_sum);
    }
    return D == 64 ? launch_decode_t<64, false, 1>(q, k, v, out, kp, stream, nb, skv_pad, row_max, row_sum)
                   : launch_decode_t<128, false, 1>(q, k, v, out, kp, stream, nb, skv_pad, row_max, row_sum);
}

}  // namespace ia
