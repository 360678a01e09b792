// Decode-step K/V cache update (gfx950): the keys and values of T new tokens
// per (batch, K/V head), float32, are coded to int8 under the cache's
// per-tensor scale and written to cache rows pos .. pos+T-1.
//
// The pages do not describe this step; it precedes the attention call of a
// decoder's decode step, whose data flow stays INT8 (IntAttention digest
// pages, "Methodology", step 3). The code of a value x under scale s is the
// inputs' rule: clip(rint(x / s), -127, 127) with x / s the IEEE float32
// quotient (round to nearest, ties to even), rint ties to even, NaN -> 0.
//
// HBM bound: 4 bytes read and 1 byte written per value. Each thread codes 16
// consecutive values of one token row (four 16-byte loads, one 16-byte
// store); consecutive threads cover consecutive 16-value chunks, so a wave
// reads 4 KB and writes 1 KB contiguously within a head's rows.
#include "ia_device.h"

namespace ia {
namespace {

constexpr int kAppendThreads = 256;

__device__ __forceinline__ uint32_t code4(float4 x, float s) {
    auto one = [&](float v) -> uint32_t {
        float y = rintf(__fdiv_rn(v, s));
        y = y != y ? 0.0f : fminf(fmaxf(y, -127.0f), 127.0f);
        return static_cast<uint32_t>(static_cast<int32_t>(y)) & 0xffu;
    };
    return one(x.x) | (one(x.y) << 8) | (one(x.z) << 16) | (one(x.w) << 24);
}

// chunks: B * Hkv * T * (D / 16) per tensor; thread c < chunks codes K, the
// next `chunks` threads code V.
__global__ __launch_bounds__(kAppendThreads) void ia_kv_append_kernel(
    const float* __restrict__ k_new, const float* __restrict__ v_new, int8_t* __restrict__ k_cache,
    int8_t* __restrict__ v_cache, long long chunks, int T, int D, int capacity, int pos, float s_k, float s_v) {
    const int cpr = D / 16;                                  // chunks per token row
    for (long long c = static_cast<long long>(blockIdx.x) * kAppendThreads + threadIdx.x; c < 2 * chunks;
         c += static_cast<long long>(gridDim.x) * kAppendThreads) {
        const bool is_v = c >= chunks;
        const long long cc = is_v ? c - chunks : c;
        const long long row = cc / cpr;                      // (b, h, t) row of the new tokens
        const int part = static_cast<int>(cc - row * cpr);
        const long long bh = row / T;
        const int t = static_cast<int>(row - bh * T);
        const float* src = (is_v ? v_new : k_new) + row * D + 16 * part;
        int8_t* dst = (is_v ? v_cache : k_cache) + (bh * capacity + pos + t) * D + 16 * part;
        const float s = is_v ? s_v : s_k;
        const float4* s4 = reinterpret_cast<const float4*>(src);
        const float4 a = s4[0], b = s4[1], cq = s4[2], d = s4[3];
        uint4 o;
        o.x = code4(a, s);
        o.y = code4(b, s);
        o.z = code4(cq, s);
        o.w = code4(d, s);
        *reinterpret_cast<uint4*>(dst) = o;
    }
}

}  // namespace

int launch_kv_append(const float* k_new, const float* v_new, int8_t* k_cache, int8_t* v_cache, int B, int Hkv,
                     int T, int D, int capacity, int pos, float s_k, float s_v, void* stream) {
    const long long chunks = static_cast<long long>(B) * Hkv * T * (D / 16);
    const long long want = (2 * chunks + kAppendThreads - 1) / kAppendThreads;
    const unsigned blocks = static_cast<unsigned>(want < 8192 ? want : 8192);   // grid-stride beyond
    hipLaunchKernelGGL(ia_kv_append_kernel, dim3(blocks), dim3(kAppendThreads), 0,
                       static_cast<hipStream_t>(stream), k_new, v_new, k_cache, v_cache, chunks, T, D, capacity,
                       pos, s_k, s_v);
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

}  // namespace ia
