// Roofline calibration kernels for gfx950 (built into libintattn_probe.so,
// not part of the attention library): a pure int8 MFMA loop and a pure
// 32-bit integer VALU loop, used to confirm the MFMA and VALU peaks on the
// machine the attention kernels are measured on.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Four independent accumulator chains of v_mfma_i32_32x32x32_i8 per wave
// (65536 int8 ops per instruction), so issue never waits on a previous
// result; the sums are folded into one word per lane at the end.
__global__ __launch_bounds__(256) void probe_mfma_i8(int iters, int32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    v4i a = v4i{lane, lane + 1, lane + 2, lane + 3};
    v4i b = v4i{lane ^ 5, lane ^ 6, lane ^ 7, lane ^ 9};
    v16i c0 = v16i{}, c1 = v16i{}, c2 = v16i{}, c3 = v16i{};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int32_t s = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Eight independent chains of v_mad_u32_u24 per lane (one 32-bit integer
// multiply-add per lane per instruction).
__global__ __launch_bounds__(256) void probe_valu(int iters, int32_t* __restrict__ sink) {
    uint32_t x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = threadIdx.x * 8 + j;
    const uint32_t m = 0x1234u + blockIdx.x;
#pragma unroll 4
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __umul24(x[j], m) + static_cast<uint32_t>(j);
    }
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s ^= x[j];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = static_cast<int32_t>(s);
}

}  // namespace

extern "C" {

// blocks workgroups of 256 threads, iters loop trips each; sink holds
// blocks*256 int32 (device memory, caller-owned). Returns 0, or -1 when the
// launch fails. Work: probe_mfma: 4 * iters * 65536 ops per wave;
// probe_valu: 8 * iters multiply-adds per lane.
int intattn_probe_mfma_i8(int blocks, int iters, int32_t* sink, void* stream) {
    (void)hipGetLastError();   // report this launch's status only
    hipLaunchKernelGGL(probe_mfma_i8, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int intattn_probe_valu(int blocks, int iters, int32_t* sink, void* stream) {
    (void)hipGetLastError();   // report this launch's status only
    hipLaunchKernelGGL(probe_valu, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
