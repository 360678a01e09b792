// Device-side building blocks shared by the integer attention kernels
// (gfx950 / CDNA4): MFMA wrapper, accumulator layout helpers, workgroup
// renumbering and the requantisation step.
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology",
// steps 2-3; integer widths and roundings as stated in include/intattn.h.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include "intattn_internal.h"

namespace ia {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// S^T tiles: v_mfma_i32_32x32x32_i8 with K as the A operand (rows = keys)
// and Q^T as the B operand (columns = queries). Lane l (l32 = l % 32,
// hh = l / 32) holds the 16 accumulator registers of column l32, i.e. scores
// of a single query row for 16 keys of the 32-key block.
__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Key (relative to its 32-key block) held by accumulator register r of a
// 32x32 MFMA result in lane half hh (lanes 0-31: hh = 0, lanes 32-63: 1).
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

// Byte position of a key of a 32-key block inside a transposed V row, such
// that lane half hh reads its 16 keys (acc_row(0..15, hh)) contiguously; the
// 16 bytes are then the B operand of P.V in the order of the P operand.
__device__ __forceinline__ int vt_pos(int key_in_block) {
    const int a = key_in_block >> 3, h = (key_in_block >> 2) & 1, c = key_in_block & 3;
    return 16 * h + 4 * a + c;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Renumber them so that consecutive logical blocks run on the same XCD.
// Bijective on [0, n): the first 8*floor(n/8) ids are regrouped, the
// remainder is kept.
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

// Saturating slot word: with y = s - m <= 0 and negM4 = -4M (|4M| < 2^23),
// t = sat_int32(y * negM4 + 2^25) has the slot min(31, (x*M + 2^23) >> 24)
// in bits 26..30 (byte 3 = 4 * slot + two fraction bits): scaling numerator
// and shift by 4 keeps the quotient, the value is below 2^31 whenever the
// slot is below 31, and saturation to 2^31 - 1 lands exactly in slot 31.
__device__ __forceinline__ uint32_t slot_word_sat(int32_t y, int32_t negM4, int32_t half4) {
    int32_t t;
    asm("v_mad_i32_i24 %0, %1, %2, %3 clamp" : "=v"(t) : "v"(y), "v"(negM4), "v"(half4));
    return static_cast<uint32_t>(t);
}

// int32 accumulator -> int8: sign(a) * min(127, (|a|*M_o + 2^(sh_o-1)) >> sh_o).
__device__ __forceinline__ int8_t requantise(int32_t a, const IaKernelParams& P) {
    const uint32_t mag = static_cast<uint32_t>(a < 0 ? -a : a);
    const uint64_t prod = static_cast<uint64_t>(mag) * P.req_mul + (uint64_t(1) << (P.req_shift - 1));
    uint64_t qv = prod >> P.req_shift;
    if (qv > 127) qv = 127;
    return static_cast<int8_t>(a < 0 ? -static_cast<int32_t>(qv) : static_cast<int32_t>(qv));
}

// Entry k of the exp table from the packed kernel argument.
__device__ __forceinline__ uint32_t lut_entry(const IaKernelParams& P, int k) {
    return (P.lut2[k >> 1] >> (16 * (k & 1))) & 0xffffu;
}

__device__ __forceinline__ int32_t dpp_xor1(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true); }
__device__ __forceinline__ int32_t dpp_xor2(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true); }
__device__ __forceinline__ int32_t dpp_half_mirror(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true); }

}  // namespace ia
