// Declarations shared by the host derivation and the HIP launchers of the
// integer attention library (not part of the public C ABI).
#pragma once

#include <cstdint>

#include "intattn.h"

// Shape checks common to every entry point (no device access).
int intattn_validate_shape(const intattn_shape* s, int causal);

// Everything a kernel needs besides the tensor pointers, passed by value so
// that it lands in kernel-argument (scalar) registers.
struct IaKernelParams {
    int32_t B, H, Sq, Skv;
    int32_t causal;
    int32_t idx_mul;     // M, < 2^23
    int32_t x_clip;      // smallest relative score that lands in slot 31
    int32_t req_shift;   // sh_o, 1..63
    uint32_t req_mul;    // M_o, in [2^30, 2^31)
    uint32_t lut2[16];   // exp table, entries 2i and 2i+1 packed lo/hi
};
