// Host-side launch helpers shared by the kernel launchers of the integer
// attention library.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "intattn.h"

namespace ia {

// Host: raises a kernel's dynamic LDS limit to `bytes` on the current device,
// once per device (devices 0..63; `done` is one bit per device, owned by the
// caller per kernel instance). Safe to call from several threads: a race
// only sets the same value twice.
inline int ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return INTATTN_E_HIP;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t(1) << dev) : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return INTATTN_OK;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
        return INTATTN_E_HIP;
    done.fetch_or(bit, std::memory_order_release);
    return INTATTN_OK;
}

}  // namespace ia
