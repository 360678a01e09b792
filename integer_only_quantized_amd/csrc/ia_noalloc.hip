// intattn_forward_ex_noalloc: intattn_forward_ex for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation). The one path of intattn_forward_ex that
// uses device memory beyond its inputs and outputs, decode with keys split
// over several workgroups per head, takes it here from `scratch`, a
// file-scope device array of kIaNoAllocScratchBytes that every GPU the
// library runs on holds until the process ends, instead of from a caller
// workspace. Nothing is allocated: no hipMalloc, no allocating library call.
//
// The split kernels clear what must start at zero (the first chunk of each
// head clears its int32 accumulators before any chunk adds to them), and
// overwrite every score, chunk maximum and chunk sum they read, so the
// array's contents from an earlier call never matter. Calls that overlap on
// one GPU (different streams or threads) share its array and race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "intattn.h"
#include "intattn_internal.h"

namespace {

constexpr uint64_t kScratchBytes = INTATTN_NOALLOC_SCRATCH_BYTES;

// The device-side array. In host code this name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, per device.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (on the first call that needs it, with that device current).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return INTATTN_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return INTATTN_E_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return INTATTN_OK;
}

}  // namespace

extern "C" int intattn_forward_ex_noalloc(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                                          const intattn_shape* shape, const intattn_scales* scales, float clip,
                                          int causal, const intattn_variant* variant, void* stream,
                                          int32_t* row_max, uint32_t* row_sum) {
    if (variant != nullptr && (variant->workspace != nullptr || variant->workspace_bytes != 0))
        return INTATTN_E_WORKSPACE;   // the scratch is the library's own
    intattn_variant var{};
    if (variant != nullptr) var = *variant;
    // every argument check of intattn_forward_ex first (no HIP call), with a
    // stand-in workspace of the scratch's size that is never dereferenced
    const uint64_t need = intattn_workspace_bytes(shape, &var);
    if (need > kScratchBytes) return INTATTN_E_SCRATCH;
    const int st = intattn_validate_forward_ex(q, k, v, out, shape, scales, clip, causal, &var, row_max, row_sum);
    if (st != INTATTN_OK) return st;
    if (need > 0) {
        void* p = nullptr;
        const int sst = scratch_address(&p);
        if (sst != INTATTN_OK) return sst;
        var.workspace = p;
        var.workspace_bytes = kScratchBytes;
    }
    return intattn_forward_ex(q, k, v, out, shape, scales, clip, causal, &var, stream, row_max, row_sum);
}
