// Short-row kernel instances with uint16 probabilities (the variant the
// pages' "Limitations & Future Work" motivate: long flat rows underflow in
// uint8). The kernel itself is in ia_short_impl.h.
#include "ia_short_impl.h"

namespace ia {

int launch_short16(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                   const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum) {
    const int nbh = (kp.Skv + 63) / 64;              // 32-key blocks per half
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (D == 64) return launch_short_n<64, 1, true>(nbh, q, k, v, out, kp, s, row_max, row_sum);
    return launch_short_n<128, 1, true>(nbh, q, k, v, out, kp, s, row_max, row_sum);
}

}  // namespace ia
