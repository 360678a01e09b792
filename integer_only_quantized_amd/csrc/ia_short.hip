// Short-row kernel instances with uint8 probabilities, and the short-row
// entry (uint16 probabilities are instantiated in ia_short16.hip). The
// kernel itself is in ia_short_impl.h.
#include "ia_short_impl.h"

namespace ia {

int short_max_keys(int D) { return 64 * short_max_half_blocks(D); }

int launch_short(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                 const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum) {
    if (kp.prob_bits == 16) return launch_short16(q, k, v, out, D, kp, stream, row_max, row_sum);
    const int nbh = (kp.Skv + 63) / 64;              // 32-key blocks per half
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (D == 64) return launch_short_n<64, 1, false>(nbh, q, k, v, out, kp, s, row_max, row_sum);
    return launch_short_n<128, 1, false>(nbh, q, k, v, out, kp, s, row_max, row_sum);
}

}  // namespace ia
