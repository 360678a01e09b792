// Declarations shared by the host code and the HIP launchers of the integer
// attention library (not part of the public C ABI). Host-only types: the
// HIP stream travels as void* so this header needs no HIP headers.
#pragma once

#include <cstdint>

#include "ia_intdiv.h"
#include "intattn.h"

// Shape checks common to every entry point (no device access).
int intattn_validate_shape(const intattn_shape* s, int causal);

// Every argument check of intattn_forward_ex, without queueing anything (no
// HIP call): the status intattn_forward_ex would return before any launch.
int intattn_validate_forward_ex(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                                const intattn_shape* shape, const intattn_scales* scales, float clip, int causal,
                                const intattn_variant* variant, int32_t* row_max, uint32_t* row_sum);

// Largest exp table of the variants (32 is the pages' table).
constexpr int kIaMaxLut = 128;
// Entries of the table the kernels receive: the exp table by slot (N <= 128
// entries), or, from mu = 1/2 on, the direct table by clipped score gap
// (X_clip + 1 <= 2N - 2 entries); the rest 0.
constexpr int kIaTabEntries = 256;

// Everything a kernel needs besides the tensor pointers, passed by value so
// that it lands in kernel-argument (scalar) registers.
struct IaKernelParams {
    int32_t B, H, Sq, Skv;
    int32_t causal;
    int32_t idx_mul;     // M, <= 2^23
    int32_t idx_shift;   // sh: slot = (x*M + 2^(sh-1)) >> sh, 24 below mu = 1/2, 9..23 above
    int32_t x_clip;      // smallest relative score that lands in the last slot
    // Table index of a gap x' = min(m - s, x_clip) as the row-constant kernels
    // (decode, general) compute it: (x' * tab_mul + tab_half) >> tab_shift,
    // i.e. the slot (M, 2^23, 24), or x' itself for the direct table (1, 0, 0).
    int32_t tab_mul;
    uint32_t tab_half;
    int32_t tab_shift;
    // Operands of the table address for the layout slot_k (entry_addr):
    // slot_k > 0: -k*M and k*2^23 (saturating slot word); 0: -x_clip and 0.
    int32_t ent_a;
    int32_t ent_b;
    int32_t req_shift;   // sh_o, 1..63
    uint32_t req_mul;    // M_o, in [2^30, 2^31)
    int32_t lut_size;    // N: 32, 64 or 128 entries; entry N-1 is 0
    int32_t slot_k;      // slot-word scale k and table layout: 4 (N = 32, 4M < 2^23),
                         // 2 (N <= 64, 2M < 2^23), 1 (below mu = 1/2), or 0: the
                         // direct table by clipped score gap (from mu = 1/2 on)
    int32_t slot_k_log2; // log2(k) (0 for the direct table)
    int32_t kv_group;    // query heads per K/V head (1: one K/V head each)
    int32_t kv_rows;     // rows per K/V head in memory (>= Skv: a cache of that capacity)
    int32_t prob_bits;   // 8: uint8 probabilities; 16: the uint16 variant
    ia::InvariantDiv kvg_div;   // division by kv_group (query head -> K/V head)
    ia::InvariantDiv h_div;     // division by H (batch, head of a flat head index)
    ia::InvariantDiv qb_div;    // division by the launch's query-block count (set by the launcher)
    uint32_t lut2[kIaTabEntries / 2];   // table entries 2i and 2i+1 packed lo/hi (slot_k > 0:
                                        // the exp table by slot; 0: by score gap 0..x_clip)
};

// Host derivation of every integer the kernels receive, for a table of
// lut_size entries (32, 64 or 128) of lut_bits bits (16 or 8): the exp
// table in Q15 units (8-bit entries times 128), M and its shift, the clip
// point and the requantisation pair. Errors as intattn_derive_params (E_RANGE also for an
// unsupported lut_size, prob_bits or lut_bits).
int intattn_derive_core(const intattn_shape* shape, const intattn_scales* sc, float clip, int lut_size,
                        uint16_t* lut, int32_t* idx_mul, int32_t* idx_shift, int32_t* x_clip, int32_t* req_shift,
                        int64_t* req_mul, int prob_bits = 8, int lut_bits = 16);

namespace ia {

// Clears an error left pending in this thread by earlier, unrelated HIP
// calls, so that the status read after a launch is that launch's own.
void clear_pending_hip_error();

// Each launcher queues one kernel on `stream` (a hipStream_t) and returns
// INTATTN_OK or INTATTN_E_HIP / INTATTN_E_SHAPE. row_max / row_sum are
// optional per-row outputs [B, H, Sq] (both NULL or both set).

// Any shape; also writes the probabilities [B, H, Sq, Skv] when probs != NULL.
int launch_general(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                   const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum,
                   uint8_t* probs);

// Skv <= short_max_keys(D): K and V of a head resident in LDS.
int short_max_keys(int D);
int launch_short(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                 const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum);
// The uint16-probability instances of the short-row kernel (launch_short
// calls it for kp.prob_bits == 16).
int launch_short16(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                   const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum);

// Sq == 1: one head per workgroup, HBM streaming; past decode_max_keys() keys
// the scores are not kept and K is streamed three times.
int decode_max_keys();

// Decode over long caches, keys split into chunks over several workgroups
// per head (Sq = 1): workspace bytes for B*H heads, and the launch (four
// kernels; the workspace is caller-owned device memory of at least that size).
size_t decode_split_workspace_bytes(long long heads, int Skv, int D);
int launch_decode_split(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D, const IaKernelParams& kp,
                        void* stream, void* workspace, int32_t* row_max, uint32_t* row_sum);
int launch_decode(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                  const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum);

// Any shape (used for long rows): K/V tiles streamed through LDS, three passes.
int launch_long(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum);

// Decode-step cache update: quantise T new tokens (float32) per (b, K/V head)
// into rows pos .. pos+T-1 of the int8 caches [B, Hkv, capacity, D].
int launch_kv_append(const float* k_new, const float* v_new, int8_t* k_cache, int8_t* v_cache, int B, int Hkv,
                     int T, int D, int capacity, int pos, float s_k, float s_v, void* stream);

// Unfused pipeline stages (scores and probabilities in HBM). The softmax
// stages hold a row in registers: Skv <= stage_max_keys().
int stage_max_keys();
int launch_qk_scores(const int8_t* q, const int8_t* k, int32_t* scores, int D, const IaKernelParams& kp,
                     void* stream);
int launch_index_softmax(const int32_t* scores, uint8_t* probs, int32_t* row_max, uint32_t* row_sum,
                         const IaKernelParams& kp, void* stream);
int launch_fp_softmax(const int32_t* scores, uint8_t* probs, float alpha, const IaKernelParams& kp, void* stream);
int launch_pv(const uint8_t* probs, const int8_t* v, int8_t* out, int D, const IaKernelParams& kp, void* stream);

}  // namespace ia
