// C-ABI entry points of the integer attention library: argument checks,
// host parameter derivation and the choice of device kernel.
//
// Kernel choice (all bit-identical to the specification in include/intattn.h,
// for every table size and K/V head grouping):
//   Sq == 1                                  -> decode kernel (HBM streaming;
//                                               past 16384 keys its three-pass
//                                               form), or with a workspace
//                                               the split-decode kernels for
//                                               the shapes uses_split names
//   Skv <= 512 (d = 64) or 256 (d = 128)      -> short-row kernel (K/V in LDS)
//   otherwise                                -> long-row kernel (tiled, 3 passes)
// (table sizes, entry widths, K/V head groupings and probability widths all
// run on the same kernels: the table reaches them in Q15 units)
// intattn_forward_debug with a probability buffer runs the general kernel,
// which is the only one that materialises P.
//
// The unfused stages (intattn_qk_scores, intattn_index_softmax,
// intattn_fp_softmax, intattn_pv) keep scores and probabilities in
// caller-owned device buffers; chained, the integer ones give exactly the
// result of intattn_forward.
#include <climits>
#include <cmath>
#include <cstdint>

#include "intattn.h"
#include "intattn_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape, head size and parameter derivation shared by every entry point.
// lut_size: 32, 64 or 128; kv_heads: K/V heads (0: H), dividing H;
// kv_capacity: rows per K/V head in memory (0: Skv), at least Skv;
// prob_bits: 8 or 16; lut_bits: table entry width, 16 or 8.
int derive_kernel_params(const intattn_shape* shape, const intattn_scales* scales, float clip, int causal,
                         IaKernelParams* kp, int lut_size = 32, int kv_heads = 0, int kv_capacity = 0,
                         int prob_bits = 8, int lut_bits = 16) {
    int st = intattn_validate_shape(shape, causal);
    if (st != INTATTN_OK) return st;
    if (shape->D != 64 && shape->D != 128) return INTATTN_E_DIM;
    if (kv_heads < 0) return INTATTN_E_SHAPE;
    const int hkv = kv_heads == 0 ? shape->H : kv_heads;
    if (shape->H > 0 && (hkv < 1 || shape->H % hkv != 0)) return INTATTN_E_SHAPE;
    if (kv_capacity < 0 || (kv_capacity != 0 && kv_capacity < shape->Skv)) return INTATTN_E_SHAPE;
    const int rows = kv_capacity == 0 ? shape->Skv : kv_capacity;
    if (static_cast<double>(shape->B) * hkv * rows * shape->D > 9.0e15) return INTATTN_E_SHAPE;
    uint16_t lut[kIaMaxLut] = {};
    int32_t idx_mul = 0, idx_shift = 0, x_clip = 0, req_shift = 0;
    int64_t req_mul = 0;
    st = intattn_derive_core(shape, scales, clip, lut_size, lut, &idx_mul, &idx_shift, &x_clip, &req_shift,
                             &req_mul, prob_bits, lut_bits);
    if (st != INTATTN_OK) return st;
    kp->B = shape->B;
    kp->H = shape->H;
    kp->Sq = shape->Sq;
    kp->Skv = shape->Skv;
    kp->causal = causal ? 1 : 0;
    kp->idx_mul = idx_mul;
    kp->idx_shift = idx_shift;
    kp->x_clip = x_clip;
    kp->req_shift = req_shift;
    kp->req_mul = static_cast<uint32_t>(req_mul);
    kp->lut_size = lut_size;
    uint16_t tab[kIaTabEntries] = {};
    if (idx_shift == 24) {
        // slot word t = sat(y * -kM + k * 2^23): the largest k in {4, 2, 1}
        // with k <= 128/N (the byte holds k * (N - 1) + k - 1) and kM within
        // the 24-bit signed operand (M <= 2^23 and -M >= -2^23 for k = 1);
        // k = 4 only for the 32-entry table
        const int64_t m = idx_mul;
        int k = 1;
        if (lut_size == 32 && 4 * m < (int64_t(1) << 23)) k = 4;
        else if (lut_size <= 64 && 2 * m < (int64_t(1) << 23)) k = 2;
        kp->slot_k = k;
        kp->slot_k_log2 = k == 4 ? 2 : k - 1;
        kp->ent_a = -k * idx_mul;
        kp->ent_b = k << 23;
        kp->tab_mul = idx_mul;
        kp->tab_half = 1u << 23;
        kp->tab_shift = 24;
        for (int i = 0; i < kIaMaxLut; ++i) tab[i] = lut[i];
        // Masked keys enter the slot word as y = -2^23. When k(M + 1) >= 256
        // the word saturates (slot N - 1 or past it: entry 0). Below that
        // (M < 64 for N = 32) it lands on slot floor((M + 1) / 2), which no
        // allowed key reaches: an int8 score gap is at most 2 * 128 * 127^2,
        // whose slot floor((4129024 M + 2^23) / 2^24) is smaller for every
        // M >= 1 (checked for each M below 256). Those unreachable entries are
        // made 0, so masked keys drop out of the sum as the specification
        // says.
        if (k * (static_cast<int64_t>(idx_mul) + 1) < 256)
            for (int i = (idx_mul + 1) / 2; i < lut_size; ++i) tab[i] = 0;
    } else {
        // From mu = 1/2 on a score unit moves half a bin or more, so the
        // clip point is at most 2N - 3 units from the row max: the table is
        // indexed by the clipped gap x' = min(m - s, x_clip) itself,
        // entry x' = lut[min(N-1, (x'*M + 2^(sh-1)) >> sh)], and entry
        // x_clip is 0 (the sparse tail).
        if (x_clip < 1 || x_clip >= kIaTabEntries) return INTATTN_E_RANGE;   // not reached (x_clip <= 2N-3)
        for (int x = 0; x <= x_clip; ++x) {
            const int64_t slot = (static_cast<int64_t>(x) * idx_mul + (int64_t(1) << (idx_shift - 1))) >> idx_shift;
            tab[x] = lut[slot < lut_size - 1 ? slot : lut_size - 1];
        }
        kp->slot_k = 0;
        kp->slot_k_log2 = 0;
        kp->ent_a = -x_clip;
        kp->ent_b = 0;
        kp->tab_mul = 1;
        kp->tab_half = 0;
        kp->tab_shift = 0;
    }
    kp->kv_group = shape->H > 0 ? shape->H / hkv : 1;
    kp->kvg_div = ia::invariant_div(static_cast<uint32_t>(kp->kv_group));
    kp->h_div = ia::invariant_div(static_cast<uint32_t>(shape->H > 0 ? shape->H : 1));
    kp->kv_rows = rows;
    kp->prob_bits = prob_bits;
    for (int i = 0; i < kIaTabEntries / 2; ++i)
        kp->lut2[i] = static_cast<uint32_t>(tab[2 * i]) | (static_cast<uint32_t>(tab[2 * i + 1]) << 16);
    return INTATTN_OK;
}

int prepare(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
            const intattn_shape* shape, const intattn_scales* scales, float clip, int causal,
            IaKernelParams* kp, int lut_size = 32, int kv_heads = 0, int kv_capacity = 0, int prob_bits = 8,
            int lut_bits = 16) {
    if (!q || !k || !v || !out || !shape || !scales) return INTATTN_E_NULL;
    const int st = derive_kernel_params(shape, scales, clip, causal, kp, lut_size, kv_heads, kv_capacity,
                                        prob_bits, lut_bits);
    if (st != INTATTN_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return INTATTN_E_ALIGN;
    return INTATTN_OK;
}

long long rows_of(const IaKernelParams& kp) { return static_cast<long long>(kp.B) * kp.H * kp.Sq; }

// Decode shapes split their keys over several workgroups per head when the
// caller gives a workspace: past the single-workgroup decode kernel's key
// limit, and when the heads (a workgroup each) are few for the cache length:
// from 4096 keys on, once Skv > 128 * heads. GPU time on MI355X (128-wide
// heads, calls queued ahead of the GPU): 32 heads take 16.6 us unsplit
// against 15.9 us split at 4096 keys (a near tie, left unsplit: one launch
// instead of four costs the host less) but 29.8 against 24.3 at 8192; 64
// heads 31.6 against 34.2 at 8192 keys and 55.8 against 58.1 at 16384; 96
// heads 36.2 against 45.3 at 8192 but 106.5 against 88.6 at 16384.
bool uses_split(int B, int H, int Sq, int Skv) {
    const long long heads = static_cast<long long>(B) * H;
    return Sq == 1 && (Skv > ia::decode_max_keys() || (Skv >= 4096 && Skv > 128 * heads));
}

int dispatch(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
             const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum,
             void* workspace = nullptr) {
    if (workspace != nullptr && uses_split(kp.B, kp.H, kp.Sq, kp.Skv))
        return ia::launch_decode_split(q, k, v, out, D, kp, stream, workspace, row_max, row_sum);
    if (kp.Sq == 1)   // past decode_max_keys() keys: three passes over K, no scores kept
        return ia::launch_decode(q, k, v, out, D, kp, stream, row_max, row_sum);
    if (kp.Skv <= ia::short_max_keys(D))
        return ia::launch_short(q, k, v, out, D, kp, stream, row_max, row_sum);
    return ia::launch_long(q, k, v, out, D, kp, stream, row_max, row_sum);
}

}  // namespace

extern "C" int intattn_forward(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                               const intattn_shape* shape, const intattn_scales* scales, float clip,
                               int causal, void* stream) {
    IaKernelParams kp;
    const int st = prepare(q, k, v, out, shape, scales, clip, causal, &kp);
    if (st != INTATTN_OK) return st;
    if (static_cast<long long>(kp.B) * kp.H * kp.Sq == 0) return INTATTN_OK;
    ia::clear_pending_hip_error();
    return dispatch(q, k, v, out, shape->D, kp, stream, nullptr, nullptr);
}

extern "C" int intattn_forward_debug(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                                     const intattn_shape* shape, const intattn_scales* scales, float clip,
                                     int causal, void* stream, int32_t* row_max, uint32_t* row_sum,
                                     uint8_t* probs) {
    if (!row_max || !row_sum) return INTATTN_E_NULL;
    IaKernelParams kp;
    const int st = prepare(q, k, v, out, shape, scales, clip, causal, &kp);
    if (st != INTATTN_OK) return st;
    if (static_cast<long long>(kp.B) * kp.H * kp.Sq == 0) return INTATTN_OK;
    ia::clear_pending_hip_error();
    if (probs != nullptr)
        return ia::launch_general(q, k, v, out, shape->D, kp, stream, row_max, row_sum, probs);
    return dispatch(q, k, v, out, shape->D, kp, stream, row_max, row_sum);
}

extern "C" uint64_t intattn_workspace_bytes(const intattn_shape* shape, const intattn_variant* variant) {
    (void)variant;   // the workspace does not depend on the table or probability width
    if (!shape || intattn_validate_shape(shape, 0) != INTATTN_OK) return 0;
    if (shape->D != 64 && shape->D != 128) return 0;
    if (!uses_split(shape->B, shape->H, shape->Sq, shape->Skv)) return 0;
    return ia::decode_split_workspace_bytes(static_cast<long long>(shape->B) * shape->H, shape->Skv, shape->D);
}

namespace {

// Every check of intattn_forward_ex (no HIP call), and its kernel parameters.
int check_forward_ex(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, const intattn_shape* shape,
                     const intattn_scales* scales, float clip, int causal, const intattn_variant* variant,
                     int32_t* row_max, uint32_t* row_sum, IaKernelParams* kp) {
    if ((row_max == nullptr) != (row_sum == nullptr)) return INTATTN_E_NULL;
    const int lut_size = variant && variant->lut_size != 0 ? variant->lut_size : 32;
    const int kv_heads = variant ? variant->kv_heads : 0;
    const int kv_capacity = variant ? variant->kv_capacity : 0;
    const int prob_bits = variant && variant->prob_bits != 0 ? variant->prob_bits : 8;
    const int lut_bits = variant && variant->lut_bits != 0 ? variant->lut_bits : 16;
    const int st = prepare(q, k, v, out, shape, scales, clip, causal, kp, lut_size, kv_heads, kv_capacity,
                           prob_bits, lut_bits);
    if (st != INTATTN_OK) return st;
    void* ws = variant ? variant->workspace : nullptr;
    if (ws != nullptr && uses_split(shape->B, shape->H, shape->Sq, shape->Skv)) {
        const uint64_t need = intattn_workspace_bytes(shape, variant);
        if (variant->workspace_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return INTATTN_E_WORKSPACE;
    }
    return INTATTN_OK;
}

}  // namespace

int intattn_validate_forward_ex(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                                const intattn_shape* shape, const intattn_scales* scales, float clip, int causal,
                                const intattn_variant* variant, int32_t* row_max, uint32_t* row_sum) {
    IaKernelParams kp;
    return check_forward_ex(q, k, v, out, shape, scales, clip, causal, variant, row_max, row_sum, &kp);
}

extern "C" int intattn_forward_ex(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                                  const intattn_shape* shape, const intattn_scales* scales, float clip,
                                  int causal, const intattn_variant* variant, void* stream, int32_t* row_max,
                                  uint32_t* row_sum) {
    IaKernelParams kp;
    const int st = check_forward_ex(q, k, v, out, shape, scales, clip, causal, variant, row_max, row_sum, &kp);
    if (st != INTATTN_OK) return st;
    void* ws = variant ? variant->workspace : nullptr;
    if (rows_of(kp) == 0) return INTATTN_OK;
    ia::clear_pending_hip_error();
    return dispatch(q, k, v, out, shape->D, kp, stream, row_max, row_sum, ws);
}

extern "C" int intattn_qk_scores(const int8_t* q, const int8_t* k, int32_t* scores, const intattn_shape* shape,
                                 void* stream) {
    if (!q || !k || !scores || !shape) return INTATTN_E_NULL;
    int st = intattn_validate_shape(shape, 0);
    if (st != INTATTN_OK) return st;
    if (shape->D != 64 && shape->D != 128) return INTATTN_E_DIM;
    if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(scores) & 3u)) return INTATTN_E_ALIGN;
    IaKernelParams kp{};
    kp.B = shape->B;
    kp.H = shape->H;
    kp.Sq = shape->Sq;
    kp.Skv = shape->Skv;
    kp.kv_group = 1;
    kp.kvg_div = ia::invariant_div(1);
    kp.h_div = ia::invariant_div(static_cast<uint32_t>(shape->H > 0 ? shape->H : 1));
    kp.kv_rows = shape->Skv;
    kp.prob_bits = 8;
    if (rows_of(kp) == 0) return INTATTN_OK;
    ia::clear_pending_hip_error();
    return ia::launch_qk_scores(q, k, scores, shape->D, kp, stream);
}

extern "C" int intattn_index_softmax(const int32_t* scores, uint8_t* probs, int32_t* row_max, uint32_t* row_sum,
                                     const intattn_shape* shape, const intattn_scales* scales, float clip,
                                     int causal, void* stream) {
    if (!scores || !probs || !shape || !scales) return INTATTN_E_NULL;
    if ((row_max == nullptr) != (row_sum == nullptr)) return INTATTN_E_NULL;
    if (reinterpret_cast<uintptr_t>(scores) & 3u) return INTATTN_E_ALIGN;
    IaKernelParams kp;
    const int st = derive_kernel_params(shape, scales, clip, causal, &kp);
    if (st != INTATTN_OK) return st;
    if (kp.Skv > ia::stage_max_keys()) return INTATTN_E_SHAPE;
    if (rows_of(kp) == 0) return INTATTN_OK;
    ia::clear_pending_hip_error();
    return ia::launch_index_softmax(scores, probs, row_max, row_sum, kp, stream);
}

extern "C" int intattn_fp_softmax(const int32_t* scores, uint8_t* probs, const intattn_shape* shape,
                                  const intattn_scales* scales, int causal, void* stream) {
    if (!scores || !probs || !shape || !scales) return INTATTN_E_NULL;
    if (reinterpret_cast<uintptr_t>(scores) & 3u) return INTATTN_E_ALIGN;
    int st = intattn_validate_shape(shape, causal);
    if (st != INTATTN_OK) return st;
    if (shape->D != 64 && shape->D != 128) return INTATTN_E_DIM;
    if (!(scales->q > 0.0f) || !(scales->k > 0.0f) || !std::isfinite(scales->q) || !std::isfinite(scales->k))
        return INTATTN_E_SCALE;
    IaKernelParams kp{};
    kp.B = shape->B;
    kp.H = shape->H;
    kp.Sq = shape->Sq;
    kp.Skv = shape->Skv;
    kp.causal = causal ? 1 : 0;
    kp.kv_group = 1;
    kp.kvg_div = ia::invariant_div(1);
    kp.h_div = ia::invariant_div(static_cast<uint32_t>(shape->H > 0 ? shape->H : 1));
    kp.kv_rows = shape->Skv;
    kp.prob_bits = 8;
    if (kp.Skv > ia::stage_max_keys()) return INTATTN_E_SHAPE;
    if (rows_of(kp) == 0) return INTATTN_OK;
    // dequantisation factor of a score: s_q * s_k / sqrt(D), rounded once to float32
    const float alpha = static_cast<float>(static_cast<double>(scales->q) * static_cast<double>(scales->k) /
                                           std::sqrt(static_cast<double>(shape->D)));
    ia::clear_pending_hip_error();
    return ia::launch_fp_softmax(scores, probs, alpha, kp, stream);
}

extern "C" int intattn_pv(const uint8_t* probs, const int8_t* v, int8_t* out, const intattn_shape* shape,
                          const intattn_scales* scales, float clip, int causal, void* stream) {
    if (!probs || !v || !out || !shape || !scales) return INTATTN_E_NULL;
    if (!aligned16(v) || !aligned16(out)) return INTATTN_E_ALIGN;
    IaKernelParams kp;
    const int st = derive_kernel_params(shape, scales, clip, causal, &kp);
    if (st != INTATTN_OK) return st;
    if (rows_of(kp) == 0) return INTATTN_OK;
    ia::clear_pending_hip_error();
    return ia::launch_pv(probs, v, out, shape->D, kp, stream);
}

extern "C" int intattn_kv_append(const float* k_new, const float* v_new, int8_t* k_cache, int8_t* v_cache,
                                 int32_t B, int32_t kv_heads, int32_t T, int32_t D, int32_t capacity, int32_t pos,
                                 float s_k, float s_v, void* stream) {
    if (!k_new || !v_new || !k_cache || !v_cache) return INTATTN_E_NULL;
    if (B < 0 || kv_heads < 0 || T < 0 || capacity < 1 || capacity > 65535 || pos < 0 ||
        static_cast<int64_t>(pos) + T > capacity)
        return INTATTN_E_SHAPE;
    if (D != 64 && D != 128) return INTATTN_E_DIM;
    if (static_cast<double>(B) * kv_heads * capacity * D > 9.0e15) return INTATTN_E_SHAPE;
    if (!(s_k > 0.0f) || !(s_v > 0.0f) || !std::isfinite(s_k) || !std::isfinite(s_v)) return INTATTN_E_SCALE;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) return INTATTN_E_ALIGN;
    if (static_cast<int64_t>(B) * kv_heads * T == 0) return INTATTN_OK;
    ia::clear_pending_hip_error();
    return ia::launch_kv_append(k_new, v_new, k_cache, v_cache, B, kv_heads, T, D, capacity, pos, s_k, s_v, stream);
}
