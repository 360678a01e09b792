/*
 * intattn.h - C ABI of the MI355X (gfx950) fully-integer attention library.
 *
 * The operation is the IntAttention forward pass (IntAttention digest pages,
 * euno.news, arXiv 2511.21513v1, section "Methodology", steps 2 and 3):
 * int8 Q.K^T gives int32 scores; IndexSoftmax clips each score relative to
 * its row maximum at a sparsity-aware threshold, indexes a 32-entry exp
 * table, sums the pseudo-exponents in int32, and scales them by an integer
 * reciprocal (multiply + right shift) into uint8 probabilities; the uint8
 * probabilities multiply int8 V; the int32 result is requantised to int8.
 * No floating point is used on the device: the integer divisions (each row's
 * reciprocal, the split of a workgroup index into head and query block) run
 * on integer instructions as well. The float32 comparator and the cache
 * update below take float inputs by definition.
 *
 * Integer specification (the pages leave every width and rounding open; this
 * is the reading the library implements, bit for bit):
 *   alpha = s_q*s_k/sqrt(D), delta = clip/31, mu = alpha/delta   (binary64)
 *   lut[k] = rint(2^15 * exp(-k*delta)) for k < 31, lut[31] = 0
 *   required 2^-24 <= mu < 2^14; M = rint(mu * 2^sh) with sh = 24 for
 *   mu < 1/2, else sh = 23 - e for mu = m 2^e, m in [1/2, 1) (frexp), so
 *   that M <= 2^23 always (M in [2^22, 2^23] from mu = 1/2 on)
 *   s_ij = sum_d q_id k_jd                        (int32)
 *   m_i = max over allowed j of s_ij
 *   idx_ij = min(31, ((m_i - s_ij)*M + 2^(sh-1)) >> sh), 31 for masked keys
 *   E_i = sum_j lut[idx_ij]                        (< 2^31)
 *   R_i = (255*2^23 + E_i/2) / E_i                  (integer division)
 *   p_ij = (lut[idx_ij]*R_i + 2^22) >> 23           (uint8)
 *   a_id = sum_j p_ij v_jd                          (int32)
 *   mu_o = s_v/(255*s_o) = M_o * 2^-sh_o, M_o in [2^30, 2^31)
 *   out_id = sign(a)*min(127, (|a|*M_o + 2^(sh_o-1)) >> sh_o)
 * A key j is allowed for query i when j < Skv and, if causal, when
 * j <= i + Skv - Sq (causal masks are aligned to the bottom-right corner).
 *
 * Layout: every tensor is contiguous row-major [B, H, S, D] int8 in device
 * memory (S = Sq for q and out, Skv for k and v). Inputs are expected in the
 * symmetric range [-127, 127]; the library does not read device data to check
 * this.
 *
 * Devices and streams: every launch goes to the calling thread's current
 * HIP device, and `stream` (NULL: the null stream) must belong to it; the
 * tensors must be memory that device can read and write.
 *
 * Graph capture: the attention entry points queue only kernel launches on
 * `stream` (no allocation, memset, copy or synchronisation), so their calls
 * can be captured in a HIP graph and replayed. The long-row and decode
 * kernels raise their dynamic LDS limit once per device on first use, a
 * host-side call: make one uncaptured call of a shape before capturing it.
 *
 * Ownership: all tensor pointers are caller-owned device memory and must stay
 * valid until the work queued on `stream` has finished. Structs are
 * caller-owned host memory read during the call only. The library keeps no
 * reference to any argument after returning.
 *
 * Errors: every function returns INTATTN_OK (0) or a negative code. All
 * argument validation runs on the host before any HIP call, so an invalid
 * call queues no work and writes nothing. A failed kernel launch returns
 * INTATTN_E_HIP. Work is asynchronous: device faults surface at the next
 * synchronisation of `stream`, not in the return code.
 */
#ifndef INTATTN_H
#define INTATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct intattn_shape {
    int32_t B;    /* batch, >= 0 (0: nothing to do)                          */
    int32_t H;    /* heads, >= 0 (0: nothing to do)                          */
    int32_t Sq;   /* query rows, >= 0 (0: nothing to do)                     */
    int32_t Skv;  /* key/value rows, 1 .. 65535                              */
    int32_t D;    /* head dimension; 64 or 128 on the device                 */
} intattn_shape;

typedef struct intattn_scales {
    float q, k, v, o;  /* real value = scale * int8, each finite and > 0     */
} intattn_scales;

/* Integers derived on the host from (D, scales, clip). */
typedef struct intattn_params {
    uint16_t lut[32];   /* exp table, lut[0] = 32768, lut[31] = 0           */
    int32_t  idx_mul;   /* M                                                 */
    int32_t  idx_shift; /* sh: 24 for mu < 1/2, 9..23 from mu = 1/2 on       */
    int32_t  x_clip;    /* smallest m - s that lands in slot 31              */
    int32_t  req_shift; /* sh_o, 1 .. 63                                     */
    int64_t  req_mul;   /* M_o                                               */
} intattn_params;

enum {
    INTATTN_OK      =  0,
    INTATTN_E_NULL  = -1,  /* a required pointer is NULL                     */
    INTATTN_E_SHAPE = -2,  /* negative size, Skv outside 1..65535, causal
                              with Sq > Skv, or a size product overflowing  */
    INTATTN_E_DIM   = -3,  /* D not supported by the device kernels         */
    INTATTN_E_SCALE = -4,  /* a scale is not finite and > 0                  */
    INTATTN_E_CLIP  = -5,  /* clip is not finite and > 0                     */
    INTATTN_E_RANGE = -6,  /* mu outside [2^-24, 2^14) or sh_o outside 1..63 */
    INTATTN_E_HIP   = -7,  /* the HIP runtime reported an error              */
    INTATTN_E_ALIGN = -8,  /* a tensor pointer is not 16-byte aligned        */
    INTATTN_E_WORKSPACE = -9, /* workspace smaller than intattn_workspace_bytes,
                                 or not 256-byte aligned                    */
    INTATTN_E_SCRATCH = -10   /* intattn_forward_ex_noalloc: the shape needs
                                 more than INTATTN_NOALLOC_SCRATCH_BYTES     */
};

/* The 32-entry exp table for a clip threshold (in logit units): lut_out[k] =
 * rint(2^15 exp(-k clip/31)) for k < 31 and lut_out[31] = 0 (the table of
 * the pages' IndexSoftmax lookup step). Host only, pure. Errors: E_NULL,
 * E_CLIP. */
int intattn_build_lut(float clip, uint16_t lut_out[32]);

/* All host-derived integers for a call (the parameters the device kernels
 * receive). Host only, pure. Validates shape->D >= 1 but not the device's D
 * restriction. Errors: E_NULL, E_SHAPE, E_SCALE, E_CLIP, E_RANGE. */
int intattn_derive_params(const intattn_shape* shape, const intattn_scales* scales,
                          float clip, intattn_params* out);

/* The attention forward pass of the pages' "Methodology" steps 2-3:
 * out = IntAttention(q, k, v). q, k, v, out: device pointers (see Layout).
 * causal: 0 or 1. stream: a hipStream_t (NULL for the null stream); the
 * kernels are queued on it and the call returns without synchronising.
 * Every tensor pointer must be 16-byte aligned. Allocates no device memory.
 * Errors: E_NULL, E_SHAPE, E_DIM, E_ALIGN, E_SCALE, E_CLIP, E_RANGE, E_HIP. */
int intattn_forward(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                    const intattn_shape* shape, const intattn_scales* scales,
                    float clip, int causal, void* stream);

/* intattn_forward plus the per-row integer state of IndexSoftmax, for parity
 * checks: row_max [B,H,Sq] int32 (m_i), row_sum [B,H,Sq] uint32 (E_i), and,
 * when probs is not NULL, probs [B,H,Sq,Skv] uint8 (p_ij, 0 for masked keys).
 * row_max and row_sum are required device pointers. With probs, the general
 * kernel runs (the only one that writes P); without, the same kernel as
 * intattn_forward. Errors: as intattn_forward. */
int intattn_forward_debug(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                          const intattn_shape* shape, const intattn_scales* scales,
                          float clip, int causal, void* stream,
                          int32_t* row_max, uint32_t* row_sum, uint8_t* probs);

/* ---- Variants: finer exp tables and grouped K/V heads ----------------------
 * Finer tables: the pages' "Limitations & Future Work" (lookup-table
 * granularity) call the 32-entry table a trade-off between accuracy and
 * memory and say very large attention heads may need finer tables. With
 * lut_size N in {32, 64, 128} every step above is unchanged except
 *   delta = clip/(N-1), lut[k] = rint(2^15 exp(-k delta)) for k < N-1,
 *   lut[N-1] = 0, idx = min(N-1, ((m - s)*M + 2^(sh-1)) >> sh),
 * with (M, sh) from mu = alpha/delta as above (mu grows with N, so a finer
 * table reaches the narrower-fraction form at smaller alpha). N = 32 is the
 * specification above.
 * Grouped K/V heads (decoder serving: grouped-query and multi-query
 * attention; the pages do not describe this step): k and v hold kv_heads
 * heads, [B, kv_heads, Skv, D], and query head h reads K/V head
 * h / (H / kv_heads); kv_heads must divide H (kv_heads = H is ordinary
 * multi-head attention).
 * uint16 probabilities: the same section warns of underflow on skewed score
 * distributions; a uint8 row of 513 or more uniform keys is all zeros. With
 * prob_bits = 16: R16 = (65535*2^16 + E/2) / E, p = (lut[idx]*R16 + 2^15)
 * >> 16 (uint16, target row sum 65535), and mu_o = s_v/(65535*s_o); every
 * kernel runs it (P.V as two int8 products, high and low probability
 * bytes).
 * uint8 table entries: the lookup-table granularity item frames the table as
 * an accuracy/memory trade; lut_bits = 8 stores e8[k] = rint(255 exp(-k
 * delta)) for k < N-1 and e8[N-1] = 0 (any N), and with E8 = sum_j e8
 *   R8 = (255*2^17 + E8) / (2*E8),  p = (e8*R8 + 2^15) >> 16        (uint8)
 *   R8 = (65535*2^10 + E8) / (2*E8), p = (e8*R8 + 2^8) >> 9     (uint16 P).
 * The kernels receive the table in Q15 units, lut = 128*e8: with E = 128*E8
 * the Q15 reciprocal and product above give exactly these R8 and p (both
 * fractions reduce by 128), so every kernel serves both widths; row_sum then
 * reports E = 128*E8. */
typedef struct intattn_variant {
    int32_t lut_size;    /* exp-table entries: 32, 64 or 128; 0 means 32     */
    int32_t kv_heads;    /* K/V heads; 0 means H                             */
    int32_t kv_capacity; /* rows per K/V head in memory, >= Skv (a K/V cache
                            of that capacity whose first Skv rows are
                            attended); 0 means Skv                           */
    int32_t prob_bits;   /* probability width: 8 (uint8, the specification
                            above) or 16 (uint16 variant); 0 means 8         */
    int32_t lut_bits;    /* table entry width: 16 (Q15, the specification
                            above) or 8 (uint8 entries); 0 means 16          */
    void*    workspace;  /* device memory, caller-owned, for decode (Sq = 1)
                            with Skv > 16384, or with Skv >= 4096 and
                            Skv > 128*B*H (few heads for the cache length,
                            each a workgroup): keys are split into chunks
                            over several workgroups per head (exact: the row
                            max and sum are combined before any probability,
                            and the P.V partials are integers). NULL: those
                            shapes run one workgroup per head, on the decode
                            kernel (Skv <= 16384) or, past 16384 keys, on its
                            three-pass form that keeps no scores and reads K
                            three times (about 3x slower than split on a
                            65535-key cache at 64 heads: 1.5 against
                            4.9 TB/s of K and V). intattn_forward never
                            splits: it has no workspace                       */
    uint64_t workspace_bytes; /* size of workspace                           */
} intattn_variant;

typedef struct intattn_params_ex {
    uint16_t lut[128];  /* entries 0..lut_size-1 in Q15 units (128*e8 for
                           lut_bits 8; entry lut_size-1 is 0); the rest 0   */
    int32_t  lut_size;
    int32_t  idx_mul;   /* M                                                 */
    int32_t  idx_shift; /* sh: 24 for mu < 1/2, 9..23 from mu = 1/2 on       */
    int32_t  x_clip;    /* smallest m - s that lands in slot lut_size-1      */
    int32_t  req_shift; /* sh_o, 1 .. 63                                     */
    int64_t  req_mul;   /* M_o                                               */
    int32_t  prob_bits; /* 8 or 16                                           */
    int32_t  lut_bits;  /* 16 or 8                                           */
} intattn_params_ex;

/* The lut_size-entry exp table of lut_bits-bit entries (lut_out holds
 * lut_size entries: Q15 for 16, e8 in 0..255 for 8). Host only, pure.
 * Errors: E_NULL, E_CLIP, E_RANGE (lut_size not 32, 64 or 128, lut_bits not
 * 16 or 8). */
int intattn_build_lut_ex(float clip, int32_t lut_size, int32_t lut_bits, uint16_t* lut_out);

/* intattn_derive_params for a lut_size-entry table of lut_bits-bit entries
 * (16 or 8; out->lut holds the table in Q15 units) and prob_bits-wide
 * probabilities (8 or 16; 16 changes only M_o, sh_o). Host only, pure.
 * Errors: E_NULL, E_SHAPE, E_SCALE, E_CLIP, E_RANGE (also lut_size,
 * prob_bits, lut_bits). */
int intattn_derive_params_ex(const intattn_shape* shape, const intattn_scales* scales,
                             float clip, int32_t lut_size, int32_t prob_bits, int32_t lut_bits,
                             intattn_params_ex* out);

/* intattn_forward with a variant (NULL: lut_size 32, kv_heads H, no cache
 * padding, uint8 P, Q15 table). q and out are [B, H, Sq, D]; k and v are [B, kv_heads,
 * kv_capacity, D], of which rows 0..Skv-1 of each head are read. row_max / row_sum:
 * optional device outputs [B, H, Sq] (both NULL or both set), as in
 * intattn_forward_debug. Every tensor pointer 16-byte aligned; allocates no
 * device memory. Errors: those of intattn_forward, E_NULL for one of
 * row_max / row_sum without the other, E_SHAPE for kv_heads < 0 or not
 * dividing H or for 0 < kv_capacity < Skv, E_RANGE for lut_size, prob_bits or lut_bits,
 * E_WORKSPACE for a workspace smaller than intattn_workspace_bytes or not
 * 256-byte aligned. With a workspace, the call may queue several kernels. */
/* Bytes of workspace intattn_forward_ex uses for this shape and variant
 * (256-byte aligned; int32 scores per key and head, per-chunk maxima and
 * sums, per-head accumulators), 0 when the shape does not use one (only
 * Sq = 1 with Skv > 16384, or Skv >= 4096 and Skv > 128*B*H, does). Host only,
 * pure. Returns 0 for an invalid shape as well. */
uint64_t intattn_workspace_bytes(const intattn_shape* shape, const intattn_variant* variant);

int intattn_forward_ex(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                       const intattn_shape* shape, const intattn_scales* scales, float clip,
                       int causal, const intattn_variant* variant, void* stream,
                       int32_t* row_max, uint32_t* row_sum);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 * intattn_forward_ex with the same arguments and results, except that the
 * shapes that split their keys over several workgroups per head (those for
 * which intattn_workspace_bytes is nonzero) use the library's own device
 * scratch, a static array of INTATTN_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends, instead of a caller
 * workspace; variant->workspace must be NULL and workspace_bytes 0. Calls no
 * allocating function. Every call on a GPU shares that GPU's scratch, so
 * calls that overlap on one GPU (other streams or threads) race; the kernels
 * clear what must start at zero, so earlier contents never matter. The
 * scratch's device address is looked up once per device on the first call
 * that needs it (hipGetSymbolAddress, with that device current).
 * Errors: those of intattn_forward_ex (all checked before any HIP call),
 * E_WORKSPACE for a caller workspace, E_SCRATCH when intattn_workspace_bytes
 * exceeds the scratch size, E_HIP if the scratch address lookup fails. */
#define INTATTN_NOALLOC_SCRATCH_BYTES (32ull << 20)
int intattn_forward_ex_noalloc(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                               const intattn_shape* shape, const intattn_scales* scales, float clip,
                               int causal, const intattn_variant* variant, void* stream,
                               int32_t* row_max, uint32_t* row_sum);

/* Decode-step cache update (the step before attention in a decoder's decode
 * step; the pages do not describe it): the keys and values of T new tokens,
 * k_new and v_new float32 [B, kv_heads, T, D] in device memory, are coded to
 * int8 and written to rows pos .. pos+T-1 of the caches k_cache and v_cache,
 * int8 [B, kv_heads, capacity, D] in device memory; no other byte of the
 * caches changes. Code of a value x under the cache's per-tensor scale s
 * (s_k for keys, s_v for values): clip(rint(x / s), -127, 127), with x / s
 * the IEEE float32 quotient (round to nearest, ties to even), rint rounding
 * ties to even, NaN coded as 0 and +-inf as +-127 (the inputs' quantisation
 * rule). The caches then feed intattn_forward_ex with kv_capacity =
 * capacity and Skv = pos + T. All pointers 16-byte aligned; D 64 or 128;
 * 0 <= pos, pos + T <= capacity <= 65535. Asynchronous on stream; allocates
 * nothing. Errors: E_NULL, E_SHAPE, E_DIM, E_SCALE (s_k or s_v not finite
 * and > 0), E_ALIGN, E_HIP. */
int intattn_kv_append(const float* k_new, const float* v_new, int8_t* k_cache, int8_t* v_cache,
                      int32_t B, int32_t kv_heads, int32_t T, int32_t D, int32_t capacity, int32_t pos,
                      float s_k, float s_v, void* stream);

/* ---- The pipeline as separate stages (scores and P in device memory) ----
 * The pages' "Methodology" step 1 places the cost of an INT8 pipeline in the
 * floating-point softmax between the integer products; these entry points run
 * the three steps as separate kernels so each can be timed, and offer the
 * floating-point softmax as a comparator. Chained as
 *   intattn_qk_scores -> intattn_index_softmax -> intattn_pv
 * they give exactly intattn_forward's output. All buffers are caller-owned
 * device memory; nothing is allocated; calls queue on stream and return.
 * The softmax stages need Skv <= 4096 (a row is held in registers). */

/* Step 3, first product: scores[b,h,i,j] = sum_d q[b,h,i,d] * k[b,h,j,d]
 * as int32 [B,H,Sq,Skv], for every (i, j) (masks are applied by the
 * softmax stage). q, k 16-byte aligned; scores 4-byte aligned.
 * Errors: E_NULL, E_SHAPE, E_DIM, E_ALIGN, E_HIP. */
int intattn_qk_scores(const int8_t* q, const int8_t* k, int32_t* scores,
                      const intattn_shape* shape, void* stream);

/* Step 2, IndexSoftmax on int32 scores [B,H,Sq,Skv] (|s| < 2^30, as any
 * int8 product is): probs [B,H,Sq,Skv] uint8 p_ij (0 for keys that are not
 * allowed), and optionally row_max [B,H,Sq] int32 and row_sum [B,H,Sq]
 * uint32 (both or neither). Same integers as intattn_forward_debug.
 * scores 4-byte aligned. Errors: E_NULL, E_SHAPE (also Skv > 4096), E_DIM,
 * E_ALIGN, E_SCALE, E_CLIP, E_RANGE, E_HIP. */
int intattn_index_softmax(const int32_t* scores, uint8_t* probs, int32_t* row_max,
                          uint32_t* row_sum, const intattn_shape* shape,
                          const intattn_scales* scales, float clip, int causal,
                          void* stream);

/* Comparator for step 2 (the dequantise-softmax-requantise loop the pages
 * remove): y = alpha * s in float32 with alpha = float32(s_q*s_k/sqrt(D)),
 * softmax over the allowed keys with the row max subtracted (float32), and
 * probs = min(255, rint(255 * p)) as uint8 (0 for keys that are not
 * allowed). Floating point is used only here. scores 4-byte aligned.
 * Errors: E_NULL, E_SHAPE (also Skv > 4096), E_DIM, E_ALIGN, E_SCALE, E_HIP. */
int intattn_fp_softmax(const int32_t* scores, uint8_t* probs, const intattn_shape* shape,
                       const intattn_scales* scales, int causal, void* stream);

/* Step 3, second product: out = requantise(P.V) int8 [B,H,Sq,D] from uint8
 * probs [B,H,Sq,Skv] and int8 v, with the requantisation of intattn_forward
 * (from s_v, s_o; clip and the other scales must be valid as for
 * intattn_forward). With causal, key tiles past a query block's causal limit
 * are skipped, so probs must be 0 there (as the softmax stages write them).
 * v, out 16-byte aligned. Errors: E_NULL, E_SHAPE, E_DIM, E_ALIGN, E_SCALE,
 * E_CLIP, E_RANGE, E_HIP. */
int intattn_pv(const uint8_t* probs, const int8_t* v, int8_t* out, const intattn_shape* shape,
               const intattn_scales* scales, float clip, int causal, void* stream);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* intattn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* INTATTN_H */
