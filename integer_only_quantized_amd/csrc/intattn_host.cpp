// Host side of the integer attention library: argument validation and the
// derivation of every integer the device kernels receive.
//
// The pages (IntAttention digest, "Methodology" step 2) describe a 32-entry
// exp table indexed by the clipped integer score and an integer reciprocal
// normalisation; the widths below are this library's fixed reading of them
// (stated in include/intattn.h). Finer tables of 64 or 128 entries (the
// pages' "Limitations & Future Work", lookup-table granularity) change only
// the bin width clip/(N-1) and the table; a table of uint8 entries (the
// narrow end of the same section's accuracy/memory trade) reaches the
// kernels as 128 times its entries, which leaves every probability unchanged
// (the identity is stated in include/intattn.h). All arithmetic is IEEE binary64 from float32
// inputs with correctly rounded operations only; the file is compiled with
// -ffp-contract=off so no multiply-add is fused, and rint() (round half to
// even in the default rounding mode) is the only rounding used.
#include <cfenv>
#include <cmath>
#include <cstdint>

#include "intattn.h"
#include "intattn_internal.h"

namespace {

constexpr int kLutSize = 32;
constexpr double kLutOne = 32768.0;   // Q15 entry for a zero relative score
constexpr double kLut8One = 255.0;    // uint8 entry for a zero relative score
constexpr int kLut8Scale = 128;       // uint8 entries in Q15 units
constexpr int kIdxShift = 24;        // bin-multiplier fraction bits below mu = 1/2
constexpr int kIdxMulBits = 23;      // from mu = 1/2 on: the widest multiplier M <= 2^23
constexpr int kReqFrac = 31;

bool finite_positive(float x) { return std::isfinite(x) && x > 0.0f; }

// The derivation assumes round-to-nearest for every binary64 operation. The
// floating-point environment is per thread; a caller that changed the mode
// gets it back on return.
struct NearestRounding {
    int saved;
    NearestRounding() : saved(std::fegetround()) {
        if (saved != FE_TONEAREST) std::fesetround(FE_TONEAREST);
    }
    ~NearestRounding() {
        if (saved != FE_TONEAREST) std::fesetround(saved);
    }
};

bool valid_lut_size(int n) { return n == 32 || n == 64 || n == 128; }
bool valid_lut_bits(int b) { return b == 16 || b == 8; }

// Entries k < n-1: rint(one * exp(-k clip/(n-1))), one = 2^15 (16-bit
// entries) or 255 (8-bit); entry n-1: 0 (the sparse tail).
void fill_lut(double clip, int n, int bits, uint16_t* lut) {
    const double one = bits == 8 ? kLut8One : kLutOne;
    const double delta = clip / static_cast<double>(n - 1);
    for (int k = 0; k < n - 1; ++k) {
        const double v = std::rint(one * std::exp(-(static_cast<double>(k) * delta)));
        lut[k] = static_cast<uint16_t>(v);
    }
    lut[n - 1] = 0;
}

}  // namespace

extern "C" int intattn_build_lut(float clip, uint16_t lut_out[32]) {
    if (!lut_out) return INTATTN_E_NULL;
    if (!finite_positive(clip)) return INTATTN_E_CLIP;
    NearestRounding guard;
    fill_lut(static_cast<double>(clip), kLutSize, 16, lut_out);
    return INTATTN_OK;
}

extern "C" int intattn_build_lut_ex(float clip, int32_t lut_size, int32_t lut_bits, uint16_t* lut_out) {
    if (!lut_out) return INTATTN_E_NULL;
    if (!valid_lut_size(lut_size) || !valid_lut_bits(lut_bits)) return INTATTN_E_RANGE;
    if (!finite_positive(clip)) return INTATTN_E_CLIP;
    NearestRounding guard;
    fill_lut(static_cast<double>(clip), lut_size, lut_bits, lut_out);
    return INTATTN_OK;
}

int intattn_validate_shape(const intattn_shape* s, int causal) {
    if (!s) return INTATTN_E_NULL;
    if (s->B < 0 || s->H < 0 || s->Sq < 0) return INTATTN_E_SHAPE;
    if (s->Skv < 1 || s->Skv > 65535) return INTATTN_E_SHAPE;
    if (s->D < 1) return INTATTN_E_SHAPE;
    if (causal && s->Sq > s->Skv) return INTATTN_E_SHAPE;
    // element counts must fit size_t comfortably (64-bit indexing on device)
    const double nq = static_cast<double>(s->B) * s->H * s->Sq * s->D;
    const double nk = static_cast<double>(s->B) * s->H * s->Skv * s->D;
    if (nq > 9.0e15 || nk > 9.0e15) return INTATTN_E_SHAPE;
    return INTATTN_OK;
}

int intattn_derive_core(const intattn_shape* shape, const intattn_scales* sc, float clip, int lut_size,
                        uint16_t* lut, int32_t* idx_mul, int32_t* idx_shift, int32_t* x_clip, int32_t* req_shift,
                        int64_t* req_mul, int prob_bits, int lut_bits) {
    if (!shape || !sc || !lut || !idx_mul || !idx_shift || !x_clip || !req_shift || !req_mul) return INTATTN_E_NULL;
    if (!valid_lut_size(lut_size) || !valid_lut_bits(lut_bits)) return INTATTN_E_RANGE;
    if (prob_bits != 8 && prob_bits != 16) return INTATTN_E_RANGE;
    if (shape->D < 1) return INTATTN_E_SHAPE;
    if (!finite_positive(sc->q) || !finite_positive(sc->k) || !finite_positive(sc->v) ||
        !finite_positive(sc->o))
        return INTATTN_E_SCALE;
    if (!finite_positive(clip)) return INTATTN_E_CLIP;
    NearestRounding guard;

    const int n = lut_size;
    const double c = static_cast<double>(clip);
    const double alpha = (static_cast<double>(sc->q) * static_cast<double>(sc->k)) /
                         std::sqrt(static_cast<double>(shape->D));
    const double delta = c / static_cast<double>(n - 1);
    const double mu = alpha / delta;
    if (!(mu >= std::ldexp(1.0, -24) && mu < std::ldexp(1.0, 14))) return INTATTN_E_RANGE;

    // M = rint(mu * 2^sh): sh = 24 below mu = 1/2 (M in [1, 2^23]); from
    // 1/2 on, with mu = m 2^e (m in [1/2, 1)), sh = 23 - e so that
    // M = rint(m 2^23) lies in [2^22, 2^23]
    int sh = kIdxShift;
    if (mu >= 0.5) {
        int e = 0;
        (void)std::frexp(mu, &e);
        sh = kIdxMulBits - e;
    }
    const int64_t M = static_cast<int64_t>(std::rint(std::ldexp(mu, sh)));
    // x*M >= (2n-3)*2^(sh-1)  <=>  slot >= n-1
    const int64_t num = int64_t(2 * n - 3) << (sh - 1);

    // output multiplier: s_v / (P_one * s_o), P_one = 255 (uint8 P) or 65535
    const double p_one = prob_bits == 16 ? 65535.0 : 255.0;
    const double mu_o = static_cast<double>(sc->v) / (p_one * static_cast<double>(sc->o));
    int e_o = 0;
    const double m_o = std::frexp(mu_o, &e_o);
    int64_t Mo = static_cast<int64_t>(std::rint(std::ldexp(m_o, kReqFrac)));
    if (Mo == (int64_t(1) << kReqFrac)) {
        Mo = int64_t(1) << (kReqFrac - 1);
        e_o += 1;
    }
    const int sh_o = kReqFrac - e_o;
    if (sh_o < 1 || sh_o > 63) return INTATTN_E_RANGE;

    fill_lut(c, n, lut_bits, lut);
    if (lut_bits == 8)
        for (int i = 0; i < n; ++i) lut[i] = static_cast<uint16_t>(lut[i] * kLut8Scale);
    *idx_mul = static_cast<int32_t>(M);
    *idx_shift = sh;
    *x_clip = static_cast<int32_t>((num + M - 1) / M);
    *req_shift = sh_o;
    *req_mul = Mo;
    return INTATTN_OK;
}

extern "C" int intattn_derive_params(const intattn_shape* shape, const intattn_scales* sc,
                                     float clip, intattn_params* out) {
    if (!shape || !sc || !out) return INTATTN_E_NULL;
    intattn_params p{};
    const int st = intattn_derive_core(shape, sc, clip, kLutSize, p.lut, &p.idx_mul, &p.idx_shift, &p.x_clip,
                                       &p.req_shift, &p.req_mul);
    if (st != INTATTN_OK) return st;
    *out = p;
    return INTATTN_OK;
}

extern "C" int intattn_derive_params_ex(const intattn_shape* shape, const intattn_scales* sc, float clip,
                                        int32_t lut_size, int32_t prob_bits, int32_t lut_bits,
                                        intattn_params_ex* out) {
    if (!shape || !sc || !out) return INTATTN_E_NULL;
    intattn_params_ex p{};
    const int st = intattn_derive_core(shape, sc, clip, lut_size, p.lut, &p.idx_mul, &p.idx_shift, &p.x_clip,
                                       &p.req_shift, &p.req_mul, prob_bits, lut_bits);
    if (st != INTATTN_OK) return st;
    p.lut_size = lut_size;
    p.prob_bits = prob_bits;
    p.lut_bits = lut_bits;
    *out = p;
    return INTATTN_OK;
}

extern "C" const char* intattn_strerror(int status) {
    switch (status) {
        case INTATTN_OK: return "ok";
        case INTATTN_E_NULL: return "a required pointer is NULL";
        case INTATTN_E_SHAPE: return "invalid shape (sizes, Skv outside 1..65535, or causal with Sq > Skv)";
        case INTATTN_E_DIM: return "head dimension not supported by the device kernels (64 or 128)";
        case INTATTN_E_SCALE: return "a quantisation scale is not finite and positive";
        case INTATTN_E_CLIP: return "the clip threshold is not finite and positive";
        case INTATTN_E_RANGE: return "scales outside the encodable range (index multiplier or output shift)";
        case INTATTN_E_HIP: return "the HIP runtime reported an error";
        case INTATTN_E_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case INTATTN_E_WORKSPACE: return "workspace too small for the shape, or not 256-byte aligned";
        case INTATTN_E_SCRATCH: return "the shape needs more device scratch than the library's static scratch holds";
        default: return "unknown status";
    }
}
