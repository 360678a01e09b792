// Host-only driver for the library's C entry points, built by
// tests/test_host_sanitizers.py with g++ -fsanitize=address,undefined from
// the library's own host sources (intattn_host.cpp, intattn_api.cpp). The
// device launchers are replaced by the stubs below, which record which
// kernel family the dispatch picked and touch no memory, so every path of
// argument validation, parameter derivation and kernel choice runs on the CPU
// under the sanitizers.
//
// Input (stdin): one parameter set a line, "D s_q s_k s_v s_o clip lut_size
// prob_bits lut_bits" (floats as hexadecimal or decimal); output: one line per
// set, "status M x_clip req_shift req_mul lut[0..lut_size-1]", for the test to
// compare with the oracle. Then the built-in validation and dispatch checks
// run; the last line is "ok" when every one passed.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <string>

#include "intattn.h"
#include "intattn_internal.h"

// ---- launcher stubs (test only: the real ones are HIP code) -------------------
static std::string g_last;   // kernel family of the last launch
static int g_launches = 0;

static int stub(const char* name) {
    g_last = name;
    ++g_launches;
    return INTATTN_OK;
}

namespace ia {
void clear_pending_hip_error() {}
int launch_general(const int8_t*, const int8_t*, const int8_t*, int8_t*, int, const IaKernelParams&, void*,
                   int32_t*, uint32_t*, uint8_t*) {
    return stub("general");
}
int short_max_keys(int D) { return D == 64 ? 512 : 256; }
int launch_short(const int8_t*, const int8_t*, const int8_t*, int8_t*, int, const IaKernelParams&, void*, int32_t*,
                 uint32_t*) {
    return stub("short");
}
int decode_max_keys() { return 16384; }
size_t decode_split_workspace_bytes(long long heads, int Skv, int) {
    return static_cast<size_t>(heads) * static_cast<size_t>(Skv) * 8u + 4096u;
}
int launch_decode_split(const int8_t*, const int8_t*, const int8_t*, int8_t*, int, const IaKernelParams&, void*,
                        void*, int32_t*, uint32_t*) {
    return stub("split");
}
int launch_decode(const int8_t*, const int8_t*, const int8_t*, int8_t*, int, const IaKernelParams&, void*,
                  int32_t*, uint32_t*) {
    return stub("decode");
}
int launch_long(const int8_t*, const int8_t*, const int8_t*, int8_t*, int, const IaKernelParams&, void*, int32_t*,
                uint32_t*) {
    return stub("long");
}
int launch_kv_append(const float*, const float*, int8_t*, int8_t*, int, int, int, int, int, int, float, float,
                     void*) {
    return stub("kv_append");
}
int stage_max_keys() { return 4096; }
int launch_qk_scores(const int8_t*, const int8_t*, int32_t*, int, const IaKernelParams&, void*) {
    return stub("qk");
}
int launch_index_softmax(const int32_t*, uint8_t*, int32_t*, uint32_t*, const IaKernelParams&, void*) {
    return stub("isoftmax");
}
int launch_fp_softmax(const int32_t*, uint8_t*, float, const IaKernelParams&, void*) { return stub("fpsoftmax"); }
int launch_pv(const uint8_t*, const int8_t*, int8_t*, int, const IaKernelParams&, void*) { return stub("pv"); }
}  // namespace ia

// ---- checks -------------------------------------------------------------------
static int g_fail = 0;

static void expect(bool ok, const char* what, int line) {
    if (!ok) {
        ++g_fail;
        std::printf("FAIL line %d: %s\n", line, what);
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// Fake device addresses: never dereferenced (the launchers are stubs).
static const int8_t* const Q = reinterpret_cast<const int8_t*>(0x100000);
static const int8_t* const K = reinterpret_cast<const int8_t*>(0x200000);
static const int8_t* const V = reinterpret_cast<const int8_t*>(0x300000);
static int8_t* const O = reinterpret_cast<int8_t*>(0x400000);

static int fwd(intattn_shape s, intattn_scales sc, float clip = 6.2344107f, int causal = 0,
               const int8_t* q = Q, int8_t* o = O) {
    g_last.clear();
    return intattn_forward(q, K, V, o, &s, &sc, clip, causal, nullptr);
}

static void validation_checks() {
    const intattn_scales ok{0.05f, 0.05f, 0.05f, 0.05f};
    const float inf = std::numeric_limits<float>::infinity();
    const float nan = std::numeric_limits<float>::quiet_NaN();
    const int before = g_launches;
    EXPECT(fwd({1, 1, 8, 0, 64}, ok) == INTATTN_E_SHAPE);
    EXPECT(fwd({1, 1, 8, 65536, 64}, ok) == INTATTN_E_SHAPE);
    EXPECT(fwd({-1, 1, 8, 8, 64}, ok) == INTATTN_E_SHAPE);
    EXPECT(fwd({1, 1, 9, 8, 64}, ok, 6.2344107f, 1) == INTATTN_E_SHAPE);
    EXPECT(fwd({1 << 30, 1 << 30, 8, 8, 64}, ok) == INTATTN_E_SHAPE);
    EXPECT(fwd({1, 1, 8, 8, 96}, ok) == INTATTN_E_DIM);
    EXPECT(fwd({1, 1, 8, 8, 64}, ok, 6.2344107f, 0, nullptr) == INTATTN_E_NULL);
    EXPECT(fwd({1, 1, 8, 8, 64}, ok, 6.2344107f, 0, Q + 1) == INTATTN_E_ALIGN);
    EXPECT(fwd({1, 1, 8, 8, 64}, ok, 6.2344107f, 0, Q, O + 8) == INTATTN_E_ALIGN);
    for (float bad : {0.0f, -1.0f, inf, nan}) {
        EXPECT(fwd({1, 1, 8, 8, 64}, {bad, 0.05f, 0.05f, 0.05f}) == INTATTN_E_SCALE);
        EXPECT(fwd({1, 1, 8, 8, 64}, {0.05f, 0.05f, 0.05f, bad}) == INTATTN_E_SCALE);
        EXPECT(fwd({1, 1, 8, 8, 64}, ok, bad) == INTATTN_E_CLIP);
    }
    EXPECT(fwd({1, 1, 8, 8, 64}, {0.05f, 0.05f, 1e-30f, 1.0f}) == INTATTN_E_RANGE);
    EXPECT(intattn_forward(Q, K, V, O, nullptr, &ok, 6.2f, 0, nullptr) == INTATTN_E_NULL);
    EXPECT(intattn_forward(Q, K, V, O, nullptr, nullptr, 6.2f, 0, nullptr) == INTATTN_E_NULL);
    intattn_shape s{1, 1, 8, 8, 64};
    int32_t rm = 0;
    uint32_t rs = 0;
    EXPECT(intattn_forward_debug(Q, K, V, O, &s, &ok, 6.2f, 0, nullptr, nullptr, &rs, nullptr) == INTATTN_E_NULL);
    EXPECT(intattn_forward_debug(Q, K, V, O, &s, &ok, 6.2f, 0, nullptr, &rm, nullptr, nullptr) == INTATTN_E_NULL);
    // variants
    intattn_variant var{};
    var.lut_size = 48;
    EXPECT(intattn_forward_ex(Q, K, V, O, &s, &ok, 6.2f, 0, &var, nullptr, nullptr, nullptr) == INTATTN_E_RANGE);
    var = intattn_variant{};
    var.kv_heads = 3;
    intattn_shape s4{1, 4, 8, 8, 64};
    EXPECT(intattn_forward_ex(Q, K, V, O, &s4, &ok, 6.2f, 0, &var, nullptr, nullptr, nullptr) == INTATTN_E_SHAPE);
    var = intattn_variant{};
    var.kv_capacity = 7;
    EXPECT(intattn_forward_ex(Q, K, V, O, &s, &ok, 6.2f, 0, &var, nullptr, nullptr, nullptr) == INTATTN_E_SHAPE);
    var = intattn_variant{};
    var.prob_bits = 12;
    EXPECT(intattn_forward_ex(Q, K, V, O, &s, &ok, 6.2f, 0, &var, nullptr, nullptr, nullptr) == INTATTN_E_RANGE);
    var = intattn_variant{};
    var.lut_bits = 4;
    EXPECT(intattn_forward_ex(Q, K, V, O, &s, &ok, 6.2f, 0, &var, nullptr, nullptr, nullptr) == INTATTN_E_RANGE);
    EXPECT(intattn_forward_ex(Q, K, V, O, &s, &ok, 6.2f, 0, nullptr, nullptr, &rm, nullptr) == INTATTN_E_NULL);
    // workspace too small or misaligned for a split decode shape
    intattn_shape sd{1, 4, 1, 20000, 128};
    const uint64_t need = intattn_workspace_bytes(&sd, nullptr);
    EXPECT(need > 0);
    var = intattn_variant{};
    var.workspace = reinterpret_cast<void*>(0x10000);
    var.workspace_bytes = need - 1;
    EXPECT(intattn_forward_ex(Q, K, V, O, &sd, &ok, 6.2f, 0, &var, nullptr, nullptr, nullptr) ==
           INTATTN_E_WORKSPACE);
    var.workspace = reinterpret_cast<void*>(0x10010);
    var.workspace_bytes = need;
    EXPECT(intattn_forward_ex(Q, K, V, O, &sd, &ok, 6.2f, 0, &var, nullptr, nullptr, nullptr) ==
           INTATTN_E_WORKSPACE);
    // stages
    int32_t* sc32 = reinterpret_cast<int32_t*>(0x500000);
    uint8_t* pr = reinterpret_cast<uint8_t*>(0x600000);
    EXPECT(intattn_qk_scores(nullptr, K, sc32, &s, nullptr) == INTATTN_E_NULL);
    EXPECT(intattn_qk_scores(Q, K, sc32 + 0, nullptr, nullptr) == INTATTN_E_NULL);
    EXPECT(intattn_qk_scores(Q, K, reinterpret_cast<int32_t*>(0x500002), &s, nullptr) == INTATTN_E_ALIGN);
    intattn_shape sl{1, 1, 8, 4097, 64};
    EXPECT(intattn_index_softmax(sc32, pr, nullptr, nullptr, &sl, &ok, 6.2f, 0, nullptr) == INTATTN_E_SHAPE);
    EXPECT(intattn_fp_softmax(sc32, pr, &sl, &ok, 0, nullptr) == INTATTN_E_SHAPE);
    EXPECT(intattn_index_softmax(sc32, pr, &rm, nullptr, &s, &ok, 6.2f, 0, nullptr) == INTATTN_E_NULL);
    EXPECT(intattn_fp_softmax(sc32, pr, &s, &ok, 1, nullptr) == INTATTN_OK);
    intattn_shape sc9{1, 1, 9, 8, 64};
    EXPECT(intattn_fp_softmax(sc32, pr, &sc9, &ok, 1, nullptr) == INTATTN_E_SHAPE);
    EXPECT(intattn_pv(pr, V, O, &s, &ok, nan, 0, nullptr) == INTATTN_E_CLIP);
    EXPECT(intattn_pv(pr, V + 1, O, &s, &ok, 6.2f, 0, nullptr) == INTATTN_E_ALIGN);
    // cache update
    const float* f = reinterpret_cast<const float*>(0x700000);
    int8_t* kc = reinterpret_cast<int8_t*>(0x800000);
    int8_t* vc = reinterpret_cast<int8_t*>(0x900000);
    EXPECT(intattn_kv_append(nullptr, f, kc, vc, 1, 1, 1, 64, 8, 0, 0.1f, 0.1f, nullptr) == INTATTN_E_NULL);
    EXPECT(intattn_kv_append(f, f, kc, vc, 1, 1, 2, 64, 8, 7, 0.1f, 0.1f, nullptr) == INTATTN_E_SHAPE);
    EXPECT(intattn_kv_append(f, f, kc, vc, 1, 1, 1, 64, 65536, 0, 0.1f, 0.1f, nullptr) == INTATTN_E_SHAPE);
    EXPECT(intattn_kv_append(f, f, kc, vc, 1, 1, 1, 80, 8, 0, 0.1f, 0.1f, nullptr) == INTATTN_E_DIM);
    EXPECT(intattn_kv_append(f, f, kc, vc, 1, 1, 1, 64, 8, 0, nan, 0.1f, nullptr) == INTATTN_E_SCALE);
    EXPECT(intattn_kv_append(f + 1, f, kc, vc, 1, 1, 1, 64, 8, 0, 0.1f, 0.1f, nullptr) == INTATTN_E_ALIGN);
    // host-only helpers
    uint16_t lut[128];
    EXPECT(intattn_build_lut(6.2f, nullptr) == INTATTN_E_NULL);
    EXPECT(intattn_build_lut(-1.0f, lut) == INTATTN_E_CLIP);
    EXPECT(intattn_build_lut_ex(6.2f, 48, 16, lut) == INTATTN_E_RANGE);
    EXPECT(intattn_build_lut_ex(6.2f, 32, 12, lut) == INTATTN_E_RANGE);
    intattn_params p{};
    EXPECT(intattn_derive_params(&s, &ok, 6.2f, nullptr) == INTATTN_E_NULL);
    EXPECT(intattn_derive_params(nullptr, &ok, 6.2f, &p) == INTATTN_E_NULL);
    // only the one valid fp_softmax call above launched anything
    EXPECT(g_launches == before + 1);
}

static void dispatch_checks() {
    const intattn_scales ok{0.05f, 0.05f, 0.05f, 0.05f};
    struct Case {
        intattn_shape s;
        int causal;
        const char* kernel;
    };
    const Case cases[] = {
        {{8, 12, 512, 512, 64}, 0, "short"},   {{32, 12, 197, 197, 64}, 0, "short"},
        {{1, 2, 256, 256, 128}, 1, "short"},   {{1, 2, 257, 257, 128}, 1, "long"},
        {{1, 32, 4096, 4096, 128}, 1, "long"}, {{16, 32, 1, 8192, 128}, 0, "decode"},
        {{2, 3, 1, 16384, 128}, 0, "decode"},  {{1, 2, 1, 16385, 64}, 1, "decode"},
        {{1, 1, 513, 513, 64}, 0, "long"},
    };
    for (const Case& c : cases) {
        const int st = fwd(c.s, ok, 6.2344107f, c.causal);
        EXPECT(st == INTATTN_OK);
        if (g_last != c.kernel) {
            ++g_fail;
            std::printf("FAIL dispatch B=%d H=%d Sq=%d Skv=%d D=%d: %s, want %s\n", c.s.B, c.s.H, c.s.Sq, c.s.Skv,
                        c.s.D, g_last.c_str(), c.kernel);
        }
    }
    // empty problems launch nothing
    const int before = g_launches;
    EXPECT(fwd({0, 12, 512, 512, 64}, ok) == INTATTN_OK);
    EXPECT(fwd({2, 3, 0, 7, 128}, ok, 6.2344107f, 1) == INTATTN_OK);
    EXPECT(g_launches == before);
    // a workspace routes long and few-heads decode to the split kernels
    intattn_shape sd{2, 32, 1, 65535, 128};
    intattn_variant var{};
    var.workspace = reinterpret_cast<void*>(0x1000000);
    var.workspace_bytes = intattn_workspace_bytes(&sd, &var);
    g_last.clear();
    EXPECT(intattn_forward_ex(Q, K, V, O, &sd, &ok, 6.2f, 0, &var, nullptr, nullptr, nullptr) == INTATTN_OK);
    EXPECT(g_last == "split");
    g_last.clear();
    EXPECT(intattn_forward(Q, K, V, O, &sd, &ok, 6.2f, 0, nullptr) == INTATTN_OK);
    EXPECT(g_last == "decode");   // no workspace: the three-pass decode kernel
    // the debug entry point with probabilities runs the general kernel
    intattn_shape s{1, 1, 8, 8, 64};
    int32_t* rm = reinterpret_cast<int32_t*>(0xa00000);
    uint32_t* rs = reinterpret_cast<uint32_t*>(0xb00000);
    uint8_t* pr = reinterpret_cast<uint8_t*>(0xc00000);
    g_last.clear();
    EXPECT(intattn_forward_debug(Q, K, V, O, &s, &ok, 6.2f, 0, nullptr, rm, rs, pr) == INTATTN_OK);
    EXPECT(g_last == "general");
    for (int code = 1; code >= -12; --code) EXPECT(intattn_strerror(code) != nullptr && intattn_strerror(code)[0]);
}

static float parse_float(const char* tok) { return std::strtof(tok, nullptr); }

int main() {
    char line[512];
    while (std::fgets(line, sizeof line, stdin)) {
        char* tok[9];
        int n = 0;
        for (char* t = std::strtok(line, " \t\r\n"); t && n < 9; t = std::strtok(nullptr, " \t\r\n")) tok[n++] = t;
        if (n != 9) continue;
        intattn_shape s{1, 1, 1, 1, std::atoi(tok[0])};
        intattn_scales sc{parse_float(tok[1]), parse_float(tok[2]), parse_float(tok[3]), parse_float(tok[4])};
        intattn_params_ex p{};
        const int st = intattn_derive_params_ex(&s, &sc, parse_float(tok[5]), std::atoi(tok[6]), std::atoi(tok[7]),
                                                std::atoi(tok[8]), &p);
        std::printf("%d %d %d %d %lld", st, p.idx_mul, p.x_clip, p.req_shift, static_cast<long long>(p.req_mul));
        if (st == INTATTN_OK)
            for (int i = 0; i < p.lut_size; ++i) std::printf(" %u", static_cast<unsigned>(p.lut[i]));
        std::printf("\n");
    }
    validation_checks();
    dispatch_checks();
    std::printf(g_fail == 0 ? "ok\n" : "failed %d\n", g_fail);
    return g_fail == 0 ? 0 : 1;
}
