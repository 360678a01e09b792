// Host check of the kernels' integer division (ia_intdiv.h), compiled with
// g++ by tests/test_intdiv.py. Prints "ok" when every check passes.
//   1. the reciprocal for every normalised divisor in [2^31, 2^32);
//   2. the row reciprocals the kernels take, for every row sum E in
//      [1, 2^31): floor((255*2^23 + floor(E/2)) / E) and
//      floor((65535*2^16 + floor(E/2)) / E), by the general division, and
//      by the 24-bit row division (udiv_row) for every E in [2^14, 2^31);
//   3. quotient and remainder on edge cases and 2*10^7 seeded random pairs;
//   4. division by launch-invariant divisors (every divisor below 2^16 and
//      random larger ones) for dividends below 2^31.
#include <atomic>
#include <cstdio>
#include <random>
#include <thread>
#include <vector>

#include "ia_intdiv.h"

static std::atomic<long> g_bad{0};

static void report(const char* what, unsigned long long a, unsigned long long b, unsigned long long got,
                   unsigned long long want) {
    if (g_bad++ < 8) std::printf("%s: %llu %llu got %llu want %llu\n", what, a, b, got, want);
}

template <class F>
static void parallel(unsigned long long lo, unsigned long long hi, F f) {
    const int T = 8;
    std::vector<std::thread> th;
    const unsigned long long n = hi - lo;
    for (int t = 0; t < T; ++t)
        th.emplace_back([=] { for (unsigned long long x = lo + n * t / T; x < lo + n * (t + 1) / T; ++x) f(x); });
    for (auto& x : th) x.join();
}

int main() {
    parallel(1ull << 31, 1ull << 32, [](unsigned long long d) {
        const unsigned __int128 all = ~static_cast<unsigned __int128>(0) >> 64;   // 2^64 - 1
        const unsigned long long want = static_cast<unsigned long long>(all / d) - (1ull << 32);
        const uint32_t got = ia::intdiv_reciprocal(static_cast<uint32_t>(d));
        if (got != want) report("reciprocal", d, 0, got, want);
    });
    parallel(1, 1ull << 31, [](unsigned long long E) {
        const uint32_t e = static_cast<uint32_t>(E);
        const uint32_t n8 = (255u << 23) + (e >> 1);
        const ia::UDivMod a = ia::udivmod32(n8, e);
        if (a.q != n8 / e || a.r != n8 % e) report("uint8 reciprocal", n8, e, a.q, n8 / e);
        const ia::UDivMod b = ia::udivmod32(0xFFFF0000u, e);
        const unsigned long long want16 = (0xFFFF0000ull + (e >> 1)) / e;
        const unsigned long long got16 = b.q + (b.r + (e >> 1) >= e ? 1u : 0u);
        if (got16 != want16) report("uint16 reciprocal", e, 0, got16, want16);
        if (e >= (1u << 14)) {   // the 24-bit row division's range
            const uint32_t r8 = ia::udiv_row(n8, e);
            if (r8 != n8 / e) report("row division, uint8", n8, e, r8, n8 / e);
            const uint32_t r16 = ia::udiv_row(0xFFFF0000u, e);
            if (r16 != 0xFFFF0000u / e) report("row division, uint16", e, 0, r16, 0xFFFF0000u / e);
        }
    });
    const uint32_t edge[] = {0u, 1u, 2u, 3u, 7u, 255u, 256u, 32767u, 32768u, 32640u, 65535u, 65536u,
                             0x7fffffffu, 0x80000000u, 0x80000001u, 0xfffffffeu, 0xffffffffu};
    for (uint32_t n : edge)
        for (uint32_t d : edge) {
            if (d == 0) continue;
            const ia::UDivMod a = ia::udivmod32(n, d);
            if (a.q != n / d || a.r != n % d) report("edge", n, d, a.q, n / d);
        }
    // invariant divisors: every d below 2^16 and random larger ones, each
    // with dividends at the ends of [0, 2^31) and at multiples of d +- 1
    std::mt19937_64 rng(20261203);
    auto check_inv = [&](uint32_t d) {
        const ia::InvariantDiv v = ia::invariant_div(d);
        auto one = [&](uint32_t n) {
            const ia::UDivMod a = ia::divmod_invariant(n, v);
            if (a.q != n / d || a.r != n % d) report("invariant", n, d, a.q, n / d);
        };
        one(0); one(1); one(0x7fffffffu); one(0x7ffffffeu);
        for (uint32_t k : {1u, 2u, 3u, 1000u, 0x7fffffffu / d}) {
            const uint64_t x = uint64_t(k) * d;
            for (int64_t e = -1; e <= 1; ++e)
                if (int64_t(x) + e >= 0 && int64_t(x) + e < (int64_t(1) << 31)) one(uint32_t(int64_t(x) + e));
        }
        for (int i = 0; i < 8; ++i) one(static_cast<uint32_t>(rng()) >> 1);
    };
    for (uint32_t d = 1; d < 65536; ++d) check_inv(d);
    for (int i = 0; i < 200000; ++i) check_inv((static_cast<uint32_t>(rng()) >> (rng() % 31)) | 1u);
    check_inv(0x7fffffffu); check_inv(0x80000000u); check_inv(0xffffffffu);

    for (int i = 0; i < 20000000; ++i) {
        const uint64_t w = rng();
        const uint32_t n = static_cast<uint32_t>(w);
        uint32_t d = static_cast<uint32_t>(w >> 32) >> (rng() % 32);   // divisors of every size
        if (d == 0) d = 1;
        const ia::UDivMod a = ia::udivmod32(n, d);
        if (a.q != n / d || a.r != n % d) report("random", n, d, a.q, n / d);
    }
    if (g_bad == 0) std::printf("ok\n");
    return g_bad == 0 ? 0 : 1;
}
