// Unsigned integer division without floating point, for device and host.
//
// The compiler lowers an integer division by a run-time value to a sequence
// built on the float reciprocal unit. The kernels of this library divide with
// the routines below instead, so that their instruction stream stays
// integer-only, as the method requires of the whole attention path.
//
// Method: normalise the divisor (top bit set), compute its reciprocal
// v = floor((2^64 - 1) / d) - 2^32 by Newton-Raphson from the linear start
// 48/17 - 32/17 x (relative error at most 1/17 on [1/2, 1)), three steps
// with the error term scaled to its expected size, then make v exact with one
// check in each direction; divide with the two-by-one reciprocal step of
// Moller and Granlund, "Improved division by invariant integers" (IEEE
// Transactions on Computers 60(2), 2011), Algorithm 4. The reciprocal is
// checked against exact division for every normalised divisor on the host.
//
// Plain constexpr C++ on 32- and 64-bit integers: HIP compiles it for the
// device, and the host test compiles the same text with g++.
#pragma once

#include <cstdint>

namespace ia {

// v = floor((2^64 - 1) / dn) - 2^32 for dn in [2^31, 2^32).
constexpr uint32_t intdiv_reciprocal(uint32_t dn) {
    // z ~ 2^63 / dn in (2^31, 2^32]: 48/17 - 32/17 x at x = dn / 2^32, in Q31
    const uint64_t c48 = 6063298184ull;   // round(48/17 * 2^31)
    const uint64_t c32 = 4042198789ull;   // round(32/17 * 2^31)
    const uint64_t z0 = c48 - ((c32 * (dn >> 16)) >> 16);
    // Newton-Raphson z' = z + z e / 2^63 with e = 2^63 - dn z; |e| shrinks
    // from below 2^59 to below 2^55 and 2^47, so each step shifts e to about
    // 28 bits before the product (which stays below 2^61)
    const int64_t e0 = static_cast<int64_t>((uint64_t(1) << 63) - uint64_t(dn) * z0);
    const uint64_t z1 =
        static_cast<uint64_t>(static_cast<int64_t>(z0) + ((static_cast<int64_t>(z0) * (e0 >> 31)) >> 32));
    const int64_t e1 = static_cast<int64_t>((uint64_t(1) << 63) - uint64_t(dn) * z1);
    const uint64_t z2 =
        static_cast<uint64_t>(static_cast<int64_t>(z1) + ((static_cast<int64_t>(z1) * (e1 >> 27)) >> 36));
    const int64_t e2 = static_cast<int64_t>((uint64_t(1) << 63) - uint64_t(dn) * z2);
    // last step in Q32: y = 2^64 / dn ~ 2 z2 (1 + e2 / 2^63); it lands within
    // [-2, 0] of floor((2^64 - 1) / dn), so +1 centres it on [-1, 1]
    const uint64_t y = 2 * z2 + static_cast<uint64_t>((static_cast<int64_t>(z2) * (e2 >> 19)) >> 43) + 1;
    uint64_t v = y - (uint64_t(1) << 32);
    if (v > 0xffffffffull) v = 0xffffffffull;
    // exact: the largest v with dn (2^32 + v) <= 2^64 - 1
    const uint64_t lim = ((uint64_t(1) << 32) - dn) * (uint64_t(1) << 32) - 1;   // 2^64 - 1 - dn 2^32
    if (uint64_t(dn) * v > lim) --v;
    if (v < 0xffffffffull && uint64_t(dn) * (v + 1) <= lim) ++v;
    return static_cast<uint32_t>(v);
}

struct UDivMod {
    uint32_t q, r;
};

// floor(n / d) and n mod d for d >= 1.
constexpr UDivMod udivmod32(uint32_t n, uint32_t d) {
    const int s = __builtin_clz(d);
    const uint32_t dn = d << s;
    const uint32_t v = intdiv_reciprocal(dn);
    // the two words of n 2^s; u1 < dn
    const uint32_t u1 = s == 0 ? 0u : n >> (32 - s);
    const uint32_t u0 = n << s;
    // two-by-one step with the reciprocal (q1, q0) = v u1 + (u1, u0)
    const uint64_t qq = uint64_t(v) * u1 + ((uint64_t(u1) << 32) | u0);
    uint32_t q1 = static_cast<uint32_t>(qq >> 32) + 1;
    const uint32_t q0 = static_cast<uint32_t>(qq);
    uint32_t r = u0 - q1 * dn;
    if (r > q0) {
        q1 -= 1;
        r += dn;
    }
    if (r >= dn) {
        q1 += 1;
        r -= dn;
    }
    return UDivMod{q1, r >> s};
}

constexpr uint32_t udiv32(uint32_t n, uint32_t d) { return udivmod32(n, d).q; }

// floor(n / d) for the row reciprocals: 2^14 <= d < 2^31, 2^30 <= n < 2^32
// and a quotient below 2^18, on 24-bit multiplies only (full rate on the
// device, where 32-bit multiplies run at a quarter of it). With s = clz(d),
// d24 = (d << s) >> 8 in [2^23, 2^24) and n24 = n >> 8, the quotient is about
// n24 2^s / d24. x approaches 2^46 / d24 from below: the start
// (46 - 32 y) / 17 (y = d24 / 2^24 in [1/2, 1)) lies within -3/17 and 0 of
// 1/y, and each Newton-Raphson step x + x (2^46 - d24 x) / 2^46 squares the
// relative error and stays below; three steps leave it under 2^-19. The
// estimate is then within one of the quotient and two checks make it exact.
constexpr uint64_t mul24(uint32_t a, uint32_t b) {   // a, b < 2^24
    return uint64_t(a & 0xffffffu) * (b & 0xffffffu);
}

constexpr uint32_t udiv_row(uint32_t n, uint32_t d) {
    const int s = __builtin_clz(d);
    const uint32_t d24 = (d << s) >> 8;
    uint32_t x = 11222737u - static_cast<uint32_t>(mul24(7895097u, d24) >> 24);   // (46 - 32 y) / 17, Q22
    // steps: e = 2^46 - d24 x >= 0 stays below 2^43.5, 2^41.1 and 2^36.1
    // (relative errors 3/17, (3/17)^2, (3/17)^4); x += x e / 2^46, with e
    // shifted to under 2^24 first
    uint64_t e = (uint64_t(1) << 46) - mul24(d24, x);
    x += static_cast<uint32_t>(mul24(x, static_cast<uint32_t>(e >> 20)) >> 26);
    e = (uint64_t(1) << 46) - mul24(d24, x);
    x += static_cast<uint32_t>(mul24(x, static_cast<uint32_t>(e >> 18)) >> 28);
    e = (uint64_t(1) << 46) - mul24(d24, x);
    x += static_cast<uint32_t>(mul24(x, static_cast<uint32_t>(e >> 13)) >> 33);
    // q ~ n24 x 2^s / 2^46 (s <= 17)
    uint32_t q = static_cast<uint32_t>(mul24(n >> 8, x) >> 29) >> (17 - s);
    const uint64_t p = uint64_t(q) * d;
    if (p > n) --q;
    else if (p + d <= n) ++q;
    return q;
}

// Division by a divisor fixed for a whole launch (block counts, heads per
// group), with a multiplier the host derives once: Granlund and Montgomery,
// "Division by invariant integers using multiplication" (PLDI 1994),
// round-up method for dividends below 2^31. With l = ceil(log2 d) and
// m = floor(2^(31+l) / d) + 1 < 2^32, m d lies in (2^(31+l), 2^(31+l) + 2^l],
// so floor(n m / 2^(31+l)) = floor(n / d) for 0 <= n < 2^31. d = 1 keeps m = 0
// and passes n through.
struct InvariantDiv {
    uint32_t m;      // multiplier; 0 for d = 1
    uint32_t shift;  // l - 1
    uint32_t d;
};

// Host only (it divides once to derive the multiplier).
inline InvariantDiv invariant_div(uint32_t d) {
    if (d <= 1) return InvariantDiv{0u, 0u, 1u};
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << (31 + l)) / d) + 1;
    return InvariantDiv{static_cast<uint32_t>(m), l - 1, d};
}

// floor(n / d) and n mod d for 0 <= n < 2^31.
constexpr UDivMod divmod_invariant(uint32_t n, const InvariantDiv& v) {
    const uint32_t q = v.m == 0 ? n : static_cast<uint32_t>((uint64_t(n) * v.m) >> 32) >> v.shift;
    return UDivMod{q, n - q * v.d};
}

}  // namespace ia
