// Device-side building blocks shared by the integer attention kernels
// (gfx950 / CDNA4): MFMA wrapper, accumulator layout helpers, workgroup
// renumbering and the requantisation step.
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology",
// steps 2-3; integer widths and roundings as stated in include/intattn.h.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "ia_intdiv.h"
#include "intattn_internal.h"

namespace ia {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Wait states around v_mfma_i32_32x32x32_i8 that the compiler inserts only
// between instructions it emits itself (inline asm is opaque to its hazard
// checks): a VALU read of the MFMA's result needs 12 (s_nop 11, what it emits
// before a VALU consumer), and an MFMA reading a VGPR that a VALU op just
// wrote needs 2. These asm statements carry the wait states and are tied to
// the registers by their operands, so they sit after the producer and before
// the consumer: mfma_result_guard where inline asm (the slot word) reads
// fresh scores, mfma_source_guard where an asm-built P operand feeds P.V.
__device__ __forceinline__ void mfma_result_guard(v16i& s) { asm volatile("s_nop 11" : "+v"(s)); }
__device__ __forceinline__ void mfma_result_guard(v16i& s0, v16i& s1) {
    asm volatile("s_nop 11" : "+v"(s0), "+v"(s1));
}
__device__ __forceinline__ void mfma_source_guard(v4i& a) { asm volatile("s_nop 1" : "+v"(a)); }

// S^T tiles: v_mfma_i32_32x32x32_i8 with K as the A operand (rows = keys)
// and Q^T as the B operand (columns = queries). Lane l (l32 = l % 32,
// hh = l / 32) holds the 16 accumulator registers of column l32, i.e. scores
// of a single query row for 16 keys of the 32-key block.
__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Key (relative to its 32-key block) held by accumulator register r of a
// 32x32 MFMA result in lane half hh (lanes 0-31: hh = 0, lanes 32-63: 1).
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

// Byte position of a key of a 32-key block inside a transposed V row, such
// that lane half hh reads its 16 keys (acc_row(0..15, hh)) contiguously; the
// 16 bytes are then the B operand of P.V in the order of the P operand.
__device__ __forceinline__ int vt_pos(int key_in_block) {
    const int a = key_in_block >> 3, h = (key_in_block >> 2) & 1, c = key_in_block & 3;
    return 16 * h + 4 * a + c;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Renumber them so that consecutive logical blocks run on the same XCD.
// Bijective on [0, n): the first 8*floor(n/8) ids are regrouped, the
// remainder is kept.
__device__ __forceinline__ int xcd_local_block(int bid, int n) {
    const int full = n & ~7;
    if (bid >= full) return bid;
    const int per = full >> 3;
    return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; }

// Table index of a score under the row constants: the clip is s' = max(s, lo)
// with lo = m - x_clip, so the gap x' = m - s' is at most x_clip; then
// idx = (x' * tab_mul + tab_half) >> tab_shift, computed as
// (C - s' * tab_mul) mod 2^32 >> tab_shift with C = m * tab_mul + tab_half
// mod 2^32 and negM = -tab_mul (the true value is below 2^31, and every
// operand fits the 24-bit signed multiplier). With (M, 2^23, 24) this is the
// slot (x'*M + 2^23) >> 24, for the exp table by slot; with (1, 0, 0) it is
// x' itself, for the direct table by gap (from mu = 1/2 on).
__device__ __forceinline__ uint32_t slot_of(int32_t s, int32_t lo, uint32_t C, int32_t negM, uint32_t shift) {
    const int32_t sp = max(s, lo);
    return (C + static_cast<uint32_t>(__mul24(sp, negM))) >> shift;
}

// Saturating slot word for a table of N entries: with y = s - m <= 0, a
// scale k (4, 2 or 1, with k <= 128/N and kM < 2^23; the layouts below) and
// negMk = -kM, halfk = k * 2^23, t = sat_int32(y * negMk + halfk) =
// sat(k (x M + 2^23)) has top byte floor(k (x M + 2^23) / 2^24), whose
// quotient by k is the raw slot (x*M + 2^23) >> 24: scaling numerator and
// shift by k keeps the quotient. The value is below 2^31 whenever the raw
// slot is below 128/k, and saturation to 2^31 - 1 gives byte 127, i.e. slot
// 127/k >= N - 1.
__device__ __forceinline__ uint32_t slot_word_sat(int32_t y, int32_t negMk, int32_t halfk) {
    int32_t t;
    asm("v_mad_i32_i24 %0, %1, %2, %3 clamp" : "=v"(t) : "v"(y), "s"(negMk), "v"(halfk));
    return static_cast<uint32_t>(t);
}

// Exp-table layouts in LDS (at byte address 0), chosen by the slot scale
// KM = k, each bank-conflict free on the 64-bank LDS (lanes that read
// different slots never meet in one bank) and addressed from a top byte in
// one SDWA op:
//   KM = 4 (N = 32, 4M < 2^23): u32[32], byte = 4 slot + fraction, address
//          byte & 0x7c;
//   KM = 2 (N <= 64, 2M < 2^23): u16[128], byte = 2 slot + fraction,
//          address byte & 0x7e;
//   KM = 1: u16[128], byte = slot, address 2 * byte.
// u16 entries past slot N - 1 are 0 (the clipped tail); a saturated byte
// (127) always lands on such an entry or on slot N - 1.
//   KM = 0 (from mu = 1/2 on, see entry_addr): u16[256] indexed by the
//          clipped gap itself.
template <int KM>
__device__ __forceinline__ uint32_t lut_byte_addr(uint32_t t) {
    uint32_t a;
    if constexpr (KM == 1) {
        asm("v_lshlrev_b32_sdwa %0, 1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
            : "=v"(a) : "v"(t));
    } else {
        const uint32_t m = KM == 4 ? 0x7cu : 0x7eu;
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
            : "=v"(a) : "v"(t), "s"(m));
    }
    return a;
}

// LDS address of the table entry of a relative score y = s - m <= 0 (a
// masked key has y = -2^23), for layout KM with a = P.ent_a, b = P.ent_b:
//   KM = 4, 2, 1: the top byte of the saturating slot word (a = -kM,
//     b = k 2^23), two VALU ops;
//   KM = 0: from mu = 1/2 on a score unit moves half a bin or more, so the
//     clip point x_clip is at most 2N - 3 units from the row max and the
//     table is indexed by the clipped gap x' = min(-y, x_clip) itself
//     (u16 entries, entry x' = lut[slot(x')], entry x_clip = 0): a = -x_clip,
//     address 2 x' = -2 max(y, a), again two VALU ops.
template <int KM>
__device__ __forceinline__ uint32_t entry_addr(int32_t y, int32_t a, int32_t b) {
    if constexpr (KM == 0) {
        (void)b;
        return static_cast<uint32_t>(__mul24(max(y, a), -2));
    } else {
        return lut_byte_addr<KM>(slot_word_sat(y, a, b));
    }
}

// int32 accumulator -> int8: sign(a) * min(127, (|a|*M_o + 2^(sh_o-1)) >> sh_o).
// One signed product instead of magnitude and sign: with h = 2^(sh-1),
// -floor((|a|M + h) / 2^sh) = floor((aM + 2^sh - 1 - h) / 2^sh) for a < 0, so
// the result is clamp(floor((aM + h + s) / 2^sh), -127, 127) with s = a >> 31
// (0 or -1). M_o < 2^31 and |a| < 2^31 keep |aM + h + s| < 2^63.
__device__ __forceinline__ int8_t requantise(int32_t a, const IaKernelParams& P) {
    const int64_t x = static_cast<int64_t>(a) * static_cast<int32_t>(P.req_mul) +
                      ((int64_t(1) << (P.req_shift - 1)) + (a >> 31));
    const int32_t r = static_cast<int32_t>(max(min(x >> P.req_shift, int64_t(127)), int64_t(-127)));
    return static_cast<int8_t>(r);
}

// The same for shifts sh >= 33: h + s = (2^(sh-33) + s) * 2^32 + (s mod 2^32),
// and floor(x / 2^sh) = floor(hi32(x) / 2^(sh-32)), hi32(x) in (-2^31, 2^31).
// add = 2^(sh-33), rsh = sh - 32.
__device__ __forceinline__ int32_t requantise_hi(int32_t a, uint32_t mul, uint32_t add, uint32_t rsh) {
    const int32_t s = a >> 31;
    const uint64_t c = static_cast<uint64_t>(static_cast<uint32_t>(s)) |
                       (static_cast<uint64_t>(add + static_cast<uint32_t>(s)) << 32);
    const int64_t x = static_cast<int64_t>(a) * static_cast<int32_t>(mul) + static_cast<int64_t>(c);
    const int32_t r = static_cast<int32_t>(static_cast<uint64_t>(x) >> 32) >> rsh;
    return min(max(r, -127), 127);
}

__device__ __forceinline__ int32_t dpp_xor1(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true); }
__device__ __forceinline__ int32_t dpp_xor2(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true); }
__device__ __forceinline__ int32_t dpp_half_mirror(int32_t x) { return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true); }


// f(std::integral_constant<int, i>{}) for i = 0 .. N-1 (compile-time indices).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The packed exp table as one register of the wave: lane i holds argument
// word i (entries 2i and 2i+1). The argument words are wave-uniform (scalar
// registers); writing them lane by lane keeps a per-lane index from turning
// into a vector load of the argument segment (whose wait would also cover any
// loads issued before it).
template <int NW = kIaMaxLut / 2, int OFF = 0>
__device__ __forceinline__ uint32_t lut_words(const IaKernelParams& P) {
    static_assert(NW % 16 == 0 && NW <= 64 && OFF + NW <= kIaTabEntries / 2, "words come in groups of 16");
    uint32_t all = 0;
    // the lane number must be an inline constant (one scalar operand per VOP3)
#define IA_WL(i) asm volatile("v_writelane_b32 %0, %1, " #i : "+v"(all) : "s"(P.lut2[OFF + i]));
    IA_WL(0) IA_WL(1) IA_WL(2) IA_WL(3) IA_WL(4) IA_WL(5) IA_WL(6) IA_WL(7)
    IA_WL(8) IA_WL(9) IA_WL(10) IA_WL(11) IA_WL(12) IA_WL(13) IA_WL(14) IA_WL(15)
    if constexpr (NW > 16) {
        IA_WL(16) IA_WL(17) IA_WL(18) IA_WL(19) IA_WL(20) IA_WL(21) IA_WL(22) IA_WL(23)
        IA_WL(24) IA_WL(25) IA_WL(26) IA_WL(27) IA_WL(28) IA_WL(29) IA_WL(30) IA_WL(31)
    }
    if constexpr (NW > 32) {
        IA_WL(32) IA_WL(33) IA_WL(34) IA_WL(35) IA_WL(36) IA_WL(37) IA_WL(38) IA_WL(39)
        IA_WL(40) IA_WL(41) IA_WL(42) IA_WL(43) IA_WL(44) IA_WL(45) IA_WL(46) IA_WL(47)
        IA_WL(48) IA_WL(49) IA_WL(50) IA_WL(51) IA_WL(52) IA_WL(53) IA_WL(54) IA_WL(55)
        IA_WL(56) IA_WL(57) IA_WL(58) IA_WL(59) IA_WL(60) IA_WL(61) IA_WL(62) IA_WL(63)
    }
#undef IA_WL
    return all;
}

// Exp-table entry idx (0..127) from lut_words: lut[idx] for idx < N, else 0.
// A cross-lane read: every lane of the wave must be active.
__device__ __forceinline__ uint32_t lut_value(const IaKernelParams& P, uint32_t words, int idx) {
    const uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute((idx >> 1) << 2, static_cast<int>(words)));
    const uint32_t e = (w >> (16 * (idx & 1))) & 0xffffu;
    return idx < P.lut_size ? e : 0u;
}

// Fills the u16 table at t (LDS, kIaTabEntries entries) from one whole wave:
// the exp table by slot (entries 0..127; the host leaves entries past N - 1
// zero), and entries 128..255 as well for the direct table (slot_k = 0).
__device__ __forceinline__ void fill_lut_u16(const IaKernelParams& P, uint16_t* t, int lane) {
    uint32_t* t32 = reinterpret_cast<uint32_t*>(t);
    t32[lane] = lut_words<64, 0>(P);
    if (P.slot_k == 0) t32[64 + lane] = lut_words<64, 64>(P);
}

// Fills the table of layout KM (see lut_byte_addr, entry_addr) at LDS t
// (512 bytes) from one whole wave.
template <int KM>
__device__ __forceinline__ void fill_lut_table(const IaKernelParams& P, void* t, int lane) {
    uint32_t* t32 = static_cast<uint32_t*>(t);
    if constexpr (KM == 4) {
        const uint32_t v = lut_value(P, lut_words<16>(P), lane & 31);   // N = 32: words 0..15
        if (lane < 32) t32[lane] = v;
    } else if constexpr (KM == 0) {
        t32[lane] = lut_words<64, 0>(P);
        t32[64 + lane] = lut_words<64, 64>(P);
    } else {
        t32[lane] = lut_words<64, 0>(P);
    }
}


typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;


// LDS tiles of K and V rows (D bytes per row, 16-byte chunks). 16-byte reads
// are served 16 lanes per cycle over 64 four-byte banks, so the 16 rows read
// by one 16-lane phase must land in 16 distinct 16-byte bank groups.
//
// Chunk position of logical chunk c of K row r: c ^ k_swz<D>(r).
template <int D>
__device__ __forceinline__ int k_swz(int r) {
    return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
// Chunk position of logical chunk c of V row (key) r: c ^ v_swz<D>(r); the 8
// keys of one ds_read_b64_tr_b8 (for the P.V operand order below) land in 8
// distinct bank groups.
template <int D>
__device__ __forceinline__ int v_swz(int r) {
    return D == 128 ? ((r & 3) | ((r >> 1) & 4)) : (((r >> 1) & 1) | ((r >> 2) & 2));
}

// s_waitcnt vmcnt(N) for a compile-time N <= 63 (vmcnt bits [3:0] and
// [15:14]; lgkmcnt and expcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
    static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same for a count known only at run time (wave-uniform); a constant
// argument folds to the one s_waitcnt. Counts above 31 wait for everything.
__device__ __forceinline__ void wait_vmcnt(int n) {
#define IA_VMCNT_CASE(N) \
    case N: wait_vmcnt_c<N>(); break;
    switch (n) {
        IA_VMCNT_CASE(0) IA_VMCNT_CASE(1) IA_VMCNT_CASE(2) IA_VMCNT_CASE(3) IA_VMCNT_CASE(4) IA_VMCNT_CASE(5)
        IA_VMCNT_CASE(6) IA_VMCNT_CASE(7) IA_VMCNT_CASE(8) IA_VMCNT_CASE(9) IA_VMCNT_CASE(10) IA_VMCNT_CASE(11)
        IA_VMCNT_CASE(12) IA_VMCNT_CASE(13) IA_VMCNT_CASE(14) IA_VMCNT_CASE(15) IA_VMCNT_CASE(16)
        IA_VMCNT_CASE(17) IA_VMCNT_CASE(18) IA_VMCNT_CASE(19) IA_VMCNT_CASE(20) IA_VMCNT_CASE(21)
        IA_VMCNT_CASE(22) IA_VMCNT_CASE(23) IA_VMCNT_CASE(24) IA_VMCNT_CASE(25) IA_VMCNT_CASE(26)
        IA_VMCNT_CASE(27) IA_VMCNT_CASE(28) IA_VMCNT_CASE(29) IA_VMCNT_CASE(30) IA_VMCNT_CASE(31)
        default: wait_vmcnt_c<0>(); break;
    }
#undef IA_VMCNT_CASE
}

// Workgroup barrier: this wave's LDS operations complete, then all waves
// meet. Outstanding global->LDS loads are not waited for here (the caller
// waits for exactly the loads it needs with wait_vmcnt first).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS byte address of a __shared__ object (its offset in the workgroup's LDS).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)(const_cast<void*>(p))));
}

// 32-bit LDS load from a byte address (the kernel's LDS block starts at 0).
__device__ __forceinline__ uint32_t lds_u32(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(static_cast<uintptr_t>(addr));
}

// 16-bit LDS load (zero-extended) from a byte address.
__device__ __forceinline__ uint32_t lds_u16(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(static_cast<uintptr_t>(addr));
}

// Table entry at a byte address produced by entry_addr<KM>.
template <int KM>
__device__ __forceinline__ uint32_t lut_load(uint32_t addr) {
    if constexpr (KM == 4) return lds_u32(addr);
    else return lds_u16(addr);
}

// Scheduling fence over 16 values: every load feeding them completes here,
// together (one wait for the batch instead of one per value).
__device__ __forceinline__ void pin16(int32_t (&a)[16]) {
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                      "+v"(a[7]), "+v"(a[8]), "+v"(a[9]), "+v"(a[10]), "+v"(a[11]), "+v"(a[12]), "+v"(a[13]),
                      "+v"(a[14]), "+v"(a[15]));
}

// P.V B operand from a row-major V block of 32 keys in LDS (rows of D bytes,
// chunks placed by v_swz): lane (l32, hh) needs V[key(b)][32db + l32] for its
// 16 keys key(b) = acc_row(b, hh), b = 0..15, in that byte order. Two
// ds_read_b64_tr_b8 per 32-column block provide them: within each 16-lane
// group, lane pair (2i, 2i+1) supplies the two 8-byte halves of row key(b)
// (b = i for the first read, 8 + i for the second), and lane j of the group
// receives column j of those 8 rows. tr8_lane_addr gives this lane's byte
// offset from the start of the block for read rd of column block db.
template <int D>
__device__ __forceinline__ uint32_t tr8_lane_addr(int lane, int db, int rd) {
    const int hh = lane >> 5;
    const int i = (lane & 15) >> 1;
    const int key = acc_row(8 * rd + i, hh);
    const int col = 32 * db + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
    return static_cast<uint32_t>(key * D + 16 * ((col >> 4) ^ v_swz<D>(key)) + (col & 15));
}

// One ds_read_b64_tr_b8 at LDS byte address addr + OFF (a compiler builtin,
// so the compiler counts it and places the wait before the first use; OFF is
// applied to the LDS pointer, which lets it fold into the offset field).
template <int OFF>
__device__ __forceinline__ v2i tr8_read(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
    typedef __attribute__((address_space(3))) char lds_char;
    const lds_char* p = reinterpret_cast<const lds_char*>(static_cast<uintptr_t>(addr)) + OFF;
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        reinterpret_cast<__attribute__((address_space(3))) v2i*>(const_cast<lds_char*>(p)));
}

// All 2*DB transpose reads of one key block at LDS byte addresses va[i] + OFF;
// vb[db] is the B operand of column block db.
template <int DB, int OFF>
__device__ __forceinline__ void tr8_operands(const uint32_t (&va)[2 * DB], v4i (&vb)[DB]) {
    static_assert(DB == 2 || DB == 4, "column blocks per head: 2 (d = 64) or 4 (d = 128)");
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const v2i r0 = tr8_read<OFF>(va[2 * db]);
        const v2i r1 = tr8_read<OFF>(va[2 * db + 1]);
        vb[db] = v4i{r0[0], r0[1], r1[0], r1[1]};
    }
}

// Top byte of the probability word: for a table entry e <= E and R2 = 2R,
// e * R2 + 2^23 < 2^32, so the top byte of e * R2 + 2^23 is
// p = (e * R + 2^22) >> 23, and adding 2^31 flips its top bit: the byte is
// p ^ 0x80, i.e. p - 128 as int8.
__device__ __forceinline__ uint32_t prob_word(uint32_t e, uint32_t R2) { return __umul24(e, R2) + 0x80800000u; }

// P operand word (p - 128 as int8 for four keys) from two words that each
// hold two table entries e (bits 0..15 and 16..31), for a row reciprocal
// R < 2^16 and p <= 255. With x = e * R + 2^22 + 2^30
// (< 2^32; v_mad_u32_u16, op_sel picking the entry's half), bits 23..30 of
// x are p ^ 0x80 for p = (e * R + 2^22) >> 23: adding 2^30 adds 128 to
// x >> 23 and leaves nothing below bit 23 changed. Each byte is shifted into
// place by an SDWA byte write that keeps the other bytes, so one key costs
// two VALU ops and no table read.
__device__ __forceinline__ uint32_t prob_bytes4(uint32_t pw0, uint32_t pw1, uint32_t R) {
    const uint32_t c = (1u << 22) + (1u << 30);
    uint32_t x0, x1, x2, x3;
    asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(x0) : "v"(pw0), "v"(R), "s"(c));
    asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(x1) : "v"(pw0), "v"(R), "s"(c));
    asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(x2) : "v"(pw1), "v"(R), "s"(c));
    asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(x3) : "v"(pw1), "v"(R), "s"(c));
    uint32_t d = x0 >> 23;             // byte 0 (bit 8 is overwritten below)
    asm("v_lshrrev_b32_sdwa %0, 23, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(x1));
    asm("v_lshrrev_b32_sdwa %0, 23, %1 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(x2));
    asm("v_lshrrev_b32_sdwa %0, 23, %1 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(x3));
    return d;
}

// Two table entries (each < 2^16) in one word: a in bits 0..15, b above.
__device__ __forceinline__ uint32_t entry_pair(uint32_t a, uint32_t b) { return a | (b << 16); }

// Top bytes of four words packed into one (byte i from word i).
__device__ __forceinline__ uint32_t pack_top_bytes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0703u);
    const uint32_t hi = __builtin_amdgcn_perm(w3, w2, 0x07030c0cu);
    return lo | hi;
}

// uint16 probabilities: the word e * R16 + 2^15 + 2^31 holds p in bits
// 16..31 with the top bit flipped (e * R16 + 2^15 < 2^32, so adding 2^31
// flips bit 31 alone): byte 3 is (p >> 8) ^ 0x80, byte 2 is p & 0xff.
__device__ __forceinline__ uint32_t prob16_word(uint32_t e, uint32_t R16) { return __umul24(e, R16) + 0x80008000u; }

// Bytes 3 and 2 of four words: hi = their bytes 3, lo = their bytes 2 (in
// word order), four v_perm.
__device__ __forceinline__ void pack_bytes_32(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t& hi,
                                              uint32_t& lo) {
    const uint32_t a = __builtin_amdgcn_perm(w1, w0, 0x07030602u);   // w0.b2 w1.b2 w0.b3 w1.b3
    const uint32_t b = __builtin_amdgcn_perm(w3, w2, 0x07030602u);   // w2.b2 w3.b2 w2.b3 w3.b3
    lo = __builtin_amdgcn_perm(b, a, 0x05040100u);
    hi = __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Every row that exists has E >= 128 * 255 (its max key alone contributes the
// first table entry, 2^15 or 128 * 255), so the row reciprocals below take
// E at least that (a row that does not exist, and is never stored, may have
// E = 0) and divide with the 24-bit row division.
constexpr uint32_t kRowSumMin = 128u * 255u;

// Row reciprocal R = floor((255 * 2^23 + floor(E/2)) / E) for E < 2^31 (the
// numerator stays below 2^32), by integer division.
__device__ __forceinline__ uint32_t reciprocal8(uint32_t E) {
    const uint32_t e = max(E, kRowSumMin);
    return udiv_row((255u << 23) + (e >> 1), e);
}

// R16 = floor((65535 * 2^16 + floor(E/2)) / E) (below 2^18 for E >= 128*255,
// a 24-bit operand): with 65535 * 2^16 = q E + r, adding floor(E/2) < E
// carries into the quotient at most once.
__device__ __forceinline__ uint32_t reciprocal16(uint32_t E) {
    const uint32_t e = max(E, kRowSumMin);
    const uint32_t q = udiv_row(0xFFFF0000u, e);
    const uint32_t r = 0xFFFF0000u - q * e;
    return q + (r + (e >> 1) >= e ? 1u : 0u);
}

}  // namespace ia
