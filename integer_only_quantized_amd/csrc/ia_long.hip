// Long-row integer attention kernel (gfx950 / CDNA4): key/value tiles
// streamed into LDS by asynchronous global->LDS loads, three exact passes per
// query block. Used for rows longer than the short-row kernel holds (e.g.
// causal prefill at S = 4096).
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology",
// steps 2-3; integer widths and roundings as stated in include/intattn.h.
//
// Structure:
//   * one workgroup = 4 waves = 128 query rows of one (b, h); in the row-sum
//     and P.V passes each wave owns 32 rows, holds their Q fragments, and
//     produces S^T blocks (32 keys x 32 queries) on v_mfma_i32_32x32x32_i8,
//     so each lane holds one row; in the row-max pass each wave takes 64
//     rows and one of the tile's two key blocks;
//   * keys and values arrive in tiles of 64 rows through an LDS ring filled
//     by global_load_lds_dwordx4 (no register staging). The P.V pass uses
//     three K+V stages: tile t+2 is requested while tile t is computed, and
//     only tile t+1 is waited for (s_waitcnt vmcnt) before the per-tile
//     barrier. The two passes over K alone use the V stages as well (six K
//     stages): two tiles between barriers, loads four tiles ahead;
//   * LDS reads are bank-conflict free on the 64-bank LDS (16 lanes per
//     cycle for 16-byte reads): K rows have their 16-byte chunks XOR-swizzled
//     by the row; V rows stay row-major (chunks swizzled by the key) and the
//     P.V B operand (16 keys of one value column) comes from two
//     ds_read_b64_tr_b8 transpose reads;
//   * the row max must be known before any slot and the row sum before any
//     probability, so there are three passes over the tiles with Q.K^T
//     recomputed in each: (1) row max; (2) the MFMA accumulator is seeded
//     with -m, so it yields y = s - m directly; a clamped 24-bit
//     multiply-add turns y into the slot word, whose top byte addresses the
//     shared exp table; the entries are summed into E; (3) the same table
//     entry e gives the probability byte arithmetically: the top byte of
//     e * 2R + 2^23 + 2^31 (mod 2^32) is p XOR 0x80, i.e. p - 128 as int8,
//     which is the P operand of P.V (with uint8 P the tile's two key blocks
//     are interleaved: one block's MFMAs run under the other's integer
//     work). The +128 * colsum(V) correction is summed from the same B
//     operands, each tile by one wave in turn;
//   * rows past Skv read in-bounds bytes of the last valid row; their scores
//     are masked to p = 0, and since colsum covers exactly the rows fed,
//     their values cancel: sum (p - 128) v + 128 sum v = sum p v;
//   * causal workgroups are dispatched heaviest first, and when the head
//     count allows, every XCD owns a fixed subset of heads (L2 locality).
// Slot word, y = s - m in [-2^23, 0], for a table of N entries (32, or a
// finer 64 or 128): t = sat(y * -kM + k * 2^23) with k = 4 (N = 32,
// 4M < 2^23), 2 (N <= 64, 2M < 2^23) or 1; byte 3 is k * slot + fraction
// bits (127 when saturated), and the table layout KM = k in LDS is
// addressed from it in one SDWA op (u32[32]: byte & 0x7c; u16[128]:
// byte & 0x7e or 2 * byte).
#include <type_traits>

#include "ia_device.h"
#include "ia_launch.h"

namespace ia {
namespace {

constexpr int kLongWaves = 4;
constexpr int kLongRows = 32 * kLongWaves;   // query rows per workgroup
constexpr int kLongTile = 64;                // keys per tile
constexpr int kStages = 3;                   // LDS ring depth
// Table words in LDS for layout KM: 64 (u32[32] or u16[128]), 128 for the
// direct table (u16[256]).
constexpr int table_words(int KM) { return KM == 0 ? kIaTabEntries / 2 : kIaMaxLut / 2; }

template <int D, int KM>
struct LongLds {
    static constexpr int TB = kLongTile * D;        // bytes per K or V tile
    uint32_t lut[table_words(KM)];                  // exp table (layout KM); first member: LDS address 0
    int32_t colsum[kLongWaves][D];
    int8_t k[kStages][TB];
    int8_t v[kStages][TB];
};

template <int D, int KM, bool P16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(P16 ? 2 : 3))) void ia_long_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int nqb, InvariantDiv map_div, int32_t* __restrict__ row_max,
    uint32_t* __restrict__ row_sum) {
    using L = LongLds<D, KM>;
    constexpr int KS = D / 32;
    constexpr int DB = D / 32;
    constexpr int CPR = D / 16;                              // 16-byte chunks per row
    constexpr int LOADS = L::TB / 1024 / kLongWaves;          // 1 KB load instructions per wave per tile
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    L& lds = *reinterpret_cast<L*>(lds_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // ---- workgroup -> (head, query block) ---------------------------------
    const int nheads = P.B * P.H;
    const int bid = blockIdx.x;
    int head_i, qb;
    if (P.causal && (nheads & 7) == 0) {
        const int j = bid >> 3;
        const UDivMod t = divmod_invariant(static_cast<uint32_t>(j), map_div);   // by nheads / 8
        head_i = (bid & 7) + 8 * static_cast<int>(t.r);
        qb = nqb - 1 - static_cast<int>(t.q);
    } else if (P.causal) {
        const UDivMod t = divmod_invariant(static_cast<uint32_t>(bid), map_div);   // by nheads
        head_i = static_cast<int>(t.r);
        qb = nqb - 1 - static_cast<int>(t.q);
    } else {
        const int lb = xcd_local_block(bid, static_cast<int>(gridDim.x));
        const UDivMod t = divmod_invariant(static_cast<uint32_t>(lb), map_div);   // by nqb
        qb = static_cast<int>(t.r);
        head_i = static_cast<int>(t.q);
    }
    const size_t head = static_cast<size_t>(head_i);
    const int8_t* qh = q + head * P.Sq * D;
    const size_t kvhead = divmod_invariant(static_cast<uint32_t>(head_i), P.kvg_div).q;   // grouped K/V heads
    const int8_t* kh = k + kvhead * P.kv_rows * D;
    const int8_t* vh = v + kvhead * P.kv_rows * D;

    const int shift = P.Skv - P.Sq;
    const int q0 = qb * kLongRows;
    const int qw0 = q0 + wave * 32;
    const int qrow = qw0 + l32;
    const int kend_row = P.causal ? min(P.Skv, qrow + shift + 1) : P.Skv;
    const int kend_wave = P.causal ? min(P.Skv, qw0 + shift + 1) : P.Skv;
    const int qlast = min(q0 + kLongRows, P.Sq) - 1;
    const int kend_wg = P.causal ? min(P.Skv, qlast + shift + 1) : P.Skv;
    const int ntiles = (kend_wg + kLongTile - 1) / kLongTile;

    if (wave == 0) fill_lut_table<KM>(P, lds.lut, lane);

    v4i qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (qrow < P.Sq)
            qf[ks] = *reinterpret_cast<const v4i*>(qh + static_cast<size_t>(qrow) * D + 32 * ks + 16 * hh);
        else
            qf[ks] = v4i{0, 0, 0, 0};
    }

    // ---- asynchronous tile loads -------------------------------------------
    // Wave w, instruction i fills LDS bytes [(w*LOADS + i) KB, +1 KB) of the
    // stage; lane l writes 16 bytes at l*16, i.e. row (1 KB offset)/D + l/CPR,
    // stored chunk l % CPR, which holds logical chunk (l % CPR) ^ swizzle(row).
    // Per-lane source offsets within a tile are fixed; a tile adds t*64*D.
    uint32_t koff[LOADS], voff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int row = (wave * LOADS + i) * (1024 / D) + lane / CPR;
        const int pos = lane % CPR;
        koff[i] = static_cast<uint32_t>(row * D + 16 * (pos ^ k_swz<D>(row)));
        voff[i] = static_cast<uint32_t>(row * D + 16 * (pos ^ v_swz<D>(row)));
    }
    auto issue = [&](const int8_t* src, int8_t* dst, const uint32_t (&off)[LOADS], int t) {
        const int8_t* base = src + static_cast<size_t>(t) * kLongTile * D;
        const bool tail = (t + 1) * kLongTile > P.Skv;
        const uint32_t lim = static_cast<uint32_t>((P.Skv - t * kLongTile) * D - 16);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            // rows past Skv: any in-bounds bytes (masked, and cancelled by colsum)
            const uint32_t o = tail ? min(off[i], lim) : off[i];
            __builtin_amdgcn_global_load_lds(base + o, (lds_void_t*)(dst + (wave * LOADS + i) * 1024), 16, 0, 0);
        }
    };

    // K tile stage st: 0..2 in the K ring; the passes that read K alone also
    // use the V ring, as stages 3..5 (the two rings are contiguous)
    static_assert(offsetof(L, v) == offsetof(L, k) + kStages * L::TB, "K and V rings adjacent");
    auto kstage = [&](int st) -> int8_t* {
        return reinterpret_cast<int8_t*>(&lds) + offsetof(L, k) + static_cast<size_t>(st) * L::TB;
    };

    // S^T block kb (0 or 1) of the K tile in stage ST, from accumulator c0.
    // The swizzle of row 32 kb + l32 depends on l32 alone, so each fragment's
    // address is a per-lane register (kfo) plus a constant that folds into the
    // instruction's offset field: the stages are compile-time constants (the
    // tile loops below are unrolled over the ring), and no address is
    // recomputed per tile.
    uint32_t kfo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        kfo[ks] = static_cast<uint32_t>(l32 * D + 16 * ((2 * ks + hh) ^ k_swz<D>(l32)));
    auto scores = [&](auto st_c, int kb, const v16i& c0) {
        constexpr int ST = decltype(st_c)::value;
        v16i s = c0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v4i a = *reinterpret_cast<const v4i*>(lds_raw + kfo[ks] + (offsetof(L, k) + ST * L::TB) +
                                                        32 * kb * D);
            s = mfma_i8_32x32x32(a, qf[ks], s);
        }
        return s;
    };
    // Both S^T blocks of the tile in stage ST: all eight fragment reads are
    // issued before the first MFMA (one LDS round trip per tile, not one per
    // pair of fragments)
    auto scores2 = [&](auto st_c, const v16i& c0, v16i& s0, v16i& s1) {
        constexpr int ST = decltype(st_c)::value;
        v4i a[2][KS];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a[kb][ks] = *reinterpret_cast<const v4i*>(lds_raw + kfo[ks] + (offsetof(L, k) + ST * L::TB) +
                                                          32 * kb * D);
        // every fragment is an operand here, so all reads are issued (and
        // waited for once) before the MFMAs
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(a[0][ks]), "+v"(a[1][ks]));
        s0 = c0;
        s1 = c0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s0 = mfma_i8_32x32x32(a[0][ks], qf[ks], s0);
            s1 = mfma_i8_32x32x32(a[1][ks], qf[ks], s1);
        }
    };
    // key j0 + acc_row(r, hh) is allowed iff 8(r/4) + (r%4) < kend_row - j0 - 4hh
    auto mask = [&](v16i& s, int j0, int32_t fill) {
        if (j0 + 32 > kend_wave) {
            const int lim = kend_row - j0 - 4 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) >= lim) s[r] = fill;
        }
    };

    // P.V B operand addresses for stage 0, key block 0 (see tr8_lane_addr);
    // the stage and key block add immediate offsets
    uint32_t vaddr[2 * DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
            vaddr[2 * db + rd] = static_cast<uint32_t>(offsetof(L, v)) + tr8_lane_addr<D>(lane, db, rd);
    }

    // The pass over K and V: three stages, one tile between workgroup
    // barriers, loads requested two tiles ahead.
    auto run_kv_tiles = [&](auto&& body) {
        // prologue: tiles 0 and 1 requested, tile 0 waited for
        constexpr int per_tile = 2 * LOADS;
        wait_vmcnt(0);                       // nothing else in flight when counting
        issue(kh, lds.k[0], koff, 0);
        issue(vh, lds.v[0], voff, 0);
        if (ntiles > 1) {
            issue(kh, lds.k[1], koff, 1);
            issue(vh, lds.v[1], voff, 1);
            wait_vmcnt(per_tile);
        } else {
            wait_vmcnt(0);
        }
        lds_barrier();
        for (int t0 = 0; t0 < ntiles; t0 += kStages) {
            static_for<kStages>([&](auto sc) {
                constexpr int ST = decltype(sc)::value;
                const int t = t0 + ST;
                if (t >= ntiles) return;
                if (t + 2 < ntiles) {
                    constexpr int ST2 = (ST + 2) % kStages;
                    issue(kh, lds.k[ST2], koff, t + 2);
                    issue(vh, lds.v[ST2], voff, t + 2);
                }
                body(t, sc);
                // tile t+1 must have landed; tile t+2 may stay in flight
                if (t + 2 < ntiles) wait_vmcnt(per_tile);
                else wait_vmcnt(0);
                lds_barrier();
            });
        }
    };

    // Passes over K alone: six stages, two tiles between workgroup barriers,
    // loads requested four tiles ahead. Tiles t+4 and t+5 go to the stages of
    // t-2 and t-1, which every wave finished before the last barrier; at the
    // end of a pair, tiles t+2 and t+3 must have landed.
    auto run_k_tiles = [&](auto&& body) {
        wait_vmcnt(0);                       // nothing else in flight when counting
        const int pre = min(ntiles, 4);
        for (int t = 0; t < pre; ++t) issue(kh, kstage(t), koff, t);
        wait_vmcnt(max(0, pre - 2) * LOADS);  // tiles 0 and 1 landed
        lds_barrier();
        for (int t0 = 0; t0 < ntiles; t0 += 2 * kStages) {
            static_for<kStages>([&](auto pc) {
                constexpr int S0 = 2 * decltype(pc)::value;   // stages of tiles t and t+1
                const int t = t0 + S0;
                if (t >= ntiles) return;
                int issued = 0;
                if (t + 4 < ntiles) {
                    issue(kh, kstage((S0 + 4) % (2 * kStages)), koff, t + 4);
                    ++issued;
                }
                if (t + 5 < ntiles) {
                    issue(kh, kstage((S0 + 5) % (2 * kStages)), koff, t + 5);
                    ++issued;
                }
                body(t, std::integral_constant<int, S0>{});
                if (t + 1 < ntiles) body(t + 1, std::integral_constant<int, S0 + 1>{});
                wait_vmcnt(issued * LOADS);
                lds_barrier();
            });
        }
    };

    // ---- pass 1: row max ---------------------------------------------------
    // Wave w takes the 64 rows of row groups g0 = 2 (w & 1) and g0 + 1 (the
    // 32-row groups of waves g0 and g0 + 1 in the other passes) and key block
    // kbw = w >> 1 of every tile: each K fragment set feeds two MFMA chains,
    // so a wave reads half the fragments that its own 32 rows over both key
    // blocks would need. The two key blocks' maxima of a row meet through
    // LDS (the column-sum area, unused until the end).
    const v16i zero16 = v16i{};
    const int g0 = 2 * (wave & 1);
    const int kbw = wave >> 1;
    v4i qg[2][KS];
    int kend_gw[2], kend_gr[2], kend_gl[2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
        const int qa = q0 + 32 * (g0 + gi);
        const int row = qa + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (row < P.Sq)
                qg[gi][ks] = *reinterpret_cast<const v4i*>(qh + static_cast<size_t>(row) * D + 32 * ks + 16 * hh);
            else
                qg[gi][ks] = v4i{0, 0, 0, 0};
        }
        kend_gw[gi] = P.causal ? min(P.Skv, qa + shift + 1) : P.Skv;
        kend_gr[gi] = P.causal ? min(P.Skv, row + shift + 1) : P.Skv;
        kend_gl[gi] = P.causal ? min(P.Skv, qa + 31 + shift + 1) : P.Skv;
    }
    uint32_t kfw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kfw[ks] = kfo[ks] + static_cast<uint32_t>(32 * kbw * D);
    auto mask_g = [&](v16i& sc, int j0, int kw, int kr) {
        if (j0 + 32 > kw) {
            const int lim = kr - j0 - 4 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) >= lim) sc[r] = INT_MIN;
        }
    };
    int32_t mg0 = INT_MIN, mg1 = INT_MIN;
    run_k_tiles([&](int t, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        const int jb = t * kLongTile + 32 * kbw;
        if (jb >= kend_gl[1]) return;        // no row of either group attends this block
        v4i a[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            a[ks] = *reinterpret_cast<const v4i*>(lds_raw + kfw[ks] + (offsetof(L, k) + ST * L::TB));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(a[ks]));
        v16i s0 = zero16, s1 = zero16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s0 = mfma_i8_32x32x32(a[ks], qg[0][ks], s0);
            s1 = mfma_i8_32x32x32(a[ks], qg[1][ks], s1);
        }
        mask_g(s0, jb, kend_gw[0], kend_gr[0]);
        mask_g(s1, jb, kend_gw[1], kend_gr[1]);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            mg0 = max(max(mg0, s0[r]), s0[r + 1]);
            mg1 = max(max(mg1, s1[r]), s1[r + 1]);
        }
    });
    mg0 = max(mg0, __shfl_xor(mg0, 32));
    mg1 = max(mg1, __shfl_xor(mg1, 32));
    int32_t* const xm = &lds.colsum[0][0];   // [row group][key block][row]
    static_assert(sizeof(lds.colsum) >= 4 * 2 * 32 * sizeof(int32_t), "row-max exchange fits");
    if (hh == 0) {
        xm[(g0 * 2 + kbw) * 32 + l32] = mg0;
        xm[((g0 + 1) * 2 + kbw) * 32 + l32] = mg1;
    }
    lds_barrier();
    const int32_t mrow = max(xm[(wave * 2) * 32 + l32], xm[(wave * 2 + 1) * 32 + l32]);

    // row constants of the slot arithmetic
    v16i cinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = -mrow;
    auto table_entry = [&](int32_t y) -> uint32_t { return lut_load<KM>(entry_addr<KM>(y, P.ent_a, P.ent_b)); };
    constexpr int32_t kMasked = -(1 << 23);   // y of a masked key: saturates to the last slot

    // ---- pass 2: row sum of the table entries ------------------------------
    uint32_t E = 0;
    run_k_tiles([&](int t, auto st) {
        v16i s0, s1;
        scores2(st, cinit, s0, s1);
        mfma_result_guard(s0, s1);           // the slot word (inline asm) reads them
        mask(s0, t * kLongTile, kMasked);
        mask(s1, t * kLongTile + 32, kMasked);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const uint32_t e0 = table_entry(s0[r]);
            const uint32_t e1 = table_entry(s0[r + 1]);
            const uint32_t e2 = table_entry(s1[r]);
            const uint32_t e3 = table_entry(s1[r + 1]);
            E += (e0 + e1) + (e2 + e3);
        }
    });
    E += __shfl_xor(E, 32);
    // uint8 P: R2 = 2R <= 2^17; uint16 P: R16 < 2^18 (E >= 128*255; both 24-bit operands)
    const uint32_t R2 = P16 ? reciprocal16(E) : 2 * reciprocal8(E);
    if (row_max != nullptr && hh == 0 && qrow < P.Sq) {
        row_max[head * P.Sq + qrow] = mrow;
        row_sum[head * P.Sq + qrow] = E;
    }

    // ---- pass 3: P from the table, P.V on the MFMA --------------------------
    // uint16 P: o holds the high probability bytes' product, o16 the low ones'
    v16i o[DB];
    v16i o16[P16 ? DB : 1];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = v16i{};
#pragma unroll
    for (int db = 0; db < (P16 ? DB : 1); ++db) o16[db] = v16i{};
    int32_t cs[DB];                          // this lane's part of the column sums
#pragma unroll
    for (int db = 0; db < DB; ++db) cs[db] = 0;
    auto pword = [&](int32_t y) -> uint32_t { return prob_word(table_entry(y), R2); };
    auto pack = [&](const v16i& s, int w4) -> int {
        return static_cast<int>(pack_top_bytes(pword(s[4 * w4]), pword(s[4 * w4 + 1]), pword(s[4 * w4 + 2]),
                                               pword(s[4 * w4 + 3])));
    };
    // uint16 P: signed operands (p >> 8) - 128 and (p & 0xff) - 128 of four keys
    auto pack16 = [&](const v16i& s, int w4, int& hi, int& lo) {
        auto pw = [&](int32_t y) -> uint32_t { return prob16_word(table_entry(y), R2); };
        uint32_t h, l;
        pack_bytes_32(pw(s[4 * w4]), pw(s[4 * w4 + 1]), pw(s[4 * w4 + 2]), pw(s[4 * w4 + 3]), h, l);
        hi = static_cast<int>(h);
        lo = static_cast<int>(l ^ 0x80808080u);
    };
    run_kv_tiles([&](int t, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        const bool colsum_turn = (t % kLongWaves) == wave;
        auto kblock = [&](auto kbc) {
            constexpr int kb = decltype(kbc)::value;
            auto& st = st_c;
            v16i s = scores(st, kb, cinit);
            mfma_result_guard(s);            // the slot word (inline asm) reads them
            mask(s, t * kLongTile + 32 * kb, kMasked);
            v4i pa, pl;
            if constexpr (P16) {
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    int h, l;
                    pack16(s, w4, h, l);
                    pa[w4] = h;
                    pl[w4] = l;
                }
            } else {
                pa = v4i{pack(s, 0), pack(s, 1), pack(s, 2), pack(s, 3)};
            }
            v4i vb[DB];
            tr8_operands<DB, ST * L::TB + kb * 32 * D>(vaddr, vb);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma_i8_32x32x32(pa, vb[db], o[db]);
            if constexpr (P16) {
#pragma unroll
                for (int db = 0; db < DB; ++db) o16[db] = mfma_i8_32x32x32(pl, vb[db], o16[db]);
            }
            if (colsum_turn) {
                // one wave per tile; the asm keeps the sums from being
                // computed on every wave and selected afterwards
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    asm volatile("" : "+v"(cs[db]));
                    cs[db] = __builtin_amdgcn_sdot4(vb[db][0], 0x01010101, cs[db], false);
                    cs[db] = __builtin_amdgcn_sdot4(vb[db][1], 0x01010101, cs[db], false);
                    cs[db] = __builtin_amdgcn_sdot4(vb[db][2], 0x01010101, cs[db], false);
                    cs[db] = __builtin_amdgcn_sdot4(vb[db][3], 0x01010101, cs[db], false);
                }
            }
        };
        if constexpr (P16) {
            kblock(std::integral_constant<int, 0>{});
            kblock(std::integral_constant<int, 1>{});
        } else {
            // uint8 P, the two blocks interleaved in four steps so that each
            // step's MFMAs run under the other block's integer work and LDS
            // waits: (A) block 0's scores and table reads; (B) block 1's
            // scores while block 0's P operand is formed and its V operands
            // read; (C) block 0's P.V while block 1's table reads go out;
            // (D) block 1's P operand and P.V
            const int j0 = t * kLongTile;
            auto& st = st_c;
            uint32_t e[16];
            v16i s = scores(st, 0, cinit);
            mfma_result_guard(s);            // the slot word (inline asm) reads them
            mask(s, j0, kMasked);
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = table_entry(s[i]);
            __builtin_amdgcn_sched_barrier(0);
            s = scores(st, 1, cinit);
            v4i pa0;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4)
                pa0[w4] = static_cast<int>(pack_top_bytes(prob_word(e[4 * w4], R2), prob_word(e[4 * w4 + 1], R2),
                                                          prob_word(e[4 * w4 + 2], R2),
                                                          prob_word(e[4 * w4 + 3], R2)));
            auto colsum_add = [&](const v4i (&vb)[DB]) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    asm volatile("" : "+v"(cs[db]));
#pragma unroll
                    for (int w = 0; w < 4; ++w) cs[db] = __builtin_amdgcn_sdot4(vb[db][w], 0x01010101, cs[db], false);
                }
            };
            {
                v4i vb0[DB];
                tr8_operands<DB, ST * L::TB>(vaddr, vb0);
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db] = mfma_i8_32x32x32(pa0, vb0[db], o[db]);
                if (colsum_turn) colsum_add(vb0);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma_result_guard(s);
            mask(s, j0 + 32, kMasked);
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = table_entry(s[i]);
            __builtin_amdgcn_sched_barrier(0);
            v4i pa1;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4)
                pa1[w4] = static_cast<int>(pack_top_bytes(prob_word(e[4 * w4], R2), prob_word(e[4 * w4 + 1], R2),
                                                          prob_word(e[4 * w4 + 2], R2),
                                                          prob_word(e[4 * w4 + 3], R2)));
            v4i vb1[DB];
            tr8_operands<DB, ST * L::TB + 32 * D>(vaddr, vb1);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma_i8_32x32x32(pa1, vb1[db], o[db]);
            if (colsum_turn) colsum_add(vb1);
        }
    });
    // column sums: lanes l and l^32 hold the two key halves; waves hold tiles
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int32_t tot = cs[db] + __shfl_xor(cs[db], 32);
        if (hh == 0) lds.colsum[wave][32 * db + l32] = tot;
    }
    __syncthreads();

    // ---- requantise and store -----------------------------------------------
    // rows of this lane: qw0 + 4hh + acc_row(r, 0); full groups skip the checks
    int8_t* const obase = out + (head * P.Sq + qw0 + 4 * hh) * D;
    const bool full = qw0 + 32 <= P.Sq;
    const uint32_t rq_add = P.req_shift >= 33 ? (1u << (P.req_shift - 33)) : 0u;
    const uint32_t rq_sh = static_cast<uint32_t>(P.req_shift - 32);
    auto store_rows = [&](const v16i& acc, int8_t* op) {
        auto put = [&](auto rq) {
            if (full) {
#pragma unroll
                for (int r = 0; r < 16; ++r) op[acc_row(r, 0) * D] = static_cast<int8_t>(rq(acc[r]));
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (qw0 + 4 * hh + acc_row(r, 0) < P.Sq) op[acc_row(r, 0) * D] = static_cast<int8_t>(rq(acc[r]));
            }
        };
        if (P.req_shift >= 33) put([&](int32_t x) { return requantise_hi(x, P.req_mul, rq_add, rq_sh); });
        else put([&](int32_t x) { return static_cast<int32_t>(requantise(x, P)); });
    };
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + l32;
        const int32_t c128 = 128 * (lds.colsum[0][d] + lds.colsum[1][d] + lds.colsum[2][d] + lds.colsum[3][d]);
        v16i acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // uint16 P: sum p v = 256 (sum hi v) + sum lo v, each byte sum
            // corrected by its own 128 * colsum (|.| < 2^24)
            if constexpr (P16) acc[r] = 256 * (o[db][r] + c128) + (o16[db][r] + c128);
            else acc[r] = o[db][r] + c128;
        }
        store_rows(acc, obase + d);
    }
}

template <int D, int KM, bool P16>
int launch_long_t(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, const IaKernelParams& kp,
                  hipStream_t s, int nqb, unsigned blocks, int32_t* row_max, uint32_t* row_sum) {
    static std::atomic<uint64_t> lds_set{0};
    const size_t shm = sizeof(LongLds<D, KM>);
    const int st = ensure_dynamic_lds(reinterpret_cast<const void*>(&ia_long_kernel<D, KM, P16>),
                                      static_cast<int>(shm), lds_set);
    if (st != INTATTN_OK) return st;
    // the divisor of the workgroup -> (head, query block) split the kernel takes
    const int nheads = kp.B * kp.H;
    const uint32_t map_d = kp.causal ? ((nheads & 7) == 0 ? nheads >> 3 : nheads) : nqb;
    hipLaunchKernelGGL((ia_long_kernel<D, KM, P16>), dim3(blocks), dim3(256), shm, s, q, k, v, out, kp, nqb,
                       invariant_div(map_d), row_max, row_sum);
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

}  // namespace

int launch_long(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum) {
    const int nqb = (kp.Sq + kLongRows - 1) / kLongRows;
    const long long blocks = static_cast<long long>(nqb) * kp.H * kp.B;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned nb = static_cast<unsigned>(blocks);
    auto go = [&](auto d_c, auto p16_c) -> int {
        constexpr int DD = decltype(d_c)::value;
        constexpr bool PP = decltype(p16_c)::value;
        if (kp.slot_k == 4) return launch_long_t<DD, 4, PP>(q, k, v, out, kp, s, nqb, nb, row_max, row_sum);
        if (kp.slot_k == 2) return launch_long_t<DD, 2, PP>(q, k, v, out, kp, s, nqb, nb, row_max, row_sum);
        if (kp.slot_k == 1) return launch_long_t<DD, 1, PP>(q, k, v, out, kp, s, nqb, nb, row_max, row_sum);
        return launch_long_t<DD, 0, PP>(q, k, v, out, kp, s, nqb, nb, row_max, row_sum);
    };
    using D64 = std::integral_constant<int, 64>;
    using D128 = std::integral_constant<int, 128>;
    if (kp.prob_bits == 16) return D == 64 ? go(D64{}, std::true_type{}) : go(D128{}, std::true_type{});
    return D == 64 ? go(D64{}, std::false_type{}) : go(D128{}, std::false_type{});
}

}  // namespace ia
