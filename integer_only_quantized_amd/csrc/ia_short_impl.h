// Short-row integer attention kernel (gfx950 / CDNA4), shared by the uint8-P
// (ia_short.hip) and uint16-P (ia_short16.hip) translation units: the whole key range
// of a head resident in LDS (Skv <= 512 at d = 64, <= 256 at d = 128), each
// row's keys split over two waves.
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology",
// steps 2-3; integer widths and roundings as stated in include/intattn.h.
//
// Work split: one workgroup = 4 waves = 2 query groups of 32 rows x 2 key
// halves (NBH blocks of 32 keys each, a compile-time count). Wave w takes
// query group w & 1 and key half w >> 1, so a head of S = 512 gives 8
// workgroups of 4 waves, and every row's max, sum and P.V partials are
// combined across the two key halves through LDS once per pass.
//   staging: K of both halves via global_load_lds (rows XOR-swizzled for the
//            64-bank LDS; rows past Skv read in-bounds bytes of the last row,
//            masked below);
//   pass 1:  S^T blocks of the wave's half (K fragments from LDS, Q^T
//            fragments in registers) -> row max; exchange with the other half;
//   pass 2:  the MFMA accumulator starts from -m, so it yields y = s - m;
//            slot word -> shared exp table -> row sum; the table entry of
//            every score is kept in registers, two 16-bit entries a word;
//            exchange the sums;
//   V:       row-major V replaces K in LDS (global_load_lds again; chunks
//            swizzled for the transpose reads);
//   pass 3:  P bytes from the kept entries, two VALU ops a key and no table
//            read: bits 23..30 of e * R + 2^22 + 2^30 are p - 128 as int8,
//            written into the P operand by SDWA byte writes;
//            V operand by ds_read_b64_tr_b8; P.V on the MFMA; the column sums
//            of the V rows fed come from the same operands (sdot4), and
//            o + 128 * colsum = sum p v;
//   combine: each wave sends the output columns the other half's wave
//            finishes through LDS, adds the partials it receives,
//            requantises and stores its own columns.
// Slot word, y = s - m in [-2^23, 0], for a table of N entries (32, or a
// finer 64 or 128): t = sat(y * -kM + k * 2^23) with k = 4 (N = 32,
// 4M < 2^23), 2 (N <= 64, 2M < 2^23) or 1; its top byte is k * slot +
// fraction bits (127 when saturated), and the table layout KM = k in LDS is
// addressed from that byte in one SDWA op (u32[32]: byte & 0x7c; u16[128]:
// byte & 0x7e or 2 * byte).
#pragma once

#include <type_traits>

#include "ia_device.h"

namespace ia {
namespace {

// Staging of a key block: split between the two query-group waves of its key
// half (each loads part of it; a workgroup barrier per block makes the other
// part visible), or loaded whole by both (identical bytes; each wave waits
// only for its own loads, no barrier). Splitting halves the L2->LDS traffic
// of the start-up burst, which pays only for the longest full rows (measured:
// 512 keys at d = 64); elsewhere the per-block barriers cost more.
template <int NBH, bool SKIP>
constexpr bool split_k_staging() { return NBH >= 8 && !SKIP; }

// Table words in LDS for layout KM: 64 (u32[32] or u16[128]), 128 for the
// direct table (u16[256]).
constexpr int table_words(int KM) { return KM == 0 ? kIaTabEntries / 2 : kIaMaxLut / 2; }

template <int D, int NBH, int KM>
struct ShortLds {
    static constexpr int DB = D / 32;
    static constexpr int KVBytes = 2 * NBH * 32 * D;                 // K (later V) of both halves
    static constexpr int XOBytes = 4 * (DB / 2) * 16 * 64 * 4;       // output partials, 4 waves
    static constexpr int Region = KVBytes > XOBytes ? KVBytes : XOBytes;
    uint32_t lut[table_words(KM)];           // exp table (layout KM); first member: LDS address 0
    int32_t xm[2][2][32];                    // row max exchange [query group][half][row]
    uint32_t xe[2][2][32];                   // row sum exchange
    int32_t xcs[4][D];                       // column-sum partials, one per wave
    int8_t q[2][32 * D];                     // Q rows of each query group (K-block layout)
    int8_t kv[Region];                       // K, then V, then the output partials
};

template <int D, int NBH, bool SKIP, int KM, bool P16>
__global__ __launch_bounds__(256) void ia_short_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int nqb, int32_t* __restrict__ row_max,
    uint32_t* __restrict__ row_sum) {
    using L = ShortLds<D, NBH, KM>;
    constexpr int KS = D / 32;
    constexpr int DB = D / 32;
    constexpr int HDB = DB / 2;                        // output column blocks finished per wave
    constexpr int CPR = D / 16;                        // 16-byte chunks per row
    __shared__ __attribute__((aligned(16))) L lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qg = wave & 1;
    const int half = wave >> 1;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int bid = xcd_local_block(blockIdx.x, static_cast<int>(gridDim.x));
    const UDivMod hq = divmod_invariant(static_cast<uint32_t>(bid), P.qb_div);
    const int qb = static_cast<int>(hq.r);
    const size_t head = hq.q;
    const int8_t* qh = q + head * P.Sq * D;
    const size_t kvhead = divmod_invariant(static_cast<uint32_t>(head), P.kvg_div).q;   // grouped K/V heads
    const int8_t* kh = k + kvhead * P.kv_rows * D;
    const int8_t* vh = v + kvhead * P.kv_rows * D;

    // ---- staging ---------------------------------------------------------------
    // Each wave stages the key blocks of its own half that it reads (the two
    // query-group waves of a half write the same bytes to the same place), so
    // a wave waits only for its own loads, block by block, and no barrier
    // precedes pass 1 or pass 3. Block j of half h is LPB loads of 1 KB; load
    // i of it fills LDS KB blk = (h*NBH + j)*LPB + i: lane l writes row
    // blk*(1024/D) + l/CPR, stored chunk l % CPR = logical chunk
    // (l % CPR) ^ swizzle(row).
    // The source offset of load blk is blk*1024 plus a per-lane constant that
    // depends only on the parity of blk (the swizzles use the row's low bits),
    // so the loads take a scalar base; rows past Skv (a uniform tail case)
    // are clamped per lane.
    constexpr int LPB = D / 32;
    uint32_t koff[2], voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int row = par * (1024 / D) + lane / CPR;
        koff[par] = static_cast<uint32_t>(row * D + 16 * ((lane % CPR) ^ k_swz<D>(row)) - par * 1024);
        voff[par] = static_cast<uint32_t>(row * D + 16 * ((lane % CPR) ^ v_swz<D>(row)) - par * 1024);
    }
    const bool stage_tail = L::KVBytes / D > P.Skv;     // some staged rows lie past Skv
    // One wave's loads of a run of 1 KB pieces: piece lb (a compile-time
    // index) goes from gsrc + lb KB + off[parity] to ldst + lb KB. Four
    // consecutive pieces share one scalar base and one M0 value: the
    // instruction's immediate offset (applied to the global and the LDS
    // address alike) selects the piece within its 4 KB window, so a piece
    // costs no scalar address arithmetic of its own. par0 is the parity of
    // the run's first piece (the per-lane offsets alternate with the parity).
    auto load_run = [&](const int8_t* gsrc, int8_t* ldst, uint32_t off0, uint32_t off1, int par0, auto lb_c) {
        constexpr int lb = decltype(lb_c)::value;
        constexpr int w = lb >> 2;
        const uint32_t o = ((par0 + lb) & 1) ? off1 : off0;
        __builtin_amdgcn_global_load_lds(gsrc + w * 4096 + o, (lds_void_t*)(ldst + w * 4096), 16, (lb & 3) * 1024, 0);
    };
    auto stage = [&](const int8_t* src, bool is_v, int kb_first, int nblk, auto split_c) {
        constexpr bool split = decltype(split_c)::value;
        const uint32_t off0 = is_v ? voff[0] : koff[0];
        const uint32_t off1 = is_v ? voff[1] : koff[1];
        // split: this wave loads pieces i0 .. i0 + LPB/2 - 1 of every block
        const int i0 = split ? qg * (LPB / 2) : 0;
        constexpr int NI = split ? LPB / 2 : LPB;
        if (!stage_tail) {
            const int first = kb_first * LPB + i0;
            const int8_t* g = src + static_cast<size_t>(first) * 1024;
            int8_t* l = lds.kv + first * 1024;
            if constexpr (split && NI == 1) {
                // one piece a block, LPB apart: piece j of the run is block j
                static_for<NBH>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    if (j < nblk) load_run(g, l, off0, off1, first, std::integral_constant<int, j * LPB>{});
                });
            } else {
                static_for<NBH>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    if (j < nblk) {
                        static_for<NI>([&](auto ic) {
                            constexpr int ii = decltype(ic)::value;
                            load_run(g, l, off0, off1, first, std::integral_constant<int, j * LPB + ii>{});
                        });
                    }
                });
            }
            // distinct markers keep the two paths apart (a merged last load
            // would hide the count of loads in flight from the compiler)
            asm volatile("; staged, no tail");
        } else {
            // blocks wholly below Skv as above; only a block holding rows
            // past Skv clamps its rows per lane
            const int first = kb_first * LPB + i0;
            const int8_t* g = src + static_cast<size_t>(first) * 1024;
            int8_t* l = lds.kv + first * 1024;
            static_for<NBH>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if (j < nblk) {
                    if ((kb_first + j + 1) * 32 <= P.Skv) {
                        static_for<NI>([&](auto ic) {
                            load_run(g, l, off0, off1, first, std::integral_constant<int, j * LPB + decltype(ic)::value>{});
                        });
                    } else {
#pragma unroll
                        for (int ii = 0; ii < NI; ++ii) {
                            const int i = i0 + ii;
                            const int blk = (kb_first + j) * LPB + i;
                            const int row = blk * (1024 / D) + lane / CPR;
                            const int chunk = (lane % CPR) ^ (is_v ? v_swz<D>(row) : k_swz<D>(row));
                            __builtin_amdgcn_global_load_lds(
                                src + static_cast<size_t>(min(row, P.Skv - 1)) * D + 16 * chunk,
                                (lds_void_t*)(lds.kv + blk * 1024), 16, 0, 0);
                        }
                    }
                }
            });
            asm volatile("; staged, tail rows clamped");
        }
    };

    const int shift = P.Skv - P.Sq;
    const int qw0 = qb * 64 + qg * 32;
    const int qrow = qw0 + l32;
    const int kend_row = P.causal ? min(P.Skv, qrow + shift + 1) : P.Skv;
    const int kend_wave = P.causal ? min(P.Skv, qw0 + shift + 1) : P.Skv;
    const int kb0 = half * NBH;                        // first key block of this wave
    // 32-key blocks of key half h that some row of query group g attends
    // (none for a group past Sq; causal: up to the group's last row); blocks
    // past that are skipped in every pass (their p would all be 0). Without
    // SKIP every block of both halves is attended by both groups.
    auto nvalid_of = [&](int g, int h) -> int {
        const int qa = qb * 64 + 32 * g;
        if (qa >= P.Sq) return 0;
        const int kmax = P.causal ? min(P.Skv, min(qa + 31, P.Sq - 1) + shift + 1) : P.Skv;
        return min(NBH, max(0, (kmax - 32 * h * NBH + 31) / 32));
    };
    const int nvalid = SKIP ? nvalid_of(qg, half) : NBH;
    // column sums shared between the two query groups (each sums every other
    // block) only when both groups feed the same blocks in both halves
    const bool share_cs = !SKIP || (nvalid_of(0, 0) == nvalid_of(1, 0) && nvalid_of(0, 1) == nvalid_of(1, 1));

    // Q rows of this wave's query group, staged like a K block (both key-half
    // waves of the group write the same bytes); rows past Sq read the last
    // row and are computed but never stored. Q goes through LDS rather than
    // straight into registers so that no register load is in flight behind
    // the block-by-block waits below.
    if (nvalid > 0) {
        if (qw0 + 32 <= P.Sq) {
            static_for<LPB>([&](auto ic) {
                load_run(qh + static_cast<size_t>(qw0) * D, &lds.q[qg][0], koff[0], koff[1], 0, ic);
            });
            asm volatile("; Q staged");
        } else {
#pragma unroll
            for (int i = 0; i < LPB; ++i) {
                const int row = i * (1024 / D) + lane / CPR;
                const int chunk = (lane % CPR) ^ k_swz<D>(row);
                __builtin_amdgcn_global_load_lds(qh + static_cast<size_t>(min(qw0 + row, P.Sq - 1)) * D + 16 * chunk,
                                                 (lds_void_t*)(&lds.q[qg][i * 1024]), 16, 0, 0);
            }
            asm volatile("; Q staged, tail rows clamped");
        }
    }
    // blocks of this half that either query group reads (split staging
    // loads these), and the most blocks any wave reads (the number of
    // per-block barriers, the same in every wave)
    const int nvp = SKIP ? max(nvalid_of(0, half), nvalid_of(1, half)) : NBH;
    const int nv_max = SKIP ? max(nvp, max(nvalid_of(0, half ^ 1), nvalid_of(1, half ^ 1))) : NBH;
    // K after Q: waiting for a K block also covers the (older) Q loads
    constexpr bool kSplitK = split_k_staging<NBH, SKIP>();
    stage(kh, false, kb0, kSplitK ? nvp : nvalid, std::integral_constant<bool, kSplitK>{});
    v4i qf[KS];                          // Q^T fragments, read from LDS in pass 1
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = v4i{0, 0, 0, 0};
    if (wave == 0) fill_lut_table<KM>(P, lds.lut, lane);
    // block j of this wave's half is in LDS: loads complete in issue order;
    // whole-block staging issued nvalid blocks of LPB loads, split staging
    // nvp blocks of LPB/2 loads, and then every wave meets at a barrier
    // (executed for j < nv_max by all waves alike)
    auto sync_block = [&](int j, bool split) {
        if (!split) {
            if (j < nvalid) wait_vmcnt((nvalid - 1 - j) * LPB);
        } else if (j < nv_max) {
            if (j < nvp) wait_vmcnt((nvp - 1 - j) * (LPB / 2));
            lds_barrier();
        }
    };

    // S^T block kb (absolute) from accumulator c0
    auto scores = [&](int kb, const v16i& c0) {
        v16i s = c0;
        const int r = 32 * kb + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = (2 * ks + hh) ^ k_swz<D>(r);
            const v4i a = *reinterpret_cast<const v4i*>(&lds.kv[r * D + 16 * c]);
            s = mfma_i8_32x32x32(a, qf[ks], s);
        }
        return s;
    };
    // key 32kb + acc_row(r, hh) is allowed iff 8(r/4) + (r%4) < kend_row - 32kb - 4hh
    auto mask = [&](v16i& s, int kb, int32_t fill) {
        if (32 * kb + 32 > kend_wave) {
            const int lim = kend_row - 32 * kb - 4 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) >= lim) s[r] = fill;
        }
    };

    // Each pass is software-pipelined (MFMAs of block j+1 issued before the
    // integer work on block j) and fenced per block with a scheduling barrier.

    // ---- pass 1: row max ---------------------------------------------------
    const v16i zero16 = v16i{};
    int32_t mrow = INT_MIN;
    {
        v16i cur = zero16;
        sync_block(0, kSplitK);
        if (nvalid > 0) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = *reinterpret_cast<const v4i*>(&lds.q[qg][l32 * D + 16 * ((2 * ks + hh) ^ k_swz<D>(l32))]);
            cur = scores(kb0, zero16);
        }
#pragma unroll
        for (int j = 0; j < NBH; ++j) {
            v16i nxt = zero16;
            if (j + 1 < NBH) sync_block(j + 1, kSplitK);
            if (j + 1 < nvalid) nxt = scores(kb0 + j + 1, zero16);
            if (j < nvalid) {
                mask(cur, kb0 + j, INT_MIN);
#pragma unroll
                for (int r = 0; r < 16; r += 2) mrow = max(max(mrow, cur[r]), cur[r + 1]);
                // keep the reduction per block (not one cross-block tree at the end)
                asm volatile("" : "+v"(mrow));
            }
            if (j + 1 < NBH) cur = nxt;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    mrow = max(mrow, __shfl_xor(mrow, 32));
    if (hh == 0) lds.xm[qg][half][l32] = mrow;
    lds_barrier();
    mrow = max(mrow, lds.xm[qg][half ^ 1][l32]);

    // ---- pass 2: slots, table entries, row sum; slot bytes kept ------------
    constexpr int32_t kMasked = -(1 << 23);   // y of a masked key: saturates to the last slot
    uint32_t ew[NBH][8];                 // table entries of this wave's keys, two a word
    uint32_t E = 0;
    {
        v16i cinit;
#pragma unroll
        for (int r = 0; r < 16; ++r) cinit[r] = -mrow;
        // the slot word (inline asm) reads each block's scores one block after
        // its MFMAs, with a whole block of integer work in between, except
        // for the first block, which is guarded
        // d = 64 with up to 4 blocks a half (e.g. S = 197): no software
        // pipelining, which saves 8 VGPRs there and measured 2 % faster on
        // ViT's shape (14.43 against 14.72 us)
        constexpr bool kPipe2 = NBH > 4 || D != 64;
        v16i cur = cinit;
        if (kPipe2 && nvalid > 0) {
            cur = scores(kb0, cinit);
            mfma_result_guard(cur);
        }
#pragma unroll
        for (int j = 0; j < NBH; ++j) {
            v16i nxt = cinit;
            if (kPipe2) {
                if (j + 1 < nvalid) nxt = scores(kb0 + j + 1, cinit);
            } else if (j < nvalid) {
                cur = scores(kb0 + j, cinit);
                mfma_result_guard(cur);
            }
            if (j >= nvalid) {
#pragma unroll
                for (int i = 0; i < 8; ++i) ew[j][i] = 0;   // never read
                if (kPipe2 && j + 1 < NBH) cur = nxt;
                __builtin_amdgcn_sched_barrier(0);
                continue;
            }
            mask(cur, kb0 + j, kMasked);
            uint32_t e[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = lut_load<KM>(entry_addr<KM>(cur[i], P.ent_a, P.ent_b));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ew[j][i] = entry_pair(e[2 * i], e[2 * i + 1]);
                // keep the pair word (not the two entries it came from) live
                asm volatile("" : "+v"(ew[j][i]));
            }
#pragma unroll
            for (int i = 0; i < 16; i += 4) E += (e[i] + e[i + 1]) + (e[i + 2] + e[i + 3]);
            asm volatile("" : "+v"(E));
            if (kPipe2 && j + 1 < NBH) cur = nxt;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    E += __shfl_xor(E, 32);
    if (hh == 0) lds.xe[qg][half][l32] = E;
    lds_barrier();                       // every wave is also done with K (and its K loads)
    stage(vh, true, kb0, nvalid, std::false_type{});   // V replaces K (whole blocks)
    E += lds.xe[qg][half ^ 1][l32];
    // E >= 128*255 for every row that exists (it attends at least one key,
    // whose entry is 2^15, or 128*255 for a table of uint8 entries); rows
    // past Sq may have E = 0 and are never stored. R <= 65280 once
    // E >= 2^15; the one larger value, R = 65536 at E = 128*255, is clamped
    // to the 16-bit operand's 65535 without changing any p: the entries are
    // then multiples of 128, and (e*R + 2^22) >> 23 is e/128 for R = 2^16
    // and for R = 2^16 - 1 alike (e <= 2^15 < 2^22).
    // uint16 P: R16 = floor((65535 * 2^16 + floor(E/2)) / E) < 2^18
    const uint32_t R = P16 ? reciprocal16(E) : min(reciprocal8(E), 65535u);
    if (row_max != nullptr && half == 0 && hh == 0 && qrow < P.Sq) {
        row_max[head * P.Sq + qrow] = mrow;
        row_sum[head * P.Sq + qrow] = E;
    }
    uint32_t vaddr[2 * DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
            vaddr[2 * db + rd] = static_cast<uint32_t>(offsetof(L, kv)) + static_cast<uint32_t>(kb0 * 32 * D) +
                                 tr8_lane_addr<D>(lane, db, rd);
    }

    // ---- pass 3: P from the kept table entries, P.V on the MFMA ------------
    // P operand of block j: byte c of word w4 is key 4 w4 + c of the block
    auto pbytes = [&](const uint32_t (&w)[8]) {
        v4i pa;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) pa[w4] = static_cast<int>(prob_bytes4(w[2 * w4], w[2 * w4 + 1], R));
        return pa;
    };
    // uint16 P: the word e * R16 + 2^15 + 2^31 holds (p >> 8) ^ 0x80 in byte 3
    // and p & 0xff in byte 2; four words give the signed operands of the high
    // bytes (hi) and, flipped, of the low bytes (lo), each p byte minus 128
    auto pbytes16 = [&](const uint32_t (&w)[8], v4i& hi, v4i& lo) {
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            const uint32_t a = w[2 * w4], b = w[2 * w4 + 1];
            uint32_t h, l;
            pack_bytes_32(prob16_word(a & 0xffffu, R), prob16_word(a >> 16, R), prob16_word(b & 0xffffu, R),
                          prob16_word(b >> 16, R), h, l);
            hi[w4] = static_cast<int>(h);
            lo[w4] = static_cast<int>(l ^ 0x80808080u);
        }
    };
    v16i o[DB];
    v16i o16[P16 ? DB : 1];              // uint16 P: the low bytes' product
    int32_t cs[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        o[db] = v16i{};
        cs[db] = 0;
    }
#pragma unroll
    for (int db = 0; db < (P16 ? DB : 1); ++db) o16[db] = v16i{};
    {
        v4i pa = v4i{0, 0, 0, 0};
        v4i pl = v4i{0, 0, 0, 0};
        if (nvalid > 0) {
            if constexpr (P16) pbytes16(ew[0], pa, pl);
            else pa = pbytes(ew[0]);
        }
        static_for<NBH>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            sync_block(j, false);
            if (j >= nvalid) return;
            v4i vb[DB];
            tr8_operands<DB, j * 32 * D>(vaddr, vb);
            // the next block's P operand while the transpose reads land
            v4i pnext = v4i{0, 0, 0, 0};
            v4i plnext = v4i{0, 0, 0, 0};
            if constexpr (j + 1 < NBH) {
                if (j + 1 < nvalid) {
                    if constexpr (P16) pbytes16(ew[j + 1], pnext, plnext);
                    else pnext = pbytes(ew[j + 1]);
                }
            }
            mfma_source_guard(pa);               // built by inline asm (uint8 P)
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma_i8_32x32x32(pa, vb[db], o[db]);
            if constexpr (P16) {
#pragma unroll
                for (int db = 0; db < DB; ++db) o16[db] = mfma_i8_32x32x32(pl, vb[db], o16[db]);
            }
            // column sums of the V rows fed: when both query groups feed the
            // same blocks, each sums every other block (asm: no speculation)
            if (!share_cs || (j & 1) == qg) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    asm volatile("" : "+v"(cs[db]));
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        cs[db] = __builtin_amdgcn_sdot4(vb[db][w], 0x01010101, cs[db], false);
                }
            }
            if constexpr (j + 1 < NBH) {
                pa = pnext;
                if constexpr (P16) pl = plnext;
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    // uint16 P: sum p v = 256 (sum hi v) + sum lo v, with hi and lo each
    // offset by -128 and corrected by 128 * colsum at the end (257 * that in
    // all). The combined partial 256 o + o16 is formed in wrapping 32-bit
    // arithmetic: its pieces may pass 2^31 while the final sum, |sum p v| <
    // 2^31, is exact modulo 2^32.
    if constexpr (P16) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o[db][r] = static_cast<int32_t>(256u * static_cast<uint32_t>(o[db][r]) + static_cast<uint32_t>(o16[db][r]));
    }
    // column-sum partials of this wave (both key halves of the lane pair)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int32_t c = cs[db] + __shfl_xor(cs[db], 32);
        if (hh == 0) lds.xcs[wave][32 * db + l32] = c;
    }

    // ---- combine the halves, requantise, store -------------------------------
    // The wave of half h finishes column blocks [h*HDB, (h+1)*HDB); partial of
    // column block j of that set, from the wave (qg, src half), at
    // kv + (((qg*2 + src)*HDB + j)*16 + r)*256 + 4*lane. Every row gets
    // o_half0 + o_half1 + 128 * (sum of the four column-sum partials): the
    // column sums cover exactly the V rows fed, so this is sum p v.
    lds_barrier();                       // every wave is done with V
    auto xo_addr = [&](int src, int j, int r) {
        return static_cast<uint32_t>(offsetof(L, kv)) +
               static_cast<uint32_t>((((qg * 2 + src) * HDB + j) * 16 + r) * 256 + 4 * lane);
    };
    // rows of this lane: qw0 + 4hh + acc_row(r, 0); full groups skip the checks
    int8_t* const obase = out + (head * P.Sq + qw0 + 4 * hh) * D;
    const bool full = qw0 + 32 <= P.Sq;
    // requantise 16 accumulators and store them at op + acc_row(r, 0) * D
    const uint32_t rq_add = P.req_shift >= 33 ? (1u << (P.req_shift - 33)) : 0u;
    const uint32_t rq_sh = static_cast<uint32_t>(P.req_shift - 32);
    auto store_rows = [&](const int32_t (&acc)[16], int8_t* op) {
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
        if (P.req_shift >= 33) put([&](int32_t a) { return requantise_hi(a, P.req_mul, rq_add, rq_sh); });
        else put([&](int32_t a) { return static_cast<int32_t>(requantise(a, P)); });
    };
    auto finish = [&](auto hc) {
        constexpr int H = decltype(hc)::value;
        static_for<HDB>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int db = (1 - H) * HDB + j;     // columns the other wave finishes
#pragma unroll
            for (int r = 0; r < 16; ++r)
                *reinterpret_cast<__attribute__((address_space(3))) int32_t*>(
                    static_cast<uintptr_t>(xo_addr(H, j, r))) = o[db][r];
        });
        lds_barrier();
        static_for<HDB>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int db = H * HDB + j;
            const int d = 32 * db + l32;
            // shared sums: all four waves' partials; otherwise this query
            // group's two waves (wave = 2 * half + query group)
            const int32_t csum = share_cs ? lds.xcs[0][d] + lds.xcs[1][d] + lds.xcs[2][d] + lds.xcs[3][d]
                                          : lds.xcs[qg][d] + lds.xcs[2 + qg][d];
            const uint32_t c128 = (P16 ? 257u : 1u) * 128u * static_cast<uint32_t>(csum);
            int32_t acc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = static_cast<int32_t>(lds_u32(xo_addr(1 - H, j, r)));
            // all 16 reads in flight together, one wait (not one per read)
            pin16(acc);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r] = static_cast<int32_t>(static_cast<uint32_t>(acc[r]) + static_cast<uint32_t>(o[db][r]) + c128);
            store_rows(acc, obase + d);
        });
    };
    if (half == 0) finish(std::integral_constant<int, 0>{});
    else finish(std::integral_constant<int, 1>{});
}

template <int D, int NBH, bool P16>
int launch_short_t(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                   const IaKernelParams& kp, hipStream_t stream, int32_t* row_max, uint32_t* row_sum) {
    const int nqb = (kp.Sq + 63) / 64;
    const long long blocks = static_cast<long long>(kp.B) * kp.H * nqb;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    // some 32-key block goes unattended by a whole query group: causal rows,
    // an empty trailing query group, or a second key half shorter than NBH
    // blocks
    const int tail_rows = kp.Sq % 64;
    const bool skip = kp.causal || (tail_rows != 0 && tail_rows <= 32) || kp.Skv <= 64 * NBH - 32;
    const dim3 grid(static_cast<unsigned>(blocks));
    IaKernelParams kq = kp;
    kq.qb_div = invariant_div(static_cast<uint32_t>(nqb));
    auto go = [&](auto skip_c, auto km_c) {
        hipLaunchKernelGGL((ia_short_kernel<D, NBH, decltype(skip_c)::value, decltype(km_c)::value, P16>), grid,
                           dim3(256), 0, stream, q, k, v, out, kq, nqb, row_max, row_sum);
    };
    using T = std::true_type;
    using F = std::false_type;
    using K4 = std::integral_constant<int, 4>;
    using K2 = std::integral_constant<int, 2>;
    using K1 = std::integral_constant<int, 1>;
    using K0 = std::integral_constant<int, 0>;
    if (kp.slot_k == 4) skip ? go(T{}, K4{}) : go(F{}, K4{});
    else if (kp.slot_k == 2) skip ? go(T{}, K2{}) : go(F{}, K2{});
    else if (kp.slot_k == 1) skip ? go(T{}, K1{}) : go(F{}, K1{});
    else skip ? go(T{}, K0{}) : go(F{}, K0{});
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

// Largest number of 32-key blocks per key half served by the short-row
// kernel, per head size (K, later V, of a head in 32 KB of LDS).
constexpr int short_max_half_blocks(int D) { return D == 64 ? 8 : 4; }

template <int D, int NBH, bool P16>
int launch_short_n(int nbh, const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                   const IaKernelParams& kp, hipStream_t stream, int32_t* row_max, uint32_t* row_sum) {
    if constexpr (NBH > short_max_half_blocks(D)) {
        return INTATTN_E_SHAPE;
    } else {
        if (nbh == NBH) return launch_short_t<D, NBH, P16>(q, k, v, out, kp, stream, row_max, row_sum);
        return launch_short_n<D, NBH + 1, P16>(nbh, q, k, v, out, kp, stream, row_max, row_sum);
    }
}

}  // namespace
}  // namespace ia
