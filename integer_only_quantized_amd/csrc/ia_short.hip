// Short-row integer attention kernel (gfx950 / CDNA4): the whole key range
// of a head resident in LDS (Skv <= 512 at d = 64, <= 256 at d = 128).
//
// Method: IntAttention digest pages (arXiv 2511.21513v1), "Methodology",
// steps 2-3; integer widths and roundings as stated in include/intattn.h.
#include "ia_device.h"

namespace ia {
namespace {

// Short-row kernel: the whole key range of a head (NKB blocks of 32 keys, a
// compile-time count) stays resident in LDS for the whole workgroup: K
// row-major (padded rows) and V transposed in the P-operand key order. Each
// wave owns 32 query rows.
//   pass 1: S^T blocks from K in LDS -> per-lane row max;
//   pass 2: S^T - m (the MFMA accumulator starts from -m) -> slot -> table
//           lookup -> row sum; each score's slot is kept in registers as one
//           byte (4 * slot);
//   tables: each row's 32 probabilities (p ^ 0x80, i.e. p - 128 as int8) in
//           LDS, reusing the K area;
//   pass 3: P operand = per-row table indexed by the stored slot bytes, then
//           P.V on the MFMA with V^T from LDS, plus one MFMA against an
//           all-ones operand that yields the column sums of the V rows fed.
// V is prefetched into registers before pass 1 and written to LDS after
// pass 2, so its load latency hides behind passes 1 and 2.
//
// Slot arithmetic (FAST, used when M < 2^21): with y = s - m <= 0,
//   t = sat_int32(y * (-4M) + 2^25),  slot = t >> 26.
// Scaling the spec's (x*M + 2^23) >> 24 by 4 gives the same quotient; the
// value is below 2^31 whenever slot < 31, and saturation to 2^31 - 1 lands
// exactly in slot 31, so the clip costs nothing. Masked keys use y = -2^23.
// Otherwise the explicit clip s' = max(s, m - x_clip) is used and the slot is
// moved to the same bit position with one shift.
template <int D, int NKB>
struct ShortLds {
    static constexpr int KPAD = 32 * NKB;
    static constexpr int KStride = D + 16;     // padded K row: conflict-free 16-byte reads
    static constexpr int VStride = KPAD + 16;  // padded V^T row
    static constexpr int PTBlock = 132;        // 4 interleaved row tables (bank spread)
    static constexpr int KBytes = KPAD * KStride > 8 * 8 * PTBlock ? KPAD * KStride : 8 * 8 * PTBlock;
    uint32_t lut[32];                          // first member: LDS byte address 0
    int8_t k[KBytes];                          // K, later the probability tables
    int8_t vt[D * VStride];
};

template <int D, int NKB, bool FAST>
__global__ __launch_bounds__(512) void ia_short_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, const int8_t* __restrict__ v,
    int8_t* __restrict__ out, const IaKernelParams P, int nqb, int32_t* __restrict__ row_max,
    uint32_t* __restrict__ row_sum) {
    using L = ShortLds<D, NKB>;
    constexpr int KPAD = L::KPAD;
    constexpr int KS = D / 32;
    constexpr int DB = D / 32;
    constexpr int KStride = L::KStride;
    constexpr int VStride = L::VStride;

    __shared__ __attribute__((aligned(16))) L lds;

    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nw = nthreads >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    int bid = xcd_local_block(blockIdx.x, gridDim.x);
    const int qb = bid % nqb;
    bid /= nqb;
    const int h = bid % P.H;
    const int b = bid / P.H;
    const size_t head = static_cast<size_t>(b) * P.H + h;
    const int8_t* qh = q + head * P.Sq * D;
    const int8_t* kh = k + head * P.Skv * D;
    const int8_t* vh = v + head * P.Skv * D;

    // ---- stage K (rounds of eight 16-byte loads in flight per thread) -------
    constexpr int KCH = KPAD * (D / 16);
    for (int base = 0; base < KCH; base += 8 * nthreads) {
        v4i val[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = base + u * nthreads + tid;
            const int row = c / (D / 16), ch = c % (D / 16);
            val[u] = v4i{0, 0, 0, 0};
            if (c < KCH && row < P.Skv)
                val[u] = *reinterpret_cast<const v4i*>(kh + static_cast<size_t>(row) * D + 16 * ch);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = base + u * nthreads + tid;
            const int row = c / (D / 16), ch = c % (D / 16);
            if (c < KCH) *reinterpret_cast<v4i*>(&lds.k[row * KStride + 16 * ch]) = val[u];
        }
    }
    // ---- prefetch V (4 keys x 16 value columns per item, two items/thread) --
    constexpr int VIT = (KPAD / 4) * (D / 16);
    auto load_v = [&](int c, v4i (&r)[4]) {
        const int dc = c % (D / 16), key0 = 4 * (c / (D / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[i] = v4i{0, 0, 0, 0};
            if (c < VIT && key0 + i < P.Skv)
                r[i] = *reinterpret_cast<const v4i*>(vh + static_cast<size_t>(key0 + i) * D + 16 * dc);
        }
    };
    auto store_vt = [&](int c, const v4i (&r)[4]) {
        if (c >= VIT) return;
        const int dc = c % (D / 16), key0 = 4 * (c / (D / 16));
        const int pos = 32 * (key0 >> 5) + vt_pos(key0 & 31);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // 4x4 byte transpose: keys key0..key0+3, value columns 16dc+4w..+3
            const uint32_t r0 = r[0][w], r1 = r[1][w], r2 = r[2][w], r3 = r[3][w];
            const uint32_t u0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
            const uint32_t u1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
            const uint32_t u2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
            const uint32_t u3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
            const int d0 = 16 * dc + 4 * w;
            *reinterpret_cast<uint32_t*>(&lds.vt[(d0 + 0) * VStride + pos]) = __builtin_amdgcn_perm(u2, u0, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&lds.vt[(d0 + 1) * VStride + pos]) = __builtin_amdgcn_perm(u2, u0, 0x07060302u);
            *reinterpret_cast<uint32_t*>(&lds.vt[(d0 + 2) * VStride + pos]) = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&lds.vt[(d0 + 3) * VStride + pos]) = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
        }
    };
    v4i vpre[2][4];
    load_v(tid, vpre[0]);
    load_v(tid + nthreads, vpre[1]);

    if (tid < 32) lds.lut[tid] = lut_entry(P, tid);
    __syncthreads();

    const int shift = P.Skv - P.Sq;
    const int qw0 = qb * 32 * nw + wave * 32;
    const int qrow = qw0 + l32;
    const int kend_row = P.causal ? min(P.Skv, qrow + shift + 1) : P.Skv;
    const int kend_wave = P.causal ? min(P.Skv, qw0 + shift + 1) : P.Skv;

    v4i qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (qrow < P.Sq)
            qf[ks] = *reinterpret_cast<const v4i*>(qh + static_cast<size_t>(qrow) * D + 32 * ks + 16 * hh);
        else
            qf[ks] = v4i{0, 0, 0, 0};
    }

    // S^T block (MFMA only) starting from accumulator c0
    auto scores = [&](int kb, const v16i& c0) {
        v16i s = c0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v4i a = *reinterpret_cast<const v4i*>(&lds.k[(32 * kb + l32) * KStride + 32 * ks + 16 * hh]);
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

    // Each pass is software-pipelined by hand (MFMAs of block kb+1 issued
    // before the integer work on block kb) and fenced per block with a
    // scheduling barrier; empty asm statements pin per-block reductions so
    // the compiler cannot defer them into one cross-block tree.

    // ---- pass 1: row max ---------------------------------------------------
    const v16i zero16 = v16i{};
    int32_t mrow = INT_MIN;
    {
        v16i cur = scores(0, zero16);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            v16i nxt;
            if (kb + 1 < NKB) nxt = scores(kb + 1, zero16);
            mask(cur, kb, INT_MIN);
#pragma unroll
            for (int r = 0; r < 16; r += 2) mrow = max(mrow, max(cur[r], cur[r + 1]));
            asm volatile("" : "+v"(mrow));
            if (kb + 1 < NKB) cur = nxt;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    mrow = max(mrow, __shfl_xor(mrow, 32));
    asm volatile("" ::: "memory");   // re-read K fragments in pass 2

    // ---- pass 2: slots, table lookups, row sum; slot bytes kept ------------
    const uint8_t* const ldsb_c = reinterpret_cast<const uint8_t*>(&lds);
    uint32_t idxw[NKB][4];
    uint32_t E = 0;
    {
        v16i cinit;
        int32_t negM4 = 0, half4 = 1 << 25, lo = 0, negM = 0;
        uint32_t C = 0;
        if constexpr (FAST) {
#pragma unroll
            for (int r = 0; r < 16; ++r) cinit[r] = -mrow;
            negM4 = -4 * P.idx_mul;
        } else {
            cinit = zero16;
            lo = mrow - P.x_clip;
            C = static_cast<uint32_t>(mrow) * static_cast<uint32_t>(P.idx_mul) + (1u << 23);
            negM = -P.idx_mul;
        }
        // 4 * slot of each score, in bits 26..30 of t (byte 3 = 4 * slot + fraction)
        auto slot_word = [&](int32_t y) -> uint32_t {
            if constexpr (FAST) {
                int32_t t;
                asm("v_mad_i32_i24 %0, %1, %2, %3 clamp" : "=v"(t) : "v"(y), "v"(negM4), "v"(half4));
                return static_cast<uint32_t>(t);
            } else {
                const int32_t sp = max(y, lo);
                return (C + static_cast<uint32_t>(__mul24(sp, negM))) << 2;
            }
        };
        v16i cur = scores(0, cinit);
        uint32_t ep[16];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            v16i nxt;
            if (kb + 1 < NKB) nxt = scores(kb + 1, cinit);
            mask(cur, kb, FAST ? -(1 << 23) : INT_MIN);
            uint32_t en[16];
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                uint32_t t[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    t[c] = slot_word(cur[4 * w4 + c]);
                    // table entry at byte 4 * slot = (t >> 24) & 0x7c
                    en[4 * w4 + c] = *reinterpret_cast<const uint32_t*>(ldsb_c + ((t[c] >> 24) & 0x7cu));
                }
                const uint32_t w01 = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0703u);
                const uint32_t w23 = __builtin_amdgcn_perm(t[3], t[2], 0x0c0c0703u);
                idxw[kb][w4] = __builtin_amdgcn_perm(w23, w01, 0x05040100u) & 0x7c7c7c7cu;
                // keep the packed word (not the four values it came from)
                // live until pass 3
                asm volatile("" : "+v"(idxw[kb][w4]));
            }
            // lookups of the previous block are summed one block later
            if (kb > 0) {
#pragma unroll
                for (int i = 0; i < 16; i += 2) E += ep[i] + ep[i + 1];
                asm volatile("" : "+v"(E));
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) ep[i] = en[i];
            if (kb + 1 < NKB) cur = nxt;
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) E += ep[i] + ep[i + 1];
    }
    E += __shfl_xor(E, 32);
    const uint32_t R = ((255u << 23) + (E >> 1)) / E;
    if (row_max != nullptr && hh == 0 && qrow < P.Sq) {
        row_max[head * P.Sq + qrow] = mrow;
        row_sum[head * P.Sq + qrow] = E;
    }

    // ---- V^T into LDS (prefetched items, then any remaining ones) -----------
    store_vt(tid, vpre[0]);
    store_vt(tid + nthreads, vpre[1]);
    for (int c = tid + 2 * nthreads; c < VIT; c += nthreads) {
        v4i r[4];
        load_v(c, r);
        store_vt(c, r);
    }
    __syncthreads();   // V^T complete; every wave is done with K

    // ---- per-row probability tables (wave-private, in the K area) -----------
    // Rows are interleaved four to a 132-byte block: entry (row, slot) at
    // byte block*132 + 4*slot + (row & 3), so equal slots of different
    // blocks fall in different banks.
    uint32_t pbase = static_cast<uint32_t>(offsetof(L, k)) + (wave * 8 + (l32 >> 2)) * L::PTBlock + (l32 & 3);
    asm volatile("" : "+v"(pbase));
    uint8_t* const ldsb = reinterpret_cast<uint8_t*>(&lds);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int kslot = 16 * hh + j;
        const uint32_t p = (lds.lut[kslot] * R + (1u << 22)) >> 23;
        ldsb[pbase + 4 * kslot] = static_cast<uint8_t>(p ^ 0x80u);
    }
    // the tables are read only by the wave that wrote them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- pass 3: P from the tables, P.V and column sums on the MFMA ---------
    // Three stages in flight: table lookups for block kb+2, byte packing of
    // block kb+1, MFMAs of block kb.
    auto plookup = [&](int kb, uint32_t (&pl)[16]) {
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            const uint32_t x = idxw[kb][w4];
            pl[4 * w4 + 0] = ldsb[pbase + (x & 0xffu)];
            pl[4 * w4 + 1] = ldsb[pbase + ((x >> 8) & 0xffu)];
            pl[4 * w4 + 2] = ldsb[pbase + ((x >> 16) & 0xffu)];
            pl[4 * w4 + 3] = ldsb[pbase + (x >> 24)];
        }
    };
    auto ppack = [&](const uint32_t (&pl)[16]) {
        uint32_t pw[4];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            const uint32_t lo2 = __builtin_amdgcn_perm(pl[4 * w4 + 1], pl[4 * w4 + 0], 0x0c0c0400u);
            const uint32_t hi2 = __builtin_amdgcn_perm(pl[4 * w4 + 3], pl[4 * w4 + 2], 0x0c0c0400u);
            pw[w4] = __builtin_amdgcn_perm(hi2, lo2, 0x05040100u);
        }
        return v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]), static_cast<int>(pw[2]),
                   static_cast<int>(pw[3])};
    };
    const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
    v16i o[DB], oc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        o[db] = v16i{};
        oc[db] = v16i{};
    }
    {
        uint32_t pl[16];
        plookup(0, pl);
        v4i pa = ppack(pl);
        if (NKB > 1) plookup(1, pl);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            v4i pnext;
            if (kb + 1 < NKB) pnext = ppack(pl);
            if (kb + 2 < NKB) plookup(kb + 2, pl);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const v4i vb = *reinterpret_cast<const v4i*>(&lds.vt[(32 * db + l32) * VStride + 32 * kb + 16 * hh]);
                o[db] = mfma_i8_32x32x32(pa, vb, o[db]);
                oc[db] = mfma_i8_32x32x32(ones, vb, oc[db]);
            }
            if (kb + 1 < NKB) pa = pnext;
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- requantise and store -----------------------------------------------
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + l32;
        const int32_t cs = oc[db][0];   // every row of ones x V^T is the column sum
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qi = qw0 + acc_row(r, hh);
            if (qi >= P.Sq) continue;
            out[(head * P.Sq + qi) * D + d] = requantise(o[db][r] + 128 * cs, P);
        }
    }
}

template <int D, int NKB>
int launch_short_t(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                   const IaKernelParams& kp, hipStream_t stream, int32_t* row_max, uint32_t* row_sum) {
    // the saturating slot form needs 4*M to fit the 24-bit multiplier operand
    const bool fast = kp.idx_mul < (1 << 21);
    const int nqb32 = (kp.Sq + 31) / 32;
    const long long heads = static_cast<long long>(kp.B) * kp.H;
    // waves per workgroup: as many as there are 32-row query blocks (<= 8),
    // halved while the grid would leave compute units idle
    int nw = nqb32 < 8 ? nqb32 : 8;
    while (nw > 1 && heads * ((nqb32 + nw - 1) / nw) < 256) nw = (nw + 1) / 2;
    const int nqb = (nqb32 + nw - 1) / nw;
    const long long blocks = heads * nqb;
    if (blocks > INT_MAX) return INTATTN_E_SHAPE;
    if (fast)
        hipLaunchKernelGGL((ia_short_kernel<D, NKB, true>), dim3(static_cast<unsigned>(blocks)), dim3(64 * nw),
                           0, stream, q, k, v, out, kp, nqb, row_max, row_sum);
    else
        hipLaunchKernelGGL((ia_short_kernel<D, NKB, false>), dim3(static_cast<unsigned>(blocks)), dim3(64 * nw),
                           0, stream, q, k, v, out, kp, nqb, row_max, row_sum);
    return hipGetLastError() == hipSuccess ? INTATTN_OK : INTATTN_E_HIP;
}

// Largest number of 32-key blocks served by the short-row kernel, per head
// size (K, V^T and the tables stay under 80 KB of LDS: two workgroups per CU).
constexpr int short_max_blocks(int D) { return D == 64 ? 16 : 8; }

template <int D, int NKB>
int launch_short_n(int nkb, const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out,
                   const IaKernelParams& kp, hipStream_t stream, int32_t* row_max, uint32_t* row_sum) {
    if constexpr (NKB > short_max_blocks(D)) {
        return INTATTN_E_SHAPE;
    } else {
        if (nkb == NKB) return launch_short_t<D, NKB>(q, k, v, out, kp, stream, row_max, row_sum);
        return launch_short_n<D, NKB + 1>(nkb, q, k, v, out, kp, stream, row_max, row_sum);
    }
}

}  // namespace

int short_max_keys(int D) { return 32 * short_max_blocks(D); }

int launch_short(const int8_t* q, const int8_t* k, const int8_t* v, int8_t* out, int D,
                 const IaKernelParams& kp, void* stream, int32_t* row_max, uint32_t* row_sum) {
    const int nkb = (kp.Skv + 31) / 32;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (D == 64) return launch_short_n<64, 1>(nkb, q, k, v, out, kp, s, row_max, row_sum);
    return launch_short_n<128, 1>(nkb, q, k, v, out, kp, s, row_max, row_sum);
}


}  // namespace ia
