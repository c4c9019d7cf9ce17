// attn_prefill_bf16.hip -- fused causal attention forward, bf16 in/out,
// float32 accumulation, on the gfx950 matrix cores, head size 128 (the
// kernel is written for 64 too; head size 64 uses attn_prefill_d64.hip).
//
// What it computes: for every (batch b, query head hq, query row i)
//     o_i = sum_j softmax_j(scale * q_i . k_j + M_ij) v_j
// ("Transformer" (ai-notes) -- Scaled dot-product attention), with
// M_ij = -inf for keys j > q_offset + i ("Transformer" (ai-notes) -- What is
// the causal mask?; "The Transformer architecture" -- Hands-on: query rows
// of a cached step sit at cache.pos + i), and K/V head hq / (Hq / Hkv)
// ("The Transformer architecture" -- GQA groups of n_rep query heads).  The
// T x T score matrix never leaves registers ("Grasping Codes and Math 02" --
// Flash Attention).
//
// Design.  One workgroup = 8 waves in two groups of four.  Both groups cover
// the same 128 query rows (32 per wave), group g of query head 2p + g, so
// their causal extents are identical and they walk the key tiles in
// lockstep.  Waves w and w + 4 share a SIMD.
//  * Ping-pong: a group alternates an MFMA phase (scores of key tile t and
//    the P.V product of tile t - 1) with a softmax phase (mask, weights,
//    row sum of tile t).  Group 1 runs one phase behind group 0, and one
//    s_barrier separates consecutive phases, so on every SIMD one wave feeds
//    the matrix core while the other keeps the vector ALU busy.
//  * One wave issues LDS reads and HBM -> LDS copies only so fast (each
//    blocks its instruction stream for tens of cycles, and an LDS read takes
//    several hundred cycles to return), so that work is split between the
//    phases: the softmax phase reads the K fragments of the next tile into
//    registers and issues this wave's share of the tile copies between its
//    exponentials; the MFMA phase reads one V^T fragment ahead of each score
//    MFMA, for the P.V MFMAs that follow.
//  * Scores are formed transposed, S^T = K Q^T (keys on the MFMA rows,
//    queries on its columns; v_mfma_f32_32x32x16_bf16), so each lane holds
//    scores of ONE query row: the row max and row sum need only one
//    v_permlane32_swap between the two half-waves, and the running max,
//    sum and rescale factor of a row are per-lane scalars.
//  * K and V tiles of 64 keys go from HBM straight into an LDS ring
//    (global_load_lds_dwordx4; no staging registers, no LDS stores) three
//    tiles deep, copied by one group of four waves each, about three phases
//    before use.  When both query heads of a workgroup use the same K/V head
//    (GQA with an even group size) the two groups share one ring (group 1
//    copies K, group 0 V), otherwise each group has its own.  Each 16-byte
//    chunk of a tile row sits at a position XOR-swizzled by the row, so the
//    fragment reads hit distinct LDS banks.
//  * Softmax in base 2: p = 2^(s * |scale| * log2(e) - m) with the raw
//    v_exp_f32, first against the running max m as it stands: only when a
//    row's weights would exceed 2^12 (or on its first tile, where m = -inf)
//    does the row take the tile's max, rescale its accumulator and
//    recompute.  The final division by the row sum cancels whichever m was
//    used.  A negative scale is applied by negating q on load.  The row sum
//    adds the bf16-rounded weights that feed the P.V product
//    (v_dot2_f32_bf16 against (1, 1)), so V = 1 gives O = 1.
//  * P^T, rounded to bf16, is already in the B-operand layout of the second
//    product O^T += V^T P^T.  The A operand V^T is read from the row-major V
//    tile with ds_read_b64_tr_b16 (the LDS transpose read of gfx950), whose
//    four-row gather is matched to the key order of the score accumulator.
//  * Tiles past a wave's last visible key are skipped (the wave still takes
//    part in the barriers); only tiles that straddle the diagonal or the end
//    of the keys pay for masking.
//  * Workgroups are issued longest-first (largest query tile first), and,
//    when the number of head pairs is a multiple of 8, consecutive head
//    pairs (which share K/V heads under GQA) are placed on one XCD
//    (workgroup id modulo 8) so their K/V tiles are served from its L2.
#include <math.h>

#include "internal.hpp"

namespace rocattn {
namespace {

template <int D, bool DUAL>
struct Cfg {
    static constexpr int BN = 64;                        // keys per tile
    static constexpr int BMG = 128;                      // query rows per group
    static constexpr int NCH = D / 8;                    // 16-byte chunks per key row
    static constexpr int TB = BN * D * 2;                // bytes of one K or V tile
    // ring depths (tiles); a tile is copied by the four waves of one group
    static constexpr int NK = (DUAL && D == 64) ? 4 : 3;
    static constexpr int NV = (DUAL && D == 128) ? 2 : 3;
    static constexpr int NINS = BN * NCH / 256;          // copy instructions per lane per tile
    static constexpr int RSTR = 256 / NCH;               // tile rows filled by one copy instruction
    static constexpr int MAXOPS = (DUAL ? 2 : 1) * NINS; // copy instructions per lane per round
    static constexpr int RING = (NK + NV) * TB;          // K slots, then V slots, of one ring
    static constexpr int LDS = (DUAL ? 2 : 1) * RING;
    static_assert(NINS >= 1 && BN % RSTR == 0, "copy instructions must tile the key block");
    static_assert(LDS <= 160 * 1024, "LDS of one workgroup");
};

// XOR swizzles of the 16-byte chunk position within a tile row.
//  K: sixteen consecutive rows read the same logical chunk (ds_read_b128),
//     so the rows' chunks must fall in distinct 16-byte bank groups.
//  V: four consecutive rows are read 64 bytes each (transpose reads), so the
//     rows' 64-byte segments must fall in distinct 64-byte bank groups.
template <int D>
__device__ inline int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ inline int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

struct Args {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    int B, Hq, Hkv, Tq, Tk;
    int R;         // query heads per K/V head
    int HP;        // head pairs per batch entry, ceil(Hq / 2)
    int n_qt;      // query tiles (of 128 rows) per head
    float c;       // |scale| * log2(e), at least 1e-30 so that -inf * c = -inf
    unsigned neg;  // 0x80008000 when scale < 0 (q is negated on load), else 0
    int causal;
    int q_offset;
    int xcd;       // 1: place consecutive head pairs on one XCD
};

__device__ inline float pair_max(float x) {
    // max of this lane's value and the value of the lane 32 apart
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(const lds_void*)p;
}

// One 16-byte HBM -> LDS copy per lane: lane L of the wave writes LDS bytes
// [lds + 16 L, lds + 16 L + 16) with the 16 bytes at sbase + voff.  Written
// as assembly so the compiler does not guard every later LDS read with a
// wait for it; the kernel waits itself (wait_vm) before the barrier that
// publishes the tile.  Nothing else in this kernel uses m0.
__device__ inline void copy16(const void* sbase, unsigned voff, unsigned lds) {
    // base and LDS address are wave-uniform; say so, so they live in SGPRs
    const unsigned long long b = (unsigned long long)sbase;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
    const void* base = (const void*)(((unsigned long long)hi << 32) | lo);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base) : "memory");
}

// Wait until at most n of this wave's vector-memory operations are in flight.
__device__ inline void wait_vm(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    }
}

// Marks a value as read and rewritten here, so its computation stays on this
// side of the following barrier.
template <typename T>
__device__ inline void pin(T& x) {
    asm volatile("" : "+v"(x));
}

__device__ inline void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool DUAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(Args a) {
    typedef Cfg<D, DUAL> C;
    constexpr int BN = C::BN, TB = C::TB, NK = C::NK, NV = C::NV, NINS = C::NINS;
    constexpr int MAXOPS = C::MAXOPS;
    constexpr int NKB = BN / 32;       // 32-key blocks per tile
    constexpr int NDB = D / 32;        // 32-column blocks of the output
    constexpr int NQ = D / 16;         // 16-wide d slices of q.k
    constexpr int NS = NQ * NKB;       // score MFMAs per tile
    constexpr int NKC = BN / 16;       // 16-key slices of a tile
    constexpr int NP = NDB * NKC;      // P.V MFMAs per tile
    constexpr int NE = NKB * 16;       // scores per lane per tile
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7, wave-uniform
    const int grp = wave >> 2, wg = wave & 3;
    const int h = lane >> 5, li = lane & 31;

    // ---- which (query tile, batch, head pair) this workgroup owns
    int qt, unit;
    {
        const int w = blockIdx.x;
        const int P = a.B * a.HP;
        if (a.xcd) {
            const int x = w & 7, s = w >> 3, per = P >> 3;
            const int rank = s / per;
            unit = x * per + (s - rank * per);
            qt = a.n_qt - 1 - rank;
        } else {
            const int rank = w / P;
            unit = w - rank * P;
            qt = a.n_qt - 1 - rank;
        }
    }
    const int b = unit / a.HP, pp = unit - (unit / a.HP) * a.HP;
    const int hq_raw = 2 * pp + grp;
    const bool ghost = hq_raw >= a.Hq;          // odd Hq: the last pair has one head
    const int hq = ghost ? 2 * pp : hq_raw;
    const int hk = hq / a.R;
    const int i0 = qt * C::BMG;
    const int i0w = i0 + 32 * wg;
    const int iq = i0w + li;                    // this lane's query row

    // ---- Q fragment (B operand of S^T): lane holds q[iq][16m + 8h .. +7]
    bf16x8 qf[NQ];
    {
        const int row = iq < a.Tq ? iq : a.Tq - 1;
        const uint4* src = reinterpret_cast<const uint4*>(
            a.q + ((size_t)(b * a.Hq + hq) * a.Tq + row) * D + 8 * h);
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            uint4 u = src[2 * m];
            if (iq >= a.Tq) u = make_uint4(0, 0, 0, 0);
            u.x ^= a.neg; u.y ^= a.neg; u.z ^= a.neg; u.w ^= a.neg;
            qf[m] = __builtin_bit_cast(bf16x8, u);
        }
    }

    // ---- visibility limits (the wave's are wave-uniform)
    const int kv_end = a.causal ? min(a.Tk, a.q_offset + i0 + C::BMG) : a.Tk;
    const int n = (kv_end + BN - 1) / BN;       // key tiles of the workgroup
    const int row_lim = a.causal ? min(a.Tk - 1, a.q_offset + iq) : a.Tk - 1;
    const int wave_last = a.causal ? min(a.Tk - 1, a.q_offset + i0w + 31) : a.Tk - 1;
    // keys below wave_full are visible to every row of the wave
    const int wave_full = a.causal ? min(a.Tk, a.q_offset + i0w + 1) : a.Tk;
    // last tile this wave computes (-1: none)
    const int last = (ghost || i0w >= a.Tq) ? -1 : wave_last / BN;

    // ---- K/V ring: NK K slots, then NV V slots.  With a shared ring, group 1
    //      copies the K tiles and group 0 the V tiles; with one ring per
    //      group, each group copies its own.  Copy round r fills K(r + NK - 1)
    //      and V(r + NV - 2); a wave issues its part of a round during one of
    //      its softmax phases (rounds below 0 form the prologue).
    const unsigned ring = lds_addr(lds) + (DUAL ? (unsigned)(grp * C::RING) : 0u);
    const bf16* kh = a.k + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const bf16* vh = a.v + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    // copy instruction i of a tile: lane (wg, lane) fills the tile's 16-byte
    // slot 256 i + 64 wg + lane, i.e. row cp_r0 + i * RSTR at chunk cp_p
    const int cl = wg * 64 + lane;
    const int cp_r0 = cl / C::NCH, cp_p = cl % C::NCH;
    const unsigned cp_kcol = 16u * (unsigned)(cp_p ^ swz_k<D>(cp_r0));
    const unsigned cp_vcol = 16u * (unsigned)(cp_p ^ swz_v<D>(cp_r0));
    const unsigned cp_lds = (unsigned)(wg * 64 * 16);
    // slots are taken modulo the ring depth for any tile index (negative
    // ones included)
    auto kslot = [&](int t) { return ring + (unsigned)((((t % NK) + NK) % NK) * TB); };
    auto vslot = [&](int t) { return ring + (unsigned)((NK + ((t % NV) + NV) % NV) * TB); };
    auto copy_ins = [&](const bf16* head, int t, unsigned slot, unsigned col, int i) {
        // a tile outside 0 .. n-1 is never read: its copy re-reads a valid
        // tile into the slot it would occupy, which holds no live data then
        const int j0 = min(max(t, 0), n - 1) * BN;
        const char* base = reinterpret_cast<const char*>(head + (size_t)j0 * D);
        // rows past the last key re-read the last key (finite; masked)
        const int row = min(cp_r0 + i * C::RSTR, a.Tk - 1 - j0);
        copy16(base, (unsigned)row * (unsigned)(D * 2) + col, slot + (unsigned)(i * 256 * 16) + cp_lds);
    };
    // Every round issues the same MAXOPS copy instructions per lane (K ones
    // first), so the number of copies in flight after a given round is a
    // compile-time constant.
    auto copy_part = [&](int r, int q0, int q1) {
        const int tk = r + NK - 1, tv = r + NV - 2;
        // shared ring: group 1 copies K(tk), group 0 V(tv) (selected, not branched)
        const bool sk = grp == 1;
        const bf16* sh = sk ? kh : vh;
        const int st = sk ? tk : tv;
        const unsigned ss = sk ? kslot(tk) : vslot(tv);
        const unsigned sc = sk ? cp_kcol : cp_vcol;
#pragma unroll
        for (int q = 0; q < MAXOPS; ++q) {
            if (q < q0 || q >= q1) continue;
            if (DUAL) {
                if (q < NINS) copy_ins(kh, tk, kslot(tk), cp_kcol, q);
                else copy_ins(vh, tv, vslot(tv), cp_vcol, q - NINS);
            } else {
                copy_ins(sh, st, ss, sc, q);
            }
        }
    };
    // wait until this lane's copies of a round have landed while those of
    // the `later` rounds issued after it may still be in flight
    auto wait_rounds_after = [&](int later) { wait_vm(later * MAXOPS); };
    // the round a wave issues during its local phase u (odd u: a softmax or
    // idle phase); below 0: none
    auto round_of = [&](int u) { return (!DUAL && grp == 1) ? (u + 1) >> 1 : (u - 1) >> 1; };

    // ---- per-lane fragment offsets in a tile (bytes).  In both the row
    //      term, the swizzled chunk term and the in-chunk term occupy
    //      disjoint bits, so the offset for slice m (block cb) is the slice-0
    //      offset XOR 32m (64cb).
    // K operand (A of S^T): key row 32kb + li, logical chunk 2m + h
    const unsigned koff = 2u * (unsigned)(li * D + 8 * (h ^ swz_k<D>(li)));
    // V^T operand via transpose reads: supplying lane (16g + 4r + qq) points
    // at V[key_base + 4(g/2) + r][32 cb + 16(g%2) + 4qq] (logical column)
    const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
    const unsigned voff =
        2u * (unsigned)((4 * (tg >> 1) + tr) * D + 16 * (tg & 1) + 4 * tq + 8 * swz_v<D>(tr));

    f32x16 oacc[NDB];
#pragma unroll
    for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    f32x16 sacc[NKB];
    bf16x8 pb[NKC];
    float m_run = -INFINITY, l_a = 0.f, l_b = 0.f;
    const float cs = a.c;

    // K fragments of the next tile, read into registers during the softmax
    // phase (so the LDS reads of a SIMD are spread over both of its waves)
    bf16x8 kpre[NS];
    // One MFMA phase: S^T = K(t) Q^T on the prefetched K fragments (when
    // `scores`), then O^T += V^T(tv) P^T (when tv >= 0).  The V^T fragment of
    // P.V MFMA j is read before score MFMA j, so it has the whole score
    // product to arrive (an LDS read takes several hundred cycles); its
    // registers take the place of the K fragment just consumed.  Hard
    // scheduling fences keep that order.
    auto mfma_phase = [&](bool scores, int tv) {
        const unsigned vb0 = vslot(tv < 0 ? 0 : tv) + voff;
        auto vfrag = [&](int j) {
            const int kc = j / NDB, cb = j % NDB;
            const unsigned addr = (vb0 + (unsigned)(16 * kc * D * 2)) ^ (64u * cb);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr);
            const i16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(addr + 16u * D));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 vf[NP];
        if (scores) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                if (tv >= 0 && i < NP) vf[i] = vfrag(i);
                __builtin_amdgcn_sched_barrier(0);
                const int m = i / NKB, kb = i % NKB;
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kpre[i], qf[m],
                                                                   i < NKB ? f32x16{} : sacc[kb], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) pin(sacc[kb]);
        }
        if (tv >= 0) {
            constexpr int DONE = NS < NP ? NS : NP;   // fragments already read
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                if (!scores || j >= DONE) vf[j] = vfrag(j);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int kc = j / NDB, cb = j % NDB;
                oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], pb[kc], oacc[cb], 0, 0, 0);
            }
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb) pin(oacc[cb]);
        }
    };

    // key offset (within the tile) of score element e = 16 kb + r of a lane
    auto key_of = [&](int e) { return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + (e & 3); };
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    // weights p = 2^(s c - m) of 16-key slice kc in bf16 (the B operand of
    // P.V) and this lane's part of their sum
    auto weights_kc = [&](int kc, float m, float& sa, float& sb) {
        const float nm = -m;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = 8 * kc + 2 * u;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], cs, nm));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][(e + 1) & 15], cs, nm));
            bf16x2 pk;
            pk[0] = (bf16)p0;
            pk[1] = (bf16)p1;
            pb[kc][2 * u] = pk[0];
            pb[kc][2 * u + 1] = pk[1];
            if (u & 1) sb = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, sb, false);
            else sa = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, sa, false);
        }
    };
    auto kfrag_read = [&](int t, int i) {
        const int m = i / NKB, kb = i % NKB;
        const unsigned addr = (kslot(t) + koff + (unsigned)(kb * 32 * D * 2)) ^ (32u * m);
        kpre[i] = *(lds_bf16x8*)(uintptr_t)addr;
    };

    // softmax phase of tile t (issuing copy round r): mask, then
    // per 16-key slice the weights against the running max, with the K
    // fragment reads of tile t + 1 and the copy instructions spread between
    // the slices (one wave issues LDS reads and copies only so fast).  Only
    // when some weight would exceed 2^12 (or on the first tile, where the
    // running max is -inf) take the row max, raise the running max and
    // recompute.
    constexpr int CPC = (MAXOPS + NKC - 1) / NKC;              // copies per slice
    auto softmax_phase = [&](int t, int r) {
        const int j0 = t * BN;
        if (j0 + BN > wave_full) {
            const int lim = row_lim - (j0 + 4 * h);
#pragma unroll
            for (int e = 0; e < NE; ++e)
                if (key_of(e) > lim) sacc[e >> 4][e & 15] = -INFINITY;
        }
        float sa = 0.f, sb = 0.f;
        // the K fragment reads go first: an LDS read takes several hundred
        // cycles to return (a read of a tile this wave will not use is harmless)
#pragma unroll
        for (int i = 0; i < NS; ++i) kfrag_read(t + 1, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            copy_part(r, kc * CPC, (kc + 1) * CPC);
            weights_kc(kc, m_run, sa, sb);
            __builtin_amdgcn_sched_barrier(0);
        }
        const bool big = !(sa + sb <= 4096.f);
        if (__any(big)) {
            // rows (both half-wave lanes of a row) whose weights got too big
            // take their tile max; the other rows keep m_run (alpha = 1) and
            // recompute the very same weights
            const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)big, (unsigned)big, false, false);
            const bool row_big = (sw[0] | sw[1]) != 0u;
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < NE; ++e) mx = fmaxf(mx, sacc[e >> 4][e & 15]);
            const float tmax = pair_max(mx) * cs;
            const float m_new = row_big ? fmaxf(m_run, tmax) : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_a *= alpha;
            l_b *= alpha;
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) oacc[cb][rr] *= alpha;
            m_run = m_new;
            sa = 0.f;
            sb = 0.f;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) weights_kc(kc, m_run, sa, sb);
        }
        l_a += sa;
        l_b += sb;
        // the weights, sums and prefetched fragments are finished inside this
        // phase, not sunk past the barrier into the next one
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) pin(pb[kc]);
        pin(l_a);
        pin(l_b);
#pragma unroll
        for (int i = 0; i < NS; ++i) pin(kpre[i]);
    };

    // ---- prologue: copy rounds 1-NK .. -1; K(0) lands before the first barrier
    for (int r = 1 - NK; r < 0; ++r) copy_part(r, 0, MAXOPS);
    if (DUAL || grp == 1) wait_rounds_after(NK - 2);
    phase_barrier();
    if (last >= 0) {
#pragma unroll
        for (int i = 0; i < NS; ++i) kfrag_read(0, i);
    }

    // ---- phases 0 .. 2n + 1, one barrier between consecutive phases.
    //      Group g runs MFMA(t) in local phase u = p - g = 2t and softmax(t)
    //      in u = 2t + 1.  Before softmax(s) of either group K(s + 1) has
    //      landed (its fragments are read then); before MFMA(s + 1), V(s).
    //      K(s + 1) is copied in round s + 2 - NK, V(s) in round s + 2 - NV.
    const int nph = 2 * n + 2;
    auto end = [&](int p) {
        if (p + 1 >= nph) return;
        const int u = p - grp;
        if (DUAL) {
            // rounds issued so far: up to s - 1 after an MFMA phase (u = 2s),
            // up to s after a softmax phase (u = 2s + 1)
            if (u >= 0 && (u & 1) == 0) wait_rounds_after(NK - 3);   // K(s + 1)
            else if (u >= 0) wait_rounds_after(NV - 2);               // V(s)
        } else if (u & 1) {
            // group 1 has issued rounds up to s = (u + 1) / 2 and needs
            // K(s + 1); group 0 up to s = (u - 1) / 2 and needs V(s)
            wait_rounds_after(grp == 1 ? NK - 2 : NV - 2);
        }
        phase_barrier();
    };
    auto idle = [&](int p) {
        const int u = p - grp;
        if (u & 1) {
            const int r = round_of(u);
            if (r >= 0) copy_part(r, 0, MAXOPS);
        }
        end(p);
    };

    int p = 0;
    if (grp == 1) {  // group 1 idles in phase 0
        idle(0);
        p = 1;
    }
    if (last >= 0) {
        __builtin_amdgcn_s_setprio(1);
        mfma_phase(true, -1);
        __builtin_amdgcn_s_setprio(0);
        end(p);
        ++p;
        softmax_phase(0, round_of(1));
        end(p);
        ++p;
        for (int t = 1; t <= last; ++t) {
            __builtin_amdgcn_s_setprio(1);
            mfma_phase(true, t - 1);
            __builtin_amdgcn_s_setprio(0);
            end(p);
            ++p;
            softmax_phase(t, round_of(2 * t + 1));
            end(p);
            ++p;
        }
        __builtin_amdgcn_s_setprio(1);
        mfma_phase(false, last);
        __builtin_amdgcn_s_setprio(0);
        end(p);
        ++p;
    }
    for (; p < nph; ++p) idle(p);  // tiles past this wave's rows: keep the ring moving
    wait_vm(0);                     // no copy into LDS outlives the workgroup

    // ---- epilogue: O = O^T / l, lane holds columns 32cb + 8g4 + 4h .. +3 of row iq
    const float l_tot = pair_sum(l_a + l_b);
    if (!ghost && iq < a.Tq) {
        const float inv = 1.f / l_tot;
        bf16* orow = a.o + ((size_t)(b * a.Hq + hq) * a.Tq + iq) * D;
#pragma unroll
        for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = (bf16)(oacc[cb][4 * g4 + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * g4 + 4 * h) = val;
            }
        if (a.lse && h == 0)
            a.lse[(size_t)(b * a.Hq + hq) * a.Tq + iq] = (m_run + log2f(l_tot)) * kLn2;
    }
}

template <int D, bool DUAL>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
    typedef Cfg<D, DUAL> C;
    Args a;
    a.q = static_cast<const bf16*>(p.q);
    a.k = static_cast<const bf16*>(p.k);
    a.v = static_cast<const bf16*>(p.v);
    a.o = static_cast<bf16*>(p.o);
    a.lse = p.lse;
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Tq = p.Tq; a.Tk = p.Tk;
    a.R = p.Hq / p.Hkv;
    a.HP = (p.Hq + 1) / 2;
    a.n_qt = (p.Tq + C::BMG - 1) / C::BMG;
    a.c = fmaxf(fabsf(p.scale) * kLog2e, 1e-30f);
    a.neg = p.scale < 0.f ? 0x80008000u : 0u;
    a.causal = p.causal;
    a.q_offset = p.causal ? p.q_offset : 0;
    const long long units = (long long)a.B * a.HP;
    a.xcd = (units % 8 == 0) ? 1 : 0;
    const long long nwg = (long long)a.n_qt * units;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, DUAL>), dim3((unsigned)nwg), dim3(512), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16_d128(const FwdParams& p, hipStream_t stream) {
    // the two query heads 2p, 2p + 1 of a workgroup share a K/V head iff the
    // group size Hq / Hkv is even
    const bool shared = (p.Hq / p.Hkv) % 2 == 0;
    return shared ? launch_d<128, false>(p, stream) : launch_d<128, true>(p, stream);
}

}  // namespace rocattn
