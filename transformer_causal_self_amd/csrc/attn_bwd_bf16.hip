// attn_bwd_bf16.hip -- gradients of the fused causal attention, bf16 in/out,
// float32 accumulation, on the gfx950 matrix cores, head sizes 64 and 128.
//
// What it computes: for an upstream gradient dO of o = softmax(scale S + M) V,
// S = Q K^T, per (batch, query head):
//     P   = exp(scale S - lse)           (the forward's weights, rebuilt from
//                                          its log-sum-exp rows)
//     dV  = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
//     dS  = P (dP - D),   dQ = scale dS K,   dK = scale dS^T Q,
// the chain rule of the forward through the softmax ("The Transformer
// architecture" -- Softmax is a differentiable allocation; the operator is
// trained in "Transformer Math and Implementation Deep Dive" -- What To
// Implement: tiny training loop).  A K/V head sums dK and dV over the
// query heads of its group ("The Transformer architecture" -- GQA), in a
// fixed order, so results are deterministic.  D_i equals sum_j P_ij dP_ij.
//
// Two launches, each a plain adaptation of the forward's tile scheme:
//  * bwd_dq_kernel: one workgroup = 4 waves x 32 query rows.  First each
//    row's statistics: lse as a base-2 exponent and D = rowsum(dO * O),
//    which the wave also writes to the workspace, 64 floats per 32-row tile
//    (32 lse, then 32 D; rows past Tq get 0), so the dK/dV kernel finds a
//    tile's row statistics in one contiguous 256-byte block.  It then walks the
//    32-key tiles of its rows like the forward (S^T = K Q^T with keys on the
//    MFMA rows, one query per lane), forms dP^T = V dO^T the same way, then
//    dQ^T += K^T dS^T with K^T read by the LDS transpose read.  Per tile the
//    ring holds K and V with the row-read swizzle and K again with the
//    transpose-read swizzle.
//  * bwd_dkv_kernel: one workgroup = 4 waves x 32 keys; it walks the 32-row
//    query tiles of every query head of the group (S = Q K^T with queries on
//    the MFMA rows, one key per lane), and accumulates dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T and Q^T from transpose reads.  The rows' lse
//    and D values travel with the query tile through LDS.  Head size 64
//    runs this kernel (two waves per SIMD); head size 128 runs
//    bwd_dkv_pair_kernel, which splits a key block's work between two waves
//    (S, P and dV / dP, dS and dK) so that it too fits two waves per SIMD.
// Rows past Tq and keys past Tk contribute nothing; keys no query can see
// get dK = dV = 0.
#include <math.h>

#include "internal.hpp"
#include "mfma_tiles.hpp"

namespace rocattn {
namespace {

struct BwdArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const bf16* o;
    const bf16* dO;
    const float* lse;   // natural-log row log-sum-exp of the forward [B][Hq][Tq]
    float* stats;       // workspace [B * Hq][n_rt][64]: lse * log2(e), then D, of a row tile
    bf16* dq;
    bf16* dk;
    bf16* dv;
    int B, Hq, Hkv, Tq, Tk, R;
    int n_rt;           // 32-row tiles per head
    float c;            // scale * log2(e)
    float scale;
    int causal, q_offset;
};

template <int D, int NW_ = 4>
struct BCfg {
    static constexpr int BN = 32;               // keys (dq) or query rows (dkv) per tile
    static constexpr int NW = NW_;              // waves per workgroup (all of them copy)
    static constexpr int BM = 4 * 32;           // rows (dq) or keys (dkv) per workgroup
    static constexpr int NQ = D / 16;           // 16-wide d slices of a product over d
    static constexpr int NDB = D / 32;          // 32-row blocks of d in the accumulators
    static constexpr int NKC = 2;               // 16-wide slices of a 32-long tile
    static constexpr int NCH = D / 8;           // 16-byte chunks per row
    static constexpr int TB = BN * D * 2;       // bytes of one tile
    static constexpr int CPL = NW * 64;         // lanes that copy
    static constexpr int NINS = BN * NCH / CPL; // 16-byte copies per lane per tile
    static constexpr int RSTR = CPL / NCH;      // tile rows filled by one copy instruction
    static_assert(NINS >= 1 && BN * NCH == NINS * CPL, "every lane copies whole chunks of a tile");
};

// offset (before + 4h) of element e of a 32x32 accumulator block along its rows
__device__ inline int row_of(int e) { return 8 * (e >> 2) + (e & 3); }

// ---------------------------------------------------------------------------
// Per-lane tile addressing shared by the two gradient kernels.
template <int D, int NW = 4>
struct TileLanes {
    typedef BCfg<D, NW> C;
    int cp_r0;
    unsigned cp_kcol, cp_vcol, cp_lds;
    unsigned koff, voff;   // row-read and transpose-read offsets in a tile
    __device__ TileLanes(int wave, int lane) {
        const int cl = wave * 64 + lane;
        cp_r0 = cl / C::NCH;
        const int cp_p = cl % C::NCH;
        cp_kcol = 16u * (unsigned)(cp_p ^ swz_k<D>(cp_r0));
        cp_vcol = 16u * (unsigned)(cp_p ^ swz_v<D>(cp_r0));
        cp_lds = (unsigned)(wave * 64 * 16);
        const int h = lane >> 5, li = lane & 31;
        koff = 2u * (unsigned)(li * D + 8 * (h ^ swz_k<D>(li)));
        const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
        voff = 2u * (unsigned)((4 * (tg >> 1) + tr) * D + 16 * (tg & 1) + 4 * tq + 8 * swz_v<D>(tr));
    }
    // copy rows [j0, j0 + BN) of a [T][D] matrix (rows past T - 1 repeat row
    // T - 1) into the tile at `slot`, chunk positions swizzled by `col`
    __device__ void copy(const bf16* m, int T, int j0, unsigned slot, unsigned col) const {
#pragma unroll
        for (int i = 0; i < C::NINS; ++i) {
            const int row = min(cp_r0 + i * C::RSTR, T - 1 - j0);
            copy16(m + (long long)j0 * D, (unsigned)row * (unsigned)(D * 2) + col,
                   slot + (unsigned)(i * C::CPL * 16) + cp_lds);
        }
    }
    // row operand: row li of the tile, d slice m (16 wide), half h
    __device__ bf16x8 rowfrag(unsigned tile, int m) const {
        return *(lds_bf16x8*)(uintptr_t)((tile + koff) ^ (32u * m));
    }
    // transposed operand: d-block cb (32 wide) over tile rows slice kc
    // (16 rows, in the row order of an accumulator block's elements)
    __device__ bf16x8 trfrag(unsigned tile, int cb, int kc) const {
        const unsigned addr = (tile + voff + (unsigned)(16 * kc * D * 2)) ^ (64u * cb);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(addr + 16u * D));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// One copy of a tile serving both read patterns (head size 128): the
// 16-byte chunk c of row r sits at chunk position c ^ (4 (r & 3) ^ (r >> 2 & 3)).
// Sixteen consecutive rows then take sixteen distinct positions (row reads of
// one logical chunk hit distinct banks), and four consecutive rows with the
// same r >> 2 put an aligned 64-byte segment in four distinct 64-byte bank
// groups (transpose reads).  Offsets as in TileLanes; the transpose read's
// second 8-row half, rows r + 8, has the swizzle of row r with chunk bit 1
// flipped, so its address is the first half's with byte bit 5 flipped,
// 8 rows further on.
template <int D, int NW>
struct OneTileLanes {
    typedef BCfg<D, NW> C;
    static_assert(D == 128, "the combined swizzle is laid out for 256-byte rows");
    static __device__ int swz(int r) { return (4 * (r & 3)) ^ ((r >> 2) & 3); }
    int cp_r0;
    unsigned cp_col, cp_lds;
    unsigned roff, toff;
    __device__ OneTileLanes(int wave, int lane) {
        const int cl = wave * 64 + lane;
        cp_r0 = cl / C::NCH;
        cp_col = 16u * (unsigned)((cl % C::NCH) ^ swz(cp_r0));
        cp_lds = (unsigned)(wave * 64 * 16);
        const int h = lane >> 5, li = lane & 31;
        roff = 2u * (unsigned)(li * D) + 16u * (unsigned)(h ^ swz(li));
        const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
        const int c0 = 2 * (tg & 1) + (tq >> 1), r = 4 * (tg >> 1) + tr;
        toff = 2u * (unsigned)(r * D) + 16u * (unsigned)(c0 ^ swz(r)) + 8u * (unsigned)(tq & 1);
    }
    __device__ void copy(const bf16* m, int T, int j0, unsigned slot) const {
#pragma unroll
        for (int i = 0; i < C::NINS; ++i) {
            const int row = min(cp_r0 + i * C::RSTR, T - 1 - j0);
            copy16(m + (long long)j0 * D, (unsigned)row * (unsigned)(D * 2) + cp_col,
                   slot + (unsigned)(i * C::CPL * 16) + cp_lds);
        }
    }
    __device__ bf16x8 rowfrag(unsigned tile, int m) const {
        return *(lds_bf16x8*)(uintptr_t)((tile + roff) ^ (32u * m));
    }
    __device__ bf16x8 trfrag(unsigned tile, int cb, int kc) const {
        const unsigned lo_addr = (tile + (unsigned)(16 * kc * D * 2) + toff) ^ (64u * cb);
        const unsigned hi_addr = (lo_addr ^ 32u) + 16u * D;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)lo_addr);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)hi_addr);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// lane's 8 consecutive d values (16m + 8h ..) of row `row` of a [T][D] matrix
template <int D>
__device__ inline void load_row_frags(const bf16* m, int row, bool ok, int h, bf16x8 (&f)[D / 16]) {
    const uint4* src = reinterpret_cast<const uint4*>(m + (long long)(ok ? row : 0) * D + 8 * h);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
        uint4 u = src[2 * i];
        if (!ok) u = make_uint4(0, 0, 0, 0);
        f[i] = __builtin_bit_cast(bf16x8, u);
    }
}

// store 32 d-blocks' worth of a transposed accumulator (rows = d, lane = row
// of the output) times `scale` as bf16 into row `dst`
template <int D>
__device__ inline void store_rowT(bf16* dst, const f32x16 (&acc)[D / 32], float scale, int h) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 val;
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = (bf16)(acc[cb][4 * g4 + e] * scale);
            *reinterpret_cast<bf16x4*>(dst + 32 * cb + 8 * g4 + 4 * h) = val;
        }
}

// ---------------------------------------------------------------------------
// dQ: walk the key tiles of a block of 128 query rows.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
    typedef BCfg<D> C;
    constexpr int BN = C::BN, TB = C::TB, NQ = C::NQ, NDB = C::NDB, NKC = C::NKC;
    // ring slot: K (row reads) | V (row reads) | K (transpose reads).  (One
    // copy of K in the combined swizzle of OneTileLanes would do for both
    // reads, but its second-half transpose address costs the registers that
    // keep this kernel from spilling at head size 128.)
    constexpr int SLOT = 3 * TB;
    constexpr int KT = 2 * TB;   // where the transpose reads find K
    __shared__ __attribute__((aligned(1024))) char lds[2 * SLOT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, li = lane & 31;
    const int n_qt = (a.Tq + C::BM - 1) / C::BM;
    const int BH = a.B * a.Hq;
    const int qt = n_qt - 1 - (int)(blockIdx.x / BH);   // longest first
    const int bh = (int)(blockIdx.x % BH);
    const int b = bh / a.Hq, hq = bh - b * a.Hq, hk = hq / a.R;
    const int i0w = qt * C::BM + 32 * wave, iq = i0w + li;
    const bool row_ok = iq < a.Tq;
    const long long rowid = (long long)bh * a.Tq + iq;

    bf16x8 qf[NQ], gf[NQ];
    load_row_frags<D>(a.q + (long long)bh * a.Tq * D, iq, row_ok, h, qf);
    load_row_frags<D>(a.dO + (long long)bh * a.Tq * D, iq, row_ok, h, gf);
    // the row's statistics: lse as a base-2 exponent, and D = rowsum(dO * O)
    // from the lane's half of the channels plus the other half-wave's; the
    // wave's 32-row block of them goes to the workspace for the dK/dV kernel
    float Dv;
    {
        bf16x8 of[NQ];
        load_row_frags<D>(a.o + (long long)bh * a.Tq * D, iq, row_ok, h, of);
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < NQ; ++m)
#pragma unroll
            for (int j = 0; j < 8; ++j) part = fmaf((float)gf[m][j], (float)of[m][j], part);
        Dv = pair_sum(part);
    }
    const float Lr = row_ok ? a.lse[rowid] * kLog2e : 0.f;
    if ((i0w >> 5) < a.n_rt && h == 0) {
        float* tstats = a.stats + ((long long)bh * a.n_rt + (i0w >> 5)) * 64;
        tstats[li] = Lr;
        tstats[32 + li] = Dv;
    }

    const int kv_end = a.causal ? min(a.Tk, a.q_offset + qt * C::BM + C::BM) : a.Tk;
    const int n = (kv_end + BN - 1) / BN;
    const int row_lim = a.causal ? min(a.Tk - 1, a.q_offset + iq) : a.Tk - 1;
    const int wave_last = a.causal ? min(a.Tk - 1, a.q_offset + i0w + 31) : a.Tk - 1;
    const int wave_full = a.causal ? min(a.Tk, a.q_offset + i0w + 1) : a.Tk;
    const int last = i0w >= a.Tq ? -1 : wave_last / BN;

    const TileLanes<D> tl(wave, lane);
    const unsigned base = lds_addr(lds);
    const bf16* kh = a.k + (long long)(b * a.Hkv + hk) * a.Tk * D;
    const bf16* vh = a.v + (long long)(b * a.Hkv + hk) * a.Tk * D;
    auto copy_step = [&](int t, int P) {
        const int j0 = min(t, n - 1) * BN;
        const unsigned s = base + (unsigned)(P * SLOT);
        tl.copy(kh, a.Tk, j0, s, tl.cp_kcol);
        tl.copy(vh, a.Tk, j0, s + TB, tl.cp_kcol);
        tl.copy(kh, a.Tk, j0, s + KT, tl.cp_vcol);
    };

    f32x16 acc[NDB];
#pragma unroll
    for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

    copy_step(0, 0);
    wait_vm<0>();
    __syncthreads();
    auto step = [&](int t, auto slot) {
        constexpr int P = decltype(slot)::value;
        copy_step(t + 1, 1 - P);
        if (t <= last) {
            const unsigned s = base + (unsigned)(P * SLOT);
            // d 64: all fragments read ahead of the products; d 128 reads
            // them at the products (reading ahead there spills and measured
            // slower)
            constexpr bool PRE = D == 64;
            bf16x8 ka[NQ], va[NQ], kt[NKC][NDB];
            if constexpr (PRE) {
#pragma unroll
                for (int m = 0; m < NQ; ++m) {
                    ka[m] = tl.rowfrag(s, m);
                    va[m] = tl.rowfrag(s + TB, m);
                }
            }
            f32x16 st = {}, dp = {};
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(PRE ? ka[m] : tl.rowfrag(s, m), qf[m], st, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(PRE ? va[m] : tl.rowfrag(s + TB, m), gf[m], dp, 0, 0,
                                                             0);
            }
            // K^T for the second product (independent of the softmax)
            if constexpr (PRE) {
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                    for (int cb = 0; cb < NDB; ++cb) kt[kc][cb] = tl.trfrag(s + KT, cb, kc);
            }
            float p[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(st[e], a.c, -Lr));
            if ((t + 1) * BN > wave_full) {   // a tile on the diagonal or past Tk (uniform)
                const int lim = row_lim - (t * BN + 4 * h);
#pragma unroll
                for (int e = 0; e < 16; ++e) p[e] = row_of(e) <= lim ? p[e] : 0.f;
            }
            bf16x8 dsb[NKC];
#pragma unroll
            for (int e = 0; e < 16; ++e) dsb[e >> 3][e & 7] = (bf16)(p[e] * (dp[e] - Dv));
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb)
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(PRE ? kt[kc][cb] : tl.trfrag(s + KT, cb, kc),
                                                                      dsb[kc], acc[cb], 0, 0, 0);
        }
        wait_vm<0>();   // tile t + 1 has landed
        __syncthreads();
    };
    for (int t = 0; t < n; t += 2) {
        step(t, IC<0>{});
        if (t + 1 < n) step(t + 1, IC<1>{});
    }
    wait_vm<0>();
    if (row_ok) store_rowT<D>(a.dq + rowid * D, acc, a.scale, h);
}

// ---------------------------------------------------------------------------
// dK, dV: walk the query tiles of every query head of the group for a block
// of 128 keys.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
void bwd_dkv_kernel(BwdArgs a) {
    typedef BCfg<D> C;
    constexpr int BN = C::BN, TB = C::TB, NQ = C::NQ, NDB = C::NDB, NKC = C::NKC;
    // ring slot: Q (row reads) | dO (row reads) | Q (transpose reads) |
    // dO (transpose reads) | lse and D of the 32 rows (padded to 1 KiB)
    constexpr int SLOT = 4 * TB + 1024;
    __shared__ __attribute__((aligned(1024))) char lds[2 * SLOT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, li = lane & 31;
    const int G = a.B * a.Hkv;
    const int kb = (int)(blockIdx.x / G);   // ascending: early keys are seen by the most rows
    const int g = (int)(blockIdx.x % G);
    const int b = g / a.Hkv, hk = g - b * a.Hkv;
    const int j0 = kb * C::BM, jw = j0 + 32 * wave, key = jw + li;
    const bool key_ok = key < a.Tk;

    bf16x8 kf[NQ], vf[NQ];
    load_row_frags<D>(a.k + (long long)g * a.Tk * D, key, key_ok, h, kf);
    load_row_frags<D>(a.v + (long long)g * a.Tk * D, key, key_ok, h, vf);

    // query tiles that can see a key of this block; step s covers head
    // hk * R + s / per_head and row tile n_rt - 1 - s % per_head (the tiles
    // of a head from the last down, so the key blocks of a group, on one XCD
    // when B * Hkv is a multiple of 8, walk the same tiles at the same time)
    const int n_rt = (a.Tq + BN - 1) / BN;
    const int rt0 = a.causal ? min(n_rt, max(0, j0 - a.q_offset) / BN) : 0;
    const int per_head = n_rt - rt0;
    const int nsteps = a.R * per_head;
    struct Pos { int head, tile; };   // head within the group, row tile
    auto advance = [&](Pos p) {
        if (--p.tile < rt0) { p.tile = n_rt - 1; ++p.head; }
        return p;
    };

    const TileLanes<D> tl(wave, lane);
    const unsigned base = lds_addr(lds);
    const long long bh0 = (long long)b * a.Hq + (long long)hk * a.R;
    // tiles of step position p into slot P (the last position repeats past the end)
    auto copy_step = [&](Pos p, int P) {
        if (p.head >= a.R) { p.head = a.R - 1; p.tile = rt0; }
        const long long bh = bh0 + p.head;
        const int r0 = p.tile * BN;
        const unsigned sl = base + (unsigned)(P * SLOT);
        const bf16* qm = a.q + bh * a.Tq * D;
        const bf16* gm = a.dO + bh * a.Tq * D;
        tl.copy(qm, a.Tq, r0, sl, tl.cp_kcol);
        tl.copy(gm, a.Tq, r0, sl + TB, tl.cp_kcol);
        tl.copy(qm, a.Tq, r0, sl + 2 * TB, tl.cp_vcol);
        tl.copy(gm, a.Tq, r0, sl + 3 * TB, tl.cp_vcol);
    };
    // the row statistics of a step's tile into the slot, by wave 0 (one
    // dword per lane, asynchronous like the tiles)
    auto stats_step = [&](Pos p, int P) {
        if (p.head >= a.R) { p.head = a.R - 1; p.tile = rt0; }
        if (wave == 0)
            copy4(a.stats + ((bh0 + p.head) * a.n_rt + p.tile) * 64, 4u * (unsigned)lane,
                  base + (unsigned)(P * SLOT + 4 * TB));
    };

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dk[cb][r] = 0.f; dv[cb][r] = 0.f; }

    Pos cur = {0, n_rt - 1};
    if (nsteps > 0) {
        copy_step(cur, 0);
        stats_step(cur, 0);
        wait_vm<0>();
        __syncthreads();
    }
    auto step = [&](auto slot) {
        constexpr int P = decltype(slot)::value;
        const Pos nxt = advance(cur);
        copy_step(nxt, 1 - P);
        stats_step(nxt, 1 - P);
        const int r0 = cur.tile * BN;
        // some row of the tile sees a key of this wave
        const bool any = !a.causal || jw <= a.q_offset + min(r0 + BN, a.Tq) - 1;
        if (any && jw < a.Tk) {
            const unsigned sl = base + (unsigned)(P * SLOT);
            bf16x8 qa[NQ], ga[NQ];
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                qa[m] = tl.rowfrag(sl, m);
                ga[m] = tl.rowfrag(sl + TB, m);
            }
            f32x16 st = {}, dp = {};
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[m], kf[m], st, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[m], vf[m], dp, 0, 0, 0);
            }
            // dO^T and Q^T for the second products (independent of the softmax)
            bf16x8 ta[NKC][NDB], tq[NKC][NDB];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb) {
                    ta[kc][cb] = tl.trfrag(sl + 3 * TB, cb, kc);
                    tq[kc][cb] = tl.trfrag(sl + 2 * TB, cb, kc);
                }
            const float* stats = reinterpret_cast<const float*>(lds + P * SLOT + 4 * TB);
            float Ls[16], Ds[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {   // rows 8i + 4h .. + 3 of the tile
                const float4 L4 = *reinterpret_cast<const float4*>(stats + 8 * i + 4 * h);
                const float4 D4 = *reinterpret_cast<const float4*>(stats + BN + 8 * i + 4 * h);
                Ls[4 * i] = L4.x; Ls[4 * i + 1] = L4.y; Ls[4 * i + 2] = L4.z; Ls[4 * i + 3] = L4.w;
                Ds[4 * i] = D4.x; Ds[4 * i + 1] = D4.y; Ds[4 * i + 2] = D4.z; Ds[4 * i + 3] = D4.w;
            }
            float p[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(st[e], a.c, -Ls[e]));
            // every pair of the 32 x 32 block visible: no mask work (uniform)
            const bool full = jw + 31 < a.Tk && r0 + BN <= a.Tq && (!a.causal || jw + 31 <= a.q_offset + r0);
            if (!full) {
                const int lim = a.causal ? key - a.q_offset - 1 : -1;   // rows <= lim precede the key
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = r0 + row_of(e) + 4 * h;
                    const bool vis = key_ok && row < a.Tq && row > lim;
                    p[e] = vis ? p[e] : 0.f;
                }
            }
            bf16x8 pb[NKC], dsb[NKC];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                pb[e >> 3][e & 7] = (bf16)p[e];
                dsb[e >> 3][e & 7] = (bf16)(p[e] * (dp[e] - Ds[e]));
            }
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb) {
                    dv[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[kc][cb], pb[kc], dv[cb], 0, 0, 0);
                    dk[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[kc][cb], dsb[kc], dk[cb], 0, 0, 0);
                }
        }
        cur = nxt;
        wait_vm<0>();   // the next step's tiles have landed
        __syncthreads();
    };
    for (int s = 0; s < nsteps; s += 2) {
        step(IC<0>{});
        if (s + 1 < nsteps) step(IC<1>{});
    }
    wait_vm<0>();
    if (key_ok) {
        store_rowT<D>(a.dk + ((long long)g * a.Tk + key) * D, dk, a.scale, h);
        store_rowT<D>(a.dv + ((long long)g * a.Tk + key) * D, dv, 1.f, h);
    }
}

// ---------------------------------------------------------------------------
// dK, dV at head size 128 with the work of a key block split in two roles.
// Waves w and w + 4 own the same 32 keys.  Wave w forms S = Q K^T and the
// weights P of query tile s, passes P (float32) to its partner through LDS
// and accumulates dV^T += dO^T P; in the same step wave w + 4 takes tile
// s - 1: it forms dP = dO V^T, reads the P its partner wrote one step
// earlier, forms dS = P (dP - D) and accumulates dK^T += Q^T dS.  The tiles
// sit in a three-slot ring (s + 1 landing, s and s - 1 read) and the weights
// in two buffers, so one barrier per step suffices and the two waves that
// share a SIMD run independent work between barriers.  Each wave keeps one
// of the key's K / V rows and one accumulator -- half of what a wave of
// bwd_dkv_kernel keeps -- so two of them fit a SIMD.  Same products in the
// same order as bwd_dkv_kernel: the results are bit-identical.
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_pair_kernel(BwdArgs a) {
    typedef BCfg<D, 8> C;
    constexpr int BN = C::BN, TB = C::TB, NQ = C::NQ, NDB = C::NDB, NKC = C::NKC;
    // ring slot: Q | dO (one copy each, read both ways) | lse and D of the 32
    // rows (padded to 1 KiB); then two buffers of the weights of the 4 key
    // blocks ([block][4][lane] float4: the lane's 16 weights, 4 at a time)
    constexpr int SLOT = 2 * TB + 1024;
    constexpr int NSLOT = 3;
    constexpr int PX = 4 * 4 * 64 * 16;
    __shared__ __attribute__((aligned(1024))) char lds[NSLOT * SLOT + 2 * PX];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = wave >> 2, kblk = wave & 3;   // role 0: S, P, dV; role 1: dP, dS, dK
    const int h = lane >> 5, li = lane & 31;
    const int G = a.B * a.Hkv;
    const int kb = (int)(blockIdx.x / G);   // ascending: early keys are seen by the most rows
    const int g = (int)(blockIdx.x % G);
    const int b = g / a.Hkv, hk = g - b * a.Hkv;
    const int j0 = kb * C::BM, jw = j0 + 32 * kblk, key = jw + li;
    const bool key_ok = key < a.Tk;

    bf16x8 f[NQ];   // role 0: the lane's key row; role 1: its value row
    load_row_frags<D>((role ? a.v : a.k) + (long long)g * a.Tk * D, key, key_ok, h, f);

    // the same walk over the query tiles as bwd_dkv_kernel
    const int n_rt = (a.Tq + BN - 1) / BN;
    const int rt0 = a.causal ? min(n_rt, max(0, j0 - a.q_offset) / BN) : 0;
    const int per_head = n_rt - rt0;
    const int nsteps = a.R * per_head;
    struct Pos { int head, tile; };
    auto advance = [&](Pos p) {
        if (--p.tile < rt0) { p.tile = n_rt - 1; ++p.head; }
        return p;
    };

    const OneTileLanes<D, 8> tl(wave, lane);
    const unsigned base = lds_addr(lds);
    const long long bh0 = (long long)b * a.Hq + (long long)hk * a.R;
    // tiles and row statistics of step position p into ring slot `slot`
    // (positions past the end repeat the last one)
    auto copy_step = [&](Pos p, int slot) {
        if (p.head >= a.R) { p.head = a.R - 1; p.tile = rt0; }
        const long long bh = bh0 + p.head;
        const int r0 = p.tile * BN;
        const unsigned sl = base + (unsigned)(slot * SLOT);
        const bf16* qm = a.q + bh * a.Tq * D;
        const bf16* gm = a.dO + bh * a.Tq * D;
        tl.copy(qm, a.Tq, r0, sl);
        tl.copy(gm, a.Tq, r0, sl + TB);
        if (wave == 0)
            copy4(a.stats + (bh * a.n_rt + p.tile) * 64, 4u * (unsigned)lane, sl + 2 * TB);
    };
    // some row of query tile r0 sees a key of this block (the same for both roles)
    auto active = [&](int r0) { return (!a.causal || jw <= a.q_offset + min(r0 + BN, a.Tq) - 1) && jw < a.Tk; };
    // rows 8i + 4h .. + 3 of a tile's statistics (lse base 2, or D)
    auto row_stats = [&](int slot, int which, float (&rs)[16]) {
        const float* st = reinterpret_cast<const float*>(lds + slot * SLOT + 2 * TB) + which * BN;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 r4 = *reinterpret_cast<const float4*>(st + 8 * i + 4 * h);
            rs[4 * i] = r4.x; rs[4 * i + 1] = r4.y; rs[4 * i + 2] = r4.z; rs[4 * i + 3] = r4.w;
        }
    };

    f32x16 acc[NDB];   // role 0: dV^T; role 1: dK^T
#pragma unroll
    for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
    float4* const px = reinterpret_cast<float4*>(lds + NSLOT * SLOT) + kblk * 4 * 64 + lane;

    if (nsteps == 0) {   // no query row sees these keys
        if (key_ok) store_rowT<D>((role ? a.dk : a.dv) + ((long long)g * a.Tk + key) * D, acc, 1.f, h);
        return;
    }
    Pos cur = {0, n_rt - 1}, prev = cur;
    copy_step(cur, 0);
    wait_vm<0>();
    __syncthreads();
    // step s: role 0 on tile s (slot s % 3), role 1 on tile s - 1; tiles of
    // step s + 1 land in slot (s + 1) % 3, last read by role 1 in step s - 1
    int slot = 0;
    for (int s = 0; s <= nsteps; ++s) {
        const int nslot = slot == NSLOT - 1 ? 0 : slot + 1;
        const Pos nxt = advance(cur);
        if (s + 1 < nsteps) copy_step(nxt, nslot);
        f32x16 sd = {};     // role 0: S; role 1: dP
        float rs[16];       // role 0: the rows' lse (base 2); role 1: their D
        bf16x8 w[NKC];      // B operand of the second product: role 0 P, role 1 dS (bf16)
        int rslot;          // the ring slot this wave reads
        bool act;
        if (role == 0) {
            rslot = slot;
            act = s < nsteps && active(cur.tile * BN);
        } else {
            rslot = slot == 0 ? NSLOT - 1 : slot - 1;
            act = s > 0 && active(prev.tile * BN);
        }
        const unsigned sl = base + (unsigned)(rslot * SLOT);
        if (act) {
            // role 0: S = Q K^T from Q rows; role 1: dP = dO V^T from dO rows
            // everything the step reads is in LDS when it starts (role 1's
            // weights were written a step earlier): issue all the reads at
            // once, so the step waits for one LDS round trip
            const unsigned src = sl + (unsigned)(role * TB);
            const unsigned tsrc = sl + (unsigned)((1 - role) * TB);
            float4* const pbuf = px + (((s - role) & 1) ? 4 * 4 * 64 : 0);
            bf16x8 rf[NQ], tf[NKC][NDB];
            float4 pw[4];
#pragma unroll
            for (int m = 0; m < NQ; ++m) rf[m] = tl.rowfrag(src, m);
            if (role)
#pragma unroll
                for (int i = 0; i < 4; ++i) pw[i] = pbuf[64 * i];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb) tf[kc][cb] = tl.trfrag(tsrc, cb, kc);
            row_stats(rslot, role, rs);
#pragma unroll
            for (int m = 0; m < NQ; ++m) sd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf[m], f[m], sd, 0, 0, 0);
            if (role == 0) {
                const int r0 = cur.tile * BN;
                float p[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sd[e], a.c, -rs[e]));
                const bool full =
                    jw + 31 < a.Tk && r0 + BN <= a.Tq && (!a.causal || jw + 31 <= a.q_offset + r0);
                if (!full) {
                    const int lim = a.causal ? key - a.q_offset - 1 : -1;   // rows <= lim precede the key
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = r0 + row_of(e) + 4 * h;
                        const bool vis = key_ok && row < a.Tq && row > lim;
                        p[e] = vis ? p[e] : 0.f;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pbuf[64 * i] = make_float4(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]);
#pragma unroll
                for (int e = 0; e < 16; ++e) w[e >> 3][e & 7] = (bf16)p[e];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 p4 = pw[i];
                    const float pe[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int e = 4 * i + j;
                        w[e >> 3][e & 7] = (bf16)(pe[j] * (sd[e] - rs[e]));
                    }
                }
            }
            // role 0: dV^T += dO^T P; role 1: dK^T += Q^T dS (one instruction
            // stream for both, so the accumulators stay in place)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb)
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[kc][cb], w[kc], acc[cb], 0, 0, 0);
        }
        prev = cur;
        cur = nxt;
        slot = nslot;
        wait_vm<0>();   // the next step's tiles have landed
        __syncthreads();
    }
    if (key_ok) {
        if (role) store_rowT<D>(a.dk + ((long long)g * a.Tk + key) * D, acc, a.scale, h);
        else store_rowT<D>(a.dv + ((long long)g * a.Tk + key) * D, acc, 1.f, h);
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
    typedef BCfg<D> C;
    hipError_t e;
    const long long n_qt = (a.Tq + C::BM - 1) / C::BM;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)(n_qt * a.B * a.Hq)), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long n_kb = (a.Tk + C::BM - 1) / C::BM;
    if constexpr (D == 128)
        hipLaunchKernelGGL(bwd_dkv_pair_kernel<D>, dim3((unsigned)(n_kb * a.B * a.Hkv)), dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL(bwd_dkv_kernel<D>, dim3((unsigned)(n_kb * a.B * a.Hkv)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int Hq, int Tq) {
    return sizeof(float) * 64 * (size_t)B * Hq * (size_t)((Tq + 31) / 32);
}

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
    BwdArgs a;
    a.q = static_cast<const bf16*>(p.q);
    a.k = static_cast<const bf16*>(p.k);
    a.v = static_cast<const bf16*>(p.v);
    a.o = static_cast<const bf16*>(p.o);
    a.dO = static_cast<const bf16*>(p.dO);
    a.lse = p.lse;
    a.stats = static_cast<float*>(p.workspace);
    a.dq = static_cast<bf16*>(p.dq);
    a.dk = static_cast<bf16*>(p.dk);
    a.dv = static_cast<bf16*>(p.dv);
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Tq = p.Tq; a.Tk = p.Tk;
    a.R = p.Hq / p.Hkv;
    a.n_rt = (p.Tq + 31) / 32;
    a.c = p.scale * kLog2e;
    a.scale = p.scale;
    a.causal = p.causal;
    a.q_offset = p.causal ? p.q_offset : 0;
    return p.d == 64 ? launch_bwd_d<64>(a, stream) : launch_bwd_d<128>(a, stream);
}

}  // namespace rocattn
