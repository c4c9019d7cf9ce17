// attn_prefill_d64.hip -- fused causal attention forward, bf16 in/out,
// float32 accumulation, on the gfx950 matrix cores, head size 64.  (Head
// size 128 has its own kernel, attn_prefill_bf16.hip: with half the matrix
// work per score, head size 64 is bound by the vector ALU, and this
// four-wave, two-workgroups-per-CU design overlaps it best.)
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
// Design (one workgroup = 4 waves = 128 query rows of one (b, hq)):
//  * Each wave owns 32 query rows.  Its Q fragment stays in registers for
//    the whole kernel as the B operand of v_mfma_f32_32x32x16_bf16.
//  * Keys are visited in tiles of 64.  K and V tiles go from HBM straight
//    into LDS (global_load_lds_dwordx4: no staging registers, no LDS store
//    instructions) and are shared by the four waves.  Each 16-byte chunk of
//    a tile row is stored at a position XOR-swizzled by the row, so the
//    fragment reads below hit distinct LDS banks.
//  * Scores are formed transposed, S^T = K Q^T (keys on the MFMA rows,
//    queries on its columns), so in the accumulator layout each lane holds
//    scores of ONE query row (lane % 32) for 16 keys: the row max and row
//    sum need no cross-lane work except one v_permlane32_swap between the
//    two half-waves, and the running max / sum / rescale factor of a row
//    are per-lane scalars.
//  * Software pipeline: K runs one tile ahead of V.  In the steady state a
//    tile step is written in issue order: each score MFMA of tile t+1 is
//    followed by a slice of the exponentials of tile t, then the P.V MFMAs
//    of tile t follow with their V^T fragment reads; fragment reads are
//    issued three MFMAs ahead of their use.  Global loads run two tiles (K)
//    and one tile (V) ahead; one barrier per tile.
//  * Softmax in base 2: p = 2^(s * |scale| * log2(e) - m) with the raw
//    v_exp_f32, against the running max m as it stands (no per-tile row
//    max): only when a row's weights would exceed 2^12 does the row take
//    the tile's max, rescale its accumulator and recompute.  The running
//    max starts at tile 0's max; the final division by the row sum cancels
//    whichever m was used.  A negative scale is applied by negating q on
//    load.  The row sum adds the bf16-rounded weights that feed the P.V
//    product (v_dot2_f32_bf16 against (1, 1)), so V = 1 gives O = 1.
//  * P^T, rounded to bf16, is already in the B-operand layout of the second
//    product O^T += V^T P^T.  The A operand V^T is read from the row-major V
//    tile with ds_read_b64_tr_b16 (the LDS transpose read of gfx950), whose
//    four-row gather is matched to the key order of the score accumulator.
//  * Causal tiles past a wave's last visible key are skipped; only tiles
//    that straddle the diagonal (or the end of the keys) pay for masking.
//  * Workgroups are issued longest-first (largest query tile first), and,
//    when the number of batch x K/V heads is a multiple of 8, the query
//    heads that share a K/V head are placed on the same XCD (workgroup id
//    modulo 8) so their K/V tiles are served from that XCD's L2.
#include <math.h>

#include "internal.hpp"

namespace rocattn {
namespace {

template <int D>
struct Cfg {
    static constexpr int BN = D == 128 ? 32 : 64;  // keys per tile
    static constexpr int NW = 4;                  // waves per workgroup
    static constexpr int BM = 32 * NW;            // query rows per workgroup
    static constexpr int NCH = D / 8;             // 16-byte chunks per row
    static constexpr int TILE = BN * D;           // elements per K or V tile
    static constexpr int RSTR = 256 / NCH;        // rows filled by one 256-lane copy round
    static constexpr int NINS = BN / RSTR;        // copy rounds per tile
    static_assert(BN % RSTR == 0, "tile rows must split evenly");
};

// XOR swizzles of the 16-byte chunk position within a tile row.
//  K: sixteen consecutive rows read the same logical chunk (ds_read_b128),
//     so the rows' chunks must fall in sixteen distinct 16-byte bank groups.
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
    int G;         // B * Hkv
    int n_qt;      // query tiles per head
    float c;       // |scale| * log2(e), at least 1e-30 so that -inf * c = -inf
    unsigned neg;  // 0x80008000 when scale < 0 (q is negated on load), else 0
    int causal;
    int q_offset;
    int xcd;       // 1: group the heads of one K/V head on one XCD
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

// Hides a value from the optimiser, so offsets derived from it are formed
// next to their use instead of being hoisted out of the key loop as
// loop-invariant registers.
__device__ inline int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
__device__ __attribute__((always_inline)) inline void copy_tile_fn(
    const bf16* src, int j0, bf16* dst, unsigned lane_off, int Tk, int cp_r0, int wave) {
    typedef Cfg<D> C;
    if (j0 + C::BN <= Tk) {
        const bf16* base = src + (size_t)j0 * D;  // wave-uniform
#pragma unroll
        for (int i = 0; i < C::NINS; ++i)
            __builtin_amdgcn_global_load_lds(base + (size_t)i * C::RSTR * D + lane_off,
                                             (lds_void*)(dst + (i * 256 + wave * 64) * 8), 16, 0, 0);
    } else {  // last, partial tile: rows past the last key re-read the last key
        const unsigned col = lane_off - (unsigned)(cp_r0 * D);
#pragma unroll
        for (int i = 0; i < C::NINS; ++i) {
            const int row = min(j0 + cp_r0 + i * C::RSTR, Tk - 1);
            __builtin_amdgcn_global_load_lds(src + (size_t)row * D + col,
                                             (lds_void*)(dst + (i * 256 + wave * 64) * 8), 16, 0, 0);
        }
    }
}

template <int D>
struct Tile {
    static constexpr int NKB = Cfg<D>::BN / 32;  // 32-key blocks per tile
    f32x16 s[NKB];
};

struct Even { static constexpr int value = 0; };
struct Odd { static constexpr int value = 1; };

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(Args a) {
    typedef Cfg<D> C;
    constexpr int BN = C::BN, BM = C::BM;
    constexpr int NKB = BN / 32;       // 32-key blocks per tile
    constexpr int NDB = D / 32;        // 32-column blocks of the output
    constexpr int NQ = D / 16;         // 16-wide d slices of q.k
    constexpr int NS = NQ * NKB;       // score MFMAs per tile
    constexpr int NP = NDB * NKB * 2;  // P.V MFMAs per tile
    constexpr int NE = NKB * 16;       // scores per lane per tile
    constexpr int EA = NE / NS;        // exponentials per score MFMA
    constexpr int AHEAD = D == 128 ? 2 : 3;  // fragment reads in flight
    // VALU instructions the steady state places after each score MFMA: 3 per
    // exponential (fma, exp, half a pack, half a sum)
    constexpr int VA = 3 * EA;
    static_assert(NE % NS == 0 && EA % 2 == 0 && (8 % EA == 0), "slices must divide");
    // four distinct LDS objects, always addressed by compile-time parity, so
    // the compiler can tell that reads of one buffer do not alias the
    // asynchronous HBM -> LDS copies into another (and need not wait for them)
    __shared__ __attribute__((aligned(16))) bf16 kbuf0[C::TILE];
    __shared__ __attribute__((aligned(16))) bf16 kbuf1[C::TILE];
    __shared__ __attribute__((aligned(16))) bf16 vbuf0[C::TILE];
    __shared__ __attribute__((aligned(16))) bf16 vbuf1[C::TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int h = lane >> 5, li = lane & 31;

    // ---- which (query tile, batch, query head) this workgroup owns
    int qt, g, rep;
    {
        const int w = blockIdx.x;
        if (a.xcd) {
            const int x = w & 7, s = w >> 3;
            const int per = (a.G >> 3) * a.R;
            const int rank = s / per, rem = s - rank * per;
            g = x * (a.G >> 3) + rem / a.R;
            rep = rem % a.R;
            qt = a.n_qt - 1 - rank;
        } else {
            const int per = a.G * a.R;
            const int rank = w / per, rem = w - rank * per;
            g = rem / a.R;
            rep = rem % a.R;
            qt = a.n_qt - 1 - rank;
        }
    }
    const int b = g / a.Hkv, hk = g - (g / a.Hkv) * a.Hkv;
    const int hq = hk * a.R + rep;
    const int i0 = qt * BM;
    const int i0w = i0 + 32 * wave;
    const int iq = i0w + li;               // this lane's query row

    // ---- Q fragment (B operand): lane holds q[iq][16m + 8h .. +7]
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

    // ---- K/V tile copy, HBM -> LDS directly.  In copy round i, lane L of
    //      wave w fills the tile's 16-byte slot i*256 + 64w + L, i.e. row
    //      r0 + i*RSTR at chunk position cp_p, with the logical chunk that
    //      the swizzle puts there.  Rows past the last key re-read the last
    //      key (finite values; those keys are masked).
    const bf16* kh = a.k + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const bf16* vh = a.v + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const int cp_slot = wave * 64 + lane;
    const int cp_r0 = cp_slot / C::NCH, cp_p = cp_slot % C::NCH;
    const int cp_ck = cp_p ^ swz_k<D>(cp_r0), cp_cv = cp_p ^ swz_v<D>(cp_r0);
    const unsigned cp_koff = (unsigned)(cp_r0 * D + 8 * cp_ck);  // elements within a tile
    const unsigned cp_voff = (unsigned)(cp_r0 * D + 8 * cp_cv);
    auto copy_tile = [&](const bf16* src, int j0, bf16* dst, unsigned lane_off) {
        copy_tile_fn<D>(src, j0, dst, lane_off, a.Tk, cp_r0, wave);
    };

    // ---- per-lane fragment offsets in a tile (elements).  In both the row
    //      term, the swizzled chunk term and the in-chunk term occupy
    //      disjoint bits, so the offset for slice m (block cb) is the slice-0
    //      offset XOR 16m (32cb): one register and one v_xor per read.
    // K operand (A of S^T): key row 32kb + li, logical chunk 2m + h
    const int koff0 = li * D + 8 * (h ^ swz_k<D>(li));
    // V^T operand via transpose reads: supplying lane (16g + 4r + qq) points
    // at V[key_base + 4(g/2) + r][32 cb + 16(g%2) + 4qq] (logical column)
    const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
    const int voff0 = (4 * (tg >> 1) + tr) * D + 16 * (tg & 1) + 4 * tq + 8 * swz_v<D>(tr);

    // the same offsets in bytes (the XOR terms double with them)
    int koff = 2 * koff0, voff = 2 * voff0;  // re-hidden at every tile step
    auto kfrag = [&](const bf16* Ks, int i) -> bf16x8 {  // score MFMA i = (m, kb)
        const int m = i / NKB, kb = i % NKB;
        const char* p = reinterpret_cast<const char*>(Ks + kb * 32 * D) + (koff ^ (32 * m));
        return *reinterpret_cast<const bf16x8*>(p);
    };
    auto vfrag = [&](const bf16* Vs, int j) -> bf16x8 {  // P.V MFMA j = (kb, cc, cb)
        const int cb = j % NDB, kc = j / NDB;            // kc = 2 kb + cc
        const char* vp = reinterpret_cast<const char*>(Vs + 16 * kc * D) + (voff ^ (64 * cb));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 16 * D));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // ---- visibility limits (the wave's are wave-uniform)
    const int kv_end = a.causal ? min(a.Tk, a.q_offset + i0 + BM) : a.Tk;
    const int n_tiles = (kv_end + BN - 1) / BN;
    const int row_lim = a.causal ? min(a.Tk - 1, a.q_offset + iq) : a.Tk - 1;
    const int wave_last = a.causal ? min(a.Tk - 1, a.q_offset + i0w + 31) : a.Tk - 1;
    // keys below wave_full are visible to every row of the wave
    const int wave_full = a.causal ? min(a.Tk, a.q_offset + i0w + 1) : a.Tk;

    f32x16 oacc[NDB];
#pragma unroll
    for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float cs = a.c;

    // key offset (within the tile) of score element e = 16 kb + r of a lane
    auto key_of = [&](int e) { return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + (e & 3); };

    auto zero_tile = [&](Tile<D>& T) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) T.s[kb][r] = 0.f;
    };

    // S^T(tile) = K(tile) Q^T (plain order; edge steps)
    auto scores = [&](const bf16* Ks, Tile<D>& T) {
        zero_tile(T);
#pragma unroll
        for (int i = 0; i < NS; ++i)
            T.s[i % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(Ks, i), qf[i / NKB],
                                                                   T.s[i % NKB], 0, 0, 0);
    };

    // masked score element (key past the row's limit) -> -inf
    auto mask_elem = [&](float s, int e, int lim) { return key_of(e) > lim ? -INFINITY : s; };

    // p = 2^(s c - m) for the score pair (e, e + 1), rounded to bf16 into the
    // B operand of the P.V product; the row sum adds those rounded weights
    // (v_dot2_f32_bf16 against (1, 1)), so V = 1 gives O = 1
    bf16x8 pb[NKB][2];
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    auto exp_pair = [&](const Tile<D>& T, int e, float nm, float& sa, float& sb) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(T.s[e >> 4][e & 15], cs, nm));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(T.s[e >> 4][(e + 1) & 15], cs, nm));
        bf16x2 pk;
        pk[0] = (bf16)p0;
        pk[1] = (bf16)p1;
        pb[e >> 4][(e >> 3) & 1][e & 7] = pk[0];
        pb[e >> 4][(e >> 3) & 1][(e & 7) + 1] = pk[1];
        if (e & 2) sb = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, sb, false);
        else sa = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, sa, false);
    };
    // weights of a whole tile against the running max; when some weight would
    // exceed 2^12 (a score above the running max by ~12 in log2 units), the
    // rows concerned (both half-wave lanes of a row) take the tile's max,
    // rescale, and every row recomputes (unchanged rows get the very same
    // weights)
    auto fix_weights = [&](const Tile<D>& T, float& sa, float& sb) {
        const bool big = !(sa + sb <= 4096.f);
        if (__any(big)) {
            const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)big, (unsigned)big, false, false);
            const bool row_big = (sw[0] | sw[1]) != 0u;
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < NE; ++e) mx = fmaxf(mx, T.s[e >> 4][e & 15]);
            const float tmax = pair_max(mx) * cs;
            const float m_new = row_big ? fmaxf(m_run, tmax) : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
            m_run = m_new;
            sa = 0.f;
            sb = 0.f;
#pragma unroll
            for (int e = 0; e < NE; e += 2) exp_pair(T, e, -m_run, sa, sb);
        }
        l_run += sa + sb;
    };
    auto mask_tile = [&](Tile<D>& T, int j0) {
        const int lim = row_lim - (j0 + 4 * h);
#pragma unroll
        for (int e = 0; e < NE; ++e) T.s[e >> 4][e & 15] = mask_elem(T.s[e >> 4][e & 15], e, lim);
    };

    // O^T += V^T P^T (plain order; edge steps)
    auto pv_tile = [&](const bf16* Vs) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int cb = j % NDB, kc = j / NDB;
            oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(Vs, j), pb[kc >> 1][kc & 1],
                                                               oacc[cb], 0, 0, 0);
        }
    };

    // ---- prologue: K(0), V(0), K(1) into LDS; scores and max of tile 0
    copy_tile(kh, 0, kbuf0, cp_koff);
    copy_tile(vh, 0, vbuf0, cp_voff);
    if (n_tiles > 1) copy_tile(kh, BN, kbuf1, cp_koff);
    __syncthreads();

    Tile<D> SA, SB;
    scores(kbuf0, SA);  // tile 0 is visible to every wave (key 0 is)
    if (BN > wave_full) mask_tile(SA, 0);
    {   // the running max starts at tile 0's max
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < NE; ++e) mx = fmaxf(mx, SA.s[e >> 4][e & 15]);
        m_run = pair_max(mx) * cs;
    }

    // One pipeline step.  On entry `cur` holds the (masked) scores of tile t
    // and m_run already covers tile t.  The step forms the weights of tile t
    // and adds P V(t), computes the scores of tile t+1 into `nxt`, and
    // brings m_run up to date for tile t+1.
    auto step = [&](int t, Tile<D>& cur, Tile<D>& nxt, auto parity_tag) {
        constexpr int PAR = decltype(parity_tag)::value;  // t & 1, known at compile time
        bf16* const k_this = PAR ? kbuf1 : kbuf0;   // held K(t); receives K(t+2)
        const bf16* const Kn = PAR ? kbuf0 : kbuf1; // K(t+1)
        const bf16* const Vc = PAR ? vbuf1 : vbuf0; // V(t)
        bf16* const v_next = PAR ? vbuf0 : vbuf1;   // receives V(t+1)
        const int j0 = t * BN;
        koff = opaque(2 * koff0);
        voff = opaque(2 * voff0);
        const bool more_k = t + 2 < n_tiles, more_v = t + 1 < n_tiles;
        if (more_k) copy_tile(kh, j0 + 2 * BN, k_this, cp_koff);
        if (more_v) copy_tile(vh, j0 + BN, v_next, cp_voff);
        const bool next_active = more_v && j0 + BN <= wave_last;
        const bool next_masked = j0 + 2 * BN > wave_full;
        const float nm = -m_run;
        float sa = 0.f, sb = 0.f;
        auto steady = [&]() {
            // ---- steady state: one basic block per phase, in issue order
            // phase A: score MFMAs of tile t+1 | weights of tile t.
            // Key block by key block (MFMA i = (kb, m) with kb = i / NQ), so
            // the second score block starts only once the first half of
            // tile t is spent: the two tiles never hold all their registers
            // at once.
            zero_tile(nxt);
            auto kfrag_kb = [&](int i) { return kfrag(Kn, (i % NQ) * NKB + i / NQ); };
            bf16x8 kq[AHEAD];
#pragma unroll
            for (int i = 0; i < AHEAD; ++i) kq[i] = kfrag_kb(i);
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const bf16x8 kf = kq[i % AHEAD];
                if (i + AHEAD < NS) kq[i % AHEAD] = kfrag_kb(i + AHEAD);
                nxt.s[i / NQ] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[i % NQ],
                                                                        nxt.s[i / NQ], 0, 0, 0);
#pragma unroll
                for (int u = 0; u < EA; u += 2) exp_pair(cur, i * EA + u, nm, sa, sb);
            }
            // keep that order: per score MFMA one fragment read and its
            // share of the exponential work
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, VA, 0); // VALU
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            }
            fix_weights(cur, sa, sb);
            // phase B: P.V MFMAs of tile t
            bf16x8 vq[AHEAD];
#pragma unroll
            for (int j = 0; j < AHEAD; ++j) vq[j] = vfrag(Vc, j);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const bf16x8 vf = vq[j % AHEAD];
                if (j + AHEAD < NP) vq[j % AHEAD] = vfrag(Vc, j + AHEAD);
                const int cb = j % NDB, kc = j / NDB;
                oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kc >> 1][kc & 1], oacc[cb],
                                                                   0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // LDS (transpose) reads
            }
        };
        if (next_active && !next_masked && j0 + BN <= wave_full) {
            steady();
        } else {
            // ---- edge steps: diagonal tiles, the last tile, skipped tiles
            if (next_active) scores(Kn, nxt);
            if (j0 <= wave_last) {
#pragma unroll
                for (int e = 0; e < NE; e += 2) exp_pair(cur, e, nm, sa, sb);
                fix_weights(cur, sa, sb);
                pv_tile(Vc);
            }
            if (next_active && next_masked) mask_tile(nxt, j0 + BN);
        }
        __syncthreads();
    };

    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
        step(t, SA, SB, Even());
        step(t + 1, SB, SA, Odd());
    }
    if (t < n_tiles) step(t, SA, SB, Even());

    // ---- epilogue: O = O^T / l, lane holds columns 32cb + 8g4 + 4h .. +3 of row iq
    const float l_tot = pair_sum(l_run);
    if (iq < a.Tq) {
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

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
    typedef Cfg<D> C;
    Args a;
    a.q = static_cast<const bf16*>(p.q);
    a.k = static_cast<const bf16*>(p.k);
    a.v = static_cast<const bf16*>(p.v);
    a.o = static_cast<bf16*>(p.o);
    a.lse = p.lse;
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Tq = p.Tq; a.Tk = p.Tk;
    a.R = p.Hq / p.Hkv;
    a.G = p.B * p.Hkv;
    a.n_qt = (p.Tq + C::BM - 1) / C::BM;
    a.c = fmaxf(fabsf(p.scale) * kLog2e, 1e-30f);
    a.neg = p.scale < 0.f ? 0x80008000u : 0u;
    a.causal = p.causal;
    a.q_offset = p.causal ? p.q_offset : 0;
    a.xcd = (a.G % 8 == 0) ? 1 : 0;
    const long long n = (long long)a.n_qt * a.G * a.R;
    hipLaunchKernelGGL(prefill_bf16_kernel<D>, dim3((unsigned)n), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16_d64(const FwdParams& p, hipStream_t stream) {
    return launch_d<64>(p, stream);
}

}  // namespace rocattn
