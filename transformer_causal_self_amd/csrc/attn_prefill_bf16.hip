// attn_prefill_bf16.hip -- fused causal attention forward, bf16 in/out,
// float32 accumulation, on the gfx950 matrix cores, head sizes 64 and 128.
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
// Design (one workgroup = 4 waves = 128 query rows of one (b, hq); several
// workgroups per CU -- or, for long dense launches at head size 128, 12
// waves = 384 rows, one workgroup per CU, so that each tile copied into LDS
// serves three times the rows):
//  * Each wave owns 32 query rows; its Q fragment stays in registers as the
//    B operand of v_mfma_f32_32x32x16_bf16.  The kernel is kept small so
//    that several waves share each SIMD (four at head size 64, about 120
//    VGPRs; three at head size 128, about 145): the latency of LDS reads,
//    copies and barriers is hidden by the other waves rather than by a
//    software pipeline inside one wave.  Measured faster than a two-group
//    ping-pong kernel with a three-tile ring (two workgroups per CU) at both
//    head sizes, and than 64-row waves at head size 64.
//  * Keys are visited in tiles of 64 (head size 64) or 32 (head size 128).
//    K and V tiles go from HBM straight into two LDS rings of two tiles
//    (global_load_lds_dwordx4: two 16-byte copies per lane fill a tile at
//    either head size), issued one tile ahead.  Each 16-byte
//    chunk of a tile row sits at a position XOR-swizzled by the row, so the
//    fragment reads hit distinct banks.
//  * Scores are formed transposed, S^T = K Q^T (keys on the MFMA rows,
//    queries on its columns), so each lane holds 16 scores of one query row
//    per 32-key block: the row max and row sum need no cross-lane work except
//    one v_permlane32_swap between the two half-waves.
//  * Tile step t: scores of tile t (K fragments from LDS), mask when the
//    tile straddles the diagonal, weights, P.V (V^T fragments from LDS);
//    one barrier per tile.
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
//  * Tiles past a wave's last visible key are skipped (the wave still takes
//    part in the barriers and copies); only tiles that straddle the
//    diagonal or the end of the keys pay for masking.
//  * Workgroups are issued longest-first (largest query tile first), and,
//    when the number of batch x K/V heads is a multiple of 8, the query
//    heads that share a K/V head are placed on the same XCD (workgroup id
//    modulo 8) so their K/V tiles are served from that XCD's L2.
#include <math.h>

#include "internal.hpp"
#include "mfma_tiles.hpp"
#include "rope_math.hpp"

namespace rocattn {
namespace {

// Tile shape and occupancy per head size (chosen by measurement); DK is the
// width of q and k rows, DV that of v and o rows:
//   DK = DV = 64:  64-key tiles, four waves per SIMD (about 120 VGPRs)
//   otherwise:     32-key tiles, three waves per SIMD (about 145-160 VGPRs)
// NWS waves per workgroup: 4 (several workgroups per CU), or at head size
// 128, 12 -- one workgroup fills a CU at three waves per SIMD and each K/V
// tile copied into LDS serves 384 query rows (long launches; see
// wide_prefill below).
template <int DK, int DV, int NWS = 4>
struct Cfg {
    static constexpr bool SMALL = DK == 64 && DV == 64;
    static constexpr int BN = SMALL ? 64 : 32;      // keys per tile
    static constexpr int WPE = SMALL ? 4 : 3;       // waves per SIMD
    static constexpr int NW = NWS;                  // waves per workgroup
    static_assert(NW == 4 || (NW == 12 && !SMALL), "4-wave workgroups, or 12 at head size 128");
    static constexpr int RB = 1;                    // 32-row blocks per wave (the code allows more)
    static constexpr int BM = NW * RB * 32;         // query rows per workgroup
    static constexpr int NCHK = DK / 8;             // 16-byte chunks per key row
    static constexpr int NCHV = DV / 8;             // 16-byte chunks per value row
    static constexpr int TBK = BN * DK * 2;         // bytes of one K tile
    static constexpr int TBV = BN * DV * 2;         // bytes of one V tile
    static constexpr int NRING = 2;                 // tiles per ring
    static constexpr int NQ = DK / 16;              // 16-wide slices of q.k
    static constexpr int NDB = DV / 32;             // 32-column blocks of the output
    static constexpr int NKC = BN / 16;             // 16-key slices of a tile
    static constexpr int NKB = BN / 32;             // 32-key blocks of a tile
    static constexpr int NE = 16 * NKB;             // scores per lane per row block and tile
    static constexpr int CPL = NW * 64;             // lanes of a workgroup (all of them copy)
    static constexpr int NINSK = BN * NCHK / CPL;   // 16-byte copies per lane per K tile
    static constexpr int NINSV = BN * NCHV / CPL;   // ... per V tile
    static constexpr int RSTRK = CPL / NCHK;        // K tile rows filled by one copy instruction
    static constexpr int RSTRV = CPL / NCHV;        // ... V tile rows
    // When the lanes do not divide a tile's 16-byte chunks (12 waves), the
    // chunks of a K tile and then a V tile are numbered 0 .. NCP-1 and lane
    // l of copy instruction i moves chunk i * CPL + l (GEN).
    static constexpr int NCK = BN * NCHK, NCP = NCK + BN * NCHV;
    static constexpr bool GEN = NCK % CPL != 0 || (NCP - NCK) % CPL != 0;
    static constexpr int NCI = (NCP + CPL - 1) / CPL;   // copy instructions per lane (GEN)
    static_assert(BN % 32 == 0 && NCK % 64 == 0 && (GEN || (NINSK >= 1 && NINSV >= 1)),
                  "tiles of whole 32-key blocks, each wave's chunks all K or all V");
};

struct Args {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    int B, Hq, Hkv, Tq, Tk;
    int R;         // query heads per K/V head
    int G;         // B * Hkv
    int n_qt;      // query tiles (of BM rows) per head
    float c;       // |scale| * log2(e), at least 1e-30 so that -inf * c = -inf
    unsigned neg;  // 0x80008000 when scale < 0 (q is negated on load), else 0
    int causal;
    int q_offset;
    int xcd;       // 1: group the heads of one K/V head on one XCD
    // element strides between batches and heads, and (32-bit) between tokens
    long long qsb, qsh, ksb, ksh, vsb, vsh, osb, osh;
    int qst, kst, vst, ost;
    // RoPE of q at load: (cos, sin) table [position][D/2] or null; query row
    // i at position rope_pos0 + i; rope_adj picks the channel pairing
    const float2* rope;
    int rope_adj, rope_pos0;
    // split over the keys: ks workgroups per (query tile, head), each writing
    // its unnormalised output [row][ks][DV] and (max, weight sum) [row][ks][2]
    int ks;
    float* part_o;
    float* part_ml;
};

// RoPE of a lane's query fragments (channels 16m + 8h .. +7 of one row)
// from the row's (cos, sin) table entries: the turn in float32, rounded once
// to bf16 -- the same arithmetic as the RoPE pass.  Split-half pair
// p = (p, p + D/2) joins fragment m with fragment m + D/32 (entries
// 16m + 8h .. +7); adjacent pair p = (2p, 2p + 1) lies inside fragment m
// (entries 8m + 4h .. +3).  Entries are loaded per fragment and used at
// once (loading all of them ahead spills at d = 128 and measured no faster).
template <int D>
__device__ inline void rope_q_frags(bf16x8 (&f)[D / 16], const float2* tab, int adj, int h) {
    constexpr int NQ = D / 16;
    float y1, y2;
    if (!adj) {
#pragma unroll
        for (int m = 0; m < NQ / 2; ++m) {
            float4 t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] = reinterpret_cast<const float4*>(tab + 16 * m + 8 * h)[i];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 x = t[j / 2];
                const float c = (j & 1) ? x.z : x.x, sn = (j & 1) ? x.w : x.y;
                rope_turn((float)f[m][j], (float)f[m + NQ / 2][j], c, sn, y1, y2);
                f[m][j] = (bf16)y1;
                f[m + NQ / 2][j] = (bf16)y2;
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            float4 t[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) t[i] = reinterpret_cast<const float4*>(tab + 8 * m + 4 * h)[i];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                rope_turn((float)f[m][4 * i], (float)f[m][4 * i + 1], t[i].x, t[i].y, y1, y2);
                f[m][4 * i] = (bf16)y1;
                f[m][4 * i + 1] = (bf16)y2;
                rope_turn((float)f[m][4 * i + 2], (float)f[m][4 * i + 3], t[i].z, t[i].w, y1, y2);
                f[m][4 * i + 2] = (bf16)y1;
                f[m][4 * i + 3] = (bf16)y2;
            }
        }
    }
}

template <int DK, int DV>
struct Scores {
    f32x16 s[Cfg<DK, DV>::RB][Cfg<DK, DV>::NKB];   // RB and NKB do not depend on the workgroup size
};

// DENSE: q and k are dense [B][H][T][DK], v and o dense [B][H][T][DV], so
// every token stride is a compile-time constant (the strided instantiation
// reads the strides from Args).
// ROPE: the query rows are turned by RoPE at load (a.rope holds the table).
// SPLIT: a.ks workgroups share a (query tile, head), each taking one
// contiguous run of its key tiles and writing partial results that
// combine_kernel merges (for launches too small to fill the chip).
template <int DK, int DV, bool DENSE, bool ROPE, bool SPLIT = false, int NWS = 4>
__global__ __launch_bounds__((Cfg<DK, DV, NWS>::NW * 64))
__attribute__((amdgpu_waves_per_eu(Cfg<DK, DV, NWS>::WPE, Cfg<DK, DV, NWS>::WPE)))
void prefill_kernel(Args a) {
    typedef Cfg<DK, DV, NWS> C;
    constexpr int BN = C::BN, NW = C::NW, RB = C::RB, BM = C::BM, NCHK = C::NCHK, NCHV = C::NCHV;
    constexpr int TBK = C::TBK, TBV = C::TBV;
    constexpr int NRING = C::NRING, NQ = C::NQ, NDB = C::NDB, NKC = C::NKC, NKB = C::NKB;
    constexpr int NE = C::NE, CPL = C::CPL;
    (void)NW;
    __shared__ __attribute__((aligned(1024))) char lds[NRING * (TBK + TBV)];  // K ring, then V ring

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int h = lane >> 5, li = lane & 31;

    // ---- which (query tile, batch, query head) this workgroup owns
    int qt, g, rep, split = 0;
    if constexpr (SPLIT) {   // longest first, the splits of a tile side by side
        split = (int)(blockIdx.x % a.ks);
        const int w = (int)(blockIdx.x / a.ks);
        const int per = a.G * a.R;
        const int rank = w / per, rem = w - rank * per;
        g = rem / a.R;
        rep = rem % a.R;
        qt = a.n_qt - 1 - rank;
    } else {
        // Workgroup w runs on XCD w % 8, as the (w / 8)-th of that XCD, and
        // an XCD hands its workgroups round-robin to its 32 CUs.  Sizes go
        // longest-first; reversing every other run of 32 evens out the sum
        // each CU receives.
        const int nwg = a.n_qt * a.G * a.R;
        const int x = blockIdx.x & 7;
        const int per_x = (nwg - x + 7) >> 3;
        int s = blockIdx.x >> 3;
        if ((s >> 5) & 1) s = min(per_x, (s | 31) + 1) - 1 - (s & 31);
        const int w = 8 * s + x;
        if (a.xcd) {
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
    const int i0w = i0 + 32 * RB * wave;      // first row of this wave
    int iq[RB];                               // this lane's query rows
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) iq[rb] = i0w + 32 * rb + li;

    // ---- Q fragments (B operand): lane holds q[iq[rb]][16m + 8h .. +7],
    //      turned by RoPE at position rope_pos0 + iq[rb] when a table is given
    bf16x8 qf[RB][NQ];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = iq[rb] < a.Tq ? iq[rb] : a.Tq - 1;
        const uint4* src = reinterpret_cast<const uint4*>(
            a.q + b * a.qsb + hq * a.qsh + (long long)row * (DENSE ? DK : a.qst) + 8 * h);
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            uint4 u = src[2 * m];
            if (iq[rb] >= a.Tq) u = make_uint4(0, 0, 0, 0);
            qf[rb][m] = __builtin_bit_cast(bf16x8, u);
        }
        if constexpr (ROPE)
            rope_q_frags<DK>(qf[rb], a.rope + (size_t)(a.rope_pos0 + row) * (DK / 2), a.rope_adj, h);
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            uint4 u = __builtin_bit_cast(uint4, qf[rb][m]);
            u.x ^= a.neg; u.y ^= a.neg; u.z ^= a.neg; u.w ^= a.neg;
            qf[rb][m] = __builtin_bit_cast(bf16x8, u);
        }
    }

    // ---- visibility limits (the wave's are wave-uniform)
    const int kv_end = a.causal ? min(a.Tk, a.q_offset + i0 + BM) : a.Tk;
    const int n = (kv_end + BN - 1) / BN;    // key tiles of the workgroup
    int t_lo = 0, t_hi = n;                  // the tiles this workgroup visits
    if constexpr (SPLIT) {
        const int per = (n + a.ks - 1) / a.ks;
        t_lo = min(n, split * per);
        t_hi = min(n, t_lo + per);
    }
    int row_lim[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) row_lim[rb] = a.causal ? min(a.Tk - 1, a.q_offset + iq[rb]) : a.Tk - 1;
    const int wave_last = a.causal ? min(a.Tk - 1, a.q_offset + i0w + 32 * RB - 1) : a.Tk - 1;
    // keys below wave_full are visible to every row of the wave
    const int wave_full = a.causal ? min(a.Tk, a.q_offset + i0w + 1) : a.Tk;
    const int last = i0w >= a.Tq ? -1 : wave_last / BN;  // last tile this wave computes

    // ---- K/V rings.  Copy of tile t: lane (wave, lane) fills the tile's
    //      16-byte slot 64 wave + lane, i.e. row cp_r0 at chunk position
    //      cp_p, with the logical chunk the swizzle puts there.  A tile at or
    //      past n is never read: its copy re-reads tile n-1 into the slot it
    //      would occupy, which holds no live data then.  Rows past the last
    //      key re-read the last key (finite values; those keys are masked).
    const unsigned kring = lds_addr(lds), vring = kring + NRING * TBK;
    const bf16* kh = a.k + b * a.ksb + hk * a.ksh;
    const bf16* vh = a.v + b * a.vsb + hk * a.vsh;
    const int kst = DENSE ? DK : a.kst, vst = DENSE ? DV : a.vst;   // elements between key rows
    const int cl = wave * 64 + lane;
    const int cpk_r0 = cl / NCHK, cpk_p = cl % NCHK;   // K tile slot of this lane
    const int cpv_r0 = cl / NCHV, cpv_p = cl % NCHV;   // V tile slot
    const unsigned cp_kcol = 16u * (unsigned)(cpk_p ^ swz_k<DK>(cpk_r0));
    const unsigned cp_vcol = 16u * (unsigned)(cpv_p ^ swz_v<DV>(cpv_r0));
    const unsigned cp_lds = (unsigned)(wave * 64 * 16);
    auto kslot = [&](int t) { return kring + (unsigned)((t % NRING) * TBK); };
    auto vslot = [&](int t) { return vring + (unsigned)((t % NRING) * TBV); };
    // Offset of the copies of a tile that lies wholly inside the keys: the
    // same for every such tile and copy instruction (the swizzle repeats
    // every RSTR rows; only the scalar source base moves).
    const unsigned cpk = (unsigned)cpk_r0 * (unsigned)(kst * 2) + cp_kcol;
    const unsigned cpv = (unsigned)cpv_r0 * (unsigned)(vst * 2) + cp_vcol;
    // NI copy instructions per lane, RS tile rows apart (C::NINSK / RSTRK for
    // K tiles, C::NINSV / RSTRV for V tiles)
    auto copy_full = [&](const bf16* head, int rs, int t, unsigned slot, unsigned off, auto ni, auto rstr) {
        constexpr int NI = decltype(ni)::value, RS = decltype(rstr)::value;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            copy16(head + (long long)(t * BN + i * RS) * rs, off, slot + (unsigned)(i * CPL * 16) + cp_lds);
    };
    auto copy_tile = [&](const bf16* head, int rs, int t, unsigned slot, unsigned col, int r0, auto ni,
                         auto rstr) {
        constexpr int NI = decltype(ni)::value, RS = decltype(rstr)::value;
        const int j0 = min(t, n - 1) * BN;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = min(r0 + i * RS, a.Tk - 1 - j0);
            copy16(head + (long long)j0 * rs, (unsigned)row * (unsigned)(rs * 2) + col,
                   slot + (unsigned)(i * CPL * 16) + cp_lds);
        }
    };
    // GEN: lane l of copy instruction i moves chunk g = i CPL + 64 wave + l
    // of the tile pair (K chunks first); a wave's 64 chunks are all K or all
    // V, so the wave picks the tensor and the LDS destination uniformly
    int gen_row[C::NCI];
    unsigned gen_col[C::NCI];
#pragma unroll
    for (int i = 0; i < C::NCI; ++i) {
        const int g = i * CPL + 64 * wave + lane;
        const bool isk = g < C::NCK;
        const int c = isk ? g : g - C::NCK, nch = isk ? NCHK : NCHV;
        gen_row[i] = c / nch;
        gen_col[i] = 16u * (unsigned)((c % nch) ^ (isk ? swz_k<DK>(c / nch) : swz_v<DV>(c / nch)));
    }
    auto copy_gen = [&](int t, int P) {
        const int j0 = min(t, n - 1) * BN;
#pragma unroll
        for (int i = 0; i < C::NCI; ++i) {
            const int gw = i * CPL + 64 * wave;   // the wave's first chunk
            if (gw < C::NCP) {
                const bool isk = gw < C::NCK;
                const int row = min(gen_row[i], a.Tk - 1 - j0);
                const int rs = isk ? kst : vst;
                const unsigned dst = isk ? kring + (unsigned)(P * TBK + 16 * gw)
                                         : vring + (unsigned)(P * TBV + 16 * (gw - C::NCK));
                copy16((isk ? kh : vh) + (long long)j0 * rs, (unsigned)row * (unsigned)(rs * 2) + gen_col[i], dst);
            }
        }
    };
    (void)copy_gen;
    constexpr IC<C::NINSK> nik{};
    constexpr IC<C::NINSV> niv{};
    constexpr IC<C::RSTRK> rsk{};
    constexpr IC<C::RSTRV> rsv{};

    // ---- per-lane fragment offsets in a tile (bytes).  The row term, the
    //      swizzled chunk term and the in-chunk term occupy disjoint bits, so
    //      slice m (block cb) is the slice-0 offset XOR 32m (64cb).
    // K operand (A of S^T): key row li, logical chunk 2m + h
    const unsigned koff = 2u * (unsigned)(li * DK + 8 * (h ^ swz_k<DK>(li)));
    // V^T operand via transpose reads: supplying lane (16g + 4r + qq) points
    // at V[key_base + 4(g/2) + r][32 cb + 16(g%2) + 4qq] (logical column)
    const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
    const unsigned voff =
        2u * (unsigned)((4 * (tg >> 1) + tr) * DV + 16 * (tg & 1) + 4 * tq + 8 * swz_v<DV>(tr));
    // The ring bases are 1024-byte aligned and the slot, block and slice
    // strides are multiples of 1024, so the XOR (bits 5-7) commutes with
    // adding them: every fragment read is a per-lane base plus a constant
    // offset once the slot is known at compile time (P = slot).
    unsigned kaddr[NQ], vaddr[NDB];
#pragma unroll
    for (int m = 0; m < NQ; ++m) kaddr[m] = kring + (koff ^ (32u * m));
#pragma unroll
    for (int cb = 0; cb < NDB; ++cb) vaddr[cb] = vring + (voff ^ (64u * cb));
    auto kfrag = [&](int P, int kb, int m) {
        return *(lds_bf16x8*)(uintptr_t)(kaddr[m] + (unsigned)(P * TBK + kb * 32 * DK * 2));
    };
    auto vfrag = [&](int P, int cb, int kc) {
        const unsigned addr = vaddr[cb] + (unsigned)(P * TBV + 16 * kc * DV * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(addr + 16u * DV));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x16 oacc[RB][NDB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[rb][cb][r] = 0.f;
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) { m_run[rb] = -INFINITY; l_run[rb] = 0.f; }
    const float cs = a.c;
    bf16x8 pb[RB][NKC];
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    // key offset (within the tile, before + 4h) of score element e
    auto key_of = [&](int e) { return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + (e & 3); };

    // S^T(tile in slot P) = K Q^T, plain order
    auto scores = [&](int P, Scores<DK, DV>& S) {
#pragma unroll
        for (int m = 0; m < NQ; ++m)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8 kf = kfrag(P, kb, m);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    S.s[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        kf, qf[rb][m], m == 0 ? f32x16{} : S.s[rb][kb], 0, 0, 0);
            }
    };
    auto mask_scores = [&](Scores<DK, DV>& S, int t) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int lim = row_lim[rb] - (t * BN + 4 * h);
#pragma unroll
            for (int e = 0; e < NE; ++e)
                if (key_of(e) > lim) S.s[rb][e >> 4][e & 15] = -INFINITY;
        }
    };
    // p = 2^(s c - m) for the score pair (e, e + 1) of row block rb, rounded
    // to bf16 into the B operand of P.V; the row sum adds the rounded weights
    auto exp_pair = [&](const Scores<DK, DV>& S, int rb, int e, float nm, float& sa, float& sb) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(S.s[rb][e >> 4][e & 15], cs, nm));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(S.s[rb][e >> 4][(e + 1) & 15], cs, nm));
        bf16x2 pk;
        pk[0] = (bf16)p0;
        pk[1] = (bf16)p1;
        pb[rb][e >> 3][e & 7] = pk[0];
        pb[rb][e >> 3][(e & 7) + 1] = pk[1];
        if (e & 2) sb = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, sb, false);
        else sa = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, sa, false);
    };
    // After the weights of a tile were formed against the running max: when
    // some weight would exceed 2^12, the rows concerned (both half-wave
    // lanes of a row) take the tile's max, rescale, and recompute (the other
    // rows get the very same weights); then add the tile to the row sums.
    auto fix_weights = [&](const Scores<DK, DV>& S, float (&sa)[RB], float (&sb)[RB]) {
        bool big[RB], any = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            big[rb] = !(sa[rb] + sb[rb] <= 4096.f);
            any = any || big[rb];
        }
        if (__any(any)) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)big[rb], (unsigned)big[rb], false, false);
                const bool row_big = (sw[0] | sw[1]) != 0u;
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < NE; ++e) mx = fmaxf(mx, S.s[rb][e >> 4][e & 15]);
                const float tmax = pair_max(mx) * cs;
                const float m_new = row_big ? fmaxf(m_run[rb], tmax) : m_run[rb];
                const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
                l_run[rb] *= alpha;
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[rb][cb][r] *= alpha;
                m_run[rb] = m_new;
                sa[rb] = 0.f;
                sb[rb] = 0.f;
#pragma unroll
                for (int e = 0; e < NE; e += 2) exp_pair(S, rb, e, -m_run[rb], sa[rb], sb[rb]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) l_run[rb] += sa[rb] + sb[rb];
    };

    // ---- prologue: copies of tiles t_lo .. t_lo + NRING-2 (slot = tile - t_lo);
    //      tile t_lo lands before the barrier
#pragma unroll
    for (int t = 0; t < NRING - 1; ++t) {
        if constexpr (C::GEN) {
            copy_gen(t_lo + t, t);
        } else {
            copy_tile(kh, kst, t_lo + t, kslot(t), cp_kcol, cpk_r0, nik, rsk);
            copy_tile(vh, vst, t_lo + t, vslot(t), cp_vcol, cpv_r0, niv, rsv);
        }
    }
    static_assert(NRING == 2, "the prologue waits for every copy");
    wait_vm<0>();
    __syncthreads();

    // One tile step: issue the copies of tile t + 1 (into the slots of tile
    // t - 1, read in step t - 1), then scores, weights and P V of tile t.  At
    // its end tile t + 1 has landed.  Overlap of the matrix and vector work
    // comes from the other workgroups on the CU.  Steps come in pairs so that
    // the ring slot of each (t % 2) is a compile-time constant.
    Scores<DK, DV> S;
    bool first = true;
    auto step = [&](int t, auto slot) {
        constexpr int P = decltype(slot)::value;
        const int tc = t + 1;
        if constexpr (C::GEN) {
            copy_gen(tc, 1 - P);
        } else if (tc < n && (tc + 1) * BN <= a.Tk) {
            copy_full(kh, kst, tc, kring + (unsigned)((1 - P) * TBK), cpk, nik, rsk);
            copy_full(vh, vst, tc, vring + (unsigned)((1 - P) * TBV), cpv, niv, rsv);
        } else {
            copy_tile(kh, kst, tc, kring + (unsigned)((1 - P) * TBK), cp_kcol, cpk_r0, nik, rsk);
            copy_tile(vh, vst, tc, vring + (unsigned)((1 - P) * TBV), cp_vcol, cpv_r0, niv, rsv);
        }
        if (t <= last) {
            scores(P, S);
            if ((t + 1) * BN > wave_full) mask_scores(S, t);
            if (first) {  // the running max starts at tile 0's max
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int e = 0; e < NE; ++e) mx = fmaxf(mx, S.s[rb][e >> 4][e & 15]);
                    m_run[rb] = pair_max(mx) * cs;
                    // a split's first tile may hold no key some rows see (then
                    // none of its tiles does): keep their reference finite
                    if constexpr (SPLIT)
                        if (m_run[rb] == -INFINITY) m_run[rb] = 0.f;
                }
                first = false;
            }
            float sa[RB], sb[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                sa[rb] = 0.f;
                sb[rb] = 0.f;
#pragma unroll
                for (int e = 0; e < NE; e += 2) exp_pair(S, rb, e, -m_run[rb], sa[rb], sb[rb]);
            }
            fix_weights(S, sa, sb);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb) {
                    const bf16x8 vf = vfrag(P, cb, kc);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        oacc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[rb][kc], oacc[rb][cb],
                                                                              0, 0, 0);
                }
        }
        wait_vm<0>();   // tile t + 1 has landed
        __syncthreads();
    };
    for (int t = t_lo; t < t_hi; t += 2) {
        step(t, IC<0>{});
        if (t + 1 < t_hi) step(t + 1, IC<1>{});
    }
    wait_vm<0>();   // no copy into LDS outlives the workgroup

    if constexpr (SPLIT) {   // partial output (relative to m_run), max and weight sum
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float l_tot = pair_sum(l_run[rb]);
            if (iq[rb] < a.Tq) {
                const size_t prow = ((size_t)(b * a.Hq + hq) * a.Tq + iq[rb]) * a.ks + split;
                float* po = a.part_o + prow * DV;
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        *reinterpret_cast<float4*>(po + 32 * cb + 8 * g4 + 4 * h) =
                            make_float4(oacc[rb][cb][4 * g4], oacc[rb][cb][4 * g4 + 1],
                                        oacc[rb][cb][4 * g4 + 2], oacc[rb][cb][4 * g4 + 3]);
                if (h == 0) {
                    a.part_ml[2 * prow] = l_tot > 0.f ? m_run[rb] : -INFINITY;
                    a.part_ml[2 * prow + 1] = l_tot;
                }
            }
        }
        return;
    }

    // ---- epilogue: O = O^T / l; lane holds columns 32cb + 8g4 + 4h .. +3 of row iq[rb]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l_tot = pair_sum(l_run[rb]);
        if (iq[rb] < a.Tq) {
            const float inv = 1.f / l_tot;
            bf16* orow = a.o + b * a.osb + hq * a.osh + (long long)iq[rb] * (DENSE ? DV : a.ost);
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    bf16x4 val;
#pragma unroll
                    for (int e = 0; e < 4; ++e) val[e] = (bf16)(oacc[rb][cb][4 * g4 + e] * inv);
                    *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * g4 + 4 * h) = val;
                }
            if (a.lse && h == 0)
                a.lse[(size_t)(b * a.Hq + hq) * a.Tq + iq[rb]] = (m_run[rb] + log2f(l_tot)) * kLn2;
        }
    }
}

// 12-wave workgroups (one per CU, each K/V tile serving 384 query rows) for
// dense head-size-128 launches long enough to give every CU at least four of
// them: a third of the tile copies per MFMA of the 4-wave workgroups, at the
// price of the overlap between workgroups on a CU.  Measured: workload 4
// (B1 Hq32 Hkv8 T16384) 1.4-2.0 % faster; workload 3 (B2 Hq32 Hkv8 T4096,
// 704 such workgroups) 0.7 % slower, so it keeps the 4-wave ones.
constexpr long long kWideMinWorkgroups = 1024;
bool wide_prefill(const FwdParams& p) {
    const long long nwg = (long long)((p.Tq + 383) / 384) * p.B * p.Hq;
    return nwg >= kWideMinWorkgroups;
}

template <int DK, int DV>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
    const bool dense = p.qs.t == DK && p.ks.t == DK && p.vs.t == DV && p.os.t == DV;
    typedef Cfg<DK, DV> C;
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
    a.qsb = p.qs.b; a.qsh = p.qs.h; a.qst = (int)p.qs.t;
    a.ksb = p.ks.b; a.ksh = p.ks.h; a.kst = (int)p.ks.t;
    a.vsb = p.vs.b; a.vsh = p.vs.h; a.vst = (int)p.vs.t;
    a.osb = p.os.b; a.osh = p.os.h; a.ost = (int)p.os.t;
    a.rope = reinterpret_cast<const float2*>(p.rope_tab);
    a.rope_adj = p.rope_adj;
    a.rope_pos0 = p.rope_pos0;
    const long long nwg = (long long)a.n_qt * a.G * a.R;
    a.ks = p.nsplit;
    a.part_o = p.part_o;
    a.part_ml = p.part_ml;
    if (p.nsplit > 1) {   // split over the keys: dense, no RoPE, one width
        if constexpr (DK != DV) {
            return hipErrorInvalidValue;
        } else {
            if (p.rope_tab || !dense) return hipErrorInvalidValue;
            hipLaunchKernelGGL((prefill_kernel<DK, DV, true, false, true>), dim3((unsigned)(nwg * p.nsplit)),
                               dim3(C::NW * 64), 0, stream, a);
            return hipGetLastError();
        }
    }
    if constexpr (DK == 128 && DV == 128) {
        if (dense && wide_prefill(p)) {   // fused RoPE or not
            typedef Cfg<DK, DV, 12> W;
            Args aw = a;
            aw.n_qt = (p.Tq + W::BM - 1) / W::BM;
            const long long nww = (long long)aw.n_qt * a.G * a.R;
            if (p.rope_tab)
                hipLaunchKernelGGL((prefill_kernel<DK, DV, true, true, false, 12>), dim3((unsigned)nww),
                                   dim3(W::NW * 64), 0, stream, aw);
            else
                hipLaunchKernelGGL((prefill_kernel<DK, DV, true, false, false, 12>), dim3((unsigned)nww),
                                   dim3(W::NW * 64), 0, stream, aw);
            return hipGetLastError();
        }
    }
    if constexpr (DK != DV) {   // one instantiation: dense, no RoPE (what attn_fwd_dv takes)
        if (p.rope_tab || !dense) return hipErrorInvalidValue;
        hipLaunchKernelGGL((prefill_kernel<DK, DV, true, false>), dim3((unsigned)nwg), dim3(C::NW * 64), 0,
                           stream, a);
    } else if (p.rope_tab) {   // dense layouts only (the fused-RoPE entry takes dense tensors)
        if (!dense) return hipErrorInvalidValue;
        hipLaunchKernelGGL((prefill_kernel<DK, DV, true, true>), dim3((unsigned)nwg), dim3(C::NW * 64), 0,
                           stream, a);
    } else if (dense) {
        hipLaunchKernelGGL((prefill_kernel<DK, DV, true, false>), dim3((unsigned)nwg), dim3(C::NW * 64), 0,
                           stream, a);
    } else {
        hipLaunchKernelGGL((prefill_kernel<DK, DV, false, false>), dim3((unsigned)nwg), dim3(C::NW * 64), 0,
                           stream, a);
    }
    return hipGetLastError();
}

}  // namespace

// Key splits: the launch has n_qt * B * Hq workgroups of 128 query rows; with
// fewer than two per CU of the 256 (a short chunk of queries over a long
// cache, a single short sequence) the chip idles, so each (query tile,
// head) is split over the keys into ks workgroups -- enough for about two
// per CU, at most 8, and each keeping at least 4 key tiles.  Decided from
// the sizes alone so the workspace can be sized before the call.
int prefill_splits(int B, int Hq, int Tq, int Tk, int d, int dv) {
    constexpr long long kWant = 512;   // workgroups a split launch aims for (two per CU)
    const long long nwg = (long long)((Tq + 127) / 128) * B * Hq;
    if (nwg <= 0 || nwg >= kWant || d != dv) return 1;
    const int bn = (d == 64 && dv == 64) ? 64 : 32;
    const long long tiles = (Tk + bn - 1) / bn;
    long long ks = (kWant + nwg - 1) / nwg;
    if (ks > 8) ks = 8;
    if (ks > tiles / 4) ks = tiles / 4;
    return ks < 2 ? 1 : (int)ks;
}

size_t prefill_split_bytes(int B, int Hq, int Tq, int dv, int ks) {
    if (ks < 2) return 0;
    return sizeof(float) * (size_t)B * Hq * Tq * ks * (size_t)(dv + 2);
}

hipError_t launch_prefill_bf16(const FwdParams& p, hipStream_t stream) {
    const int dv = p.dv ? p.dv : p.d;
    if (p.d == 64) return dv == 64 ? launch_d<64, 64>(p, stream) : launch_d<64, 128>(p, stream);
    return dv == 128 ? launch_d<128, 128>(p, stream) : launch_d<128, 64>(p, stream);
}

}  // namespace rocattn
