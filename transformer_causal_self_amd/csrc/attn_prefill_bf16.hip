// attn_prefill_bf16.hip -- fused causal attention forward, bf16 in/out,
// float32 accumulation, on the gfx950 matrix cores.  Head size 64 or 128.
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
//  * Keys are visited in tiles of 64.  K and V tiles are copied from HBM
//    into LDS with 16-byte loads and shared by the four waves.
//  * Scores are formed transposed, S^T = K Q^T (keys on the MFMA rows,
//    queries on its columns), so in the accumulator layout each lane holds
//    scores of ONE query row (lane % 32) for 16 keys: the row max and row
//    sum need no cross-lane work except one v_permlane32_swap between the
//    two half-waves, and the running max / sum / rescale factor of a row
//    are per-lane scalars.
//  * Software pipeline: K runs one tile ahead of V.  While a wave turns the
//    scores of tile t into weights (VALU) and multiplies them into V(t)
//    (MFMA), the MFMAs for the scores of tile t+1 are already in flight:
//    they read K(t+1), which was staged in LDS one iteration earlier, and
//    depend on nothing the softmax produces.  Global loads run two tiles
//    (K) and one tile (V) ahead; one barrier per tile.
//  * Softmax in base 2: p = 2^(s * |scale| * log2(e) - m) with the raw
//    v_exp_f32.  The running max m is only raised when a tile's max exceeds
//    it by more than 8 (a factor 256), so the output accumulator is
//    rescaled rarely; the final division by the row sum cancels whichever m
//    was used.  A negative scale is applied by negating q on load.
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
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int NW = 4;                  // waves per workgroup
    static constexpr int BM = 32 * NW;            // query rows per workgroup
    static constexpr int SK = D + 8;              // K tile row stride (elements)
    static constexpr int SV = D + 32;             // V tile row stride (elements)
    static constexpr int K_ELEMS = BN * SK;
    static constexpr int V_ELEMS = BN * SV;
    static constexpr int CHUNKS_ROW = D / 8;      // 16-byte chunks per row
    static constexpr int ROWS_PASS = 256 / CHUNKS_ROW;
    static constexpr int PASSES = BN / ROWS_PASS;
    static_assert(BN % ROWS_PASS == 0, "tile rows must split evenly");
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

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct Tile {
    static constexpr int NKB = Cfg<D>::BN / 32;  // 32-key blocks per tile
    f32x16 s[NKB];
};

struct Unmasked { static constexpr bool value = false; };
struct Masked { static constexpr bool value = true; };

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(Args a) {
    typedef Cfg<D> C;
    constexpr int BN = C::BN, BM = C::BM, SK = C::SK, SV = C::SV;
    constexpr int NKB = BN / 32;   // 32-key blocks per tile
    constexpr int NDB = D / 32;    // 32-column blocks of the output
    constexpr int NQ = D / 16;     // 16-wide d slices of q.k
    __shared__ __attribute__((aligned(16))) bf16 kbuf[2][C::K_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 vbuf[2][C::V_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
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

    // ---- K/V tile copy: thread -> (row, 16-byte chunk)
    const bf16* kh = a.k + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const bf16* vh = a.v + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const int cp_chunk = tid % C::CHUNKS_ROW, cp_row = tid / C::CHUNKS_ROW;
    auto load_rows = [&](const bf16* src, int j0, uint4* reg) {
#pragma unroll
        for (int pp = 0; pp < C::PASSES; ++pp) {
            const int key = j0 + cp_row + pp * C::ROWS_PASS;
            reg[pp] = key < a.Tk
                          ? *reinterpret_cast<const uint4*>(src + (size_t)key * D + cp_chunk * 8)
                          : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_rows = [&](bf16* dst, int stride, const uint4* reg) {
#pragma unroll
        for (int pp = 0; pp < C::PASSES; ++pp)
            *reinterpret_cast<uint4*>(dst + (cp_row + pp * C::ROWS_PASS) * stride + cp_chunk * 8) =
                reg[pp];
    };

    // ---- per-lane LDS offsets
    // K operand (A of S^T): key row 32kb + li, columns 16m + 8h .. +7
    const int k_off = li * SK + 8 * h;
    // V^T operand via transpose reads: supplying lane (16g + 4r + qq) points
    // at V[key_base + 4(g/2) + r][32 cb + 16(g%2) + 4qq]
    const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
    const int v_off = (4 * (tg >> 1) + tr) * SV + 16 * (tg & 1) + 4 * tq;

    // ---- visibility limits of this lane's row and of the wave
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

    // S^T(tile) = K(tile) Q^T from the K tile at Ks
    auto scores = [&](const bf16* Ks, Tile<D>& T) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) T.s[kb][r] = 0.f;
#pragma unroll
        for (int m = 0; m < NQ; ++m)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + k_off + kb * 32 * SK + 16 * m);
                T.s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[m], T.s[kb], 0, 0, 0);
            }
    };

    // weights of one tile and O^T += V^T P^T
    auto softmax_pv = [&](Tile<D>& T, const bf16* Vs, int j0, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        float mx = -INFINITY;
        if constexpr (MASKED) {
            const int lim = row_lim - (j0 + 4 * h);  // key offsets above lim are masked
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                    T.s[kb][r] = off > lim ? -INFINITY : T.s[kb][r];
                }
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, T.s[kb][r]);
        mx = pair_max(mx);
        const float tmax = mx * cs;
        // raise the running max only when it grew by more than 2^8
        const bool need = tmax > m_run + 8.f;
        if (__any(need)) {
            const float m_new = need ? tmax : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
            m_run = m_new;
        }
        const float nm = -m_run;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                bf16x8 pb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(T.s[kb][8 * cc + e], cs, nm));
                    l_run += pv;
                    pb[e] = (bf16)pv;
                }
#pragma unroll
                for (int cb = 0; cb < NDB; ++cb) {
                    const bf16* vp = Vs + v_off + (32 * kb + 16 * cc) * SV + 32 * cb;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * SV));
                    const bf16x8 vf = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, oacc[cb], 0, 0, 0);
                }
            }
    };

    // ---- prologue: K(0), V(0), K(1) into LDS; scores of tile 0
    uint4 kreg[C::PASSES], vreg[C::PASSES];
    load_rows(kh, 0, kreg);
    load_rows(vh, 0, vreg);
    store_rows(kbuf[0], SK, kreg);
    store_rows(vbuf[0], SV, vreg);
    if (n_tiles > 1) {
        load_rows(kh, BN, kreg);
        store_rows(kbuf[1], SK, kreg);
    }
    __syncthreads();

    Tile<D> SA, SB;
    scores(kbuf[0], SA);  // tile 0 is visible to every wave (key 0 is)

    // one pipeline step: softmax/PV of tile t (scores in cur) while the
    // scores of tile t+1 go into nxt
    auto step = [&](int t, Tile<D>& cur, Tile<D>& nxt) {
        const int j0 = t * BN;
        const bool more_k = t + 2 < n_tiles, more_v = t + 1 < n_tiles;
        if (more_k) load_rows(kh, j0 + 2 * BN, kreg);
        if (more_v) load_rows(vh, j0 + BN, vreg);
        if (more_v && j0 + BN <= wave_last) scores(kbuf[(t + 1) & 1], nxt);
        if (j0 <= wave_last) {
            if (j0 + BN > wave_full)
                softmax_pv(cur, vbuf[t & 1], j0, Masked());
            else
                softmax_pv(cur, vbuf[t & 1], j0, Unmasked());
        }
        if (more_k) store_rows(kbuf[t & 1], SK, kreg);
        if (more_v) store_rows(vbuf[(t + 1) & 1], SV, vreg);
        __syncthreads();
    };

    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
        step(t, SA, SB);
        step(t + 1, SB, SA);
    }
    if (t < n_tiles) step(t, SA, SB);

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

hipError_t launch_prefill_bf16(const FwdParams& p, hipStream_t stream) {
    if (p.d == 64) return launch_d<64>(p, stream);
    return launch_d<128>(p, stream);
}

}  // namespace rocattn
