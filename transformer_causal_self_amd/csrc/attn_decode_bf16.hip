// attn_decode_bf16.hip -- one-token decode step over a key/value cache,
// bf16 in/out, float32 accumulation.  Head size 64 or 128, up to 16 query
// heads per K/V head.
//
// A decode step computes one new query row per query head at position
// q_offset (cache.pos) against the cached keys 0 .. q_offset ("The
// Transformer architecture" -- Hands-on; "Transformer" (ai-notes) -- Notes on
// compute: the KV cache makes each new token step incremental).  The work is
// dominated by reading the cache once, so the kernels are built for HBM
// bandwidth, not arithmetic:
//
//  * Split-K: the visible keys of each (batch, K/V head) are cut into chunks
//    and each chunk is one workgroup, so thousands of workgroups stream the
//    cache at once.  A workgroup serves all n_rep query heads of its K/V
//    head ("The Transformer architecture" -- GQA), so every K/V byte is read
//    exactly once.
//  * Scores: one v_mfma_f32_16x16x32_bf16 per 32 channels takes 16 keys
//    straight from the 16-byte global loads (the B operand is a key row) and
//    the query heads as the A operand, so no key is staged or converted.
//  * The chunk's scores (base-2 exponent units) sit in LDS; the chunk max
//    and the weights 2^(t - m) are formed there exactly once, then each lane
//    streams 8 channels of one value row and accumulates weight x value for
//    every query head in float32.
//  * Each chunk writes its unnormalised output, its max m and its weight sum
//    l; a second small kernel merges the chunks of a row with
//        o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s,
//    which equals the softmax over the whole row.
#include <math.h>

#include <atomic>

#include "internal.hpp"
#include "rope_math.hpp"

namespace rocattn {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of cache data that is read exactly once per step: the
// non-temporal hint keeps it from displacing reused lines in the caches
// (about 5% on a 32 x 8 x 8192 x 128 cache).
__device__ __forceinline__ bf16x8 ld_once(const void* p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(static_cast<const u32x4*>(p)));
}

constexpr int kSplitMax = 2048;     // workgroups the split may use in total (bounds the workspace)
constexpr int kLdsFloats = 16384;   // 64 KiB of LDS per workgroup at most

struct DecArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    float* o_part;   // [B*Hq][S][D]
    float* ml;       // [B*Hq][S][2]  (max in base-2 units, weight sum)
    int Hq, Hkv, Tk;
    int R;           // query heads per K/V head
    int kv_len;      // visible keys (keys 0 .. kv_len-1)
    int C;           // keys per chunk (multiple of 64)
    int S;           // chunks per (batch, K/V head)
    float c;         // |scale| * log2(e)
    unsigned neg;    // sign flip for q when scale < 0
    Strides qs, ks, vs;   // element strides (batch, head, token)
    // the cached generation step in one launch (STEP): q is rotated at pos
    // on load and written back rotated by the last workgroup of each
    // (batch, K/V head); the chunk holding pos rotates the new key, appends
    // it and the new value to the caches and uses them; the last workgroup
    // to arrive (counted in cnt, zero between calls) merges the chunks
    bf16* q_rot;
    const bf16* kn;       // new keys [B][Hkv][D]
    const bf16* vn;       // new values [B][Hkv][D]
    int pos;              // position of the new token (kv_len - 1)
    double rneg;          // -log2(base) / (D / 2)
    int adj;              // RoPE pairing: 0 split-half, 1 adjacent
    unsigned* cnt;        // arrival counters [B * Hkv]
    bf16* o;
    float* lse;
    Strides os;
};


// Merge of the S partial results of one output element: M = max_s m_s, then
// sum_s 2^(m_s - M) o_s and sum_s 2^(m_s - M) l_s, in batches of 8 chunks
// (one memory round trip per batch, not per chunk).
// COHERENT: read with device-scope atomic loads (partials other workgroups
// wrote during this kernel, see the STEP merge).
template <bool COHERENT = false>
__device__ inline float ld_partial(const float* p) {
    if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}
template <bool COHERENT = false>
__device__ inline void merge_partials(const float* mlr, const float* op, int S, int D, float& M, float& den,
                                      float& acc) {
    if (S <= 8) {   // one batch: every value loaded at once (one memory round trip)
        float mv[8], lv[8], ov[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool ok = u < S;
            mv[u] = ok ? ld_partial<COHERENT>(mlr + 2 * u) : -INFINITY;
            lv[u] = ok ? ld_partial<COHERENT>(mlr + 2 * u + 1) : 0.f;
            ov[u] = ok ? ld_partial<COHERENT>(op + (size_t)u * D) : 0.f;
        }
        M = -INFINITY;
#pragma unroll
        for (int u = 0; u < 8; ++u) M = fmaxf(M, mv[u]);
        den = 0.f;
        acc = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float w = exp2f(mv[u] - M);
            den = fmaf(w, lv[u], den);
            acc = fmaf(w, ov[u], acc);
        }
        return;
    }
    M = -INFINITY;
    for (int s0 = 0; s0 < S; s0 += 8) {
        float mv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) mv[u] = s0 + u < S ? ld_partial<COHERENT>(mlr + 2 * (s0 + u)) : -INFINITY;
#pragma unroll
        for (int u = 0; u < 8; ++u) M = fmaxf(M, mv[u]);
    }
    den = 0.f;
    acc = 0.f;
    for (int s0 = 0; s0 < S; s0 += 8) {
        float mv[8], lv[8], ov[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool ok = s0 + u < S;
            mv[u] = ok ? ld_partial<COHERENT>(mlr + 2 * (s0 + u)) : -INFINITY;
            lv[u] = ok ? ld_partial<COHERENT>(mlr + 2 * (s0 + u) + 1) : 0.f;
            ov[u] = ok ? ld_partial<COHERENT>(op + (size_t)(s0 + u) * D) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float w = exp2f(mv[u] - M);
            den = fmaf(w, lv[u], den);
            acc = fmaf(w, ov[u], acc);
        }
    }
}

// RoPE of a lane's query fragments at one position (the STEP kernel's q
// load): fragment m holds channels 32 m + 8 quarter .. + 7.  Split-half pair
// p = (p, p + D/2) joins fragment m with fragment m + NM/2; adjacent pair
// p = (2p, 2p + 1) lies inside a fragment.  The turn is the RoPE pass's
// (float32, rounded once to bf16).
template <int NM>
__device__ inline void rope_q_lane(bf16x8 (&q)[NM], const float2* tab, int adj, int quarter) {
    float y1, y2;
    if (!adj) {
#pragma unroll
        for (int m = 0; m < NM / 2; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float2 t = tab[32 * m + 8 * quarter + e];
                rope_turn((float)q[m][e], (float)q[m + NM / 2][e], t.x, t.y, y1, y2);
                q[m][e] = (bf16)y1;
                q[m + NM / 2][e] = (bf16)y2;
            }
    } else {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 t = tab[16 * m + 4 * quarter + e];
                rope_turn((float)q[m][2 * e], (float)q[m][2 * e + 1], t.x, t.y, y1, y2);
                q[m][2 * e] = (bf16)y1;
                q[m][2 * e + 1] = (bf16)y2;
            }
    }
}

struct CombArgs {
    const float* o_part;
    const float* ml;
    bf16* o;
    float* lse;
    int S;
    int Hq;
    int Tq;          // query rows per head (1 for a decode step)
    Strides os;
};

template <int D, int RP, bool STEP = false>  // RP: query heads per K/V head, padded to 4, 8 or 16
__global__ __launch_bounds__(256) void decode_split_kernel(DecArgs a) {
    extern __shared__ float dsm[];
    float* St = dsm;                  // [RP][C] scores (base-2 units)
    float* Pl = dsm + RP * a.C;       // [C][RP] weights
    float* Red = Pl + RP * a.C;       // [4][RP][D] per-wave partial outputs
    // STEP: the (cos, sin) of the pairs at pos, in the per-wave partial
    // region (free before phase 3 ends and after its reduction), and the
    // last-arrival flag in the score region (free after phase 2).  The
    // split kernel's LDS size is kept: a larger one fits fewer workgroups
    // on a CU, which costs this bandwidth-bound kernel more than it saves.
    float2* tab = reinterpret_cast<float2*>(Red);
    int* last_flag = reinterpret_cast<int*>(St);
    (void)tab; (void)last_flag;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto form_angles = [&]() {   // (cos, sin) of pair tid at pos, as the RoPE pass forms them
        if (tid < D / 2) {
            const double inv_freq = exp2((double)tid * a.rneg);
            double sn, cs;
            rope_sincos((double)a.pos * inv_freq, sn, cs);
            tab[tid] = make_float2((float)cs, (float)sn);
        }
    };
    (void)form_angles;
    const int s = blockIdx.x % a.S;
    const int g = blockIdx.x / a.S;                  // b * Hkv + hk
    const int b = g / a.Hkv, hk = g - (g / a.Hkv) * a.Hkv;
    const int j_begin = s * a.C;
    const int nkeys = min(a.kv_len, j_begin + a.C) - j_begin;   // >= 1
    const int hq0 = hk * a.R;

    // ---- query heads as the A operand: for MFMA m, lane (rho, quarter)
    //      holds q[hq0 + rho][32m + 8 quarter .. +7]; key rows are read in
    //      the same channel order, so the four lanes of a key row load 64
    //      contiguous bytes per instruction.
    constexpr int NM = D / 32;
    const int rho = lane & 15, quarter = lane >> 4;

    if constexpr (STEP) {
        // the float32 (cos, sin) of every pair at position pos, formed as
        // the RoPE pass forms them; the chunk holding pos turns the new key
        // and appends it and the new value to the caches before it reads
        // them (its own stores, completed before the barrier; no other
        // workgroup reads that row)
        form_angles();
        __syncthreads();
        if (s == a.S - 1) {
            if (tid < D / 2) {
                const int c1 = a.adj ? 2 * tid : tid, c2 = a.adj ? 2 * tid + 1 : tid + D / 2;
                const bf16* kr = a.kn + (size_t)g * D;
                float y1, y2;
                rope_turn((float)kr[c1], (float)kr[c2], tab[tid].x, tab[tid].y, y1, y2);
                bf16* kc = const_cast<bf16*>(a.k) + b * a.ks.b + hk * a.ks.h + (long long)a.pos * a.ks.t;
                kc[c1] = (bf16)y1;
                kc[c2] = (bf16)y2;
            } else if (tid < D / 2 + D / 8) {
                const int c = 8 * (tid - D / 2);
                bf16* vc = const_cast<bf16*>(a.v) + b * a.vs.b + hk * a.vs.h + (long long)a.pos * a.vs.t;
                *reinterpret_cast<uint4*>(vc + c) = *reinterpret_cast<const uint4*>(a.vn + (size_t)g * D + c);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }

    bf16x8 qa[NM];
    {
        const bool ok = rho < a.R;
        const uint4* src = reinterpret_cast<const uint4*>(
            a.q + b * a.qs.b + (hq0 + (ok ? rho : 0)) * a.qs.h + 8 * quarter);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            uint4 u = src[4 * m];
            if (!ok) u = make_uint4(0, 0, 0, 0);
            qa[m] = __builtin_bit_cast(bf16x8, u);
        }
        if constexpr (STEP) rope_q_lane(qa, tab, a.adj, quarter);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            uint4 u = __builtin_bit_cast(uint4, qa[m]);
            u.x ^= a.neg; u.y ^= a.neg; u.z ^= a.neg; u.w ^= a.neg;
            qa[m] = __builtin_bit_cast(bf16x8, u);
        }
    }

    // ---- phase 1: scores of 16 keys per MFMA group
    const int ngroups = (nkeys + 15) >> 4;

    const bf16* kbase = a.k + b * a.ks.b + hk * a.ks.h + 8 * quarter;
#pragma unroll 4
    for (int gi = wave; gi < ngroups; gi += 4) {
        const int kl = gi * 16 + rho;            // key (local) whose row this lane loads
        const bool kvalid = kl < nkeys;
        const uint4* kp = reinterpret_cast<const uint4*>(
            kbase + (j_begin + (kvalid ? kl : 0)) * a.ks.t);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const bf16x8 kf = ld_once(kp + 4 * m);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[m], kf, acc, 0, 0, 0);
        }
        // acc[r] = score of query head 4*quarter + r against key gi*16 + rho
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * quarter + r;
            if (row < RP && row < a.R) St[row * a.C + kl] = kvalid ? acc[r] * a.c : -INFINITY;
        }
    }
    __syncthreads();

    // ---- phase 2: chunk max and weights, one wave per query head
    for (int row = wave; row < a.R; row += 4) {
        const float* sr = St + row * a.C;
        float mx = -INFINITY;
        for (int j = lane; j < nkeys; j += 64) mx = fmaxf(mx, sr[j]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        float sum = 0.f;
        for (int j = lane; j < nkeys; j += 64) {
            const float p = exp2f(sr[j] - mx);
            Pl[j * RP + row] = p;
            sum += p;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        if (lane == 0) {
            float* mlp = a.ml + ((size_t)(b * a.Hq + hq0 + row) * a.S + s) * 2;
            if constexpr (STEP) {   // device-coherent: another workgroup merges them
                __hip_atomic_store(mlp, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(mlp + 1, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                mlp[0] = mx;
                mlp[1] = sum;
            }
        }
    }
    __syncthreads();

    // ---- phase 3: weighted sum of value rows, 8 channels per lane
    constexpr int LPK = D / 8;       // lanes per value row
    constexpr int KPW = 64 / LPK;    // value rows per wave per step
    const int kk = lane / LPK, col = (lane % LPK) * 8;
    float acc[RP][8];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
    const bf16* vbase = a.v + b * a.vs.b + hk * a.vs.h + j_begin * a.vs.t + col;
#pragma unroll 8
    for (int j = wave * KPW + kk; j < nkeys; j += 4 * KPW) {
        const bf16x8 vv = ld_once(vbase + j * a.vs.t);
        float vf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = (float)vv[e];
        const float* pr = Pl + j * RP;
#pragma unroll
        for (int r4 = 0; r4 < RP; r4 += 4) {
            const float4 p4 = *reinterpret_cast<const float4*>(pr + r4);
            const float pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r4 + u][e] = fmaf(pp[u], vf[e], acc[r4 + u][e]);
        }
    }
    // lanes that share `col` hold different keys: fold them together
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1)
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] += __shfl_xor(acc[r][e], off);
    if (kk == 0) {
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int e = 0; e < 8; e += 4)
                *reinterpret_cast<float4*>(Red + (wave * RP + r) * D + col + e) =
                    make_float4(acc[r][e], acc[r][e + 1], acc[r][e + 2], acc[r][e + 3]);
    }
    __syncthreads();
    for (int idx = tid; idx < a.R * D; idx += 256) {
        const int r = idx / D, dd = idx - r * D;
        const float sum = Red[(0 * RP + r) * D + dd] + Red[(1 * RP + r) * D + dd] +
                          Red[(2 * RP + r) * D + dd] + Red[(3 * RP + r) * D + dd];
        float* dst = a.o_part + ((size_t)(b * a.Hq + hq0 + r) * a.S + s) * D + dd;
        if constexpr (STEP) __hip_atomic_store(dst, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *dst = sum;
    }

    if constexpr (STEP) {
        // Count this chunk's arrival once its partials are written (their
        // device-scope stores complete before the count); the last of the S
        // chunks of (b, hk) merges all of them with device-scope loads (every
        // other chunk has written its partials and read q by then), writes
        // q back rotated and leaves the counter at zero for the next call.
        // Device-scope atomics on the partials instead of plain stores and a
        // device-wide fence: the fence would write back the whole L2 of the
        // XCD, once per workgroup.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0)
            *last_flag = __hip_atomic_fetch_add(a.cnt + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                                 (unsigned)(a.S - 1)
                             ? 1
                             : 0;
        __syncthreads();
        if (*last_flag) {
            form_angles();   // the partial region is free again
            // this thread's query pairs for the write-back, loaded before the
            // merge so that the two memory round trips overlap
            constexpr int QPT = (16 * (D / 2) + 255) / 256;   // pairs per thread, for up to 16 heads
            float qx1[QPT], qx2[QPT];
#pragma unroll
            for (int u = 0; u < QPT; ++u) {
                const int idx = tid + 256 * u;
                qx1[u] = qx2[u] = 0.f;
                if (idx < a.R * (D / 2)) {
                    const int r = idx / (D / 2), p = idx - r * (D / 2);
                    const int c1 = a.adj ? 2 * p : p, c2 = a.adj ? 2 * p + 1 : p + D / 2;
                    const bf16* qr = a.q_rot + b * a.qs.b + (hq0 + r) * a.qs.h;
                    qx1[u] = (float)qr[c1];
                    qx2[u] = (float)qr[c2];
                }
            }
            for (int idx = tid; idx < a.R * D; idx += 256) {
                const int r = idx / D, col2 = idx - r * D;
                const size_t row = (size_t)(b * a.Hq + hq0 + r);
                float M, den, acc2;
                merge_partials<true>(a.ml + row * a.S * 2, a.o_part + row * a.S * D + col2, a.S, D, M, den, acc2);
                a.o[b * a.os.b + (hq0 + r) * a.os.h + col2] = (bf16)(acc2 / den);
                if (a.lse && col2 == 0) a.lse[row] = (M + log2f(den)) * kLn2;
            }
            __syncthreads();   // the angles are formed
#pragma unroll
            for (int u = 0; u < QPT; ++u) {
                const int idx = tid + 256 * u;
                if (idx < a.R * (D / 2)) {
                    const int r = idx / (D / 2), p = idx - r * (D / 2);
                    const int c1 = a.adj ? 2 * p : p, c2 = a.adj ? 2 * p + 1 : p + D / 2;
                    bf16* qr = a.q_rot + b * a.qs.b + (hq0 + r) * a.qs.h;
                    float y1, y2;
                    rope_turn(qx1[u], qx2[u], tab[p].x, tab[p].y, y1, y2);
                    qr[c1] = (bf16)y1;
                    qr[c2] = (bf16)y2;
                }
            }
            if (tid == 0) __hip_atomic_store(a.cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(CombArgs a) {
    const size_t row = blockIdx.x;             // (b * Hq + hq) * Tq + i
    const int col = threadIdx.x;
    float M, den, acc;
    merge_partials(a.ml + row * a.S * 2, a.o_part + row * a.S * D + col, a.S, D, M, den, acc);
    const size_t bh = row / a.Tq;
    const int i = (int)(row - bh * a.Tq);
    const int b = (int)(bh / a.Hq), hq = (int)(bh - (size_t)b * a.Hq);
    a.o[b * a.os.b + hq * a.os.h + (long long)i * a.os.t + col] = (bf16)(acc / den);
    if (a.lse && col == 0) a.lse[row] = (M + log2f(den)) * kLn2;
}

// The same merge for a prefill's key splits (S <= 8 partials per row, many
// rows): D / 4 lanes per row, four columns each, 256 / (D / 4) rows per
// block, every partial of a lane loaded at once.
template <int D>
__global__ __launch_bounds__(256) void combine_rows_kernel(CombArgs a, long long rows) {
    constexpr int TPR = D / 4, RPB = 256 / TPR;
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int col = (threadIdx.x % TPR) * 4;
    if (row >= rows) return;
    const float* mlr = a.ml + row * a.S * 2;
    const float* op = a.o_part + row * a.S * D + col;
    float mv[8], lv[8];
    float4 ov[8];
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const bool ok = s < a.S;
        mv[s] = ok ? mlr[2 * s] : -INFINITY;
        lv[s] = ok ? mlr[2 * s + 1] : 0.f;
        ov[s] = ok ? *reinterpret_cast<const float4*>(op + (size_t)s * D) : make_float4(0.f, 0.f, 0.f, 0.f);
        M = fmaxf(M, mv[s]);
    }
    float den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const float w = s < a.S ? exp2f(mv[s] - M) : 0.f;
        den = fmaf(w, lv[s], den);
        acc.x = fmaf(w, ov[s].x, acc.x);
        acc.y = fmaf(w, ov[s].y, acc.y);
        acc.z = fmaf(w, ov[s].z, acc.z);
        acc.w = fmaf(w, ov[s].w, acc.w);
    }
    const float inv = 1.f / den;
    const long long bh = row / a.Tq;
    const int i = (int)(row - bh * a.Tq);
    const int b = (int)(bh / a.Hq), hq = (int)(bh - (long long)b * a.Hq);
    bf16x4 val;
    val[0] = (bf16)(acc.x * inv);
    val[1] = (bf16)(acc.y * inv);
    val[2] = (bf16)(acc.z * inv);
    val[3] = (bf16)(acc.w * inv);
    *reinterpret_cast<bf16x4*>(a.o + b * a.os.b + hq * a.os.h + (long long)i * a.os.t + col) = val;
    if (a.lse && col == 0) a.lse[row] = (M + log2f(den)) * kLn2;
}

int pad_r(int R) { return R <= 4 ? 4 : (R <= 8 ? 8 : 16); }

// longest chunk whose scores, weights and partial outputs fit the LDS cap
int chunk_max(int R, int D) {
    const int rp = pad_r(R);
    return ((kLdsFloats - 4 * rp * D) / (2 * rp)) & ~63;
}

int split_target(int G) {
    const int s = (kSplitMax + G - 1) / G;
    return s < 1 ? 1 : s;
}

// Workgroups of decode_split_kernel<D, pad_r(R)> one CU holds at once by
// its registers alone (asked of the runtime once per instantiation).
int resident_by_regs(int R, int D) {
    static std::atomic<int> cache[2][3];
    const int rp = pad_r(R), i = D == 64 ? 0 : 1, j = rp == 4 ? 0 : (rp == 8 ? 1 : 2);
    int n = cache[i][j].load(std::memory_order_relaxed);
    if (n > 0) return n;
    const void* f = D == 64 ? (rp == 4 ? (const void*)decode_split_kernel<64, 4>
                                       : rp == 8 ? (const void*)decode_split_kernel<64, 8>
                                                 : (const void*)decode_split_kernel<64, 16>)
                            : (rp == 4 ? (const void*)decode_split_kernel<128, 4>
                                       : rp == 8 ? (const void*)decode_split_kernel<128, 8>
                                                 : (const void*)decode_split_kernel<128, 16>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 256, 0) != hipSuccess || n < 1) n = 1;
    cache[i][j].store(n, std::memory_order_relaxed);
    return n;
}

// Chunk length and split count for kv_len visible keys.  A chunk is one
// workgroup and the step is HBM-bound, so a CU's time is about the chunks it
// gets times their length (plus a fixed cost worth ~256 keys), as long as
// enough workgroups sit on it at once to keep the memory busy (about 3;
// fewer stretch the time in proportion).  Longer chunks need more LDS, so
// fewer fit on a CU.  The split count S is chosen to minimise
//     ceil(G S / CUs) (C + 256) max(1, 3 / resident),
//     resident = min(workgroups that fit a CU, ceil(G S / CUs)),
// over ceil(kv_len / chunk_max) <= S <= max(that, ceil(kSplitMax / G)).
// (Measured on the decode shapes tried, it ranks the splits as they time.)
void plan(int G, int R, int D, int kv_len, int* C_out, int* S_out) {
    const int c_max = chunk_max(R, D);
    const int rp = pad_r(R);
    int dev = 0, cus = 256, lds_cu = 160 * 1024;
    if (hipGetDevice(&dev) == hipSuccess) {
        int x;
        if (hipDeviceGetAttribute(&x, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && x > 0) cus = x;
        if (hipDeviceGetAttribute(&x, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
            x > 0)
            lds_cu = x;
    }
    const int by_regs = resident_by_regs(R, D);
    const int s_lo = (kv_len + c_max - 1) / c_max;
    const int s_hi = s_lo > split_target(G) ? s_lo : split_target(G);
    double best = 0.0;
    int best_C = c_max, best_S = s_lo;
    for (int S = s_lo; S <= s_hi; ++S) {
        int C = (kv_len + S - 1) / S;
        C = (C + 63) & ~63;
        if (C < 64) C = 64;
        if (C > c_max) C = c_max;
        const int S_eff = (kv_len + C - 1) / C;
        if (S_eff != S) continue;   // another S gives this chunk length
        const long long lds = (long long)sizeof(float) * (2LL * rp * C + 4LL * rp * D);
        const int fit = (int)(lds_cu / lds) < by_regs ? (int)(lds_cu / lds) : by_regs;
        const long long per_cu = ((long long)G * S + cus - 1) / cus;
        const double resident = fit < per_cu ? (double)(fit > 0 ? fit : 1) : (double)per_cu;
        const double cost = (double)per_cu * (C + 256) * (resident < 3.0 ? 3.0 / resident : 1.0);
        if (S == s_lo || cost < best) {
            best = cost;
            best_C = C;
            best_S = S;
        }
    }
    *C_out = best_C;
    *S_out = best_S;
}

template <int D, int RP, bool STEP = false>
hipError_t launch_split(const DecArgs& a, int grid, hipStream_t stream) {
    const size_t lds = sizeof(float) * ((size_t)2 * RP * a.C + (size_t)4 * RP * D);
    hipLaunchKernelGGL((decode_split_kernel<D, RP, STEP>), dim3(grid), dim3(256), lds, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dec_d(const FwdParams& p, float* o_part, float* ml, int C, int S,
                        int kv_len, hipStream_t stream) {
    DecArgs a;
    a.q = static_cast<const bf16*>(p.q);
    a.k = static_cast<const bf16*>(p.k);
    a.v = static_cast<const bf16*>(p.v);
    a.o_part = o_part;
    a.ml = ml;
    a.Hq = p.Hq; a.Hkv = p.Hkv; a.Tk = p.Tk;
    a.R = p.Hq / p.Hkv;
    a.kv_len = kv_len;
    a.C = C; a.S = S;
    a.c = fabsf(p.scale) * kLog2e;
    a.neg = p.scale < 0.f ? 0x80008000u : 0u;
    a.qs = p.qs; a.ks = p.ks; a.vs = p.vs;
    const int grid = p.B * p.Hkv * S;
    const int rp = pad_r(a.R);
    hipError_t e = rp == 4 ? launch_split<D, 4>(a, grid, stream)
                 : rp == 8 ? launch_split<D, 8>(a, grid, stream)
                           : launch_split<D, 16>(a, grid, stream);
    if (e != hipSuccess) return e;
    CombArgs c;
    c.o_part = o_part;
    c.ml = ml;
    c.o = static_cast<bf16*>(p.o);
    c.lse = p.lse;
    c.S = S;
    c.Hq = p.Hq;
    c.Tq = 1;
    c.os = p.os;
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(p.B * p.Hq), dim3(D), 0, stream, c);
    return hipGetLastError();
}

int visible_keys(int Tk, int causal, int q_offset) {
    return causal ? (q_offset + 1 < Tk ? q_offset + 1 : Tk) : Tk;
}

}  // namespace

hipError_t launch_combine_bf16(const float* part_o, const float* part_ml, void* o, float* lse,
                               long long rows, int S, int Hq, int Tq, const Strides& os, int d,
                               hipStream_t stream) {
    CombArgs c;
    c.o_part = part_o;
    c.ml = part_ml;
    c.o = static_cast<bf16*>(o);
    c.lse = lse;
    c.S = S;
    c.Hq = Hq;
    c.Tq = Tq;
    c.os = os;
    if (S > 8) return hipErrorInvalidValue;
    if (d == 64)
        hipLaunchKernelGGL(combine_rows_kernel<64>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, c,
                           rows);
    else
        hipLaunchKernelGGL(combine_rows_kernel<128>, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, stream, c,
                           rows);
    return hipGetLastError();
}

bool decode_bf16_supported(int Hq, int Hkv, int d) {
    return (d == 64 || d == 128) && Hq / Hkv <= 16;
}

// Bytes for any call with at most Tk visible keys: the split count never
// exceeds max(split_target, ceil(Tk / chunk_max)).
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int Tk, int d) {
    const int s_target = split_target(B * Hkv);
    const int c_max = chunk_max(Hq / Hkv, d);
    int S = (Tk + c_max - 1) / c_max;
    if (S < s_target) S = s_target;
    return sizeof(float) * (size_t)B * Hq * S * (d + 2);
}

size_t decode_step_counter_offset(int B, int Hq, int Hkv, int Tmax, int d) {
    return (decode_workspace_bytes(B, Hq, Hkv, Tmax, d) + 255) & ~(size_t)255;
}

size_t decode_step_workspace_bytes(int B, int Hq, int Hkv, int Tmax, int d) {
    return decode_step_counter_offset(B, Hq, Hkv, Tmax, d) + sizeof(unsigned) * (size_t)B * Hkv;
}

hipError_t launch_decode_step_bf16(const StepParams& sp, void* workspace, size_t ws_bytes, hipStream_t stream) {
    const int D = sp.d, R = sp.Hq / sp.Hkv, G = sp.B * sp.Hkv;
    const int kv_len = sp.pos + 1;
    int C, S;
    plan(G, R, D, kv_len, &C, &S);
    const size_t cnt_off = decode_step_counter_offset(sp.B, sp.Hq, sp.Hkv, sp.Tmax, D);
    if (ws_bytes < cnt_off + sizeof(unsigned) * (size_t)G) return hipErrorInvalidValue;
    DecArgs a;
    a.q = static_cast<const bf16*>(sp.q);
    a.k = static_cast<const bf16*>(sp.kc);
    a.v = static_cast<const bf16*>(sp.vc);
    a.o_part = static_cast<float*>(workspace);
    a.ml = a.o_part + (size_t)sp.B * sp.Hq * S * D;
    a.Hq = sp.Hq; a.Hkv = sp.Hkv; a.Tk = kv_len;
    a.R = R;
    a.kv_len = kv_len;
    a.C = C; a.S = S;
    a.c = fabsf(sp.scale) * kLog2e;
    a.neg = sp.scale < 0.f ? 0x80008000u : 0u;
    a.qs = {(long long)sp.Hq * D, (long long)D, D};
    a.ks = {(long long)sp.Hkv * sp.Tmax * D, (long long)sp.Tmax * D, D};
    a.vs = a.ks;
    a.q_rot = static_cast<bf16*>(sp.q);
    a.kn = static_cast<const bf16*>(sp.kn);
    a.vn = static_cast<const bf16*>(sp.vn);
    a.pos = sp.pos;
    a.rneg = -log2(sp.base) / (double)(D / 2);
    a.adj = sp.pairing;
    a.cnt = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + cnt_off);
    a.o = static_cast<bf16*>(sp.o);
    a.lse = sp.lse;
    a.os = a.qs;
    const int grid = G * S;
    const int rp = pad_r(R);
    if (D == 64)
        return rp == 4 ? launch_split<64, 4, true>(a, grid, stream)
             : rp == 8 ? launch_split<64, 8, true>(a, grid, stream)
                       : launch_split<64, 16, true>(a, grid, stream);
    return rp == 4 ? launch_split<128, 4, true>(a, grid, stream)
         : rp == 8 ? launch_split<128, 8, true>(a, grid, stream)
                   : launch_split<128, 16, true>(a, grid, stream);
}

hipError_t launch_decode_bf16(const FwdParams& p, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
    const int kv_len = visible_keys(p.Tk, p.causal, p.q_offset);
    int C, S;
    plan(p.B * p.Hkv, p.Hq / p.Hkv, p.d, kv_len, &C, &S);
    const size_t need = sizeof(float) * (size_t)p.B * p.Hq * S * (p.d + 2);
    if (ws_bytes < need) return hipErrorInvalidValue;
    float* o_part = static_cast<float*>(workspace);
    float* ml = o_part + (size_t)p.B * p.Hq * S * p.d;
    if (p.d == 64) return launch_dec_d<64>(p, o_part, ml, C, S, kv_len, stream);
    return launch_dec_d<128>(p, o_part, ml, C, S, kv_len, stream);
}

}  // namespace rocattn
