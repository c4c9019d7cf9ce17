// rope.hip -- rotary position embedding applied in place to q and k.
//
// Token t of a sequence sits at position pos = pos0 + t ("The Transformer
// architecture" -- Hands-on: RoPE is sliced from cache.pos).  Channel pair p
// of a head vector is (p, p + d/2) (split-half pairing, "The Transformer
// architecture" -- Now: RoPE, apply_rope) or (2p, 2p + 1) (adjacent
// pairing, "Transformer" (ai-notes) -- RoPE), and turns by
// theta_p = pos * base^(-2p/d) ("Transformer" (ai-notes) -- RoPE) through
// [[cos, -sin], [sin, cos]].
//
// Angles: each lane forms, in double precision, the cosine and sine of the
// few pairs it owns at one position, rounds them once to float32, and then
// rotates that (position, pairs) slot in every head and batch entry of its
// share.  On request the lanes of the first row chunk also store those
// float32 (cos, sin) values in a table [position][d/2], which the attention
// kernel's query load reads.  The work is HBM-bound
// (one read and one write of q and k); each lane moves 2 x 8 bytes (bf16) or
// 2 x 16 bytes (f32) per head row, with neighbouring lanes on neighbouring
// pairs so every head row is read and written by full, coalesced segments.
#include <math.h>

#include "internal.hpp"
#include "rope_math.hpp"

namespace rocattn {
namespace {

constexpr int kThreads = 256;

// NP consecutive elements of type T, moved as one load / store.
template <typename T, int NP>
struct __attribute__((aligned(sizeof(T) * NP))) Pack {
    T e[NP];
};

template <typename T, int NP>
__device__ inline void load_f32(const T* src, float* f) {
    Pack<T, NP> v = *reinterpret_cast<const Pack<T, NP>*>(src);
#pragma unroll
    for (int u = 0; u < NP; ++u) f[u] = (float)v.e[u];
}

template <typename T, int NP>
__device__ inline void store_f32(T* dst, const float* f) {
    Pack<T, NP> v;
#pragma unroll
    for (int u = 0; u < NP; ++u) v.e[u] = (T)f[u];
    *reinterpret_cast<Pack<T, NP>*>(dst) = v;
}

// grid.x: (token, pair-group) slots; grid.y: chunks of the head rows, the
// n_seq rows of x followed by the n_seq2 rows of x2 (q and k of one call
// share the angles of a slot, so one launch turns both).
// ADJ: adjacent pairing (the lane's 2 kPairs channels are contiguous).
template <typename T, int kPairs, bool ADJ>  // kPairs channel pairs per lane
__global__ __launch_bounds__(kThreads) void rope_kernel(T* __restrict__ x, long long n_seq,
                                                        T* __restrict__ x2, long long n_seq2,
                                                        int rows_per_chunk, int T_len, int d,
                                                        int pos0, double neg_log2_base_over_half,
                                                        float2* __restrict__ tab) {
    const int half = d >> 1;
    const int groups = half / kPairs;  // lanes per token
    const long long slot = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (slot >= (long long)T_len * groups) return;
    const int t = (int)(slot / groups);
    const int p0 = (int)(slot - (long long)t * groups) * kPairs;

    float cs[kPairs], sn[kPairs];
    const double pos = (double)pos0 + (double)t;
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
        // base^(-2p/d) = 2^(-(p / (d/2)) * log2(base))
        const double inv_freq = exp2((double)(p0 + u) * neg_log2_base_over_half);
        double s, c;
        rope_sincos(pos * inv_freq, s, c);
        cs[u] = (float)c;
        sn[u] = (float)s;
    }
    if (tab && blockIdx.y == 0) {
        float2* row = tab + (size_t)(pos0 + t) * half + p0;
#pragma unroll
        for (int u = 0; u < kPairs; ++u) row[u] = make_float2(cs[u], sn[u]);
    }

    const long long r0 = (long long)blockIdx.y * rows_per_chunk;
    const long long r1 = min(n_seq + n_seq2, r0 + rows_per_chunk);
    const size_t row_stride = (size_t)T_len * d;
    const size_t off = (size_t)t * d + (ADJ ? 2 * p0 : p0);
#pragma unroll 4
    for (long long r = r0; r < r1; ++r) {
        // split-half: the kPairs first halves, then the kPairs second halves;
        // adjacent: 2 kPairs contiguous channels, pair u = (2u, 2u + 1)
        T* lo = (r < n_seq ? x + (size_t)r * row_stride : x2 + (size_t)(r - n_seq) * row_stride) + off;
        T* hi = lo + (ADJ ? kPairs : half);
        float e[2 * kPairs], y[2 * kPairs];
        load_f32<T, kPairs>(lo, e);
        load_f32<T, kPairs>(hi, e + kPairs);
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
            const int i1 = ADJ ? 2 * u : u, i2 = ADJ ? 2 * u + 1 : u + kPairs;
            rope_turn(e[i1], e[i2], cs[u], sn[u], y[i1], y[i2]);
        }
        store_f32<T, kPairs>(lo, y);
        store_f32<T, kPairs>(hi, y + kPairs);
    }
}

template <typename T, int kPairs>
hipError_t launch_rope_t(T* x, long long n_seq, T* x2, long long n_seq2, int T_len, int d, int pos0,
                         double base, int pairing, hipStream_t stream, float* tab) {
    const long long n_rows = n_seq + n_seq2;
    const int half = d / 2;
    const int groups = half / kPairs;
    const long long slots = (long long)T_len * groups;
    const long long gx = (slots + kThreads - 1) / kThreads;
    // split the head rows so the launch has enough workgroups to fill the
    // chip; each chunk forms its own cosines and sines, so the chunks are
    // capped at 2^17 / slots (at most 2^17 lanes' worth of angles)
    long long gy = (2048 + gx - 1) / gx;
    if (gy > (1LL << 17) / slots) gy = (1LL << 17) / slots;
    if (gy > n_rows) gy = n_rows;
    if (gy < 1) gy = 1;
    const int rows_per_chunk = (int)((n_rows + gy - 1) / gy);
    gy = (n_rows + rows_per_chunk - 1) / rows_per_chunk;
    const double neg = -log2(base) / (double)half;
    dim3 grid((unsigned)gx, (unsigned)gy);
    if (pairing)
        hipLaunchKernelGGL((rope_kernel<T, kPairs, true>), grid, dim3(kThreads), 0, stream,
                           x, n_seq, x2, n_seq2, rows_per_chunk, T_len, d, pos0, neg,
                           reinterpret_cast<float2*>(tab));
    else
        hipLaunchKernelGGL((rope_kernel<T, kPairs, false>), grid, dim3(kThreads), 0, stream,
                           x, n_seq, x2, n_seq2, rows_per_chunk, T_len, d, pos0, neg,
                           reinterpret_cast<float2*>(tab));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(void* x, long long n_seq, int T_len, int d, int pos0, double base,
                       int dtype, int pairing, hipStream_t stream, float* tab, void* x2,
                       long long n_seq2) {
    // four pairs per lane (8-byte bf16 / 16-byte f32 accesses) when the half
    // head size allows it, else one pair per lane
    const bool wide = (d / 2) % 4 == 0;
    if (!x2) n_seq2 = 0;
    if (dtype == 0) {
        float* a = static_cast<float*>(x);
        float* b = static_cast<float*>(x2);
        return wide ? launch_rope_t<float, 4>(a, n_seq, b, n_seq2, T_len, d, pos0, base, pairing, stream, tab)
                    : launch_rope_t<float, 1>(a, n_seq, b, n_seq2, T_len, d, pos0, base, pairing, stream, tab);
    }
    bf16* a = static_cast<bf16*>(x);
    bf16* b = static_cast<bf16*>(x2);
    return wide ? launch_rope_t<bf16, 4>(a, n_seq, b, n_seq2, T_len, d, pos0, base, pairing, stream, tab)
                : launch_rope_t<bf16, 1>(a, n_seq, b, n_seq2, T_len, d, pos0, base, pairing, stream, tab);
}


// ---------------------------------------------------------------------------
// Per-token positions: token t of sequence b sits at pos[b * T + t] (the
// scalar pos0 + t of rope_kernel generalised, e.g. sequences of a batch at
// different cache positions).  A lane owns kPairs pairs of one (b, t), forms
// their angles once (the same arithmetic as rope_kernel) and turns that
// token in every head of sequence b.
namespace {

template <typename T, int kPairs, bool ADJ>
__global__ __launch_bounds__(kThreads) void rope_pos_kernel(T* __restrict__ x, int B, int H, int T_len,
                                                            int d, const int* __restrict__ pos,
                                                            double neg_log2_base_over_half) {
    const int half = d >> 1;
    const int groups = half / kPairs;
    const long long slot = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (slot >= (long long)B * T_len * groups) return;
    const long long bt = slot / groups;
    const int p0 = (int)(slot - bt * groups) * kPairs;
    const int b = (int)(bt / T_len), t = (int)(bt - (long long)b * T_len);
    float cs[kPairs], sn[kPairs];
    const double at = (double)pos[bt];
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
        const double inv_freq = exp2((double)(p0 + u) * neg_log2_base_over_half);
        double sv, cv;
        rope_sincos(at * inv_freq, sv, cv);
        cs[u] = (float)cv;
        sn[u] = (float)sv;
    }
    T* base = x + ((size_t)b * H * T_len + t) * d + (ADJ ? 2 * p0 : p0);
#pragma unroll 4
    for (int hh = 0; hh < H; ++hh) {
        T* lo = base + (size_t)hh * T_len * d;
        T* hi = lo + (ADJ ? kPairs : half);
        float e[2 * kPairs], y[2 * kPairs];
        load_f32<T, kPairs>(lo, e);
        load_f32<T, kPairs>(hi, e + kPairs);
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
            const int i1 = ADJ ? 2 * u : u, i2 = ADJ ? 2 * u + 1 : u + kPairs;
            rope_turn(e[i1], e[i2], cs[u], sn[u], y[i1], y[i2]);
        }
        store_f32<T, kPairs>(lo, y);
        store_f32<T, kPairs>(hi, y + kPairs);
    }
}

template <typename T, int kPairs>
hipError_t launch_rope_pos_t(T* x, int B, int H, int T_len, int d, const int* pos, double base,
                             int pairing, hipStream_t stream) {
    const int groups = (d / 2) / kPairs;
    const long long slots = (long long)B * T_len * groups;
    const dim3 grid((unsigned)((slots + kThreads - 1) / kThreads));
    const double neg = -log2(base) / (double)(d / 2);
    if (pairing)
        hipLaunchKernelGGL((rope_pos_kernel<T, kPairs, true>), grid, dim3(kThreads), 0, stream, x, B, H, T_len,
                           d, pos, neg);
    else
        hipLaunchKernelGGL((rope_pos_kernel<T, kPairs, false>), grid, dim3(kThreads), 0, stream, x, B, H, T_len,
                           d, pos, neg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_pos(void* x, int B, int H, int T_len, int d, const int* pos, double base,
                           int dtype, int pairing, hipStream_t stream) {
    const bool wide = (d / 2) % 4 == 0;
    if (dtype == 0)
        return wide ? launch_rope_pos_t<float, 4>(static_cast<float*>(x), B, H, T_len, d, pos, base, pairing, stream)
                    : launch_rope_pos_t<float, 1>(static_cast<float*>(x), B, H, T_len, d, pos, base, pairing, stream);
    return wide ? launch_rope_pos_t<bf16, 4>(static_cast<bf16*>(x), B, H, T_len, d, pos, base, pairing, stream)
                : launch_rope_pos_t<bf16, 1>(static_cast<bf16*>(x), B, H, T_len, d, pos, base, pairing, stream);
}

// ---------------------------------------------------------------------------
// Decode-step preparation ("The Transformer architecture" -- Hands-on: the new
// keys and values are written into the cache at cache.pos along the token
// axis, and RoPE is sliced from cache.pos): in one launch, rotate the Tn new
// query rows in place, rotate the new key rows into the key cache at
// positions pos .. pos + Tn - 1, and copy the new value rows into the value
// cache.  A thread owns kPairs channel pairs of one token; the block's
// threads split into SPB pair slots x (256 / SPB) row lanes, so a one-token
// step still fills every lane.  The virtual row list is [q rows | k rows |
// v rows]; the cosine and sine of a slot are formed once (as in rope_kernel:
// double precision, rounded once to float32) and reused for all its rows.
namespace {

struct PrepArgs {
    void* q;             // [B][Hq][Tn][d], rotated in place
    const void* kn;      // [B][Hkv][Tn][d]
    const void* vn;      // [B][Hkv][Tn][d]
    void* kc;            // [B][Hkv][Tmax][d]
    void* vc;            // [B][Hkv][Tmax][d]
    int Hq, Hkv, Tn, Tmax, d, pos;
    long long nq, nk;    // q rows (B Hq), k rows (B Hkv); v rows = nk
    int spb, rows_per_chunk;
    double neg;          // -log2(base) / (d / 2)
};

template <typename T, int kPairs, bool ADJ>
__global__ __launch_bounds__(kThreads) void step_prep_kernel(PrepArgs a) {
    const int half = a.d >> 1;
    const int groups = half / kPairs;
    const int rpb = kThreads / a.spb;
    const int lane_slot = threadIdx.x % a.spb, rl = threadIdx.x / a.spb;
    const long long slot = (long long)blockIdx.x * a.spb + lane_slot;
    if (slot >= (long long)a.Tn * groups) return;
    const int t = (int)(slot / groups);
    const int p0 = (int)(slot - (long long)t * groups) * kPairs;

    float cs[kPairs], sn[kPairs];
    const double pos = (double)a.pos + (double)t;
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
        const double inv_freq = exp2((double)(p0 + u) * a.neg);
        double s, c;
        rope_sincos(pos * inv_freq, s, c);
        cs[u] = (float)c;
        sn[u] = (float)s;
    }
    const int c0 = ADJ ? 2 * p0 : p0;             // first channel of the lane's slice
    const int c1 = ADJ ? c0 + kPairs : p0 + half;  // second
    const long long total = a.nq + 2 * a.nk;
    const long long r0 = (long long)blockIdx.y * a.rows_per_chunk;
    const long long r1 = min(total, r0 + a.rows_per_chunk);
    for (long long r = r0 + rl; r < r1; r += rpb) {
        const T* src;
        T* dst;
        bool rotate = true;
        if (r < a.nq) {
            dst = static_cast<T*>(a.q) + (r * a.Tn + t) * a.d;
            src = dst;
        } else {
            const bool is_k = r < a.nq + a.nk;
            const long long rk = r - a.nq - (is_k ? 0 : a.nk);   // b * Hkv + h
            src = static_cast<const T*>(is_k ? a.kn : a.vn) + (rk * a.Tn + t) * a.d;
            dst = static_cast<T*>(is_k ? a.kc : a.vc) + (rk * a.Tmax + a.pos + t) * a.d;
            rotate = is_k;
        }
        float e[2 * kPairs], y[2 * kPairs];
        load_f32<T, kPairs>(src + c0, e);
        load_f32<T, kPairs>(src + c1, e + kPairs);
        if (rotate) {
#pragma unroll
            for (int u = 0; u < kPairs; ++u) {
                const int i1 = ADJ ? 2 * u : u, i2 = ADJ ? 2 * u + 1 : u + kPairs;
                rope_turn(e[i1], e[i2], cs[u], sn[u], y[i1], y[i2]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 2 * kPairs; ++u) y[u] = e[u];
        }
        store_f32<T, kPairs>(dst + c0, y);
        store_f32<T, kPairs>(dst + c1, y + kPairs);
    }
}

template <typename T, int kPairs>
hipError_t launch_prep_t(PrepArgs a, int pairing, hipStream_t stream) {
    const int groups = (a.d / 2) / kPairs;
    const long long slots = (long long)a.Tn * groups;
    a.spb = (int)(slots < kThreads ? slots : kThreads);
    const long long gx = (slots + a.spb - 1) / a.spb;
    const long long total = a.nq + 2 * a.nk;
    const int rpb = kThreads / a.spb;
    // enough blocks to fill the chip, each row lane with a few rows
    long long gy = (2048 + gx - 1) / gx;
    const long long max_gy = (total + rpb - 1) / rpb;
    if (gy > max_gy) gy = max_gy;
    if (gy < 1) gy = 1;
    a.rows_per_chunk = (int)((total + gy - 1) / gy);
    gy = (total + a.rows_per_chunk - 1) / a.rows_per_chunk;
    dim3 grid((unsigned)gx, (unsigned)gy);
    if (pairing)
        hipLaunchKernelGGL((step_prep_kernel<T, kPairs, true>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((step_prep_kernel<T, kPairs, false>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step_prep(void* q, const void* kn, const void* vn, void* kc, void* vc, int B,
                            int Hq, int Hkv, int Tn, int Tmax, int d, int pos, double base,
                            int dtype, int pairing, hipStream_t stream) {
    PrepArgs a;
    a.q = q; a.kn = kn; a.vn = vn; a.kc = kc; a.vc = vc;
    a.Hq = Hq; a.Hkv = Hkv; a.Tn = Tn; a.Tmax = Tmax; a.d = d; a.pos = pos;
    a.nq = (long long)B * Hq;
    a.nk = (long long)B * Hkv;
    a.neg = -log2(base) / (double)(d / 2);
    a.spb = 1; a.rows_per_chunk = 1;
    const bool wide = (d / 2) % 4 == 0;
    if (dtype == 0)
        return wide ? launch_prep_t<float, 4>(a, pairing, stream) : launch_prep_t<float, 1>(a, pairing, stream);
    return wide ? launch_prep_t<bf16, 4>(a, pairing, stream) : launch_prep_t<bf16, 1>(a, pairing, stream);
}

}  // namespace rocattn
