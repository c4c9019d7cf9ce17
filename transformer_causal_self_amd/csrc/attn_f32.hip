// attn_f32.hip -- float32 causal attention forward for any head sizes
// d_k, d_v <= 256 that are multiples of 4 (q and k rows have d_k channels,
// v and o rows d_v).
//
// Computes O = softmax(scale * Q K^T + M) V ("Transformer" (ai-notes) --
// Scaled dot-product attention) in one pass over the keys without forming
// the score matrix ("Grasping Codes and Math 02" -- Flash Attention): the
// keys are visited in tiles, and each row keeps a running maximum m, a
// running denominator l and an unnormalised output, rescaled by
// exp(m_old - m_new) whenever the maximum grows, so that after the last tile
// O = acc / l equals the softmax-weighted sum.
//
// Layout of the work: a workgroup of 256 lanes owns 64 query rows of one
// (batch, query head); four neighbouring lanes share a row, each holding a
// quarter of the channels of q and of the accumulator, and combine
// their partial dot products with two lane exchanges.  Key/value tiles of 32
// rows are staged in LDS.  This kernel favours simplicity over speed: it is
// the float32 correctness path (the bf16 MFMA kernels carry the throughput).
#include <math.h>

#include "internal.hpp"

namespace rocattn {
namespace {

constexpr int kRows = 64;   // query rows per workgroup
constexpr int kKeys = 32;   // keys per LDS tile

template <int DQ>  // DQ >= max(d_k, d_v) / 4, a power of two
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(FwdParams p) {
    extern __shared__ float smem[];
    const int d = p.d, dv = p.dv ? p.dv : p.d;
    float* Ks = smem;                 // [kKeys][d]
    float* Vs = smem + kKeys * d;     // [kKeys][dv]

    const int qt = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int hk = hq / (p.Hq / p.Hkv);
    const int tid = threadIdx.x;
    const int r = tid >> 2, part = tid & 3;
    const int dq = d >> 2, dvq = dv >> 2;
    const int i = qt * kRows + r;
    const bool row_ok = i < p.Tq;

    const float* qg = static_cast<const float*>(p.q);
    const float* kg = static_cast<const float*>(p.k);
    const float* vg = static_cast<const float*>(p.v);
    const long long q_row = b * p.qs.b + hq * p.qs.h + (long long)(row_ok ? i : 0) * p.qs.t;
    const long long o_row = b * p.os.b + hq * p.os.h + (long long)(row_ok ? i : 0) * p.os.t;

    float qr[DQ], acc[DQ];
#pragma unroll
    for (int c = 0; c < DQ; ++c) {
        qr[c] = (c < dq) ? qg[q_row + part * dq + c] : 0.f;   // acc uses c < dvq
        acc[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    const long long k_base = b * p.ks.b + hk * p.ks.h, v_base = b * p.vs.b + hk * p.vs.h;
    const int row_pos = p.q_offset + i;                  // absolute position of this row
    const int kv_end = p.causal ? min(p.Tk, p.q_offset + qt * kRows + kRows) : p.Tk;

    for (int j0 = 0; j0 < kv_end; j0 += kKeys) {
        __syncthreads();
        for (int x = tid; x < kKeys * d / 4; x += 256) {
            const int e = x * 4;
            const int jj = e / d, cc = e - jj * d;
            const int j = j0 + jj;
            float4 kk = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < p.Tk) kk = *reinterpret_cast<const float4*>(kg + k_base + j * p.ks.t + cc);
            *reinterpret_cast<float4*>(Ks + e) = kk;
        }
        for (int x = tid; x < kKeys * dv / 4; x += 256) {
            const int e = x * 4;
            const int jj = e / dv, cc = e - jj * dv;
            const int j = j0 + jj;
            float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < p.Tk) vv = *reinterpret_cast<const float4*>(vg + v_base + j * p.vs.t + cc);
            *reinterpret_cast<float4*>(Vs + e) = vv;
        }
        __syncthreads();

        float s[kKeys];
        float tmax = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < DQ; ++c)
                if (c < dq) dot = fmaf(qr[c], Ks[jj * d + part * dq + c], dot);
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            const int j = j0 + jj;
            const bool vis = (j < p.Tk) && (!p.causal || j <= row_pos);
            s[jj] = vis ? dot * p.scale : -INFINITY;
            tmax = fmaxf(tmax, s[jj]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new == -INFINITY) continue;  // no visible key yet (only rows past Tq)
        const float alpha = expf(m - m_new);
        l *= alpha;
#pragma unroll
        for (int c = 0; c < DQ; ++c) acc[c] *= alpha;
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
            const float pj = expf(s[jj] - m_new);
            l += pj;
#pragma unroll
            for (int c = 0; c < DQ; ++c)
                if (c < dvq) acc[c] = fmaf(pj, Vs[jj * dv + part * dvq + c], acc[c]);
        }
        m = m_new;
    }

    if (row_ok) {
        float* og = static_cast<float*>(p.o);
        const float inv = 1.f / l;
#pragma unroll
        for (int c = 0; c < DQ; ++c)
            if (c < dvq) og[o_row + part * dvq + c] = acc[c] * inv;
        if (p.lse && part == 0)
            p.lse[(size_t)(b * p.Hq + hq) * p.Tq + i] = m + logf(l);
    }
}

template <int DQ>
hipError_t launch_dq(const FwdParams& p, hipStream_t stream) {
    dim3 grid((p.Tq + kRows - 1) / kRows, p.Hq, p.B);
    size_t lds = sizeof(float) * kKeys * (p.d + (p.dv ? p.dv : p.d));
    hipLaunchKernelGGL(attn_fwd_f32_kernel<DQ>, grid, dim3(256), lds, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
    const int dq = (p.dv > p.d ? p.dv : p.d) / 4;
    if (dq <= 4) return launch_dq<4>(p, stream);
    if (dq <= 8) return launch_dq<8>(p, stream);
    if (dq <= 16) return launch_dq<16>(p, stream);
    if (dq <= 32) return launch_dq<32>(p, stream);
    return launch_dq<64>(p, stream);
}

}  // namespace rocattn
