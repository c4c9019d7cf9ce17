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
// Layout of the work: a workgroup of 256 lanes owns 16 query rows of one
// (batch, query head); the 16 lanes of a row (one DPP row) each hold the
// 4-channel groups c * 16 + (lane mod 16) of q and of the accumulator, so a
// score is one FMA per channel held and four DPP exchanges, and a row's work
// is spread over a quarter of a wave.  Lanes whose groups lie past the row
// width read an in-range group (their q entries are zero and their
// accumulator is never stored), so no lane branches.  Key/value tiles of 32 rows are staged in LDS and
// read 16 bytes per lane (the 16 lanes of a row read 256 contiguous bytes;
// the rows of a wave read the same key).  Scores are kept in base-2 units
// (scale * log2(e) folded into the product), so each weight is one
// v_exp_f32.  This kernel is the float32 path (the bf16 MFMA kernels carry
// the throughput); it is laid out for latency, since the float32 workloads
// are small.
#include <math.h>

#include "internal.hpp"

namespace rocattn {
namespace {

constexpr int kLanes = 16;             // lanes per query row
constexpr int kRows = 256 / kLanes;    // query rows per workgroup
constexpr int kKeys = 32;              // keys per LDS tile

// x of the lane given by a DPP lane pattern (within rows of 16 lanes)
template <int CTRL>
__device__ inline float dpp_lane(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row, the same bits in every lane: pairs
// (quad_perm 1,0,3,2), quads (2,3,0,1), then the two quads of each half row
// (row_half_mirror) and the two halves (row_mirror); every addition meets
// the same two operands in both lanes it serves.
__device__ inline float sum16(float x) {
    x += dpp_lane<0xB1>(x);
    x += dpp_lane<0x4E>(x);
    x += dpp_lane<0x141>(x);
    x += dpp_lane<0x140>(x);
    return x;
}

template <int NC>  // 4-channel groups per lane: 64 NC >= max(d_k, d_v)
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(FwdParams p) {
    extern __shared__ float4 smem4[];
    const int d = p.d, dv = p.dv ? p.dv : p.d;
    const int gk = d >> 2, gv = dv >> 2;   // 4-channel groups of a k / v row
    float4* Ks = smem4;                    // [kKeys][gk]
    float4* Vs = smem4 + kKeys * gk;       // [kKeys][gv]

    const int qt = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int hk = hq / (p.Hq / p.Hkv);
    const int tid = threadIdx.x;
    const int r = tid / kLanes, part = tid % kLanes;
    const int i = qt * kRows + r;
    const bool row_ok = i < p.Tq;

    const float* qg = static_cast<const float*>(p.q);
    const float* kg = static_cast<const float*>(p.k);
    const float* vg = static_cast<const float*>(p.v);
    const long long q_row = b * p.qs.b + hq * p.qs.h + (long long)(row_ok ? i : 0) * p.qs.t;
    const long long o_row = b * p.os.b + hq * p.os.h + (long long)(row_ok ? i : 0) * p.os.t;

    float4 qr[NC], acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int gi = c * kLanes + part;
        qr[c] = gi < gk ? *reinterpret_cast<const float4*>(qg + q_row + 4 * gi) : make_float4(0.f, 0.f, 0.f, 0.f);
        acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float c2 = p.scale * kLog2e;   // score in base-2 units
    float m = -INFINITY, l = 0.f;

    const long long k_base = b * p.ks.b + hk * p.ks.h, v_base = b * p.vs.b + hk * p.vs.h;
    const int row_pos = p.q_offset + i;                  // absolute position of this row
    const int kv_end = p.causal ? min(p.Tk, p.q_offset + qt * kRows + kRows) : p.Tk;

    // a tile's K and V rows (keys past Tk as zeros), 16 bytes per lane and load
    auto k_at = [&](int j0, int x) {
        const int jj = x / gk, cc = x - jj * gk, j = j0 + jj;
        return j < p.Tk ? *reinterpret_cast<const float4*>(kg + k_base + j * p.ks.t + 4 * cc)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto v_at = [&](int j0, int x) {
        const int jj = x / gv, cc = x - jj * gv, j = j0 + jj;
        return j < p.Tk ? *reinterpret_cast<const float4*>(vg + v_base + j * p.vs.t + 4 * cc)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    // Up to d = 128 the next tile is loaded into registers while this one is
    // worked on (its load latency, paid once per tile otherwise, is what a
    // short causal row walk waits on); wider rows load each tile in turn.
    constexpr bool PF = NC <= 2;
    constexpr int NPF = PF ? kKeys * kLanes * NC / 256 : 1;   // loads per lane and tensor
    float4 kpf[NPF], vpf[NPF];
    auto prefetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < NPF; ++u) {
            const int x = tid + 256 * u;
            if (x < kKeys * gk) kpf[u] = k_at(j0, x);
            if (x < kKeys * gv) vpf[u] = v_at(j0, x);
        }
    };
    if constexpr (PF) prefetch(0);

    for (int j0 = 0; j0 < kv_end; j0 += kKeys) {
        __syncthreads();
        if constexpr (PF) {
#pragma unroll
            for (int u = 0; u < NPF; ++u) {
                const int x = tid + 256 * u;
                if (x < kKeys * gk) Ks[x] = kpf[u];
                if (x < kKeys * gv) Vs[x] = vpf[u];
            }
        } else {
            for (int x = tid; x < kKeys * gk; x += 256) Ks[x] = k_at(j0, x);
            for (int x = tid; x < kKeys * gv; x += 256) Vs[x] = v_at(j0, x);
        }
        __syncthreads();
        if constexpr (PF)
            if (j0 + kKeys < kv_end) prefetch(j0 + kKeys);

        float s[kKeys];
        float tmax = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float4 kk = Ks[jj * gk + min(c * kLanes + part, gk - 1)];
                dot = fmaf(qr[c].x, kk.x, dot);
                dot = fmaf(qr[c].y, kk.y, dot);
                dot = fmaf(qr[c].z, kk.z, dot);
                dot = fmaf(qr[c].w, kk.w, dot);
            }
            dot = sum16(dot);
            const int j = j0 + jj;
            const bool vis = (j < p.Tk) && (!p.causal || j <= row_pos);
            s[jj] = vis ? dot * c2 : -INFINITY;
            tmax = fmaxf(tmax, s[jj]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new == -INFINITY) continue;  // no visible key yet (only rows past Tq)
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            acc[c].x *= alpha; acc[c].y *= alpha; acc[c].z *= alpha; acc[c].w *= alpha;
        }
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
            const float pj = __builtin_amdgcn_exp2f(s[jj] - m_new);
            l += pj;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float4 vv = Vs[jj * gv + min(c * kLanes + part, gv - 1)];
                acc[c].x = fmaf(pj, vv.x, acc[c].x);
                acc[c].y = fmaf(pj, vv.y, acc[c].y);
                acc[c].z = fmaf(pj, vv.z, acc[c].z);
                acc[c].w = fmaf(pj, vv.w, acc[c].w);
            }
        }
        m = m_new;
    }

    if (row_ok) {
        float* og = static_cast<float*>(p.o);
        const float inv = 1.f / l;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int gi = c * kLanes + part;
            if (gi < gv)
                *reinterpret_cast<float4*>(og + o_row + 4 * gi) =
                    make_float4(acc[c].x * inv, acc[c].y * inv, acc[c].z * inv, acc[c].w * inv);
        }
        if (p.lse && part == 0)
            p.lse[(size_t)(b * p.Hq + hq) * p.Tq + i] = (m + log2f(l)) * kLn2;
    }
}

template <int NC>
hipError_t launch_nc(const FwdParams& p, hipStream_t stream) {
    dim3 grid((p.Tq + kRows - 1) / kRows, p.Hq, p.B);
    size_t lds = sizeof(float) * kKeys * (p.d + (p.dv ? p.dv : p.d));
    hipLaunchKernelGGL(attn_fwd_f32_kernel<NC>, grid, dim3(256), lds, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
    const int w = p.dv > p.d ? p.dv : p.d;
    if (w <= 64) return launch_nc<1>(p, stream);
    if (w <= 128) return launch_nc<2>(p, stream);
    return launch_nc<4>(p, stream);
}

}  // namespace rocattn
