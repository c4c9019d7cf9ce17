// calib.hip -- measured ceilings of the two units the attention kernels are
// bound by, so that their rates can be read against what the chip sustains
// as well as against its published peaks:
//   * a matrix-core loop: back-to-back v_mfma_f32_32x32x16_bf16 on
//     independent accumulators, nothing else (the bf16 MFMA ceiling);
//   * a streaming read: every byte of a large buffer read once with 16-byte
//     loads, one float per workgroup written (the HBM read ceiling);
//   * a streaming copy: read once, write once (read + write bytes).
// Built into librocattn_calib.so, a library of its own: the attention
// library does not contain or call these kernels.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rocattn_calib.h"

#define CALIB_API extern "C" __attribute__((visibility("default")))

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;   // independent accumulators per wave

// Each wave runs `iters` rounds of kChains independent 32x32x16 products on
// operands that stay in registers; the sums land in sink so nothing is
// optimised away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float seed, float* sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(lane + i));
        b[i] = (__bf16)(seed * (float)(lane - i));
    }
    f32x16 acc[kChains];
    for (int c = 0; c < kChains; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
    for (int c = 0; c < kChains; ++c)
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == 1234.5f) sink[blockIdx.x] = s;   // practically never; keeps the loop live
}

// Read of n16 16-byte vectors: workgroup w reads the contiguous block
// [w * per, (w + 1) * per), eight 16-byte loads in flight per lane
// (non-temporal: the data is used once); one value per workgroup.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, long long n16,
                                                          float* __restrict__ sink) {
    const long long per = (n16 + gridDim.x - 1) / gridDim.x;
    const long long lo = (long long)blockIdx.x * per;
    const long long hi = lo + per < n16 ? lo + per : n16;
    unsigned acc = 0;
    long long i = lo + threadIdx.x;
    for (; i + 7 * 256 < hi; i += 8 * 256) {
        u32x4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    for (; i < hi; i += 256) {
        const u32x4 x = __builtin_nontemporal_load(src + i);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    __shared__ unsigned red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)(red[0] & 0xFFFF);
}

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          long long n16) {
    const long long per = (n16 + gridDim.x - 1) / gridDim.x;
    const long long lo = (long long)blockIdx.x * per;
    const long long hi = lo + per < n16 ? lo + per : n16;
    long long i = lo + threadIdx.x;
    for (; i + 3 * 256 < hi; i += 4 * 256) {
        u32x4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(x[u], dst + i + u * 256);
    }
    for (; i < hi; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

CALIB_API int calib_mfma_loop(int n_workgroups, int iters, float* sink, void* stream) {
    if (n_workgroups <= 0 || iters <= 0 || !sink) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)n_workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), iters, 0.001f, sink);
    return hipGetLastError() == hipSuccess ? 0 : -9;
}

CALIB_API double calib_mfma_loop_flops(int n_workgroups, int iters) {
    // 4 waves per workgroup, kChains products of 32 x 32 x 16 multiply-adds
    return 2.0 * 32 * 32 * 16 * (double)kChains * iters * 4.0 * n_workgroups;
}

CALIB_API int calib_stream_read(const void* src, size_t bytes, int n_workgroups, float* sink, void* stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 || n_workgroups <= 0) return -1;
    if (reinterpret_cast<uintptr_t>(src) & 15u) return -7;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)n_workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       (long long)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : -9;
}

CALIB_API int calib_stream_copy(const void* src, void* dst, size_t bytes, int n_workgroups, void* stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 || n_workgroups <= 0) return -1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return -7;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + bytes && d0 < s0 + bytes) return -2;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)n_workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), (long long)(bytes / 16));
    return hipGetLastError() == hipSuccess ? 0 : -9;
}
