// mfma_tiles.hpp -- device helpers shared by the bf16 attention kernels that
// stage K/V-like tiles in LDS and feed them to v_mfma_f32_32x32x16_bf16:
// the LDS swizzles, the direct HBM -> LDS copy, wait counters, and the
// half-wave pair reductions.  Internal to librocattn.
#pragma once

#include "internal.hpp"

namespace rocattn {
namespace {

// XOR swizzles of the 16-byte chunk position within a tile row.
//  K: the rows of a fragment read the same logical chunk (ds_read_b128), so
//     the rows' chunks must fall in distinct 16-byte bank groups.
//  V: four consecutive rows are read 64 bytes each (transpose reads), so the
//     rows' 64-byte segments must fall in distinct 64-byte bank groups.
template <int D>
__device__ inline int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ inline int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

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
// wait for it; the kernel waits itself (wait_vm*) before the barrier that
// publishes the tile.  Nothing else in the kernels that use it touches m0.
__device__ inline void copy16(const void* sbase, unsigned voff, unsigned lds) {
    // base and LDS address are wave-uniform; say so, so they live in SGPRs
    const unsigned long long b = (unsigned long long)sbase;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
    const void* base = (const void*)(((unsigned long long)hi << 32) | lo);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base) : "memory");
}

// The same for 4 bytes per lane: the wave's 64 dwords land contiguously at
// `lds` (lane i at lds + 4 i).
__device__ inline void copy4(const void* sbase, unsigned voff, unsigned lds) {
    const unsigned long long b = (unsigned long long)sbase;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
    const void* base = (const void*)(((unsigned long long)hi << 32) | lo);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base) : "memory");
}

// Wait until at most N (0) of this wave's vector-memory operations are in flight.
template <int N>
__device__ inline void wait_vm() {
    if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int V>
struct IC {
    static constexpr int value = V;
};

}  // namespace
}  // namespace rocattn
