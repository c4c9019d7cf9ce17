// internal.hpp -- types and launcher declarations shared by the kernels and
// the host-side API of librocattn.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rocattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element strides of a [B][H][T][d] tensor between batches, heads and
// tokens; the d elements of a row are always contiguous.
struct Strides {
    long long b, h, t;
};

// Everything a forward launch needs, validated by the host API.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;      // may be null; always dense [B][Hq][Tq]
    int B, Hq, Hkv, Tq, Tk, d;
    int dv = 0;      // width of v and o rows when it differs from d (0: d)
    float scale;
    int causal;
    int q_offset;
    Strides qs, ks, vs, os;
    // RoPE of the query rows at load (bf16 prefill only): float32 (cos, sin)
    // pairs [position][d/2]; query row i sits at position rope_pos0 + i
    const float* rope_tab = nullptr;
    int rope_adj = 0;      // 0: split-half pairs (p, p + d/2); 1: adjacent (2p, 2p + 1)
    int rope_pos0 = 0;
    // bf16 prefill split over the keys (nsplit > 1): partial outputs
    // [B*Hq*Tq][nsplit][d] and (max, weight sum) [B*Hq*Tq][nsplit][2] in float32
    int nsplit = 1;
    float* part_o = nullptr;
    float* part_ml = nullptr;
};

// Prefill (any Tq) bf16 MFMA kernel, d in {64, 128}: four-wave workgroups of
// 128 query rows, several workgroups per CU.
hipError_t launch_prefill_bf16(const FwdParams& p, hipStream_t stream);

// Key splits for a bf16 prefill of this size (1: none): used when one
// workgroup per (128 query rows, head) would leave most of the chip idle.
int prefill_splits(int B, int Hq, int Tq, int Tk, int d, int dv);
size_t prefill_split_bytes(int B, int Hq, int Tq, int dv, int ks);

// Merge S <= 8 partial results per row: o = sum_s 2^(m_s - M) o_s / sum_s
// 2^(m_s - M) l_s (M = max_s m_s) into bf16 o (row r = (b Hq + hq) Tq + i
// at o + b os.b + hq os.h + i os.t) and, when lse is set, lse[r].
hipError_t launch_combine_bf16(const float* part_o, const float* part_ml, void* o, float* lse,
                               long long rows, int S, int Hq, int Tq, const Strides& os, int d,
                               hipStream_t stream);

// Split-K decode (Tq == 1) bf16 kernels; d in {64, 128}, Hq / Hkv <= 16.
bool decode_bf16_supported(int Hq, int Hkv, int d);
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int Tk, int d);
hipError_t launch_decode_bf16(const FwdParams& p, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

// One cached generation step of one new token per sequence (bf16, d 64 or
// 128, Hq / Hkv <= 16) in a single launch: q [B][Hq][1][d] rotated at pos
// (written back rotated), the new key kn [B][Hkv][1][d] rotated and, with
// the new value vn, appended to the caches kc / vc [B][Hkv][Tmax][d] at
// pos, attention over cache tokens 0 .. pos into o [B][Hq][1][d] (and lse).
// The workspace holds the split-K partials and, at
// decode_step_counter_offset, B * Hkv arrival counters that must be zero
// before the call and are zero after it.
struct StepParams {
    void* q;
    const void* kn;
    const void* vn;
    void* kc;
    void* vc;
    void* o;
    float* lse;
    int B, Hq, Hkv, Tmax, pos, d;
    float scale;
    double base;
    int pairing;
};
size_t decode_step_counter_offset(int B, int Hq, int Hkv, int Tmax, int d);
size_t decode_step_workspace_bytes(int B, int Hq, int Hkv, int Tmax, int d);
hipError_t launch_decode_step_bf16(const StepParams& sp, void* workspace, size_t ws_bytes, hipStream_t stream);

// Generic float32 kernel; d <= 256, d % 4 == 0.
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);

// RoPE in place; dtype 0 = f32, 1 = bf16; pairing 0 = split-half, 1 =
// adjacent.  x holds n_seq sequences of T rows of d elements ([n_seq][T][d])
// with token t at position pos0 + t.
// tab (optional): also store the float32 (cos, sin) of every pair at
// positions pos0 .. pos0 + T - 1 into tab[position][d/2].
// x2 (optional): a second tensor of n_seq2 sequences with the same T, d and
// positions, turned by the same launch (q and k of one call).
hipError_t launch_rope(void* x, long long n_seq, int T, int d, int pos0, double base,
                       int dtype, int pairing, hipStream_t stream, float* tab = nullptr,
                       void* x2 = nullptr, long long n_seq2 = 0);

// RoPE with per-token positions: x [B][H][T][d], token t of sequence b at
// position pos[b * T + t] (device int32 [B][T]).
hipError_t launch_rope_pos(void* x, int B, int H, int T, int d, const int* pos, double base,
                           int dtype, int pairing, hipStream_t stream);

// Everything a backward launch needs (dense [B][H][T][d] tensors), validated
// by the host API.
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dO;
    const float* lse;   // natural-log row log-sum-exp of the forward
    void* dq;
    void* dk;
    void* dv;
    void* workspace;    // bwd_workspace_bytes(B, Hq, Tq) bytes
    int B, Hq, Hkv, Tq, Tk, d;
    float scale;
    int causal;
    int q_offset;
};

// The fixed device scratch buffer of attn_fwd_noalloc: kNoAllocScratchBytes
// per device, its address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

// Gradients dq, dk, dv of the bf16 attention, d in {64, 128}.
size_t bwd_workspace_bytes(int B, int Hq, int Tq);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);

// Decode-step preparation in one launch: q [B][Hq][Tn][d] rotated in place,
// the new keys kn [B][Hkv][Tn][d] rotated into kc [B][Hkv][Tmax][d] at
// tokens pos .. pos + Tn - 1, the new values vn copied into vc there.
hipError_t launch_step_prep(void* q, const void* kn, const void* vn, void* kc, void* vc, int B,
                            int Hq, int Hkv, int Tn, int Tmax, int d, int pos, double base,
                            int dtype, int pairing, hipStream_t stream);

}  // namespace rocattn
