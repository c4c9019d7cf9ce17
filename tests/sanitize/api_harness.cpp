// api_harness.cpp -- the host validation layer of librocattn (csrc/api.cpp)
// on its own, built for the CPU with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitize_host.py.  The kernel
// launchers api.cpp calls are replaced here by stubs that launch nothing:
// they check what the validation layer hands to a kernel (sizes, the
// clamped causal offset, workspace carving) and record the call.  Every
// entry point is driven with valid arguments and with each kind of
// argument it must reject.  No GPU is touched: device pointers are fake
// addresses that nothing dereferences.  Exit status 0 when all calls
// behaved.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/rocattn.h"
#include "../../transformer_causal_self_amd/csrc/internal.hpp"

static int failures = 0;
static int launches = 0;
#define EXPECT(cond)                                                                          \
    do {                                                                                      \
        if (!(cond)) {                                                                        \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond);   \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

// ---- stand-ins for the allocator and the kernel launchers
hipError_t hipMallocAsync(void** p, size_t, hipStream_t) {
    *p = reinterpret_cast<void*>(0x7000000000ull);
    return hipSuccess;
}
hipError_t hipFreeAsync(void*, hipStream_t) { return hipSuccess; }

namespace rocattn {

static void check_fwd_params(const FwdParams& p) {
    ++launches;
    EXPECT(p.q && p.k && p.v && p.o);
    EXPECT(p.B > 0 && p.Hq > 0 && p.Hkv > 0 && p.Tq > 0 && p.Tk > 0 && p.Hq % p.Hkv == 0);
    if (p.causal) EXPECT(p.q_offset >= 0 && p.q_offset <= p.Tk);
    else EXPECT(p.q_offset == 0);
    // the kernels' 32-bit limit arithmetic: q_offset + Tq + a tile of rows
    EXPECT((long long)p.q_offset + p.Tq + 256 <= INT_MAX);
    EXPECT(p.qs.t >= p.d && p.ks.t >= p.d && p.os.t >= (p.dv ? p.dv : p.d));
}

hipError_t launch_prefill_bf16(const FwdParams& p, hipStream_t) {
    check_fwd_params(p);
    if (p.nsplit > 1) EXPECT(p.part_o && p.part_ml);
    return hipSuccess;
}
int prefill_splits(int B, int Hq, int Tq, int Tk, int d, int dv) {
    const long long nwg = (long long)((Tq + 127) / 128) * B * Hq;
    return (nwg < 512 && d == dv && Tk >= 256) ? 2 : 1;
}
size_t prefill_split_bytes(int B, int Hq, int Tq, int dv, int ks) {
    return ks < 2 ? 0 : sizeof(float) * (size_t)B * Hq * Tq * ks * (size_t)(dv + 2);
}
hipError_t launch_combine_bf16(const float* po, const float* pml, void* o, float*, long long rows, int S,
                               int, int, const Strides&, int, hipStream_t) {
    ++launches;
    EXPECT(po && pml && o && rows > 0 && S >= 2);
    return hipSuccess;
}
bool decode_bf16_supported(int Hq, int Hkv, int d) { return (d == 64 || d == 128) && Hq / Hkv <= 16; }
size_t decode_workspace_bytes(int B, int Hq, int, int Tk, int d) {
    return sizeof(float) * (size_t)B * Hq * (size_t)((Tk + 255) / 256) * (size_t)(d + 2);
}
hipError_t launch_decode_bf16(const FwdParams& p, void* ws, size_t ws_bytes, hipStream_t) {
    check_fwd_params(p);
    EXPECT(ws && ws_bytes >= decode_workspace_bytes(p.B, p.Hq, p.Hkv, p.Tk, p.d));
    return hipSuccess;
}
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t) {
    check_fwd_params(p);
    return hipSuccess;
}
hipError_t launch_rope(void* x, long long n_seq, int T, int d, int pos0, double base, int dtype, int pairing,
                       hipStream_t, float*, void* x2, long long n_seq2) {
    ++launches;
    EXPECT(x && n_seq > 0 && T > 0 && d > 0 && d % 2 == 0 && pos0 >= 0 && base > 0);
    EXPECT((long long)pos0 + T - 1 <= INT_MAX);
    EXPECT(dtype == ROCATTN_F32 || dtype == ROCATTN_BF16);
    EXPECT(pairing == 0 || pairing == 1);
    EXPECT(!x2 || n_seq2 > 0);
    return hipSuccess;
}
hipError_t launch_rope_pos(void* x, int B, int H, int T, int d, const int* pos, double, int, int,
                           hipStream_t) {
    ++launches;
    EXPECT(x && pos && B > 0 && H > 0 && T > 0 && d % 2 == 0);
    return hipSuccess;
}
size_t bwd_workspace_bytes(int B, int Hq, int Tq) { return sizeof(float) * 2 * (size_t)B * Hq * (Tq + 31); }
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t) {
    ++launches;
    if (p.causal) EXPECT(p.q_offset >= 0 && p.q_offset <= p.Tk);
    EXPECT((long long)p.q_offset + p.Tq + 256 <= INT_MAX);
    EXPECT(p.workspace != nullptr);
    return hipSuccess;
}
size_t decode_step_counter_offset(int B, int Hq, int Hkv, int Tmax, int d) {
    return (decode_workspace_bytes(B, Hq, Hkv, Tmax, d) + 255) & ~(size_t)255;
}
size_t decode_step_workspace_bytes(int B, int Hq, int Hkv, int Tmax, int d) {
    return decode_step_counter_offset(B, Hq, Hkv, Tmax, d) + sizeof(unsigned) * (size_t)B * Hkv;
}
hipError_t launch_decode_step_bf16(const StepParams& sp, void* ws, size_t ws_bytes, hipStream_t) {
    ++launches;
    EXPECT(sp.q && sp.kn && sp.vn && sp.kc && sp.vc && sp.o && ws);
    EXPECT(sp.pos >= 0 && sp.pos < sp.Tmax && sp.B > 0 && sp.Hq % sp.Hkv == 0);
    EXPECT(ws_bytes >= decode_step_workspace_bytes(sp.B, sp.Hq, sp.Hkv, sp.Tmax, sp.d));
    EXPECT(sp.pairing == 0 || sp.pairing == 1);
    return hipSuccess;
}
hipError_t noalloc_scratch(void** ptr) {
    *ptr = reinterpret_cast<void*>(0x7100000000ull);
    return hipSuccess;
}
hipError_t launch_step_prep(void* q, const void* kn, const void* vn, void* kc, void* vc, int, int, int,
                            int Tn, int Tmax, int, int pos, double, int, int, hipStream_t) {
    ++launches;
    EXPECT(q && kn && vn && kc && vc && pos >= 0 && (long long)pos + Tn <= Tmax);
    return hipSuccess;
}

}  // namespace rocattn

// ---- fake, 16-byte aligned device addresses, far apart
static void* A(unsigned i) { return reinterpret_cast<void*>(0x100000000000ull * (i + 1)); }
static const int BF = ROCATTN_BF16, F32 = ROCATTN_F32;

int main() {
    void *q = A(0), *k = A(1), *v = A(2), *o = A(3), *ws = A(4);
    float* lse = static_cast<float*>(A(5));
    // attn_fwd: valid calls of every kernel family (prefill, split prefill, decode, f32)
    EXPECT(attn_fwd(q, k, v, o, 8, 12, 12, 1024, 1024, 64, 0.125f, 1, 0, BF, nullptr) == ROCATTN_OK);
    EXPECT(attn_fwd(q, k, v, o, 1, 4, 2, 300, 2000, 128, 0.1f, 1, 1700, BF, nullptr) == ROCATTN_OK);
    EXPECT(attn_fwd(q, k, v, o, 32, 32, 8, 1, 8192, 128, 0.1f, 1, 8191, BF, nullptr) == ROCATTN_OK);
    EXPECT(attn_fwd(q, k, v, o, 1, 4, 4, 128, 128, 64, 0.125f, 1, 0, F32, nullptr) == ROCATTN_OK);
    // causal offsets far past the keys are clamped before any kernel sees them
    EXPECT(attn_fwd(q, k, v, o, 1, 4, 2, 2, 64, 128, 0.1f, 1, INT_MAX - 2, BF, nullptr) == ROCATTN_OK);
    EXPECT(attn_fwd(q, k, v, o, 1, 4, 2, 300, 700, 64, 0.1f, 1, INT_MAX - 300, BF, nullptr) == ROCATTN_OK);
    EXPECT(attn_fwd(q, k, v, o, 2, 8, 2, 1, 300, 128, 0.1f, 1, INT_MAX - 1, BF, nullptr) == ROCATTN_OK);
    EXPECT(attn_fwd(q, k, v, o, 1, 2, 1, 5, 64, 64, 0.1f, 1, INT_MAX - 5, F32, nullptr) == ROCATTN_OK);
    // rejections
    EXPECT(attn_fwd(nullptr, k, v, o, 1, 4, 2, 16, 16, 64, 0.1f, 1, 0, BF, nullptr) == ROCATTN_ERR_NULL);
    EXPECT(attn_fwd(q, k, v, o, 1, 6, 4, 16, 16, 64, 0.1f, 1, 0, BF, nullptr) == ROCATTN_ERR_SHAPE);
    EXPECT(attn_fwd(q, k, v, o, 1, 4, 2, 16, 16, 96, 0.1f, 1, 0, BF, nullptr) == ROCATTN_ERR_HEADDIM);
    EXPECT(attn_fwd(q, k, v, o, 1, 4, 2, 16, 16, 64, 0.1f, 1, -1, BF, nullptr) == ROCATTN_ERR_OFFSET);
    EXPECT(attn_fwd(q, k, v, o, 1, 4, 2, 16, 16, 64, 0.1f, 1, INT_MAX - 8, BF, nullptr) == ROCATTN_ERR_OFFSET);
    EXPECT(attn_fwd(q, k, v, o, 1, 1, 1, 1 << 30, (1 << 30) - 1000, 64, 0.1f, 1, 0, BF, nullptr) ==
           ROCATTN_ERR_SHAPE);
    EXPECT(attn_fwd(q, k, v, o, 1, 4, 2, 16, 16, 64, NAN, 1, 0, BF, nullptr) == ROCATTN_ERR_SCALE);
    EXPECT(attn_fwd(static_cast<char*>(q) + 2, k, v, o, 1, 4, 2, 16, 16, 64, 0.1f, 1, 0, BF, nullptr) ==
           ROCATTN_ERR_ALIGN);
    EXPECT(attn_fwd(q, k, v, q, 1, 4, 2, 16, 16, 64, 0.1f, 1, 0, BF, nullptr) == ROCATTN_ERR_SHAPE);
    EXPECT(attn_fwd(q, k, v, o, INT_MAX, INT_MAX, 1, INT_MAX, 1, 128, 0.1f, 1, 0, BF, nullptr) ==
           ROCATTN_ERR_SHAPE);

    // attn_fwd_ws with and without a workspace, with an lse
    const size_t need = attn_workspace_bytes(32, 32, 8, 1, 8192, 128, BF);
    EXPECT(need > 0);
    EXPECT(attn_fwd_ws(q, k, v, o, 32, 32, 8, 1, 8192, 128, 0.1f, 1, 8191, BF, nullptr, ws, need, lse) ==
           ROCATTN_OK);
    EXPECT(attn_fwd_ws(q, k, v, o, 32, 32, 8, 1, 8192, 128, 0.1f, 1, 8191, BF, nullptr, ws, need - 1, lse) ==
           ROCATTN_ERR_WORKSPACE);
    EXPECT(attn_fwd_ws(q, k, v, o, 1, 4, 2, 300, 2000, 128, 0.1f, 1, 1700, BF, nullptr, ws, 1ull << 30,
                       nullptr) == ROCATTN_OK);
    EXPECT(attn_fwd_ws(q, k, v, o, 1, 4, 2, 300, 2000, 128, 0.1f, 1, 1700, BF, nullptr, q, 1ull << 30,
                       nullptr) == ROCATTN_ERR_SHAPE);   // workspace over q
    EXPECT(attn_workspace_bytes(1, 4, 2, 16, 16, 96, BF) == 0);
    EXPECT(attn_workspace_bytes(1, 4, 2, 16, 16, 64, 7) == 0);

    // the entry point that allocates nothing: its fixed scratch serves a
    // decode step of the decode workload's size; a larger one is refused
    EXPECT(attn_fwd_noalloc(q, k, v, o, 32, 32, 8, 1, 8192, 128, 0.1f, 1, 8191, BF, nullptr, lse) == ROCATTN_OK);
    EXPECT(attn_fwd_noalloc(q, k, v, o, 1, 4, 2, 300, 2000, 128, 0.1f, 1, 1700, BF, nullptr, nullptr) ==
           ROCATTN_OK);
    EXPECT(attn_fwd_noalloc(q, k, v, o, 1024, 32, 8, 1, 1 << 20, 128, 0.1f, 1, (1 << 20) - 1, BF, nullptr,
                            nullptr) == ROCATTN_ERR_WORKSPACE);
    EXPECT(attn_fwd_noalloc(q, k, v, o, 1, 4, 2, 16, 16, 96, 0.1f, 1, 0, BF, nullptr, nullptr) ==
           ROCATTN_ERR_HEADDIM);

    // strided: BTHD views of q and o, dense k and v
    const long long st[12] = {16 * 4 * 64, 64, 4 * 64, 2 * 16 * 64, 16 * 64, 64,
                              2 * 16 * 64, 16 * 64, 64, 16 * 4 * 64, 64, 4 * 64};
    EXPECT(attn_fwd_strided(q, k, v, o, st, 1, 4, 2, 16, 16, 64, 0.1f, 1, 0, BF, nullptr, nullptr, 0, nullptr) ==
           ROCATTN_OK);
    const long long bad[12] = {16 * 4 * 64, 64, 4 * 64, 2 * 16 * 64, 16 * 64, 64,
                               2 * 16 * 64, 16 * 64, 64, 16 * 4 * 64, 0, 0};   // output rows collide
    EXPECT(attn_fwd_strided(q, k, v, o, bad, 1, 4, 2, 16, 16, 64, 0.1f, 1, 0, BF, nullptr, nullptr, 0,
                            nullptr) == ROCATTN_ERR_SHAPE);
    EXPECT(attn_fwd_strided(q, k, v, o, nullptr, 1, 4, 2, 16, 16, 64, 0.1f, 1, 0, BF, nullptr, nullptr, 0,
                            nullptr) == ROCATTN_ERR_NULL);

    // RoPE entry points
    EXPECT(rope_apply(q, k, 2, 32, 8, 4096, 128, 0, 10000.0, BF, nullptr) == ROCATTN_OK);
    EXPECT(rope_apply(q, nullptr, 2, 32, 8, 1, 128, 8191, 10000.0, BF, nullptr) == ROCATTN_OK);
    EXPECT(rope_apply(q, k, 2, 32, 8, 4096, 127, 0, 10000.0, BF, nullptr) == ROCATTN_ERR_HEADDIM);
    EXPECT(rope_apply(q, k, 2, 32, 8, 4096, 128, INT_MAX, 10000.0, BF, nullptr) == ROCATTN_ERR_OFFSET);
    EXPECT(rope_apply(q, k, 2, 32, 8, 4096, 128, 0, 0.0, BF, nullptr) == ROCATTN_ERR_SCALE);
    EXPECT(rope_apply_ex(q, k, 2, 32, 8, 16, 64, 3, 500000.0, F32, nullptr, ROCATTN_ROPE_ADJACENT) ==
           ROCATTN_OK);
    EXPECT(rope_apply_ex(q, k, 2, 32, 8, 16, 64, 3, 500000.0, F32, nullptr, 9) == ROCATTN_ERR_SHAPE);
    const int* pos = static_cast<const int*>(A(6));
    EXPECT(rope_apply_pos(q, k, 2, 4, 2, 16, 64, pos, 10000.0, BF, nullptr, 0) == ROCATTN_OK);
    EXPECT(rope_apply_pos(q, k, 2, 4, 2, 16, 64, nullptr, 10000.0, BF, nullptr, 0) == ROCATTN_ERR_NULL);

    // fused RoPE prefill
    const size_t tb = attn_fwd_rope_workspace_bytes(16384, 128);
    EXPECT(tb == (size_t)16384 * 64 * 2 * 4);
    EXPECT(attn_fwd_rope(q, k, v, o, 1, 32, 8, 16384, 16384, 128, 0.088f, 1, 0, 10000.0, 0, BF, nullptr, ws, tb,
                         nullptr) == ROCATTN_OK);
    EXPECT(attn_fwd_rope(q, k, v, o, 1, 32, 8, 16384, 16384, 128, 0.088f, 1, 0, 10000.0, 0, BF, nullptr, ws,
                         tb - 1, nullptr) == ROCATTN_ERR_WORKSPACE);
    EXPECT(attn_fwd_rope(q, k, v, o, 1, 32, 8, 100, 16384, 128, 0.088f, 1, 16300, 10000.0, 0, BF, nullptr, ws,
                         tb, nullptr) == ROCATTN_ERR_OFFSET);   // rows past the table
    EXPECT(attn_fwd_rope(q, k, v, o, 1, 32, 8, 100, 100, 128, 0.088f, 1, 0, 10000.0, 0, F32, nullptr, ws, tb,
                         nullptr) == ROCATTN_ERR_DTYPE);

    // values of their own width
    EXPECT(attn_fwd_dv(q, k, v, o, 2, 32, 8, 4096, 4096, 128, 64, 0.088f, 1, 0, BF, nullptr, lse) == ROCATTN_OK);
    EXPECT(attn_fwd_dv(q, k, v, o, 2, 32, 8, 4096, 4096, 128, 96, 0.088f, 1, 0, BF, nullptr, lse) ==
           ROCATTN_ERR_HEADDIM);

    // cached generation step
    const size_t sw = attn_decode_step_workspace_bytes(32, 32, 8, 1, 8192, 128, BF);
    EXPECT(sw > attn_workspace_bytes(32, 32, 8, 1, 8192, 128, BF));   // the partials plus the counters
    void *kn = A(7), *vn = A(8), *kc = A(9), *vc = A(10);
    EXPECT(attn_decode_step(q, kn, vn, kc, vc, o, 32, 32, 8, 1, 8192, 8191, 128, 0.088f, 10000.0, 0, BF, nullptr,
                            ws, sw - 1, nullptr) == ROCATTN_ERR_WORKSPACE);
    EXPECT(attn_decode_step(q, kn, vn, kc, vc, o, 32, 32, 8, 1, 8192, 8191, 128, 0.088f, 10000.0, 0, BF, nullptr,
                            ws, sw, nullptr) == ROCATTN_OK);
    EXPECT(attn_decode_step(q, kn, vn, kc, vc, o, 32, 32, 8, 1, 8192, 8192, 128, 0.088f, 10000.0, 0, BF, nullptr,
                            ws, sw, nullptr) == ROCATTN_ERR_OFFSET);
    EXPECT(attn_decode_step(q, kn, vn, kc, kc, o, 32, 32, 8, 1, 8192, 100, 128, 0.088f, 10000.0, 0, BF, nullptr,
                            ws, sw, nullptr) == ROCATTN_ERR_SHAPE);   // the two caches alias
    EXPECT(attn_decode_step(q, kn, vn, kc, vc, o, 1, 32, 8, 512, 4096, 3584, 128, 0.088f, 10000.0, 1, BF,
                            nullptr, nullptr, 0, nullptr) == ROCATTN_OK);

    // gradients
    const size_t bw = attn_bwd_workspace_bytes(2, 32, 8, 4096, 4096, 128, BF);
    EXPECT(bw > 0);
    void *dO = A(11), *dq = A(12), *dk = A(13), *dv = A(14);
    EXPECT(attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, 2, 32, 8, 4096, 4096, 128, 0.088f, 1, 0, BF, nullptr, ws,
                    bw) == ROCATTN_OK);
    EXPECT(attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, 1, 4, 2, 70, 200, 64, 0.125f, 1, INT_MAX - 70, BF, nullptr,
                    ws, bw) == ROCATTN_OK);
    EXPECT(attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, 2, 32, 8, 4096, 4096, 128, 0.088f, 1, 0, BF, nullptr, ws,
                    bw - 1) == ROCATTN_ERR_WORKSPACE);
    EXPECT(attn_bwd(q, k, v, o, dO, lse, q, dk, dv, 2, 32, 8, 4096, 4096, 128, 0.088f, 1, 0, BF, nullptr, ws,
                    bw) == ROCATTN_ERR_SHAPE);   // dq over q

    for (int s = -10; s <= 1; ++s) EXPECT(attn_status_string(s) != nullptr);
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("api harness: all calls behaved (%d launches reached the stubs)\n", launches);
    return 0;
}
