// api.cpp -- the C ABI of librocattn (declared in include/rocattn.h):
// argument validation, kernel choice and launch.  Every argument is checked
// on the host before anything is enqueued; a rejected call launches nothing.
#include <math.h>
#include <limits.h>
#include <stdint.h>

#include "../../include/rocattn.h"
#include "internal.hpp"

#define ROCATTN_API extern "C" __attribute__((visibility("default")))

namespace {

using rocattn::FwdParams;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p + bytes) and [q, q + qbytes) share a byte
bool overlaps(const void* p, size_t bytes, const void* q, size_t qbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + bytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + qbytes;
    return a0 < b1 && b0 < a1;
}

// element count a*b*c*d, or -1 when it would not fit comfortably in 62 bits
long long count4(long long a, long long b, long long c, long long d) {
    const long long lim = (1LL << 62);
    long long n = a;
    for (long long f : {b, c, d}) {
        if (n > lim / f) return -1;
        n *= f;
    }
    return n;
}

int check_fwd(const void* q, const void* k, const void* v, const void* o, int B, int Hq,
              int Hkv, int Tq, int Tk, int d, float scale, int causal, int q_offset,
              int dtype, const float* lse) {
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;
    if (!q || !k || !v || !o) return ROCATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || d <= 0) return ROCATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ROCATTN_ERR_SHAPE;
    if (dtype == ROCATTN_BF16) {
        if (d != 64 && d != 128) return ROCATTN_ERR_HEADDIM;
    } else {
        if (d > 256 || d % 4 != 0) return ROCATTN_ERR_HEADDIM;
        if (Hq > 65535 || B > 65535) return ROCATTN_ERR_SHAPE;   // grid y / z limits
    }
    if (causal && q_offset < 0) return ROCATTN_ERR_OFFSET;
    if (causal && (long long)q_offset + Tq > INT_MAX) return ROCATTN_ERR_OFFSET;
    if (!isfinite(scale)) return ROCATTN_ERR_SCALE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ROCATTN_ERR_ALIGN;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ROCATTN_ERR_ALIGN;
    const long long nq = count4(B, Hq, Tq, d), nkv = count4(B, Hkv, Tk, d);
    if (nq < 0 || nkv < 0) return ROCATTN_ERR_SHAPE;
    // one workgroup per 128 query rows (bf16) must fit a 1-D grid
    if (count4(B, Hq, (Tq + 127) / 128, 1) > INT_MAX) return ROCATTN_ERR_SHAPE;
    const size_t elt = dtype == ROCATTN_F32 ? 4 : 2;
    const size_t qb = (size_t)nq * elt, kvb = (size_t)nkv * elt;
    if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kvb) || overlaps(o, qb, v, kvb))
        return ROCATTN_ERR_SHAPE;
    if (lse) {
        const size_t lb = (size_t)B * Hq * Tq * sizeof(float);
        if (overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kvb) || overlaps(lse, lb, v, kvb) ||
            overlaps(lse, lb, o, qb))
            return ROCATTN_ERR_SHAPE;
    }
    return ROCATTN_OK;
}

bool uses_decode(int dtype, int Tq, int Hq, int Hkv, int d) {
    return dtype == ROCATTN_BF16 && Tq == 1 && rocattn::decode_bf16_supported(Hq, Hkv, d);
}

size_t workspace_for(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype) {
    if (!uses_decode(dtype, Tq, Hq, Hkv, d)) return 0;
    return rocattn::decode_workspace_bytes(B, Hq, Hkv, Tk, d);
}

int launch(const FwdParams& p, int dtype, hipStream_t stream, void* ws, size_t ws_bytes) {
    hipError_t e;
    if (dtype == ROCATTN_F32)
        e = rocattn::launch_fwd_f32(p, stream);
    else if (uses_decode(dtype, p.Tq, p.Hq, p.Hkv, p.d))
        e = rocattn::launch_decode_bf16(p, ws, ws_bytes, stream);
    else
        e = rocattn::launch_prefill_bf16(p, stream);
    return e == hipSuccess ? ROCATTN_OK : ROCATTN_ERR_HIP;
}

FwdParams make_params(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int Hq, int Hkv, int Tq, int Tk, int d, float scale, int causal,
                      int q_offset) {
    FwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Tq = Tq; p.Tk = Tk; p.d = d;
    p.scale = scale;
    p.causal = causal ? 1 : 0;
    p.q_offset = causal ? q_offset : 0;
    return p;
}

}  // namespace

ROCATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int Hq,
                         int Hkv, int Tq, int Tk, int d_head, float scale, int causal,
                         int q_offset, int dtype, void* stream) {
    int st = check_fwd(q, k, v, o, B, Hq, Hkv, Tq, Tk, d_head, scale, causal, q_offset, dtype,
                       nullptr);
    if (st != ROCATTN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const FwdParams p = make_params(q, k, v, o, nullptr, B, Hq, Hkv, Tq, Tk, d_head, scale,
                                    causal, q_offset);
    const size_t wsb = workspace_for(B, Hq, Hkv, Tq, Tk, d_head, dtype);
    if (wsb == 0) return launch(p, dtype, s, nullptr, 0);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, wsb, s) != hipSuccess) return ROCATTN_ERR_HIP;
    st = launch(p, dtype, s, ws, wsb);
    if (hipFreeAsync(ws, s) != hipSuccess && st == ROCATTN_OK) st = ROCATTN_ERR_HIP;
    return st;
}

ROCATTN_API size_t attn_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d_head,
                                        int dtype) {
    // the same shape checks attn_fwd applies (pointers aside)
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return 0;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || d_head <= 0) return 0;
    if (Hq % Hkv != 0) return 0;
    if (dtype == ROCATTN_BF16 && d_head != 64 && d_head != 128) return 0;
    return workspace_for(B, Hq, Hkv, Tq, Tk, d_head, dtype);
}

ROCATTN_API int attn_fwd_ws(const void* q, const void* k, const void* v, void* o, int B, int Hq,
                            int Hkv, int Tq, int Tk, int d_head, float scale, int causal,
                            int q_offset, int dtype, void* stream, void* workspace,
                            size_t ws_bytes, float* lse) {
    int st = check_fwd(q, k, v, o, B, Hq, Hkv, Tq, Tk, d_head, scale, causal, q_offset, dtype,
                       lse);
    if (st != ROCATTN_OK) return st;
    const size_t wsb = workspace_for(B, Hq, Hkv, Tq, Tk, d_head, dtype);
    if (wsb > 0) {
        if (!workspace || ws_bytes < wsb) return ROCATTN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return ROCATTN_ERR_ALIGN;
        const size_t elt = dtype == ROCATTN_F32 ? 4 : 2;
        const size_t qb = (size_t)B * Hq * Tq * d_head * elt;
        const size_t kvb = (size_t)B * Hkv * Tk * d_head * elt;
        if (overlaps(workspace, wsb, q, qb) || overlaps(workspace, wsb, k, kvb) ||
            overlaps(workspace, wsb, v, kvb) || overlaps(workspace, wsb, o, qb) ||
            (lse && overlaps(workspace, wsb, lse, (size_t)B * Hq * Tq * sizeof(float))))
            return ROCATTN_ERR_SHAPE;
    }
    const FwdParams p = make_params(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d_head, scale, causal,
                                    q_offset);
    return launch(p, dtype, static_cast<hipStream_t>(stream), workspace, ws_bytes);
}

ROCATTN_API int rope_apply(void* q, void* k, int B, int Hq, int Hkv, int T, int d_head, int pos0,
                           double base, int dtype, void* stream) {
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;
    if (!q) return ROCATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || T <= 0 || d_head <= 0) return ROCATTN_ERR_SHAPE;
    if (k && Hkv <= 0) return ROCATTN_ERR_SHAPE;
    if (d_head % 2 != 0 || d_head > 256) return ROCATTN_ERR_HEADDIM;
    if (pos0 < 0 || (long long)pos0 + T - 1 > INT_MAX) return ROCATTN_ERR_OFFSET;
    if (!isfinite(base) || !(base > 0.0)) return ROCATTN_ERR_SCALE;
    if (!aligned16(q) || (k && !aligned16(k))) return ROCATTN_ERR_ALIGN;
    const long long nq = count4(B, Hq, T, d_head);
    const long long nk = k ? count4(B, Hkv, T, d_head) : 0;
    if (nq < 0 || nk < 0) return ROCATTN_ERR_SHAPE;
    const size_t elt = dtype == ROCATTN_F32 ? 4 : 2;
    if (k && overlaps(q, (size_t)nq * elt, k, (size_t)nk * elt)) return ROCATTN_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (rocattn::launch_rope(q, (long long)B * Hq, T, d_head, pos0, base, dtype, s) != hipSuccess)
        return ROCATTN_ERR_HIP;
    if (k && rocattn::launch_rope(k, (long long)B * Hkv, T, d_head, pos0, base, dtype, s) !=
                 hipSuccess)
        return ROCATTN_ERR_HIP;
    return ROCATTN_OK;
}

ROCATTN_API const char* attn_status_string(int status) {
    switch (status) {
        case ROCATTN_OK: return "success";
        case ROCATTN_ERR_NULL: return "a required pointer is NULL";
        case ROCATTN_ERR_SHAPE: return "invalid sizes, Hq not a multiple of Hkv, or overlapping buffers";
        case ROCATTN_ERR_DTYPE: return "unknown dtype";
        case ROCATTN_ERR_HEADDIM: return "head size not supported for this dtype";
        case ROCATTN_ERR_OFFSET: return "invalid position offset (negative or too large)";
        case ROCATTN_ERR_SCALE: return "scale or RoPE base not finite (or base <= 0)";
        case ROCATTN_ERR_ALIGN: return "a pointer is not suitably aligned";
        case ROCATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case ROCATTN_ERR_HIP: return "HIP runtime error while launching";
        default: return "unknown status";
    }
}
