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

// The kernels form row and key limits such as q_offset + (first row of a
// tile) + (tile rows) in 32-bit integers, with q_offset clamped to Tk first
// (clamped_offset): Tq + Tk plus a tile's rows must stay below INT_MAX.
bool sizes_fit_int(int Tq, int Tk) { return (long long)Tq + Tk <= (long long)INT_MAX - 1024; }

// A causal offset at or past Tk - 1 makes every key visible to every row,
// exactly as Tk does; clamping keeps q_offset + Tq within 32 bits in the
// kernels' limit arithmetic (given sizes_fit_int).
int clamped_offset(int causal, int q_offset, int Tk) {
    return causal ? (q_offset < Tk ? q_offset : Tk) : 0;
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
    if (!sizes_fit_int(Tq, Tk)) return ROCATTN_ERR_SHAPE;
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

// Workspace a call cannot do without: the split-K decode's partial results.
size_t workspace_required(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype) {
    if (!uses_decode(dtype, Tq, Hq, Hkv, d)) return 0;
    return rocattn::decode_workspace_bytes(B, Hq, Hkv, Tk, d);
}

// Workspace a call uses when given: the required bytes, or for a small bf16
// prefill the partial results of its key splits (optional).
size_t workspace_for(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype) {
    const size_t req = workspace_required(B, Hq, Hkv, Tq, Tk, d, dtype);
    if (req > 0 || dtype != ROCATTN_BF16) return req;
    return rocattn::prefill_split_bytes(B, Hq, Tq, d, rocattn::prefill_splits(B, Hq, Tq, Tk, d, d));
}

// Bytes of the caller's workspace a call will use: the required bytes
// (ERR_WORKSPACE when missing or short, signalled by returning SIZE_MAX), or
// the optional bytes when the caller gave at least that much, else 0.
size_t workspace_use(size_t req, size_t want, const void* ws, size_t ws_bytes) {
    if (req > 0) return (ws && ws_bytes >= req) ? req : SIZE_MAX;
    return (want > 0 && ws && ws_bytes >= want) ? want : 0;
}

int launch(const FwdParams& p, int dtype, hipStream_t stream, void* ws, size_t ws_bytes) {
    hipError_t e;
    if (dtype == ROCATTN_F32) {
        e = rocattn::launch_fwd_f32(p, stream);
    } else if (uses_decode(dtype, p.Tq, p.Hq, p.Hkv, p.d)) {
        e = rocattn::launch_decode_bf16(p, ws, ws_bytes, stream);
    } else {
        // a small prefill is split over the keys when the caller's workspace
        // holds the partial results (and the layout is dense); otherwise one
        // workgroup per (query tile, head) as usual
        const int ks = rocattn::prefill_splits(p.B, p.Hq, p.Tq, p.Tk, p.d, p.d);
        const size_t need = rocattn::prefill_split_bytes(p.B, p.Hq, p.Tq, p.d, ks);
        const bool dense = p.qs.t == p.d && p.ks.t == p.d && p.vs.t == p.d && p.os.t == p.d;
        if (ks > 1 && ws && ws_bytes >= need && dense) {
            FwdParams q = p;
            const long long rows = (long long)p.B * p.Hq * p.Tq;
            q.nsplit = ks;
            q.part_o = static_cast<float*>(ws);
            q.part_ml = q.part_o + (size_t)rows * ks * p.d;
            e = rocattn::launch_prefill_bf16(q, stream);
            if (e == hipSuccess)
                e = rocattn::launch_combine_bf16(q.part_o, q.part_ml, p.o, p.lse, rows, ks, p.Hq, p.Tq, p.os,
                                                 p.d, stream);
        } else {
            e = rocattn::launch_prefill_bf16(p, stream);
        }
    }
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
    p.q_offset = clamped_offset(causal, q_offset, Tk);
    // dense [B][H][T][d]
    p.qs = {(long long)Hq * Tq * d, (long long)Tq * d, d};
    p.os = p.qs;
    p.ks = {(long long)Hkv * Tk * d, (long long)Tk * d, d};
    p.vs = p.ks;
    return p;
}

// Largest element offset + d of a [n0][n1][n2][d] tensor with strides s, or
// -1 when a stride is negative or the extent passes 2^62.
long long extent(int n0, int n1, int n2, int d, const rocattn::Strides& s) {
    if (s.b < 0 || s.h < 0 || s.t < 0) return -1;
    const long long lim = 1LL << 62;
    long long e = d;
    const long long n[3] = {n0, n1, n2}, st[3] = {s.b, s.h, s.t};
    for (int i = 0; i < 3; ++i) {
        if (st[i] != 0 && (n[i] - 1) > (lim - e) / st[i]) return -1;
        e += (n[i] - 1) * st[i];
    }
    return e;
}

// Rows of o never share an element: ordered by stride, each level of size > 1
// steps at least over the whole extent of the levels inside it.
bool rows_disjoint(int n0, int n1, int n2, int d, const rocattn::Strides& s) {
    long long sz[3] = {n0, n1, n2}, st[3] = {s.b, s.h, s.t};
    for (int i = 0; i < 3; ++i)          // sort by stride, ascending
        for (int j = i + 1; j < 3; ++j)
            if (st[j] < st[i]) {
                long long x = st[i]; st[i] = st[j]; st[j] = x;
                x = sz[i]; sz[i] = sz[j]; sz[j] = x;
            }
    long long inner = d;                 // extent of the levels inside the current one
    for (int i = 0; i < 3; ++i) {
        if (sz[i] <= 1) continue;
        if (st[i] < inner) return false;
        inner = st[i] * (sz[i] - 1) + inner;
    }
    return true;
}

int check_strided(const void* q, const void* k, const void* v, const void* o, int B, int Hq,
                  int Hkv, int Tq, int Tk, int d, float scale, int causal, int q_offset,
                  int dtype, const float* lse, const rocattn::Strides (&st)[4]) {
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;
    if (!q || !k || !v || !o) return ROCATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || d <= 0) return ROCATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ROCATTN_ERR_SHAPE;
    if (dtype == ROCATTN_BF16) {
        if (d != 64 && d != 128) return ROCATTN_ERR_HEADDIM;
    } else {
        if (d > 256 || d % 4 != 0) return ROCATTN_ERR_HEADDIM;
        if (Hq > 65535 || B > 65535) return ROCATTN_ERR_SHAPE;
    }
    if (causal && q_offset < 0) return ROCATTN_ERR_OFFSET;
    if (causal && (long long)q_offset + Tq > INT_MAX) return ROCATTN_ERR_OFFSET;
    if (!sizes_fit_int(Tq, Tk)) return ROCATTN_ERR_SHAPE;
    if (!isfinite(scale)) return ROCATTN_ERR_SCALE;
    const size_t elt = dtype == ROCATTN_F32 ? 4 : 2;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ROCATTN_ERR_ALIGN;
    for (const auto& x : st)
        if ((x.b * (long long)elt) % 16 || (x.h * (long long)elt) % 16 || (x.t * (long long)elt) % 16)
            return ROCATTN_ERR_ALIGN;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ROCATTN_ERR_ALIGN;
    const long long eq = extent(B, Hq, Tq, d, st[0]), ek = extent(B, Hkv, Tk, d, st[1]);
    const long long ev = extent(B, Hkv, Tk, d, st[2]), eo = extent(B, Hq, Tq, d, st[3]);
    if (eq < 0 || ek < 0 || ev < 0 || eo < 0) return ROCATTN_ERR_SHAPE;
    if (!rows_disjoint(B, Hq, Tq, d, st[3])) return ROCATTN_ERR_SHAPE;
    // the bf16 kernels address a 64-row key/value tile with 32-bit byte
    // offsets, and every kernel keeps token strides in 32 bits
    if (dtype == ROCATTN_BF16 && (st[1].t > (1LL << 24) || st[2].t > (1LL << 24)))
        return ROCATTN_ERR_SHAPE;
    for (const auto& x : st)
        if (x.t > INT_MAX) return ROCATTN_ERR_SHAPE;
    if (count4(B, Hq, (Tq + 127) / 128, 1) > INT_MAX) return ROCATTN_ERR_SHAPE;
    const size_t ob = (size_t)eo * elt;
    if (overlaps(o, ob, q, (size_t)eq * elt) || overlaps(o, ob, k, (size_t)ek * elt) ||
        overlaps(o, ob, v, (size_t)ev * elt))
        return ROCATTN_ERR_SHAPE;
    if (lse) {
        const size_t lb = (size_t)B * Hq * Tq * sizeof(float);
        if (overlaps(lse, lb, q, (size_t)eq * elt) || overlaps(lse, lb, k, (size_t)ek * elt) ||
            overlaps(lse, lb, v, (size_t)ev * elt) || overlaps(lse, lb, o, ob))
            return ROCATTN_ERR_SHAPE;
    }
    return ROCATTN_OK;
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
    if (wsb == 0) return launch(p, dtype, s, nullptr, 0);   // else allocated for the call
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
    const size_t wsb = workspace_use(workspace_required(B, Hq, Hkv, Tq, Tk, d_head, dtype),
                                     workspace_for(B, Hq, Hkv, Tq, Tk, d_head, dtype), workspace, ws_bytes);
    if (wsb == SIZE_MAX) return ROCATTN_ERR_WORKSPACE;
    if (wsb > 0) {
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
    return launch(p, dtype, static_cast<hipStream_t>(stream), wsb ? workspace : nullptr, wsb);
}

ROCATTN_API int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int Hq,
                                 int Hkv, int Tq, int Tk, int d_head, float scale, int causal,
                                 int q_offset, int dtype, void* stream, float* lse) {
    int st = check_fwd(q, k, v, o, B, Hq, Hkv, Tq, Tk, d_head, scale, causal, q_offset, dtype, lse);
    if (st != ROCATTN_OK) return st;
    const size_t req = workspace_required(B, Hq, Hkv, Tq, Tk, d_head, dtype);
    if (req > rocattn::kNoAllocScratchBytes) return ROCATTN_ERR_WORKSPACE;
    // the optional key splits of a small prefill only when their partials fit
    const size_t want = workspace_for(B, Hq, Hkv, Tq, Tk, d_head, dtype);
    const size_t use = want <= rocattn::kNoAllocScratchBytes ? want : req;
    void* scratch = nullptr;
    if (use > 0 && rocattn::noalloc_scratch(&scratch) != hipSuccess) return ROCATTN_ERR_HIP;
    const FwdParams p = make_params(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d_head, scale, causal,
                                    q_offset);
    return launch(p, dtype, static_cast<hipStream_t>(stream), use ? scratch : nullptr, use);
}

ROCATTN_API int attn_fwd_strided(const void* q, const void* k, const void* v, void* o,
                                 const long long* strides, int B, int Hq, int Hkv, int Tq,
                                 int Tk, int d_head, float scale, int causal, int q_offset,
                                 int dtype, void* stream, void* workspace, size_t ws_bytes,
                                 float* lse) {
    if (!strides) return ROCATTN_ERR_NULL;
    const rocattn::Strides st[4] = {{strides[0], strides[1], strides[2]},
                                    {strides[3], strides[4], strides[5]},
                                    {strides[6], strides[7], strides[8]},
                                    {strides[9], strides[10], strides[11]}};
    int status = check_strided(q, k, v, o, B, Hq, Hkv, Tq, Tk, d_head, scale, causal, q_offset,
                               dtype, lse, st);
    if (status != ROCATTN_OK) return status;
    const size_t wsb = workspace_use(workspace_required(B, Hq, Hkv, Tq, Tk, d_head, dtype),
                                     workspace_for(B, Hq, Hkv, Tq, Tk, d_head, dtype), workspace, ws_bytes);
    if (wsb == SIZE_MAX) return ROCATTN_ERR_WORKSPACE;
    if (wsb > 0) {
        if (!aligned16(workspace)) return ROCATTN_ERR_ALIGN;
        const size_t elt = dtype == ROCATTN_F32 ? 4 : 2;
        const size_t eq = (size_t)extent(B, Hq, Tq, d_head, st[0]) * elt;
        const size_t ek = (size_t)extent(B, Hkv, Tk, d_head, st[1]) * elt;
        const size_t ev = (size_t)extent(B, Hkv, Tk, d_head, st[2]) * elt;
        const size_t eo = (size_t)extent(B, Hq, Tq, d_head, st[3]) * elt;
        if (overlaps(workspace, wsb, q, eq) || overlaps(workspace, wsb, k, ek) ||
            overlaps(workspace, wsb, v, ev) || overlaps(workspace, wsb, o, eo) ||
            (lse && overlaps(workspace, wsb, lse, (size_t)B * Hq * Tq * sizeof(float))))
            return ROCATTN_ERR_SHAPE;
    }
    FwdParams p = make_params(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d_head, scale, causal,
                              q_offset);
    p.qs = st[0]; p.ks = st[1]; p.vs = st[2]; p.os = st[3];
    return launch(p, dtype, static_cast<hipStream_t>(stream), wsb ? workspace : nullptr, wsb);
}

ROCATTN_API int rope_apply_ex(void* q, void* k, int B, int Hq, int Hkv, int T, int d_head,
                              int pos0, double base, int dtype, void* stream, int pairing) {
    if (pairing != ROCATTN_ROPE_SPLIT_HALF && pairing != ROCATTN_ROPE_ADJACENT)
        return ROCATTN_ERR_SHAPE;
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
    // one launch turns q and k: they share every (position, pair) angle
    if (rocattn::launch_rope(q, (long long)B * Hq, T, d_head, pos0, base, dtype, pairing, s, nullptr, k,
                             k ? (long long)B * Hkv : 0) != hipSuccess)
        return ROCATTN_ERR_HIP;
    return ROCATTN_OK;
}

ROCATTN_API int rope_apply_pos(void* q, void* k, int B, int Hq, int Hkv, int T, int d_head,
                               const int* positions, double base, int dtype, void* stream,
                               int pairing) {
    if (pairing != ROCATTN_ROPE_SPLIT_HALF && pairing != ROCATTN_ROPE_ADJACENT)
        return ROCATTN_ERR_SHAPE;
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;
    if (!q || !positions) return ROCATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || T <= 0 || d_head <= 0) return ROCATTN_ERR_SHAPE;
    if (k && Hkv <= 0) return ROCATTN_ERR_SHAPE;
    if (d_head % 2 != 0 || d_head > 256) return ROCATTN_ERR_HEADDIM;
    if (!isfinite(base) || !(base > 0.0)) return ROCATTN_ERR_SCALE;
    if (!aligned16(q) || (k && !aligned16(k))) return ROCATTN_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(positions) & 3u) return ROCATTN_ERR_ALIGN;
    const long long nq = count4(B, Hq, T, d_head);
    const long long nk = k ? count4(B, Hkv, T, d_head) : 0;
    if (nq < 0 || nk < 0) return ROCATTN_ERR_SHAPE;
    if ((long long)B * T * (d_head / 2) > (long long)INT_MAX * 256) return ROCATTN_ERR_SHAPE;   // 1-D grid
    const size_t elt = dtype == ROCATTN_F32 ? 4 : 2;
    const size_t pb = (size_t)B * T * sizeof(int);
    if (k && overlaps(q, (size_t)nq * elt, k, (size_t)nk * elt)) return ROCATTN_ERR_SHAPE;
    if (overlaps(positions, pb, q, (size_t)nq * elt) || (k && overlaps(positions, pb, k, (size_t)nk * elt)))
        return ROCATTN_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (rocattn::launch_rope_pos(q, B, Hq, T, d_head, positions, base, dtype, pairing, s) != hipSuccess)
        return ROCATTN_ERR_HIP;
    if (k && rocattn::launch_rope_pos(k, B, Hkv, T, d_head, positions, base, dtype, pairing, s) != hipSuccess)
        return ROCATTN_ERR_HIP;
    return ROCATTN_OK;
}

ROCATTN_API int rope_apply(void* q, void* k, int B, int Hq, int Hkv, int T, int d_head, int pos0,
                           double base, int dtype, void* stream) {
    return rope_apply_ex(q, k, B, Hq, Hkv, T, d_head, pos0, base, dtype, stream,
                         ROCATTN_ROPE_SPLIT_HALF);
}

ROCATTN_API int attn_decode_step(void* q, const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, void* o, int B, int Hq, int Hkv, int Tn, int Tmax,
                                 int pos, int d_head, float scale, double rope_base, int pairing,
                                 int dtype, void* stream, void* workspace, size_t ws_bytes,
                                 float* lse) {
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !o) return ROCATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tn <= 0 || Tmax <= 0 || d_head <= 0)
        return ROCATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ROCATTN_ERR_SHAPE;
    if (pairing != ROCATTN_ROPE_SPLIT_HALF && pairing != ROCATTN_ROPE_ADJACENT)
        return ROCATTN_ERR_SHAPE;
    if (dtype == ROCATTN_BF16) {
        if (d_head != 64 && d_head != 128) return ROCATTN_ERR_HEADDIM;
    } else {
        if (d_head > 256 || d_head % 4 != 0) return ROCATTN_ERR_HEADDIM;
        if (Hq > 65535 || B > 65535) return ROCATTN_ERR_SHAPE;
    }
    if (pos < 0 || (long long)pos + Tn > Tmax) return ROCATTN_ERR_OFFSET;
    if (!sizes_fit_int(Tn, Tmax)) return ROCATTN_ERR_SHAPE;
    if (!isfinite(scale)) return ROCATTN_ERR_SCALE;
    if (!isfinite(rope_base) || !(rope_base > 0.0)) return ROCATTN_ERR_SCALE;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(o))
        return ROCATTN_ERR_ALIGN;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ROCATTN_ERR_ALIGN;
    const long long nq = count4(B, Hq, Tn, d_head), nn = count4(B, Hkv, Tn, d_head);
    const long long nc = count4(B, Hkv, Tmax, d_head);
    if (nq < 0 || nn < 0 || nc < 0) return ROCATTN_ERR_SHAPE;
    if (count4(B, Hq, (Tn + 127) / 128, 1) > INT_MAX) return ROCATTN_ERR_SHAPE;
    const size_t elt = dtype == ROCATTN_F32 ? 4 : 2;
    const size_t qb = (size_t)nq * elt, nb = (size_t)nn * elt, cb = (size_t)nc * elt;
    // q and the caches are written; nothing written may overlap anything else
    const void* bufs[6] = {q, k_new, v_new, k_cache, v_cache, o};
    const size_t lens[6] = {qb, nb, nb, cb, cb, qb};
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j) {
            const bool written = i == 0 || i >= 3 || j == 0 || j >= 3;
            if (written && overlaps(bufs[i], lens[i], bufs[j], lens[j])) return ROCATTN_ERR_SHAPE;
        }
    if (lse) {
        const size_t lb = (size_t)B * Hq * Tn * sizeof(float);
        for (int i = 0; i < 6; ++i)
            if (overlaps(lse, lb, bufs[i], lens[i])) return ROCATTN_ERR_SHAPE;
    }
    const int Tk = pos + Tn;
    // one new token per sequence (bf16): the whole step is one launch whose
    // workspace also holds the arrival counters of its chunk merge
    const bool fused = uses_decode(dtype, Tn, Hq, Hkv, d_head);
    const size_t wsb = fused ? ((workspace && ws_bytes >= rocattn::decode_step_workspace_bytes(B, Hq, Hkv, Tmax, d_head))
                                    ? rocattn::decode_step_workspace_bytes(B, Hq, Hkv, Tmax, d_head)
                                    : SIZE_MAX)
                             : workspace_use(workspace_required(B, Hq, Hkv, Tn, Tk, d_head, dtype),
                                             workspace_for(B, Hq, Hkv, Tn, Tk, d_head, dtype), workspace, ws_bytes);
    if (wsb == SIZE_MAX) return ROCATTN_ERR_WORKSPACE;
    if (wsb > 0) {
        if (!aligned16(workspace)) return ROCATTN_ERR_ALIGN;
        for (int i = 0; i < 6; ++i)
            if (overlaps(workspace, wsb, bufs[i], lens[i])) return ROCATTN_ERR_SHAPE;
        if (lse && overlaps(workspace, wsb, lse, (size_t)B * Hq * Tn * sizeof(float)))
            return ROCATTN_ERR_SHAPE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fused) {
        rocattn::StepParams sp;
        sp.q = q; sp.kn = k_new; sp.vn = v_new; sp.kc = k_cache; sp.vc = v_cache; sp.o = o; sp.lse = lse;
        sp.B = B; sp.Hq = Hq; sp.Hkv = Hkv; sp.Tmax = Tmax; sp.pos = pos; sp.d = d_head;
        sp.scale = scale;
        sp.base = rope_base;
        sp.pairing = pairing;
        return rocattn::launch_decode_step_bf16(sp, workspace, wsb, s) == hipSuccess ? ROCATTN_OK : ROCATTN_ERR_HIP;
    }
    if (rocattn::launch_step_prep(q, k_new, v_new, k_cache, v_cache, B, Hq, Hkv, Tn, Tmax, d_head,
                                  pos, rope_base, dtype, pairing, s) != hipSuccess)
        return ROCATTN_ERR_HIP;
    FwdParams p = make_params(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Tn, Tk, d_head, scale, 1,
                              pos);
    p.ks = {(long long)Hkv * Tmax * d_head, (long long)Tmax * d_head, d_head};
    p.vs = p.ks;
    return launch(p, dtype, s, wsb ? workspace : nullptr, wsb);
}

ROCATTN_API size_t attn_decode_step_workspace_bytes(int B, int Hq, int Hkv, int Tn, int Tmax, int d_head,
                                                   int dtype) {
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return 0;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tn <= 0 || Tmax <= 0 || d_head <= 0 || Hq % Hkv != 0) return 0;
    if (dtype == ROCATTN_BF16 && d_head != 64 && d_head != 128) return 0;
    if (uses_decode(dtype, Tn, Hq, Hkv, d_head)) return rocattn::decode_step_workspace_bytes(B, Hq, Hkv, Tmax, d_head);
    return workspace_for(B, Hq, Hkv, Tn, Tmax, d_head, dtype);
}

ROCATTN_API int attn_fwd_dv(const void* q, const void* k, const void* v, void* o, int B, int Hq,
                            int Hkv, int Tq, int Tk, int d_k, int d_v, float scale, int causal,
                            int q_offset, int dtype, void* stream, float* lse) {
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;
    if (!q || !k || !v || !o) return ROCATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || d_k <= 0 || d_v <= 0)
        return ROCATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ROCATTN_ERR_SHAPE;
    for (int d : {d_k, d_v}) {
        if (dtype == ROCATTN_BF16) {
            if (d != 64 && d != 128) return ROCATTN_ERR_HEADDIM;
        } else if (d > 256 || d % 4 != 0) {
            return ROCATTN_ERR_HEADDIM;
        }
    }
    if (dtype == ROCATTN_F32 && (Hq > 65535 || B > 65535)) return ROCATTN_ERR_SHAPE;
    if (causal && q_offset < 0) return ROCATTN_ERR_OFFSET;
    if (causal && (long long)q_offset + Tq > INT_MAX) return ROCATTN_ERR_OFFSET;
    if (!sizes_fit_int(Tq, Tk)) return ROCATTN_ERR_SHAPE;
    if (!isfinite(scale)) return ROCATTN_ERR_SCALE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ROCATTN_ERR_ALIGN;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ROCATTN_ERR_ALIGN;
    const long long nq = count4(B, Hq, Tq, d_k), nk = count4(B, Hkv, Tk, d_k);
    const long long nv = count4(B, Hkv, Tk, d_v), no = count4(B, Hq, Tq, d_v);
    if (nq < 0 || nk < 0 || nv < 0 || no < 0) return ROCATTN_ERR_SHAPE;
    if (count4(B, Hq, (Tq + 127) / 128, 1) > INT_MAX) return ROCATTN_ERR_SHAPE;
    const size_t elt = dtype == ROCATTN_F32 ? 4 : 2;
    const size_t qb = (size_t)nq * elt, kb = (size_t)nk * elt, vb = (size_t)nv * elt, ob = (size_t)no * elt;
    if (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, vb)) return ROCATTN_ERR_SHAPE;
    if (lse) {
        const size_t lb = (size_t)B * Hq * Tq * sizeof(float);
        if (overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, vb) ||
            overlaps(lse, lb, o, ob))
            return ROCATTN_ERR_SHAPE;
    }
    FwdParams p = make_params(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d_k, scale, causal, q_offset);
    p.dv = d_v;
    p.vs = {(long long)Hkv * Tk * d_v, (long long)Tk * d_v, d_v};
    p.os = {(long long)Hq * Tq * d_v, (long long)Tq * d_v, d_v};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == ROCATTN_F32 ? rocattn::launch_fwd_f32(p, s) : rocattn::launch_prefill_bf16(p, s);
    return e == hipSuccess ? ROCATTN_OK : ROCATTN_ERR_HIP;
}

ROCATTN_API size_t attn_fwd_rope_workspace_bytes(int Tk, int d_head) {
    if (Tk <= 0 || (d_head != 64 && d_head != 128)) return 0;
    return (size_t)Tk * (size_t)(d_head / 2) * 2 * sizeof(float);
}

ROCATTN_API int attn_fwd_rope(const void* q, void* k, const void* v, void* o, int B, int Hq,
                              int Hkv, int Tq, int Tk, int d_head, float scale, int causal,
                              int q_offset, double rope_base, int pairing, int dtype, void* stream,
                              void* workspace, size_t ws_bytes, float* lse) {
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;
    if (dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;   // the query-load rotation is bf16
    const int st = check_fwd(q, k, v, o, B, Hq, Hkv, Tq, Tk, d_head, scale, causal, q_offset,
                             dtype, lse);
    if (st != ROCATTN_OK) return st;
    if (pairing != ROCATTN_ROPE_SPLIT_HALF && pairing != ROCATTN_ROPE_ADJACENT) return ROCATTN_ERR_SHAPE;
    if (!(rope_base > 0.0) || !isfinite(rope_base)) return ROCATTN_ERR_SCALE;
    // query row i sits at position q_offset + i, key row j at j: every
    // query position must have a key row (the table covers [0, Tk))
    if (q_offset < 0 || (long long)q_offset + Tq > Tk) return ROCATTN_ERR_OFFSET;
    const size_t tb = attn_fwd_rope_workspace_bytes(Tk, d_head);
    if (!workspace || ws_bytes < tb) return ROCATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ROCATTN_ERR_ALIGN;
    const size_t qb = (size_t)count4(B, Hq, Tq, d_head) * 2, kvb = (size_t)count4(B, Hkv, Tk, d_head) * 2;
    const size_t lb = lse ? (size_t)B * Hq * Tq * sizeof(float) : 0;
    // k is rotated in place: it shares no byte with q or v (o and lse were
    // checked against it); the table shares none with any operand
    if (overlaps(k, kvb, q, qb) || overlaps(k, kvb, v, kvb)) return ROCATTN_ERR_SHAPE;
    if (overlaps(workspace, tb, q, qb) || overlaps(workspace, tb, k, kvb) ||
        overlaps(workspace, tb, v, kvb) || overlaps(workspace, tb, o, qb) ||
        (lse && overlaps(workspace, tb, lse, lb)))
        return ROCATTN_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* tab = static_cast<float*>(workspace);
    hipError_t e = rocattn::launch_rope(k, (long long)B * Hkv, Tk, d_head, 0, rope_base, dtype,
                                        pairing, s, tab);
    if (e != hipSuccess) return ROCATTN_ERR_HIP;
    FwdParams p = make_params(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d_head, scale, causal, q_offset);
    p.rope_tab = tab;
    p.rope_adj = pairing;
    p.rope_pos0 = q_offset;
    // the prefill kernel for every Tq (the split-K decode kernels do not rotate)
    return rocattn::launch_prefill_bf16(p, s) == hipSuccess ? ROCATTN_OK : ROCATTN_ERR_HIP;
}

ROCATTN_API size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d_head,
                                            int dtype) {
    if (dtype != ROCATTN_BF16) return 0;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || Hq % Hkv != 0) return 0;
    if (d_head != 64 && d_head != 128) return 0;
    return rocattn::bwd_workspace_bytes(B, Hq, Tq);
}

ROCATTN_API int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                         int Hq, int Hkv, int Tq, int Tk, int d_head, float scale, int causal,
                         int q_offset, int dtype, void* stream, void* workspace,
                         size_t ws_bytes) {
    if (dtype != ROCATTN_F32 && dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;
    if (dtype != ROCATTN_BF16) return ROCATTN_ERR_DTYPE;   // the gradient kernels are bf16
    if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return ROCATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || d_head <= 0) return ROCATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ROCATTN_ERR_SHAPE;
    if (d_head != 64 && d_head != 128) return ROCATTN_ERR_HEADDIM;
    if (causal && q_offset < 0) return ROCATTN_ERR_OFFSET;
    if (causal && (long long)q_offset + Tq > INT_MAX) return ROCATTN_ERR_OFFSET;
    if (!sizes_fit_int(Tq, Tk)) return ROCATTN_ERR_SHAPE;
    if (!isfinite(scale)) return ROCATTN_ERR_SCALE;
    const void* in[6] = {q, k, v, o, dO, lse};
    void* out[3] = {dq, dk, dv};
    for (const void* x : in)
        if (!aligned16(x)) return ROCATTN_ERR_ALIGN;
    for (const void* x : out)
        if (!aligned16(x)) return ROCATTN_ERR_ALIGN;
    const long long nq = count4(B, Hq, Tq, d_head), nkv = count4(B, Hkv, Tk, d_head);
    if (nq < 0 || nkv < 0) return ROCATTN_ERR_SHAPE;
    if (count4(B, Hq, (Tq + 127) / 128, 1) > INT_MAX || count4(B, Hkv, (Tk + 127) / 128, 1) > INT_MAX)
        return ROCATTN_ERR_SHAPE;
    const size_t wsb = rocattn::bwd_workspace_bytes(B, Hq, Tq);
    if (!workspace || ws_bytes < wsb) return ROCATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ROCATTN_ERR_ALIGN;
    const size_t qb = (size_t)nq * 2, kvb = (size_t)nkv * 2, lb = (size_t)B * Hq * Tq * sizeof(float);
    const size_t inb[6] = {qb, kvb, kvb, qb, qb, lb};
    const size_t outb[3] = {qb, kvb, kvb};
    // outputs and workspace overlap nothing else
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(out[i], outb[i], in[j], inb[j])) return ROCATTN_ERR_SHAPE;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(out[i], outb[i], out[j], outb[j])) return ROCATTN_ERR_SHAPE;
        if (overlaps(out[i], outb[i], workspace, wsb)) return ROCATTN_ERR_SHAPE;
    }
    for (int j = 0; j < 6; ++j)
        if (overlaps(workspace, wsb, in[j], inb[j])) return ROCATTN_ERR_SHAPE;
    rocattn::BwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv; p.workspace = workspace;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Tq = Tq; p.Tk = Tk; p.d = d_head;
    p.scale = scale;
    p.causal = causal ? 1 : 0;
    p.q_offset = clamped_offset(causal, q_offset, Tk);
    return rocattn::launch_bwd_bf16(p, static_cast<hipStream_t>(stream)) == hipSuccess ? ROCATTN_OK
                                                                                        : ROCATTN_ERR_HIP;
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
