"""Python binding of librocattn, the gfx950 causal attention library.

Argument marshalling only: every function here checks that the torch
tensors it is given are device tensors of the right dtype, shape and
layout, takes their pointers and the current HIP stream, and calls the C
ABI declared in ``include/rocattn.h``.  All arithmetic runs in the HIP
kernels; there is no fallback.  When ``librocattn.so`` has not been built,
or a call is made with CPU tensors, the call raises.

    attn_fwd(q, k, v, o=None, scale=None, causal=True, q_offset=0)
    attn_fwd_ws(q, k, v, o, workspace, lse=None, scale=None, causal=True, q_offset=0)
        (tensors that are views with contiguous rows, e.g. [B, T, H, d] memory
        transposed to [B, H, T, d], go to attn_fwd_strided)
    attn_fwd_noalloc(q, k, v, o, lse=None, scale=None, causal=True, q_offset=0)
        (no workspace, no allocation: the library's fixed device scratch)
    attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d_head, dtype)
    rope_apply(q, k=None, pos0=0, base=10000.0, pairing="split"|"adjacent")
    status_string(code)
    attn_decode_step(q, k_new, v_new, k_cache, v_cache, pos, o=None, scale=None,
                     base=10000.0, pairing="split", workspace=None, lse=None)
    attn_fwd_dv(q, k, v, o=None, scale=None, ...) -> o   (v of another width)
    attn_fwd_rope(q, k, v, o=None, ..., base=10000.0, pairing="split") -> o
    attn_bwd(q, k, v, o, dO, lse, scale=None, causal=True, q_offset=0) -> (dq, dk, dv)
    bind_attn_fwd_ws(...), bind_rope_apply(...), bind_attn_decode_step(...),
    bind_attn_fwd_rope(...), bind_attn_bwd(...) -> Bound

A Bound is one of these calls with its arguments checked and marshalled
once: calling it launches the same work again on the stream it was bound
to, with only the C call left in Python (for launch loops whose kernels are
shorter than the argument checks).
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "librocattn.so")

# the C ABI, as declared in include/rocattn.h
SYMBOLS = ("attn_fwd", "attn_fwd_ws", "attn_fwd_noalloc", "attn_fwd_strided", "attn_workspace_bytes",
           "rope_apply", "rope_apply_ex", "rope_apply_pos", "attn_decode_step", "attn_fwd_dv", "attn_fwd_rope",
           "attn_fwd_rope_workspace_bytes", "attn_bwd", "attn_decode_step_workspace_bytes",
           "attn_bwd_workspace_bytes", "attn_status_string")

F32, BF16 = 0, 1
OK = 0
STATUS = {0: "OK", -1: "ERR_NULL", -2: "ERR_SHAPE", -3: "ERR_DTYPE", -4: "ERR_HEADDIM",
          -5: "ERR_OFFSET", -6: "ERR_SCALE", -7: "ERR_ALIGN", -8: "ERR_WORKSPACE",
          -9: "ERR_HIP"}


class RocattnError(RuntimeError):
    """A librocattn entry point returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def library() -> ctypes.CDLL:
    """The loaded librocattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is missing: build it with `python -m transformer_causal_self_amd.build` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        lib = ctypes.CDLL(LIBRARY)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.attn_fwd.restype = i
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp]
        lib.attn_fwd_ws.restype = i
        lib.attn_fwd_ws.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, vp, sz, vp]
        lib.attn_fwd_noalloc.restype = i
        lib.attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, vp]
        lib.attn_fwd_strided.restype = i
        lib.attn_fwd_strided.argtypes = [vp, vp, vp, vp, ctypes.POINTER(ctypes.c_longlong),
                                         i, i, i, i, i, i, f, i, i, i, vp, vp, sz, vp]
        lib.attn_workspace_bytes.restype = sz
        lib.attn_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        lib.rope_apply.restype = i
        lib.rope_apply.argtypes = [vp, vp, i, i, i, i, i, i, ctypes.c_double, i, vp]
        lib.rope_apply_ex.restype = i
        lib.rope_apply_ex.argtypes = [vp, vp, i, i, i, i, i, i, ctypes.c_double, i, vp, i]
        lib.attn_decode_step.restype = i
        lib.attn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f,
                                         ctypes.c_double, i, i, vp, vp, sz, vp]
        lib.attn_decode_step_workspace_bytes.restype = sz
        lib.attn_decode_step_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        lib.rope_apply_pos.restype = i
        lib.rope_apply_pos.argtypes = [vp, vp, i, i, i, i, i, vp, ctypes.c_double, i, vp, i]
        lib.attn_fwd_dv.restype = i
        lib.attn_fwd_dv.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, vp, vp]
        lib.attn_fwd_rope.restype = i
        lib.attn_fwd_rope.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, ctypes.c_double, i,
                                      i, vp, vp, sz, vp]
        lib.attn_fwd_rope_workspace_bytes.restype = sz
        lib.attn_fwd_rope_workspace_bytes.argtypes = [i, i]
        lib.attn_bwd.restype = i
        lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i,
                                 i, vp, vp, sz]
        lib.attn_bwd_workspace_bytes.restype = sz
        lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_status_string.argtypes = [i]
        _lib = lib
    return _lib


def status_string(code: int) -> str:
    return library().attn_status_string(int(code)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16 only")


def _check_dev(name, t, dtype=None, rows=False):
    """rows=True accepts any strides with contiguous rows (last dimension)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device}); "
                         "there is no CPU implementation")
    if rows:
        if t.dim() == 0 or (t.stride(-1) != 1 and t.shape[-1] > 1):
            raise ValueError(f"{name} must have contiguous rows (last stride 1)")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream(t, stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _fwd_args(q, k, v, o, scale, causal, q_offset, rows=False):
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_dev(n, t, q.dtype, rows)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or o.shape != q.shape:
        raise ValueError("q, o: [B, Hq, Tq, d]; k, v: [B, Hkv, Tk, d]")
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return (B, Hq, Hkv, Tq, Tk, d, float(scale), int(bool(causal)), int(q_offset),
            _dtype_code(q))


def attn_fwd(q, k, v, o=None, scale=None, causal=True, q_offset=0, stream=None):
    """softmax(scale q k^T + M) v on the GPU; returns o ([B, Hq, Tq, d]).
    Views with contiguous rows (e.g. [B, T, H, d] tensors transposed to
    [B, H, T, d]) go through attn_fwd_strided; values of another width than
    the keys go through attn_fwd_dv."""
    import torch
    if v.dim() == 4 and q.dim() == 4 and v.shape[3] != q.shape[3]:
        return attn_fwd_dv(q, k, v, o, scale, causal, q_offset, stream=stream)
    if o is None:
        o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if not all(t.is_contiguous() for t in (q, k, v, o)):
        nb = attn_workspace_bytes(q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2],
                                  q.shape[3], q.dtype)
        ws = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
        return attn_fwd_ws(q, k, v, o, ws, None, scale, causal, q_offset, stream)
    B, Hq, Hkv, Tq, Tk, d, sc, ca, qo, dt = _fwd_args(q, k, v, o, scale, causal, q_offset)
    st = library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, Tq, Tk, d, sc, ca,
                            qo, dt, _stream(q, stream))
    if st != OK:
        raise RocattnError("attn_fwd", st)
    return o


def _fwd_dv_call(q, k, v, o, lse, scale, causal, q_offset, stream):
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_dev(n, t, q.dtype)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be dense (contiguous)")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q: [B, Hq, Tq, d_k]; k: [B, Hkv, Tk, d_k]; v: [B, Hkv, Tk, d_v]")
    B, Hq, Tq, dk = q.shape
    Hkv, Tk, dv = k.shape[1], k.shape[2], v.shape[3]
    if (k.shape[0] != B or k.shape[3] != dk or tuple(v.shape[:3]) != tuple(k.shape[:3])
            or tuple(o.shape) != (B, Hq, Tq, dv)):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}, o {tuple(o.shape)}")
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, Hq, Tq):
            raise ValueError("lse must be [B, Hq, Tq]")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, Tq, Tk, dk, dv, float(scale),
            int(bool(causal)), int(q_offset), _dtype_code(q), _stream(q, stream), _ptr(lse))
    return Bound("attn_fwd_dv", library().attn_fwd_dv, args, (q, k, v, o, lse))


def attn_fwd_dv(q, k, v, o=None, scale=None, causal=True, q_offset=0, lse=None, stream=None):
    """Attention with values of their own width: q, k [.., d_k], v [.., d_v];
    returns o [B, Hq, Tq, d_v] (scale defaults to 1/sqrt(d_k))."""
    import torch
    if o is None:
        o = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=q.device)
    _fwd_dv_call(q, k, v, o, lse, scale, causal, q_offset, stream)()
    return o


def attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d_head, dtype) -> int:
    if not isinstance(dtype, int):
        import torch
        dtype = F32 if dtype == torch.float32 else BF16
    return int(library().attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d_head, dtype))


class Bound:
    """A C-ABI entry point with its arguments marshalled once.  The tensors
    whose pointers it holds are kept alive by it; calling it repeats the
    launch on the stream it was bound to and raises on a non-zero status."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name, fn, args, keep):
        self.name, self.fn, self.args, self.keep = name, fn, args, keep

    def __call__(self):
        st = self.fn(*self.args)
        if st != OK:
            raise RocattnError(self.name, st)


def _attn_fwd_ws_call(q, k, v, o, workspace, lse, scale, causal, q_offset, stream):
    import torch
    dense = all(t is not None and t.is_contiguous() for t in (q, k, v, o))
    B, Hq, Hkv, Tq, Tk, d, sc, ca, qo, dt = _fwd_args(q, k, v, o, scale, causal, q_offset,
                                                      rows=not dense)
    ws_bytes = 0
    if workspace is not None:
        _check_dev("workspace", workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, Hq, Tq):
            raise ValueError("lse must be [B, Hq, Tq]")
    if dense:
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, Tq, Tk, d, sc, ca, qo, dt,
                _stream(q, stream), _ptr(workspace), ws_bytes, _ptr(lse))
        return Bound("attn_fwd_ws", library().attn_fwd_ws, args, (q, k, v, o, workspace, lse))
    strides = (ctypes.c_longlong * 12)(*[st for t in (q, k, v, o) for st in t.stride()[:3]])
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), strides, B, Hq, Hkv, Tq, Tk, d, sc, ca, qo, dt,
            _stream(q, stream), _ptr(workspace), ws_bytes, _ptr(lse))
    return Bound("attn_fwd_strided", library().attn_fwd_strided, args,
                 (q, k, v, o, workspace, lse, strides))


def attn_fwd_noalloc(q, k, v, o, lse=None, scale=None, causal=True, q_offset=0, stream=None):
    """attn_fwd_ws without a workspace argument and without any allocation:
    the library's fixed 64 MiB device scratch buffer of the current device
    serves the split-K partial results (dense tensors only).  Calls that
    overlap on one GPU must not be issued (they share that buffer)."""
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{n} must be dense (contiguous)")
    B, Hq, Hkv, Tq, Tk, d, sc, ca, qo, dt = _fwd_args(q, k, v, o, scale, causal, q_offset)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, Hq, Tq):
            raise ValueError("lse must be [B, Hq, Tq]")
    st = library().attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, Tq, Tk, d, sc, ca, qo, dt,
                                    _stream(q, stream), _ptr(lse))
    if st != OK:
        raise RocattnError("attn_fwd_noalloc", st)
    return o


def attn_fwd_ws(q, k, v, o, workspace=None, lse=None, scale=None, causal=True, q_offset=0,
                stream=None):
    """attn_fwd with a caller-owned workspace (a uint8 GPU tensor, or None when
    attn_workspace_bytes() is 0) and an optional float32 lse [B, Hq, Tq]."""
    _attn_fwd_ws_call(q, k, v, o, workspace, lse, scale, causal, q_offset, stream)()
    return o


def bind_attn_fwd_ws(q, k, v, o, workspace=None, lse=None, scale=None, causal=True, q_offset=0,
                     stream=None) -> Bound:
    """attn_fwd_ws's checks and marshalling now; the launch each time the
    returned Bound is called (on the current stream as of this call when
    stream is None)."""
    return _attn_fwd_ws_call(q, k, v, o, workspace, lse, scale, causal, q_offset, stream)


PAIRING = {"split": 0, "adjacent": 1}


def _rope_call(q, k, pos0, base, stream, pairing="split"):
    if pairing not in PAIRING:
        raise ValueError(f"pairing must be one of {sorted(PAIRING)}")
    _check_dev("q", q)
    if q.dim() != 4:
        raise ValueError("q must be [B, Hq, T, d]")
    B, Hq, T, d = q.shape
    Hkv = 0
    if k is not None:
        _check_dev("k", k, q.dtype)
        if k.dim() != 4 or k.shape[0] != B or k.shape[2] != T or k.shape[3] != d:
            raise ValueError("k must be [B, Hkv, T, d] with q's B, T and d")
        Hkv = k.shape[1]
    args = (_ptr(q), _ptr(k), B, Hq, Hkv, T, d, int(pos0), float(base), _dtype_code(q),
            _stream(q, stream), PAIRING[pairing])
    return Bound("rope_apply_ex", library().rope_apply_ex, args, (q, k))


def rope_apply(q, k=None, pos0=0, base=10000.0, stream=None, pairing="split"):
    """Rotate q (and k) in place by position pos0 + t; pairing "split"
    (channels p, p + d/2) or "adjacent" (channels 2p, 2p + 1)."""
    _rope_call(q, k, pos0, base, stream, pairing)()
    return q, k


def rope_apply_pos(q, k=None, positions=None, base=10000.0, stream=None, pairing="split"):
    """RoPE in place with a position per token: positions is an int32 GPU
    tensor [B, T] (token t of sequence b at positions[b, t])."""
    import torch
    if pairing not in PAIRING:
        raise ValueError(f"pairing must be one of {sorted(PAIRING)}")
    _check_dev("q", q)
    if k is not None:
        _check_dev("k", k, q.dtype)
        if k.dim() != 4 or k.shape[0] != q.shape[0] or tuple(k.shape[2:]) != tuple(q.shape[2:]):
            raise ValueError("k must be [B, Hkv, T, d] with q's B, T and d")
    if positions is None:
        raise ValueError("positions (int32 [B, T]) is required")
    _check_dev("positions", positions, torch.int32)
    B, Hq, T, d = q.shape
    if tuple(positions.shape) != (B, T):
        raise ValueError("positions must be [B, T]")
    st = library().rope_apply_pos(_ptr(q), _ptr(k), B, Hq, k.shape[1] if k is not None else 0, T, d,
                                  _ptr(positions), float(base), _dtype_code(q), _stream(q, stream),
                                  PAIRING[pairing])
    if st != OK:
        raise RocattnError("rope_apply_pos", st)
    return q, k


def bind_rope_apply(q, k=None, pos0=0, base=10000.0, stream=None, pairing="split") -> Bound:
    """rope_apply's checks and marshalling now; the launch (in place, so each
    call rotates again) each time the returned Bound is called."""
    return _rope_call(q, k, pos0, base, stream, pairing)


def _decode_step_call(q, k_new, v_new, k_cache, v_cache, pos, o, scale, base, pairing,
                      workspace, lse, stream):
    import torch
    if pairing not in PAIRING:
        raise ValueError(f"pairing must be one of {sorted(PAIRING)}")
    for n, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                 ("v_cache", v_cache), ("o", o)):
        _check_dev(n, t, q.dtype)
    if q.dim() != 4 or k_new.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q, o: [B, Hq, Tn, d]; k_new, v_new: [B, Hkv, Tn, d]; "
                         "k_cache, v_cache: [B, Hkv, Tmax, d]")
    B, Hq, Tn, d = q.shape
    Hkv, Tmax = k_cache.shape[1], k_cache.shape[2]
    if (tuple(k_new.shape) != (B, Hkv, Tn, d) or tuple(v_new.shape) != (B, Hkv, Tn, d)
            or tuple(k_cache.shape) != (B, Hkv, Tmax, d) or tuple(v_cache.shape) != (B, Hkv, Tmax, d)
            or tuple(o.shape) != tuple(q.shape)):
        raise ValueError("shape mismatch between q, k_new, v_new, the caches and o")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = 0
    if workspace is not None:
        _check_dev("workspace", workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, Hq, Tn):
            raise ValueError("lse must be [B, Hq, Tn]")
    args = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(o), B, Hq,
            Hkv, Tn, Tmax, int(pos), d, float(scale), float(base), PAIRING[pairing],
            _dtype_code(q), _stream(q, stream), _ptr(workspace), ws_bytes, _ptr(lse))
    return Bound("attn_decode_step", library().attn_decode_step, args,
                 (q, k_new, v_new, k_cache, v_cache, o, workspace, lse))


def attn_decode_step(q, k_new, v_new, k_cache, v_cache, pos, o=None, scale=None, base=10000.0,
                     pairing="split", workspace=None, lse=None, stream=None):
    """One cached step: rotate q in place and k_new into k_cache at tokens
    pos.., copy v_new into v_cache there, then attend over cache tokens
    0 .. pos + Tn - 1 (causal, q_offset = pos); returns o.  A workspace of
    attn_decode_step_workspace_bytes(B, Hq, Hkv, Tn, Tmax, d, dtype) bytes is
    needed when that is non-zero; a caller's workspace must start zeroed
    (decode_step_workspace() makes one) and is left reusable.  One is
    allocated (zeroed) here when not given."""
    import torch
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        workspace = decode_step_workspace(q, k_cache)
    _decode_step_call(q, k_new, v_new, k_cache, v_cache, pos, o, scale, base, pairing,
                      workspace, lse, stream)()
    return o


def attn_decode_step_workspace_bytes(B, Hq, Hkv, Tn, Tmax, d_head, dtype) -> int:
    if not isinstance(dtype, int):
        import torch
        dtype = F32 if dtype == torch.float32 else BF16
    return int(library().attn_decode_step_workspace_bytes(int(B), int(Hq), int(Hkv), int(Tn), int(Tmax),
                                                          int(d_head), dtype))


def decode_step_workspace(q, k_cache):
    """A zeroed workspace for attn_decode_step on tensors shaped like q
    ([B, Hq, Tn, d]) and k_cache ([B, Hkv, Tmax, d]), or None when none is
    needed.  It can serve every later step of the same sizes."""
    import torch
    nb = attn_decode_step_workspace_bytes(q.shape[0], q.shape[1], k_cache.shape[1], q.shape[2],
                                          k_cache.shape[2], q.shape[3], q.dtype)
    return torch.zeros(nb, dtype=torch.uint8, device=q.device) if nb else None


def bind_attn_decode_step(q, k_new, v_new, k_cache, v_cache, pos, o, scale=None,
                          base=10000.0, pairing="split", workspace=None, lse=None,
                          stream=None) -> Bound:
    """attn_decode_step's checks and marshalling now; each call of the
    returned Bound repeats the step (rotating q in place again)."""
    return _decode_step_call(q, k_new, v_new, k_cache, v_cache, pos, o, scale, base, pairing,
                             workspace, lse, stream)


def attn_fwd_rope_workspace_bytes(Tk, d_head) -> int:
    return int(library().attn_fwd_rope_workspace_bytes(Tk, d_head))


def _fwd_rope_call(q, k, v, o, workspace, lse, scale, causal, q_offset, base, pairing, stream):
    import torch
    if pairing not in PAIRING:
        raise ValueError(f"pairing must be one of {sorted(PAIRING)}")
    B, Hq, Hkv, Tq, Tk, d, sc, ca, qo, dt = _fwd_args(q, k, v, o, scale, causal, q_offset)
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be dense [B, H, T, d] (contiguous)")
    _check_dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, Hq, Tq):
            raise ValueError("lse must be [B, Hq, Tq]")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, Tq, Tk, d, sc, ca, qo, float(base),
            PAIRING[pairing], dt, _stream(q, stream), _ptr(workspace), ws_bytes, _ptr(lse))
    return Bound("attn_fwd_rope", library().attn_fwd_rope, args, (q, k, v, o, workspace, lse))


def attn_fwd_rope(q, k, v, o=None, scale=None, causal=True, q_offset=0, base=10000.0,
                  pairing="split", workspace=None, lse=None, stream=None):
    """Rotate k in place at positions 0.., then attention with each query row
    rotated at load (position q_offset + i; q itself is left unrotated);
    returns o.  The angle-table workspace is allocated here when not given."""
    import torch
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        nb = attn_fwd_rope_workspace_bytes(k.shape[2], q.shape[3])
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    _fwd_rope_call(q, k, v, o, workspace, lse, scale, causal, q_offset, base, pairing, stream)()
    return o


def bind_attn_fwd_rope(q, k, v, o, workspace, lse=None, scale=None, causal=True, q_offset=0,
                       base=10000.0, pairing="split", stream=None) -> Bound:
    """attn_fwd_rope's checks and marshalling now; each call of the returned
    Bound repeats it (rotating k in place again)."""
    return _fwd_rope_call(q, k, v, o, workspace, lse, scale, causal, q_offset, base, pairing,
                          stream)


def _bwd_call(q, k, v, o, dO, lse, dq, dk, dv, workspace, scale, causal, q_offset, stream):
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq), ("dk", dk),
                 ("dv", dv)):
        _check_dev(n, t, q.dtype)
    _check_dev("lse", lse, torch.float32)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, o, dO, dq: [B, Hq, Tq, d]; k, v, dk, dv: [B, Hkv, Tk, d]")
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if (tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != d
            or any(tuple(t.shape) != tuple(q.shape) for t in (o, dO, dq))
            or any(tuple(t.shape) != tuple(k.shape) for t in (dk, dv))
            or tuple(lse.shape) != (B, Hq, Tq)):
        raise ValueError("shape mismatch between the gradient operands")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = 0
    if workspace is not None:
        _check_dev("workspace", workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            B, Hq, Hkv, Tq, Tk, d, float(scale), int(bool(causal)), int(q_offset), _dtype_code(q),
            _stream(q, stream), _ptr(workspace), ws_bytes)
    return Bound("attn_bwd", library().attn_bwd, args,
                 (q, k, v, o, dO, lse, dq, dk, dv, workspace))


def attn_bwd_workspace_bytes(B, Hq, Hkv, Tq, Tk, d_head, dtype) -> int:
    if not isinstance(dtype, int):
        import torch
        dtype = F32 if dtype == torch.float32 else BF16
    return int(library().attn_bwd_workspace_bytes(B, Hq, Hkv, Tq, Tk, d_head, dtype))


def attn_bwd(q, k, v, o, dO, lse, scale=None, causal=True, q_offset=0, dq=None, dk=None,
             dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of attn_fwd for the upstream gradient dO, from
    the forward's output o and its log-sum-exp rows lse (float32 [B, Hq, Tq])."""
    import torch
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        nb = attn_bwd_workspace_bytes(q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2],
                                      q.shape[3], q.dtype)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    _bwd_call(q, k, v, o, dO, lse, dq, dk, dv, workspace, scale, causal, q_offset, stream)()
    return dq, dk, dv


def bind_attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, workspace, scale=None, causal=True,
                  q_offset=0, stream=None) -> Bound:
    """attn_bwd's checks and marshalling now; the launches at each call."""
    return _bwd_call(q, k, v, o, dO, lse, dq, dk, dv, workspace, scale, causal, q_offset, stream)
