"""Double-precision CPU oracle for causal GQA attention and RoPE.

TEST INFRASTRUCTURE ONLY.  The oracle is loaded by the test suite, by the
smoke check and by the CPU-baseline leg of the benchmark, and by nothing
else: the attention library never imports, links or calls it, and the two
share no code.  The arithmetic lives in ``attn_oracle.c`` (plain C, double
precision, one score row at a time); this module only compiles it with gcc,
widens the caller's arrays exactly to float64 and passes pointers.

Functions (each cites its passage in ``attn_oracle.c``):
    attn(q, k, v, scale, causal=True, q_offset=0, return_lse=False)
    attn_rows(q, k, v, rows, scale, causal=True, q_offset=0)
    rope(x, pos0=0, base=10000.0, pairing="split")
    rope_table(T, d, pos0=0, base=10000.0) -> float32 [T, d/2, 2] (cos, sin)
    rope_positions(x, positions, base=10000.0, pairing="split")   (rope per token)
    attn_bwd(q, k, v, dO, scale, causal=True, q_offset=0) -> (dq, dk, dv)
    decode_step(q, k_new, v_new, k_cache, v_cache, pos, scale, base=10000.0,
                pairing="split")   (a composition of rope and attn)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def compile_library(source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle C source into a shared library with gcc."""
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(os.path.abspath(out)))
    os.close(fd)
    cmd = ["gcc", *CFLAGS, source, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(tmp, out)
    return out


def _as_f64(a) -> np.ndarray:
    """Exact widening of a float32/bfloat16/float64 array (numpy or torch CPU)."""
    if hasattr(a, "detach"):  # torch tensor: bf16 has no numpy dtype, widen in torch
        import torch
        a = a.detach().to("cpu")
        a = a.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


_D = ctypes.POINTER(ctypes.c_double)
_L = ctypes.c_long


class Oracle:
    """Bindings to one compiled copy of ``attn_oracle.c``."""

    def __init__(self, lib_path: str = LIBRARY):
        self.path = lib_path
        lib = ctypes.CDLL(lib_path)
        lib.oracle_attn.restype = ctypes.c_int
        lib.oracle_attn.argtypes = [_D, _D, _D, _D, _D, _L, _L, _L, _L, _L, _L,
                                    ctypes.c_double, ctypes.c_int, _L]
        lib.oracle_attn_dv.restype = ctypes.c_int
        lib.oracle_attn_dv.argtypes = [_D, _D, _D, _D, _D, _L, _L, _L, _L, _L, _L, _L,
                                       ctypes.c_double, ctypes.c_int, _L]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_attn_rows.argtypes = [_D, _D, _D, ctypes.POINTER(ctypes.c_long), _L,
                                         _D, _D, _L, _L, _L, _L, _L, _L,
                                         ctypes.c_double, ctypes.c_int, _L]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [_D, _D, _D, _D, _D, _D, _D, _L, _L, _L, _L, _L, _L,
                                        ctypes.c_double, ctypes.c_int, _L]
        lib.oracle_rope_table.restype = ctypes.c_int
        lib.oracle_rope_table.argtypes = [ctypes.POINTER(ctypes.c_float), _L, _L, _L, ctypes.c_double]
        lib.oracle_rope.restype = ctypes.c_int
        lib.oracle_rope.argtypes = [_D, _L, _L, _L, _L, _L, ctypes.c_double, ctypes.c_int]
        self._lib = lib

    @staticmethod
    def _ptr(a: np.ndarray):
        return a.ctypes.data_as(_D)

    def attn(self, q, k, v, scale: float, causal: bool = True, q_offset: int = 0,
             return_lse: bool = False):
        """o[B,Hq,Tq,dv] (and lse[B,Hq,Tq]) for q[B,Hq,Tq,dk], k[B,Hkv,Tk,dk],
        v[B,Hkv,Tk,dv] (dv may differ from dk)."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, Hq, Tq, dk = q.shape
        _, Hkv, Tk, _ = k.shape
        dv = v.shape[3]
        if k.shape[:3] != v.shape[:3] or k.shape[0] != B or k.shape[3] != dk:
            raise ValueError("shape mismatch")
        o = np.empty((B, Hq, Tq, dv), dtype=np.float64)
        lse = np.empty((B, Hq, Tq), dtype=np.float64) if return_lse else None
        st = self._lib.oracle_attn_dv(self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(o),
                                      self._ptr(lse) if lse is not None else None,
                                      B, Hq, Hkv, Tq, Tk, dk, dv, float(scale), int(bool(causal)),
                                      int(q_offset))
        if st != 0:
            raise ValueError(f"oracle_attn rejected its arguments (status {st})")
        return (o, lse) if return_lse else o

    def attn_rows(self, q, k, v, rows, scale: float, causal: bool = True,
                  q_offset: int = 0, return_lse: bool = False):
        """Selected rows: rows is an (n, 3) integer array of (b, hq, i)."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, Hq, Tq, d = q.shape
        _, Hkv, Tk, _ = k.shape
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n = rows.shape[0]
        o = np.empty((n, d), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64) if return_lse else None
        st = self._lib.oracle_attn_rows(
            self._ptr(q), self._ptr(k), self._ptr(v),
            rows.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), n, self._ptr(o),
            self._ptr(lse) if lse is not None else None,
            B, Hq, Hkv, Tq, Tk, d, float(scale), int(bool(causal)), int(q_offset))
        if st != 0:
            raise ValueError(f"oracle_attn_rows rejected its arguments (status {st})")
        return (o, lse) if return_lse else o

    def attn_bwd(self, q, k, v, dO, scale: float, causal: bool = True, q_offset: int = 0):
        """(dq, dk, dv): gradients of sum(dO * attn(q, k, v)) (attn_oracle.c:
        oracle_attn_bwd, the chain rule of the forward)."""
        q, k, v, dO = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dO)
        B, Hq, Tq, d = q.shape
        _, Hkv, Tk, _ = k.shape
        if k.shape != v.shape or dO.shape != q.shape or k.shape[0] != B or k.shape[3] != d:
            raise ValueError("shape mismatch")
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        st = self._lib.oracle_attn_bwd(self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dO),
                                       self._ptr(dq), self._ptr(dk), self._ptr(dv),
                                       B, Hq, Hkv, Tq, Tk, d, float(scale), int(bool(causal)),
                                       int(q_offset))
        if st != 0:
            raise ValueError(f"oracle_attn_bwd rejected its arguments (status {st})")
        return dq, dk, dv

    def rope(self, x, pos0: int = 0, base: float = 10000.0, pairing: str = "split"):
        """Rotated copy of x[B,H,T,d] (token t at position pos0 + t)."""
        y = _as_f64(x).copy()
        B, H, T, d = y.shape
        pm = {"split": 0, "adjacent": 1}[pairing]
        st = self._lib.oracle_rope(self._ptr(y), B, H, T, d, int(pos0), float(base), pm)
        if st != 0:
            raise ValueError(f"oracle_rope rejected its arguments (status {st})")
        return y

    def rope_table(self, T: int, d: int, pos0: int = 0, base: float = 10000.0):
        """float32 [T, d/2, 2]: (cos, sin) of pair p at position pos0 + t."""
        out = np.zeros((T, d // 2, 2), dtype=np.float32)
        st = self._lib.oracle_rope_table(out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), T, d,
                                         int(pos0), float(base))
        if st != 0:
            raise ValueError(f"oracle_rope_table rejected its arguments (status {st})")
        return out

    def rope_positions(self, x, positions, base: float = 10000.0, pairing: str = "split"):
        """Rotated copy of x[B,H,T,d] with token t of sequence b at position
        positions[b][t]: oracle_rope applied to each token at its own pos0
        (a composition of the function above, no arithmetic of its own)."""
        x = _as_f64(x)
        B, H, T, d = x.shape
        pos = np.asarray(positions, dtype=np.int64).reshape(B, T)
        y = np.empty_like(x)
        for b in range(B):
            for t in range(T):
                y[b:b + 1, :, t:t + 1] = self.rope(np.ascontiguousarray(x[b:b + 1, :, t:t + 1]),
                                                   int(pos[b, t]), base, pairing)
        return y

    def decode_step(self, q, k_new, v_new, k_cache, v_cache, pos, scale, base=10000.0,
                    pairing="split"):
        """One cached generation step, as "The Transformer architecture" --
        Hands-on states it: the Tn new query rows sit at positions pos + i and RoPE
        is sliced from cache.pos, so q and the new keys are rotated at pos + t;
        the new keys and values are written into the caches along the token axis
        at pos ("Transformer Math and Implementation Deep Dive" -- Implementation
        Bugs To Expect: the cache grows along the token axis); then causal
        attention over cache tokens 0 .. pos + Tn - 1 with q_offset = pos.

        Returns (o, q_rot, k_cache', v_cache') in float64 (the caches as copies
        with the new rows written).  Only rope() and attn() do arithmetic."""
        q_rot = self.rope(q, pos0=pos, base=base, pairing=pairing)
        k_rot = self.rope(k_new, pos0=pos, base=base, pairing=pairing)
        kc = _as_f64(k_cache).copy()
        vc = _as_f64(v_cache).copy()
        Tn = q_rot.shape[2]
        kc[:, :, pos:pos + Tn] = k_rot
        vc[:, :, pos:pos + Tn] = _as_f64(v_new)
        o = self.attn(q_rot, kc[:, :, :pos + Tn], vc[:, :, :pos + Tn], scale, causal=True, q_offset=pos)
        return o, q_rot, kc, vc


_default: Oracle | None = None


def _stale() -> bool:
    return (not os.path.exists(LIBRARY)
            or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))


def default() -> Oracle:
    """The oracle built from ``attn_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        if _stale():
            compile_library()
        _default = Oracle(LIBRARY)
    return _default


def attn(*args, **kwargs):
    return default().attn(*args, **kwargs)


def attn_rows(*args, **kwargs):
    return default().attn_rows(*args, **kwargs)


def rope(*args, **kwargs):
    return default().rope(*args, **kwargs)


def rope_table(*args, **kwargs):
    return default().rope_table(*args, **kwargs)


def rope_positions(*args, **kwargs):
    return default().rope_positions(*args, **kwargs)


def attn_bwd(*args, **kwargs):
    return default().attn_bwd(*args, **kwargs)


def decode_step(*args, **kwargs):
    return default().decode_step(*args, **kwargs)


def threads_used() -> int:
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS, else all cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.strip().isdigit():
        return int(env)
    return os.cpu_count() or 1


if __name__ == "__main__":  # pragma: no cover
    print(compile_library(), file=sys.stderr)
