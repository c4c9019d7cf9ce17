"""Compile librocattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc,
and librocattn_calib.so (the matrix-core and streaming microbenchmarks the
benchmark quotes beside the published peaks).

    python -m transformer_causal_self_amd.build

Objects are compiled in parallel into ``_build/`` and linked in place, so
the shared libraries sit next to the Python binding that loads them.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(HERE, "librocattn.so")
SOURCES = ["api.cpp", "attn_f32.hip", "attn_prefill_bf16.hip",
           "attn_decode_bf16.hip", "attn_bwd_bf16.hip", "rope.hip", "noalloc.hip"]
CALIB_LIBRARY = os.path.join(HERE, "librocattn_calib.so")
CALIB_SOURCES = ["calib.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-command-line-argument",
    # keep the compiler away from packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build librocattn")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n" + "\n".join(noise))
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link librocattn.so and librocattn_calib.so;
    returns the attention library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIBRARY)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIBRARY)
    if verbose:
        print(LIBRARY, CALIB_LIBRARY, file=sys.stderr)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
