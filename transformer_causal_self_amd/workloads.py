"""Seeded synthetic inputs for the attention hot path.

This module only draws random numbers and names shapes; it holds none of
the method's arithmetic (no attention, no rotation), so both the HIP path's
tests/benchmark and the CPU oracle can take their inputs from it.

Draw recipe (identical for every workload): a CPU ``torch.Generator`` seeded
with the workload's seed draws q, then k, then v, each as float32 standard
normals times ``sigma``; bfloat16 workloads then round each array to bf16
(round-to-nearest-even).  Keys of a cached decode step are raw draws: each
side (library or oracle) rotates them with its own RoPE before attention.

Workloads (shapes of the pages' examples):
  1  f32 causal MHA          B1  H4        T128   d64   scale 1/8
  2  bf16 causal MHA         B8  H12       T1024  d64   scale 1/sqrt(64)
     (GPT-2-small attention: d_model 768 split into 12 heads of 64)
  3  bf16 GQA + RoPE prefill B2  Hq32 Hkv8 T4096  d128  scale 1/sqrt(128)
  4  bf16 GQA + RoPE prefill B1  Hq32 Hkv8 T16384 d128  sigma 0.5
  5  bf16 decode step        B32 Hq32 Hkv8 Tq1 at position Tk-1, Tk8192, d128,
     RoPE-rotated key cache (keys at positions 0..Tk-1)
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    key: int
    name: str
    dtype: str          # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    d: int
    scale: float        # exactly representable in float32 (the value passed to the kernel)
    causal: bool
    q_offset: int
    sigma: float
    rope: bool          # rotate q (positions q_offset..) and k (positions 0..) before attention
    rope_base: float
    seed: int

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def shapes(self):
        return ((self.B, self.Hq, self.Tq, self.d), (self.B, self.Hkv, self.Tk, self.d))


def f32(x: float) -> float:
    """Round a Python float to the nearest float32 value."""
    return float(torch.tensor(x, dtype=torch.float32).item())


WORKLOADS = {
    1: Workload(1, "mha_f32_B1_H4_T128_d64", "f32", 1, 4, 4, 128, 128, 64,
                0.125, True, 0, 1.0, False, 10000.0, 1001),
    2: Workload(2, "mha_bf16_B8_H12_T1024_d64", "bf16", 8, 12, 12, 1024, 1024, 64,
                f32(1.0 / math.sqrt(64)), True, 0, 1.0, False, 10000.0, 1002),
    3: Workload(3, "gqa_rope_bf16_B2_Hq32_Hkv8_T4096_d128", "bf16", 2, 32, 8, 4096, 4096, 128,
                f32(1.0 / math.sqrt(128)), True, 0, 1.0, True, 10000.0, 1003),
    4: Workload(4, "gqa_rope_bf16_B1_Hq32_Hkv8_T16384_d128", "bf16", 1, 32, 8, 16384, 16384, 128,
                f32(1.0 / math.sqrt(128)), True, 0, 0.5, True, 10000.0, 1004),
    5: Workload(5, "decode_bf16_B32_Hq32_Hkv8_Tk8192_d128", "bf16", 32, 32, 8, 1, 8192, 128,
                f32(1.0 / math.sqrt(128)), True, 8191, 1.0, True, 10000.0, 1005),
}


def draw(shape_q, shape_kv, dtype=torch.bfloat16, seed: int = 0, sigma: float = 1.0):
    """q, k, v drawn in that order from one seeded CPU generator."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn(shape_q, generator=g, dtype=torch.float32) * sigma
    k = torch.randn(shape_kv, generator=g, dtype=torch.float32) * sigma
    v = torch.randn(shape_kv, generator=g, dtype=torch.float32) * sigma
    return q.to(dtype), k.to(dtype), v.to(dtype)


def inputs(w: Workload):
    """The workload's raw (unrotated) q, k, v on the CPU."""
    sq, skv = w.shapes()
    return draw(sq, skv, w.torch_dtype, w.seed, w.sigma)


def random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=torch.bfloat16, seed=0, sigma=1.0):
    """Inputs for a parity case of any shape."""
    return draw((B, Hq, Tq, d), (B, Hkv, Tk, d), dtype, seed, sigma)
