"""GPU parity: the HIP kernels, called through the C ABI, against the fp64
CPU oracle on the same seeded inputs, plus invariants the pages fix.

Tolerances (max |gpu - oracle| over the compared outputs): 1e-5 for float32,
1.5e-2 for bfloat16 with float32 accumulation.  The oracle reads the very
arrays the GPU reads (bf16 widened exactly to float64); end-to-end RoPE cases
rotate on each side with that side's own RoPE.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_self_amd as ra
from transformer_causal_self_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 1.5e-2}
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def gpu(*ts):
    return [t.to(DEV) for t in ts]


def run_attn(q, k, v, scale, causal=True, q_offset=0, lse=False):
    qd, kd, vd = gpu(q, k, v)
    od = torch.empty_like(qd)
    if lse:
        B, Hq, Tq, d = q.shape
        ws_b = ra.attn_workspace_bytes(B, Hq, k.shape[1], Tq, k.shape[2], d, q.dtype)
        ws = torch.empty(max(ws_b, 1), dtype=torch.uint8, device=DEV)
        lsed = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
        ra.attn_fwd_ws(qd, kd, vd, od, ws if ws_b else None, lsed, scale=scale, causal=causal,
                       q_offset=q_offset)
        torch.cuda.synchronize()
        return od.cpu(), lsed.cpu()
    ra.attn_fwd(qd, kd, vd, od, scale=scale, causal=causal, q_offset=q_offset)
    torch.cuda.synchronize()
    return od.cpu()


def check(q, k, v, scale, causal=True, q_offset=0, tol=None):
    got = run_attn(q, k, v, scale, causal, q_offset)
    want = oracle.attn(q, k, v, scale, causal=causal, q_offset=q_offset)
    err = float(np.max(np.abs(f64(got) - want)))
    tol = TOL[q.dtype] if tol is None else tol
    assert np.all(np.isfinite(f64(got)))
    assert err <= tol, f"max abs err {err:.3e} > {tol:.1e}"
    return err


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def rope_tol(want, dtype):
    if dtype == torch.float32:
        return 1e-5
    # one bf16 ulp of the exact result (round-to-nearest of a float32 value
    # that is itself within a few float32 ulps of the exact rotation)
    return np.abs(want) * 2.0 ** -7 + 1e-6


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [2, 6, 64, 128])
@pytest.mark.parametrize("pos0", [0, 4093, 16300])
def test_rope_matches_oracle(dtype, d, pos0):
    say("rope", dtype, d, pos0)
    q, k, _ = wl.random_qkv(2, 4, 2, 37, 37, d, dtype=dtype, seed=10 + d + pos0)
    qd, kd = gpu(q, k)
    ra.rope_apply(qd, kd, pos0=pos0, base=10000.0)
    torch.cuda.synchronize()
    for got, x in ((qd, q), (kd, k)):
        want = oracle.rope(x, pos0=pos0, base=10000.0)
        diff = np.abs(f64(got) - want)
        assert np.all(diff <= rope_tol(want, dtype)), float(diff.max())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [2, 6, 64, 128])
@pytest.mark.parametrize("pos0", [0, 16300])
def test_rope_adjacent_matches_oracle(dtype, d, pos0):
    say("rope adjacent", dtype, d, pos0)
    q, k, _ = wl.random_qkv(2, 4, 2, 37, 37, d, dtype=dtype, seed=20 + d + pos0)
    qd, kd = gpu(q, k)
    ra.rope_apply(qd, kd, pos0=pos0, base=10000.0, pairing="adjacent")
    torch.cuda.synchronize()
    for got, x in ((qd, q), (kd, k)):
        want = oracle.rope(x, pos0=pos0, base=10000.0, pairing="adjacent")
        diff = np.abs(f64(got) - want)
        assert np.all(diff <= rope_tol(want, dtype)), float(diff.max())


def test_rope_adjacent_is_split_half_on_interleaved_channels():
    """Adjacent pairing on channels (x0, y0, x1, y1, ...) equals split-half
    pairing on (x0, x1, ..., y0, y1, ...), bit for bit (same angles, same
    float32 arithmetic per pair)."""
    say("rope adjacent vs split permuted")
    d = 128
    q, _, _ = wl.random_qkv(2, 3, 1, 50, 50, d, dtype=torch.bfloat16, seed=23)
    perm = torch.cat([torch.arange(0, d, 2), torch.arange(1, d, 2)])   # adjacent -> split order
    qa = q.clone().cuda()
    qs = q[..., perm].contiguous().cuda()
    ra.rope_apply(qa, None, pos0=321, pairing="adjacent")
    ra.rope_apply(qs, None, pos0=321, pairing="split")
    torch.cuda.synchronize()
    assert torch.equal(qa[..., perm].cpu(), qs.cpu())


def test_rope_q_only_and_other_base():
    say("rope q only, base 5e5")
    q, k, _ = wl.random_qkv(1, 3, 1, 5, 5, 128, dtype=torch.bfloat16, seed=77)
    qd, kd = gpu(q, k)
    ra.rope_apply(qd, None, pos0=9, base=500000.0)
    torch.cuda.synchronize()
    want = oracle.rope(q, pos0=9, base=500000.0)
    assert np.all(np.abs(f64(qd) - want) <= rope_tol(want, torch.bfloat16))
    assert torch.equal(kd.cpu(), k)  # untouched


def test_rope_position_zero_is_identity():
    say("rope pos 0 identity")
    q, k, _ = wl.random_qkv(1, 2, 2, 1, 1, 64, dtype=torch.bfloat16, seed=5)
    qd, kd = gpu(q, k)
    ra.rope_apply(qd, kd, pos0=0)
    torch.cuda.synchronize()
    assert torch.equal(qd.cpu(), q) and torch.equal(kd.cpu(), k)


def test_rope_full_workload3_shape():
    """Every element of the GQA prefill workload's q and k (positions 0..4095)."""
    w = wl.WORKLOADS[3]
    say("rope full", w.name)
    q, k, _ = wl.inputs(w)
    qd, kd = gpu(q, k)
    ra.rope_apply(qd, kd, pos0=0, base=w.rope_base)
    torch.cuda.synchronize()
    for got, x in ((qd, q), (kd, k)):
        want = oracle.rope(x, pos0=0, base=w.rope_base)
        assert np.all(np.abs(f64(got) - want) <= rope_tol(want, torch.bfloat16))


# --------------------------------------------------------------------------
# float32 path
# --------------------------------------------------------------------------

def test_attn_f32_workload1():
    w = wl.WORKLOADS[1]
    say("f32", w.name)
    q, k, v = wl.inputs(w)
    err = check(q, k, v, w.scale)
    say("max abs err", err)


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal,qo,scale", [
    (2, 4, 2, 100, 100, 64, True, 0, 0.125),
    (1, 6, 3, 37, 200, 128, True, 163, 0.0884),
    (1, 2, 1, 130, 130, 256, True, 0, 0.0625),
    (1, 2, 2, 33, 70, 8, False, 0, 0.35),
    (1, 4, 1, 1, 513, 64, True, 512, 0.125),
    (1, 2, 2, 65, 65, 36, True, 0, -0.2),
    (1, 2, 2, 40, 40, 64, True, 0, 0.0),
])
def test_attn_f32_shapes(B, Hq, Hkv, Tq, Tk, d, causal, qo, scale):
    say("f32", B, Hq, Hkv, Tq, Tk, d, causal, qo, scale)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=torch.float32, seed=Tq + Tk + d)
    check(q, k, v, scale, causal, qo)


# --------------------------------------------------------------------------
# bf16 prefill (MFMA kernel)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal,qo,scale", [
    (2, 4, 2, 300, 300, 64, True, 0, 0.125),        # several tiles + ragged tail
    (1, 8, 2, 257, 257, 128, True, 0, 0.0884),
    (1, 2, 2, 1, 1, 128, True, 0, 0.0884),          # single row / key
    (1, 4, 4, 64, 64, 64, True, 0, 0.125),
    (1, 4, 1, 100, 357, 128, True, 257, 0.0884),    # chunk appended to a cache
    (1, 3, 3, 129, 200, 64, False, 0, 0.125),       # no mask, Tq != Tk
    (2, 16, 16, 128, 128, 64, True, 0, 0.125),      # K/V heads a multiple of 8 (XCD grouping)
    (1, 16, 8, 200, 200, 128, True, 0, 0.0884),
    (1, 2, 1, 150, 150, 64, True, 0, -0.125),       # negative temperature
    (1, 2, 1, 150, 150, 128, True, 0, 0.0),         # scale 0: prefix means
    (1, 2, 2, 190, 190, 128, True, 0, 0.5),         # peaky softmax
    (2, 6, 2, 300, 300, 128, True, 0, 0.0884),      # 3 query heads per K/V head: pairs span K/V heads
    (1, 3, 1, 200, 200, 128, True, 0, 0.0884),      # odd head count: a lone head in the last pair
    (1, 5, 5, 130, 130, 128, True, 0, 0.0884),      # odd head count, one query head per K/V head
    (1, 4, 2, 100, 357, 64, True, 257, 0.125),      # d 64: chunk appended to a cache
    (1, 2, 1, 1000, 1000, 64, True, 0, 0.125),      # d 64: many tiles, ragged last tile
    (1, 2, 1, 70, 1030, 64, False, 0, 0.125),       # d 64: no mask, ragged keys
    (1, 4, 2, 70, 1030, 128, False, 0, 0.0884),     # d 128: no mask, ragged keys
])
def test_attn_bf16_shapes(B, Hq, Hkv, Tq, Tk, d, causal, qo, scale):
    say("bf16", B, Hq, Hkv, Tq, Tk, d, causal, qo, scale)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=torch.bfloat16, seed=B * Tq + Tk + d)
    check(q, k, v, scale, causal, qo)


def test_attn_bf16_workload2_full():
    """GPT-2-small attention shape, every output element."""
    w = wl.WORKLOADS[2]
    say("bf16 full", w.name)
    q, k, v = wl.inputs(w)
    err = check(q, k, v, w.scale)
    say("max abs err", err)


def test_end_to_end_workload3_full():
    """RoPE then GQA causal attention on the B2 Hq32 Hkv8 T4096 d128
    workload, every output element."""
    w = wl.WORKLOADS[3]
    say("rope+attn full", w.name)
    q, k, v = wl.inputs(w)
    qd, kd, vd = gpu(q, k, v)
    ra.rope_apply(qd, kd, pos0=0, base=w.rope_base)
    od = ra.attn_fwd(qd, kd, vd, scale=w.scale)
    torch.cuda.synchronize()
    want = oracle.attn(oracle.rope(q, 0, w.rope_base), oracle.rope(k, 0, w.rope_base), v, w.scale)
    err = float(np.max(np.abs(f64(od) - want)))
    say("max abs err", err)
    assert err <= TOL[torch.bfloat16]


def _workload4_rows(w):
    """Every row of query heads 0, 9, 22 and 31 (K/V heads 0, 2, 5, 7) plus
    256 seeded random rows of every query head."""
    rng = np.random.default_rng(4)
    rows = []
    for hq in (0, 9, 22, 31):
        rows += [(0, hq, i) for i in range(w.Tq)]
    for hq in range(w.Hq):
        rows += [(0, hq, int(i)) for i in rng.integers(0, w.Tq, 256)]
    return np.array(rows)


def test_end_to_end_workload4_sampled():
    """Long-context workload (B1 Hq32 Hkv8 T16384 d128, sigma 0.5) through
    both GPU paths -- attn_fwd_rope (the RoPE pass on k, then the prefill
    that rotates each query row as it loads it: the path the benchmark
    times) and rope_apply then attn_fwd -- against the oracle's fp64 RoPE and
    attention on every row of four query heads (one per K/V head pair) plus
    256 seeded random rows of every head."""
    w = wl.WORKLOADS[4]
    say("rope+attn sampled", w.name)
    q, k, v = wl.inputs(w)
    qd, kd, vd = gpu(q, k, v)
    o_fused = ra.attn_fwd_rope(qd, kd.clone(), vd, scale=w.scale, causal=True, q_offset=0,
                               base=w.rope_base)
    ra.rope_apply(qd, kd, pos0=0, base=w.rope_base)
    o_sep = ra.attn_fwd(qd, kd, vd, scale=w.scale)
    torch.cuda.synchronize()
    rows = _workload4_rows(w)
    qr = oracle.rope(q, 0, w.rope_base)
    kr = oracle.rope(k, 0, w.rope_base)
    want = oracle.attn_rows(qr, kr, v, rows, w.scale)
    for name, o in (("attn_fwd_rope", o_fused), ("rope_apply + attn_fwd", o_sep)):
        got = f64(o)
        assert np.all(np.isfinite(got))
        err = float(np.max(np.abs(got[rows[:, 0], rows[:, 1], rows[:, 2]] - want)))
        say(name, "max abs err over", len(rows), "rows", err)
        assert err <= TOL[torch.bfloat16], (name, err)


def test_end_to_end_workload4_full():
    """The long-context workload on the full tensor (every row of every head,
    about 2.2e12 fp64 FLOPs for the oracle, some 20-30 s on the host's
    cores): attn_fwd_rope -- the path the benchmark times, with its 12-wave
    workgroups -- against the oracle's fp64 RoPE and attention."""
    w = wl.WORKLOADS[4]
    say("rope+attn full", w.name)
    q, k, v = wl.inputs(w)
    qd, kd, vd = gpu(q, k, v)
    o = ra.attn_fwd_rope(qd, kd, vd, scale=w.scale, causal=True, q_offset=0, base=w.rope_base)
    torch.cuda.synchronize()
    got = f64(o)
    del qd, kd, vd, o
    want = oracle.attn(oracle.rope(q, 0, w.rope_base), oracle.rope(k, 0, w.rope_base), v, w.scale)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    say("max abs err over the full tensor", err)
    assert err <= TOL[torch.bfloat16], err


# --------------------------------------------------------------------------
# bf16 decode (split-K kernels)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,Hq,Hkv,Tk,d,causal,qo", [
    (2, 8, 2, 1000, 128, True, 999),
    (3, 4, 4, 37, 64, True, 36),
    (1, 16, 1, 5000, 128, True, 4999),      # 16 query heads per K/V head
    (2, 8, 1, 700, 64, True, 400),          # query earlier than the cache end
    (1, 6, 2, 1, 128, True, 0),             # one cached key
    (4, 8, 8, 300, 128, False, 0),          # no mask
    (1, 2, 1, 20000, 64, True, 19999),      # long cache, few heads: many chunks
    (1, 24, 2, 513, 128, True, 512),        # 12 query heads per K/V head
])
def test_decode_shapes(B, Hq, Hkv, Tk, d, causal, qo):
    say("decode", B, Hq, Hkv, Tk, d, causal, qo)
    q, k, v = wl.random_qkv(B, Hq, Hkv, 1, Tk, d, dtype=torch.bfloat16, seed=Tk + Hq)
    check(q, k, v, 1.0 / math.sqrt(d), causal, qo)


def test_decode_workload5_full():
    """The decode workload (B32 Hq32 Hkv8 Tk8192 d128, RoPE-rotated cache):
    the GPU rotates the cache and the new query rows, then attends with the
    split-K kernels; the oracle rotates with its fp64 RoPE and attends; every
    output element of all 32 sequences is compared."""
    w = wl.WORKLOADS[5]
    say("decode", w.name)
    q, k, v = wl.inputs(w)
    qd, kd, vd = gpu(q, k, v)
    ra.rope_apply(kd, None, pos0=0, base=w.rope_base)
    ra.rope_apply(qd, None, pos0=w.Tk - 1, base=w.rope_base)
    od = ra.attn_fwd(qd, kd, vd, scale=w.scale, causal=True, q_offset=w.q_offset)
    torch.cuda.synchronize()
    got = f64(od)
    qr = oracle.rope(q, w.Tk - 1, w.rope_base)
    kr = oracle.rope(k, 0, w.rope_base)
    want = oracle.attn(qr, kr, v, w.scale, causal=True, q_offset=w.q_offset)
    err = float(np.max(np.abs(got - want)))
    say("max abs err", err)
    assert np.all(np.isfinite(got))
    assert err <= TOL[torch.bfloat16]


# ---- causal offsets far past the keys: every key is visible to every row
#      (the host clamps the offset to Tk before the kernels' 32-bit limit
#      arithmetic, so q_offset + row can no longer wrap)

@pytest.mark.parametrize("dtype,B,Hq,Hkv,Tq,Tk,d", [
    (torch.bfloat16, 1, 4, 2, 2, 64, 128),
    (torch.bfloat16, 1, 4, 2, 300, 700, 64),
    (torch.bfloat16, 2, 8, 2, 1, 300, 128),     # split-K decode
    (torch.float32, 1, 2, 1, 5, 64, 64),
])
def test_causal_offset_near_int_max(dtype, B, Hq, Hkv, Tq, Tk, d):
    qo = 2 ** 31 - 1 - Tq
    say("offset near INT_MAX", dtype, B, Hq, Hkv, Tq, Tk, d, qo)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=dtype, seed=40 + Tq)
    scale = d ** -0.5
    got = run_attn(q, k, v, scale, causal=True, q_offset=qo, lse=True)[0]
    want = oracle.attn(q, k, v, scale, causal=True, q_offset=qo)
    assert np.all(np.isfinite(f64(got)))
    err = float(np.max(np.abs(f64(got) - want)))
    assert err <= TOL[dtype], err
    if dtype == torch.bfloat16 and Tq > 1:   # the same masking as no mask at all
        assert torch.equal(got, run_attn(q, k, v, scale, causal=False))


def test_bwd_causal_offset_near_int_max():
    B, Hq, Hkv, Tq, Tk, d = 1, 4, 2, 70, 200, 64
    qo = 2 ** 31 - 1 - Tq
    say("bwd offset near INT_MAX", qo)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=torch.bfloat16, seed=44)
    dO = wl.random_qkv(B, Hq, Hkv, Tq, 1, d, dtype=torch.bfloat16, seed=45)[0]
    scale = d ** -0.5
    o, lse = run_attn(q, k, v, scale, causal=True, q_offset=qo, lse=True)
    qd, kd, vd, od, gd, lsed = gpu(q, k, v, o, dO, lse)
    grads = ra.attn_bwd(qd, kd, vd, od, gd, lsed, scale=scale, causal=True, q_offset=qo)
    torch.cuda.synchronize()
    want = oracle.attn_bwd(q, k, v, dO, scale, causal=True, q_offset=qo)
    for name, g, w in zip(("dq", "dk", "dv"), grads, want):
        gg = f64(g)
        assert np.all(np.isfinite(gg))
        err = float(np.max(np.abs(gg - w))) / max(1.0, float(np.max(np.abs(w))))
        assert err <= TOL[torch.bfloat16], (name, err)


# --------------------------------------------------------------------------
# invariants fixed by the pages
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_row0_is_v0_bit_exact(dtype, d):
    """Row 0 sees only key 0: its weight is exactly 1 and o_0 = v_0."""
    say("row0", dtype, d)
    q, k, v = wl.random_qkv(2, 8, 2, 150, 150, d, dtype=dtype, seed=3)
    o = run_attn(q, k, v, 1.0 / math.sqrt(d))
    for hq in range(8):
        assert torch.equal(o[:, hq, 0], v[:, hq // 4, 0]), hq


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_causal_prefix_invariance_bit_exact(dtype, d):
    """Changing token t and later leaves the outputs of rows < t bit-identical
    (the page's causality check: logits before the changed token differ by
    exactly 0)."""
    say("prefix invariance", dtype, d)
    T, t = 300, 137
    q, k, v = wl.random_qkv(1, 4, 2, T, T, d, dtype=dtype, seed=8)
    o1 = run_attn(q, k, v, 0.1)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    g = torch.Generator().manual_seed(9)
    for x in (q2, k2, v2):
        x[:, :, t:] = torch.randn(x[:, :, t:].shape, generator=g).to(dtype) * 3
    o2 = run_attn(q2, k2, v2, 0.1)
    assert torch.equal(o1[:, :, :t], o2[:, :, :t])
    assert not torch.equal(o1[:, :, t:], o2[:, :, t:])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_rows_equal_prefill_rows(dtype):
    """Incremental decode (one query at position t over keys 0..t) equals row
    t of the one-shot forward; chunked prefill equals the same rows too."""
    say("decode == prefill", dtype)
    T, d = 260, 128
    q, k, v = wl.random_qkv(1, 8, 2, T, T, d, dtype=dtype, seed=21)
    full = run_attn(q, k, v, 0.0884)
    tol = 1e-5 if dtype == torch.float32 else 2 * TOL[torch.bfloat16]
    for t in (0, 1, 63, 64, 127, 200, 259):
        step = run_attn(q[:, :, t:t + 1], k[:, :, :t + 1], v[:, :, :t + 1], 0.0884, q_offset=t)
        assert float((step[:, :, 0].double() - full[:, :, t].double()).abs().max()) <= tol
    for c0, c1 in ((0, 70), (70, 200), (200, 260)):
        part = run_attn(q[:, :, c0:c1], k[:, :, :c1], v[:, :, :c1], 0.0884, q_offset=c0)
        assert float((part.double() - full[:, :, c0:c1].double()).abs().max()) <= tol


def test_gqa_equals_mha_on_repeat_interleave_bit_exact():
    """Grouped heads read their K/V head by index: the result is bit-identical
    to MHA on K/V expanded with repeat_interleave, and differs from the
    tiled (wrong) expansion."""
    say("gqa == mha")
    q, k, v = wl.random_qkv(2, 8, 2, 200, 200, 128, dtype=torch.bfloat16, seed=31)
    o_gqa = run_attn(q, k, v, 0.0884)
    o_mha = run_attn(q, k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1), 0.0884)
    o_bad = run_attn(q, k.repeat(1, 4, 1, 1), v.repeat(1, 4, 1, 1), 0.0884)
    assert torch.equal(o_gqa, o_mha)
    assert float((o_gqa.double() - o_bad.double()).abs().max()) > 0.1


@pytest.mark.parametrize("dtype,Tq", [(torch.float32, 90), (torch.bfloat16, 300), (torch.bfloat16, 1)])
def test_constant_values_give_constant_output(dtype, Tq):
    """Weights of a row sum to 1, so V = 1 gives O = 1."""
    say("V=1", dtype, Tq)
    q, k, _ = wl.random_qkv(2, 4, 2, Tq, 300, 128, dtype=dtype, seed=41)
    v = torch.ones(2, 2, 300, 128, dtype=dtype)
    o = run_attn(q, k, v, 0.0884, q_offset=300 - Tq)
    tol = 1e-6 if dtype == torch.float32 else 2.0 ** -8
    assert float((o.double() - 1.0).abs().max()) <= tol


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_softmax_worked_example(dtype, d):
    """softmax([2, 1, 0]) ~ [0.665, 0.245, 0.090]: with v_j = e_j the output
    row is the weight row."""
    say("worked example", dtype, d)
    q = torch.zeros(1, 1, 3, d); k = torch.zeros(1, 1, 3, d); v = torch.zeros(1, 1, 3, d)
    q[0, 0, 2, 0] = 1.0
    for j, s in enumerate((2.0, 1.0, 0.0)):
        k[0, 0, j, 0] = s
        v[0, 0, j, j] = 1.0
    o = run_attn(q.to(dtype), k.to(dtype), v.to(dtype), 1.0)
    w = o[0, 0, 2, :3].double().numpy()
    tol = 5e-4 + (1e-5 if dtype == torch.float32 else 2.0 ** -8)
    assert np.all(np.abs(w - np.array([0.665, 0.245, 0.090])) <= tol), w


@pytest.mark.parametrize("dtype,Tq,Tk,qo", [(torch.float32, 100, 100, 0), (torch.bfloat16, 300, 300, 0),
                                            (torch.bfloat16, 1, 3000, 2999),
                                            (torch.bfloat16, 50, 250, 200)])
def test_lse_matches_oracle(dtype, Tq, Tk, qo):
    say("lse", dtype, Tq, Tk, qo)
    q, k, v = wl.random_qkv(1, 8, 2, Tq, Tk, 128, dtype=dtype, seed=51)
    o, lse = run_attn(q, k, v, 0.0884, q_offset=qo, lse=True)
    want_o, want_lse = oracle.attn(q, k, v, 0.0884, q_offset=qo, return_lse=True)
    assert float(np.max(np.abs(f64(o) - want_o))) <= TOL[dtype]
    # bf16: the row sum adds the bf16-rounded weights that also feed the P.V
    # product (V = 1 gives O = 1), each within a relative 2^-8 (bf16 keeps 8
    # significant bits) of the exact weight, so ln(sum) moves by at most
    # ln(1 + 2^-8) = 3.9e-3, reached when one weight dominates the row.
    lse_tol = 1e-4 if dtype == torch.float32 else 4.0e-3
    assert float(np.max(np.abs(lse.double().numpy() - want_lse))) <= lse_tol


def test_bf16_deterministic():
    say("determinism")
    q, k, v = wl.random_qkv(2, 8, 2, 333, 333, 128, dtype=torch.bfloat16, seed=61)
    a = run_attn(q, k, v, 0.0884)
    b = run_attn(q, k, v, 0.0884)
    assert torch.equal(a, b)
    qd, kd, vd = wl.random_qkv(4, 8, 2, 1, 4000, 128, dtype=torch.bfloat16, seed=62)
    assert torch.equal(run_attn(qd, kd, vd, 0.0884, q_offset=3999),
                       run_attn(qd, kd, vd, 0.0884, q_offset=3999))


@pytest.mark.parametrize("Tq", [1, 300])
def test_bound_calls_repeat_the_plain_calls(Tq):
    """A Bound call (arguments marshalled once) launches the very work the
    plain call does, each time it is called."""
    say(f"bound calls Tq={Tq}")
    q, k, v = wl.random_qkv(2, 8, 2, Tq, 700, 128, dtype=torch.bfloat16, seed=73)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    qo = 700 - Tq
    nb = ra.attn_workspace_bytes(2, 8, 2, Tq, 700, 128, torch.bfloat16)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    want = torch.empty_like(qd)
    ra.attn_fwd_ws(qd, kd, vd, want, ws, None, 0.0884, True, qo)
    o = torch.full_like(qd, float("nan"))
    call = ra.bind_attn_fwd_ws(qd, kd, vd, o, ws, None, 0.0884, True, qo)
    for _ in range(3):
        o.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        assert torch.equal(o, want)
    # RoPE in place: two bound calls rotate twice, like two plain calls
    k2 = kd.clone()
    ra.rope_apply(k2, None, pos0=5)
    ra.rope_apply(k2, None, pos0=5)
    k3 = kd.clone()
    rot = ra.bind_rope_apply(k3, None, pos0=5)
    rot()
    rot()
    torch.cuda.synchronize()
    assert torch.equal(k2, k3)


def test_decode_with_caller_workspace_matches_internal():
    say("decode ws vs internal")
    q, k, v = wl.random_qkv(4, 16, 4, 1, 3000, 128, dtype=torch.bfloat16, seed=71)
    a = run_attn(q, k, v, 0.0884, q_offset=2999)
    b, _ = run_attn(q, k, v, 0.0884, q_offset=2999, lse=True)
    assert torch.equal(a, b)


# ---- strided layouts (attn_fwd_strided): the kernels read and write rows at
#      any batch / head / token strides; the values must equal the dense call
#      bit for bit, and the oracle within the tolerance.

def _dense_and_strided(q, k, v, scale, causal, q_offset, make_views, lse=False):
    """GPU result on dense tensors and on the strided views make_views builds
    (it returns q, k, v views holding the same values, and an output view)."""
    qd, kd, vd = gpu(q, k, v)
    B, Hq, Tq, d = q.shape
    # only the workspace a call requires (a decode step's): with the optional
    # one a small dense prefill splits over the keys and a strided one does
    # not, and the two then round differently
    nb = ra.attn_workspace_bytes(B, Hq, k.shape[1], Tq, k.shape[2], d, q.dtype) if Tq == 1 else 0
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV) if nb else None
    want = torch.empty_like(qd)
    lw = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV) if lse else None
    ra.attn_fwd_ws(qd, kd, vd, want, ws, lw, scale, causal, q_offset)
    qs, ks, vs, os_ = make_views(qd, kd, vd)
    os_.fill_(float("nan"))
    lg = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV) if lse else None
    ra.attn_fwd_ws(qs, ks, vs, os_, ws, lg, scale, causal, q_offset)
    torch.cuda.synchronize()
    return want.cpu(), os_.cpu(), (lw.cpu() if lse else None), (lg.cpu() if lse else None)


def _bthd(x):
    """The same values held as [B, T, H, d] memory, viewed as [B, H, T, d]."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("dtype,B,Hq,Hkv,Tq,Tk,d,causal,qo", [
    (torch.bfloat16, 2, 8, 2, 300, 300, 64, True, 0),
    (torch.bfloat16, 1, 8, 4, 257, 257, 128, True, 0),
    (torch.bfloat16, 2, 8, 2, 100, 700, 128, True, 600),
    (torch.bfloat16, 2, 6, 6, 90, 333, 64, False, 0),
    (torch.bfloat16, 3, 16, 4, 1, 2000, 128, True, 1999),   # decode
    (torch.float32, 2, 4, 2, 70, 70, 64, True, 0),
])
def test_bthd_layout_bit_exact(dtype, B, Hq, Hkv, Tq, Tk, d, causal, qo):
    say("bthd", dtype, B, Hq, Hkv, Tq, Tk, d, causal, qo)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=dtype, seed=81)

    def views(qd, kd, vd):
        o = torch.empty(B, Tq, Hq, d, dtype=dtype, device=DEV).transpose(1, 2)
        return _bthd(qd), _bthd(kd), _bthd(vd), o

    scale = d ** -0.5
    want, got, lw, lg = _dense_and_strided(q, k, v, scale, causal, qo, views, lse=True)
    assert torch.equal(got, want)
    assert torch.equal(lg, lw)
    err = float(np.max(np.abs(f64(got) - oracle.attn(q, k, v, scale, causal=causal,
                                                      q_offset=qo))))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("Tq,Tk,qo", [(512, 512, 0), (1, 1500, 1499), (64, 1000, 936)])
def test_fused_qkv_views_bit_exact(Tq, Tk, qo):
    """q, k and v sliced from one [B, T, Hq + 2 Hkv, d] buffer (a fused
    projection), output written as [B, T, Hq * d]."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    say("fused qkv", Tq, Tk, qo)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=torch.bfloat16, seed=83)

    def views(qd, kd, vd):
        # keys and values live in a cache buffer [B, Tk, 2 Hkv, d]; the new
        # queries in their own [B, Tq, Hq, d] projection output
        kv = torch.empty(B, Tk, 2 * Hkv, d, dtype=torch.bfloat16, device=DEV)
        kv[:, :, :Hkv] = kd.transpose(1, 2)
        kv[:, :, Hkv:] = vd.transpose(1, 2)
        qb = torch.empty(B, Tq, Hq + 8, d, dtype=torch.bfloat16, device=DEV)   # padded heads
        qb[:, :, :Hq] = qd.transpose(1, 2)
        o = torch.empty(B, Tq, Hq * d, dtype=torch.bfloat16, device=DEV)
        o4 = o.view(B, Tq, Hq, d).transpose(1, 2)
        return (qb[:, :, :Hq].transpose(1, 2), kv[:, :, :Hkv].transpose(1, 2),
                kv[:, :, Hkv:].transpose(1, 2), o4)

    want, got, _, _ = _dense_and_strided(q, k, v, 0.0884, True, qo, views)
    assert torch.equal(got, want)


def test_kv_broadcast_over_batch_bit_exact():
    """A zero batch stride shares one K/V across the batch."""
    say("kv broadcast")
    B, Hq, Hkv, T, d = 3, 4, 2, 200, 64
    q, k1, v1 = wl.random_qkv(B, Hq, Hkv, T, T, d, dtype=torch.bfloat16, seed=85)
    k = k1[:1].expand(B, -1, -1, -1).contiguous()
    v = v1[:1].expand(B, -1, -1, -1).contiguous()

    def views(qd, kd, vd):
        return qd, kd[:1].expand(B, -1, -1, -1), vd[:1].expand(B, -1, -1, -1), torch.empty_like(qd)

    want, got, _, _ = _dense_and_strided(q, k, v, 0.125, True, 0, views)
    assert torch.equal(got, want)


# ---- the cached generation step (attn_decode_step): RoPE at cache.pos, cache
#      append along the token axis, attention over the cache

def _rand(shape, dtype, seed, sigma=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sigma).to(dtype)


@pytest.mark.parametrize("dtype,B,Hq,Hkv,Tn,Tmax,pos,d,pairing", [
    (torch.bfloat16, 4, 32, 8, 1, 4096, 3000, 128, "split"),     # decode, split-K kernels
    (torch.bfloat16, 2, 12, 12, 1, 700, 0, 64, "adjacent"),       # first token of a sequence
    (torch.bfloat16, 2, 8, 2, 100, 1000, 500, 64, "split"),       # chunked prefill on a cache
    (torch.bfloat16, 1, 16, 4, 257, 600, 300, 128, "adjacent"),
    (torch.float32, 2, 4, 2, 3, 64, 17, 64, "split"),
])
def test_decode_step_matches_oracle(dtype, B, Hq, Hkv, Tn, Tmax, pos, d, pairing):
    say("decode step", dtype, B, Hq, Hkv, Tn, Tmax, pos, d, pairing)
    q = _rand((B, Hq, Tn, d), dtype, 91)
    kn = _rand((B, Hkv, Tn, d), dtype, 92)
    vn = _rand((B, Hkv, Tn, d), dtype, 93)
    kc = _rand((B, Hkv, Tmax, d), dtype, 94)
    vc = _rand((B, Hkv, Tmax, d), dtype, 95)
    scale = d ** -0.5
    qd, knd, vnd, kcd, vcd = gpu(q, kn, vn, kc, vc)
    o = ra.attn_decode_step(qd, knd, vnd, kcd, vcd, pos, scale=scale, base=10000.0,
                            pairing=pairing)
    torch.cuda.synchronize()
    want_o, want_q, want_kc, want_vc = oracle.decode_step(q, kn, vn, kc, vc, pos, scale,
                                                          base=10000.0, pairing=pairing)
    # q rotated in place; the new cache rows rotated (k) or copied (v); the
    # rest of the caches untouched
    assert np.all(np.abs(f64(qd) - want_q) <= rope_tol(want_q, dtype))
    got_kc, got_vc = kcd.cpu(), vcd.cpu()
    new = slice(pos, pos + Tn)
    assert np.all(np.abs(f64(got_kc[:, :, new]) - want_kc[:, :, new])
                  <= rope_tol(want_kc[:, :, new], dtype))
    assert torch.equal(got_vc[:, :, new], vn)
    for got, old in ((got_kc, kc), (got_vc, vc)):
        assert torch.equal(got[:, :, :pos], old[:, :, :pos])
        assert torch.equal(got[:, :, pos + Tn:], old[:, :, pos + Tn:])
    # the attention reads the GPU-rotated inputs: compare it to the oracle on them
    want = oracle.attn(qd.cpu(), got_kc[:, :, :pos + Tn], got_vc[:, :, :pos + Tn], scale,
                       causal=True, q_offset=pos)
    err = float(np.max(np.abs(f64(o) - want)))
    assert err <= TOL[dtype], err
    # and the end-to-end step to the oracle's own composition (fp64 RoPE,
    # unrounded), at the same contract tolerance
    err2 = float(np.max(np.abs(f64(o) - want_o)))
    say("end to end max abs err", err2)
    assert err2 <= TOL[dtype], err2


@pytest.mark.parametrize("Tn,pos", [(1, 2047), (64, 1000)])
def test_decode_step_equals_unfused_calls_bit_exact(Tn, pos):
    """One attn_decode_step gives the same bits as rope_apply on q and on the
    new keys, copies into the caches, and attention over the cache prefix."""
    say("decode step vs unfused", Tn, pos)
    B, Hq, Hkv, Tmax, d = 2, 16, 4, 2048 + 64, 128
    q = _rand((B, Hq, Tn, d), torch.bfloat16, 101).cuda()
    kn = _rand((B, Hkv, Tn, d), torch.bfloat16, 102).cuda()
    vn = _rand((B, Hkv, Tn, d), torch.bfloat16, 103).cuda()
    kc = _rand((B, Hkv, Tmax, d), torch.bfloat16, 104).cuda()
    vc = _rand((B, Hkv, Tmax, d), torch.bfloat16, 105).cuda()
    q1, kc1, vc1 = q.clone(), kc.clone(), vc.clone()
    o1 = ra.attn_decode_step(q1, kn, vn, kc1, vc1, pos, scale=0.0884)
    q2, k2 = q.clone(), kn.clone()
    ra.rope_apply(q2, None, pos0=pos)
    ra.rope_apply(k2, None, pos0=pos)
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[:, :, pos:pos + Tn] = k2
    vc2[:, :, pos:pos + Tn] = vn
    o2 = ra.attn_fwd(q2, kc2[:, :, :pos + Tn], vc2[:, :, :pos + Tn], scale=0.0884, q_offset=pos)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(kc1, kc2) and torch.equal(vc1, vc2)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("B,Hq,Hkv,Tmax,pos,d,pairing,scale", [
    (32, 32, 8, 8192, 8191, 128, "split", 0.0884),      # the decode workload's step
    (3, 12, 1, 700, 0, 64, "adjacent", 0.125),          # first token, 12 query heads per K/V head
    (2, 16, 1, 3000, 2500, 128, "split", -0.0884),      # 16 per K/V head, negative scale
    (4, 8, 4, 1024, 1023, 64, "split", 0.125),          # 2 per K/V head
    (1, 6, 2, 20000, 19999, 128, "adjacent", 0.0884),   # long cache, few heads: many chunks
    (2, 4, 4, 100, 37, 128, "split", 0.0884),           # one query head per K/V head, short cache
])
def test_one_launch_decode_step(B, Hq, Hkv, Tmax, pos, d, pairing, scale):
    """A one-token attn_decode_step is one launch: the same bits (o, lse, the
    rotated q, both caches) as rope_apply on q and the new key, the cache
    writes and attn_fwd_ws over the cache prefix; its arrival counters are
    back at zero afterwards; o is within the contract of the oracle's
    composition."""
    say("one-launch step", B, Hq, Hkv, Tmax, pos, d, pairing, scale)
    q = _rand((B, Hq, 1, d), torch.bfloat16, 121).cuda()
    kn = _rand((B, Hkv, 1, d), torch.bfloat16, 122).cuda()
    vn = _rand((B, Hkv, 1, d), torch.bfloat16, 123).cuda()
    kc = _rand((B, Hkv, Tmax, d), torch.bfloat16, 124).cuda()
    vc = _rand((B, Hkv, Tmax, d), torch.bfloat16, 125).cuda()
    q0, kc0, vc0 = q.clone(), kc.clone(), vc.clone()
    ws = ra.decode_step_workspace(q, kc)
    lse1 = torch.empty(B, Hq, 1, dtype=torch.float32, device=DEV)
    o1 = ra.attn_decode_step(q, kn, vn, kc, vc, pos, scale=scale, pairing=pairing, workspace=ws, lse=lse1)
    # the same step as separate calls
    q2, k2 = q0.clone(), kn.clone()
    ra.rope_apply(q2, None, pos0=pos, pairing=pairing)
    ra.rope_apply(k2, None, pos0=pos, pairing=pairing)
    kc2, vc2 = kc0.clone(), vc0.clone()
    kc2[:, :, pos:pos + 1] = k2
    vc2[:, :, pos:pos + 1] = vn
    nb = ra.attn_workspace_bytes(B, Hq, Hkv, 1, pos + 1, d, torch.bfloat16)
    ws2 = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(q2)
    lse2 = torch.empty_like(lse1)
    ra.attn_fwd_ws(q2, kc2[:, :, :pos + 1], vc2[:, :, :pos + 1], o2, ws2, lse2, scale=scale, q_offset=pos)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(kc, kc2) and torch.equal(vc, vc2)
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    assert int(ws[-4 * B * Hkv:].count_nonzero()) == 0   # counters left at zero
    want = oracle.decode_step(q0.cpu(), kn.cpu(), vn.cpu(), kc0.cpu(), vc0.cpu(), pos, scale, pairing=pairing)[0]
    err = float(np.max(np.abs(f64(o1) - want)))
    say("max abs err", err)
    assert err <= TOL[torch.bfloat16], err


def test_decode_steps_replay_the_prefill():
    """The pages' KV-cache check ("The Transformer architecture" -- Hands-on):
    a sequence fed one token at a time (then a chunk) through the cached step
    gives the rows of the one-shot causal forward over the rotated sequence."""
    say("decode replay")
    B, Hq, Hkv, T, d, Tmax = 2, 8, 2, 300, 128, 512
    q = _rand((B, Hq, T, d), torch.bfloat16, 111).cuda()
    k = _rand((B, Hkv, T, d), torch.bfloat16, 112).cuda()
    v = _rand((B, Hkv, T, d), torch.bfloat16, 113).cuda()
    qf, kf = q.clone(), k.clone()
    ra.rope_apply(qf, kf, pos0=0)
    full = ra.attn_fwd(qf, kf, v, scale=0.0884)
    kc = torch.zeros(B, Hkv, Tmax, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    ws = ra.decode_step_workspace(q[:, :, :1], kc)   # zeroed once, reused by every one-token step
    outs = []
    for c0, c1 in [(t, t + 1) for t in range(200)] + [(200, 300)]:
        qs = q[:, :, c0:c1].contiguous()
        outs.append(ra.attn_decode_step(qs, k[:, :, c0:c1].contiguous(), v[:, :, c0:c1].contiguous(),
                                        kc, vc, c0, scale=0.0884,
                                        workspace=ws if c1 - c0 == 1 else None))
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2)
    assert torch.equal(kc[:, :, :T], kf) and torch.equal(vc[:, :, :T], v)
    # both GPU results against the oracle's one-shot forward on the rotated
    # sequence (each is within the tolerance; they may differ by one bf16
    # rounding step from each other)
    want = oracle.attn(qf.cpu(), kf.cpu(), v.cpu(), 0.0884)
    for res in (got, full):
        err = float(np.max(np.abs(f64(res) - want)))
        assert err <= TOL[torch.bfloat16], err


# ---- gradients (attn_bwd): the chain rule of the forward, against the
#      oracle's fp64 gradients on the same bf16 inputs and the GPU forward's
#      own o and lse (the oracle recomputes its forward in fp64)
#
# Tolerance: the kernels round P and dS to bf16 (relative 2^-8) before the
# matrix products and the results to bf16, so the error of a gradient entry
# scales with the size of its terms; the bound is the forward's 1.5e-2 taken
# relative to the tensor's largest entry (at least 1).

def _bwd_inputs(B, Hq, Hkv, Tq, Tk, d, seed):
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16, seed=seed)
    dO = _rand((B, Hq, Tq, d), torch.bfloat16, seed + 7)
    return q, k, v, dO


def _gpu_bwd(q, k, v, dO, scale, causal, qo):
    qd, kd, vd, gd = gpu(q, k, v, dO)
    o, lse = run_attn(q, k, v, scale, causal, qo, lse=True)
    od, lsed = gpu(o, lse)
    dq, dk, dv = ra.attn_bwd(qd, kd, vd, od, gd, lsed, scale=scale, causal=causal, q_offset=qo)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _grad_err(got, want):
    g = f64(got)
    assert np.all(np.isfinite(g))
    return float(np.max(np.abs(g - want))) / max(1.0, float(np.max(np.abs(want))))


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal,qo", [
    (1, 4, 2, 300, 300, 64, True, 0),        # GQA, ragged tail of keys and rows
    (1, 4, 2, 300, 300, 128, True, 0),
    (2, 2, 2, 129, 200, 64, False, 0),       # no mask, Tq != Tk
    (1, 2, 2, 129, 200, 128, False, 0),
    (1, 8, 2, 70, 1030, 128, True, 960),     # a chunk at the end of a long context
    (1, 4, 4, 100, 600, 64, True, 500),
    (1, 2, 1, 1, 77, 64, True, 76),          # one query row
    (1, 3, 3, 33, 31, 128, False, 0),        # fewer keys than one tile
    (1, 4, 1, 513, 513, 64, True, 0),        # four query heads per K/V head
])
def test_bwd_matches_oracle(B, Hq, Hkv, Tq, Tk, d, causal, qo):
    say("bwd", B, Hq, Hkv, Tq, Tk, d, causal, qo)
    q, k, v, dO = _bwd_inputs(B, Hq, Hkv, Tq, Tk, d, 200 + Tq)
    scale = d ** -0.5
    got = _gpu_bwd(q, k, v, dO, scale, causal, qo)
    want = oracle.attn_bwd(q, k, v, dO, scale, causal=causal, q_offset=qo)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        err = _grad_err(g, w)
        assert err <= TOL[torch.bfloat16], f"{name}: relative max err {err:.3e}"
    if causal and Tk > qo + Tq:
        # keys past the last visible one get exactly zero
        for g in got[1:]:
            assert not torch.any(g[:, :, qo + Tq:].float() != 0)


def test_bwd_deterministic():
    say("bwd determinism")
    q, k, v, dO = _bwd_inputs(1, 8, 2, 700, 700, 128, 31)
    a = _gpu_bwd(q, k, v, dO, 0.0884, True, 0)
    b = _gpu_bwd(q, k, v, dO, 0.0884, True, 0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_workload2_full():
    """The GPT-2-small-shaped case at full size: dq of the last 64 rows of
    every head against the oracle (a row's dq needs only that row), and the
    column sums the softmax fixes for dk and dv (sum over keys of dk is 0;
    sum over keys of dv equals the sum over rows of dO)."""
    w = wl.WORKLOADS[2]
    say("bwd", w.name)
    q, k, v = wl.inputs(w)
    dO = _rand(q.shape, torch.bfloat16, 2002)
    dq, dk, dv = _gpu_bwd(q, k, v, dO, w.scale, True, 0)
    T = w.Tq
    tail = slice(T - 64, T)
    want_dq, _, _ = oracle.attn_bwd(q[:, :, tail], k, v, dO[:, :, tail], w.scale, causal=True,
                                    q_offset=T - 64)
    assert _grad_err(dq[:, :, tail], want_dq) <= TOL[torch.bfloat16]
    dk64, dv64, dO64 = f64(dk), f64(dv), f64(dO)
    # bf16 rounding of each entry bounds the error of the sums
    bound_k = 2.0 ** -8 * np.abs(dk64).sum(axis=2) + 1e-3
    assert np.all(np.abs(dk64.sum(axis=2)) <= bound_k)
    bound_v = 2.0 ** -8 * (np.abs(dv64).sum(axis=2) + np.abs(dO64).sum(axis=2)) + 1e-3
    assert np.all(np.abs(dv64.sum(axis=2) - dO64.sum(axis=2)) <= bound_v)


# ---- RoPE fused into the attention: attn_fwd_rope rotates k in place and
#      each query row as the kernel loads it

@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal,qo,pairing", [
    (2, 8, 2, 300, 300, 64, True, 0, "split"),
    (1, 8, 2, 300, 300, 128, True, 0, "adjacent"),
    (1, 16, 4, 129, 1000, 128, True, 871, "split"),       # a chunk at the end of a context
    (2, 4, 4, 200, 200, 64, True, 0, "adjacent"),
    (1, 4, 2, 70, 333, 64, False, 50, "split"),           # no mask: positions still q_offset + i
])
def test_attn_fwd_rope_equals_rope_then_attention_bit_exact(B, Hq, Hkv, Tq, Tk, d, causal, qo,
                                                            pairing):
    """One attn_fwd_rope call gives the same bits as rope_apply_ex on q (at
    pos0 = q_offset) and on k (at 0) followed by attn_fwd_ws, leaves q as it
    was and k rotated exactly as rope_apply_ex rotates it; and it agrees with
    the oracle's RoPE followed by its attention."""
    say("attn_fwd_rope", B, Hq, Hkv, Tq, Tk, d, causal, qo, pairing)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16, seed=300 + Tq)
    scale = d ** -0.5
    qd, kd, vd = gpu(q, k, v)
    lse1 = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    o1 = ra.attn_fwd_rope(qd, kd, vd, scale=scale, causal=causal, q_offset=qo, pairing=pairing,
                          lse=lse1)
    q2, k2 = gpu(q, k)
    ra.rope_apply(q2, None, pos0=qo, pairing=pairing)
    ra.rope_apply(k2, None, pos0=0, pairing=pairing)
    o2 = torch.empty_like(q2)
    lse2 = torch.empty_like(lse1)
    ra.attn_fwd_ws(q2, k2, vd, o2, None, lse2, scale=scale, causal=causal, q_offset=qo)
    torch.cuda.synchronize()
    assert torch.equal(qd.cpu(), q)
    assert torch.equal(kd, k2)
    assert torch.equal(o1, o2)
    assert torch.equal(lse1, lse2)
    want = oracle.attn(oracle.rope(q, pos0=qo, pairing=pairing), oracle.rope(k, pos0=0, pairing=pairing),
                       v, scale, causal=causal, q_offset=qo)
    err = float(np.max(np.abs(f64(o1) - want)))
    assert err <= TOL[torch.bfloat16], err


def test_attn_fwd_rope_one_row_matches_oracle():
    """Tq = 1 runs on the prefill kernel with the query-load rotation."""
    say("attn_fwd_rope Tq=1")
    B, Hq, Hkv, Tk, d = 4, 32, 8, 777, 128
    q, k, v = wl.random_qkv(B, Hq, Hkv, 1, Tk, d, torch.bfloat16, seed=77)
    qd, kd, vd = gpu(q, k, v)
    o = ra.attn_fwd_rope(qd, kd, vd, scale=0.0884, q_offset=Tk - 1)
    torch.cuda.synchronize()
    want = oracle.attn(oracle.rope(q, pos0=Tk - 1), oracle.rope(k, pos0=0), v, 0.0884,
                       q_offset=Tk - 1)
    err = float(np.max(np.abs(f64(o) - want)))
    assert err <= TOL[torch.bfloat16], err


def test_attn_fwd_rope_workload3_full():
    """The GQA + RoPE prefill of workload 3 through the fused entry, against
    the oracle on the whole output."""
    w = wl.WORKLOADS[3]
    say("attn_fwd_rope", w.name)
    q, k, v = wl.inputs(w)
    qd, kd, vd = gpu(q, k, v)
    o = ra.attn_fwd_rope(qd, kd, vd, scale=w.scale, causal=True, q_offset=0, base=w.rope_base)
    torch.cuda.synchronize()
    want = oracle.attn(oracle.rope(q, pos0=0, base=w.rope_base), oracle.rope(k, pos0=0, base=w.rope_base),
                       v, w.scale)
    err = float(np.max(np.abs(f64(o) - want)))
    assert err <= TOL[torch.bfloat16], err


@pytest.mark.parametrize("Tk,d,base", [(4096, 128, 10000.0), (1024, 64, 10000.0), (16384, 128, 500000.0)])
def test_rope_angle_table_matches_oracle(Tk, d, base):
    """The float32 (cos, sin) table attn_fwd_rope leaves in its workspace:
    every entry within one float32 ulp of the oracle's (double-precision
    angle, cosine and sine, rounded once), almost all of them equal."""
    say("rope table", Tk, d, base)
    q, k, v = wl.random_qkv(1, 1, 1, 1, Tk, d, torch.bfloat16, seed=9)
    qd, kd, vd = gpu(q, k, v)
    nb = ra.attn_fwd_rope_workspace_bytes(Tk, d)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    ra.attn_fwd_rope(qd, kd, vd, q_offset=Tk - 1, base=base, workspace=ws)
    torch.cuda.synchronize()
    got = ws.cpu().view(torch.float32).numpy().reshape(Tk, d // 2, 2)
    want = oracle.rope_table(Tk, d, 0, base)
    ulp = np.spacing(np.abs(want).astype(np.float32))
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert np.all(diff <= ulp), float(np.max(diff / ulp))
    assert np.mean(got == want) > 0.999


# ---- values of their own width (d_v != d_k)

@pytest.mark.parametrize("dtype,B,Hq,Hkv,Tq,Tk,dk,dv,causal,qo", [
    (torch.bfloat16, 2, 8, 2, 300, 300, 64, 128, True, 0),
    (torch.bfloat16, 1, 8, 4, 300, 300, 128, 64, True, 0),
    (torch.bfloat16, 1, 4, 2, 70, 1030, 128, 64, True, 960),
    (torch.bfloat16, 2, 4, 4, 129, 200, 64, 128, False, 0),
    (torch.bfloat16, 4, 32, 8, 1, 777, 64, 128, True, 776),     # one row: the prefill kernel
    (torch.float32, 1, 4, 2, 100, 100, 64, 32, True, 0),
    (torch.float32, 2, 2, 1, 33, 70, 8, 24, False, 0),
    (torch.float32, 1, 2, 2, 17, 40, 256, 4, True, 23),
])
def test_attn_fwd_dv_matches_oracle(dtype, B, Hq, Hkv, Tq, Tk, dk, dv, causal, qo):
    say("attn_fwd_dv", dtype, B, Hq, Hkv, Tq, Tk, dk, dv, causal, qo)
    q, k, _ = wl.random_qkv(B, Hq, Hkv, Tq, Tk, dk, dtype, seed=400 + Tq)
    v = _rand((B, Hkv, Tk, dv), dtype, 401 + dv)
    scale = dk ** -0.5
    qd, kd, vd = gpu(q, k, v)
    lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    o = ra.attn_fwd_dv(qd, kd, vd, scale=scale, causal=causal, q_offset=qo, lse=lse)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, Hq, Tq, dv)
    want, want_lse = oracle.attn(q, k, v, scale, causal=causal, q_offset=qo, return_lse=True)
    err = float(np.max(np.abs(f64(o) - want)))
    assert err <= TOL[dtype], err
    lse_tol = 1e-4 if dtype == torch.float32 else 4.0e-3
    assert float(np.max(np.abs(f64(lse) - want_lse))) <= lse_tol


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 64), (torch.bfloat16, 128), (torch.float32, 64)])
def test_attn_fwd_dv_equal_widths_is_attn_fwd_bit_exact(dtype, d):
    say("attn_fwd_dv equal widths", dtype, d)
    q, k, v = gpu(*wl.random_qkv(2, 8, 2, 300, 300, d, dtype, seed=41))
    a = ra.attn_fwd_dv(q, k, v, scale=0.1)
    # attn_fwd_ws without a workspace: the kernel attn_fwd_dv runs (attn_fwd
    # itself would split this small prefill over the keys)
    b = ra.attn_fwd_ws(q, k, v, torch.empty_like(q), None, None, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bwd_workload3_full():
    """The GQA shape the bench times the gradients on (B2 Hq32 Hkv8 T4096
    d128, causal): dq of the last 32 rows of every head against the oracle,
    and the softmax's column sums for dk and dv."""
    w = wl.WORKLOADS[3]
    say("bwd", w.name)
    q, k, v = wl.inputs(w)
    dO = _rand(q.shape, torch.bfloat16, 3003)
    dq, dk, dv = _gpu_bwd(q, k, v, dO, w.scale, True, 0)
    T = w.Tq
    tail = slice(T - 32, T)
    want_dq, _, _ = oracle.attn_bwd(q[:, :, tail], k, v, dO[:, :, tail], w.scale, causal=True,
                                    q_offset=T - 32)
    assert _grad_err(dq[:, :, tail], want_dq) <= TOL[torch.bfloat16]
    dk64, dv64, dO64 = f64(dk), f64(dv), f64(dO)
    R = w.Hq // w.Hkv
    dO_grp = dO64.reshape(w.B, w.Hkv, R, T, w.d).sum(axis=2)   # rows of a K/V head's group
    bound_k = 2.0 ** -8 * np.abs(dk64).sum(axis=2) + 1e-3
    assert np.all(np.abs(dk64.sum(axis=2)) <= bound_k)
    bound_v = 2.0 ** -8 * (np.abs(dv64).sum(axis=2) + np.abs(dO_grp).sum(axis=2)) + 1e-3
    assert np.all(np.abs(dv64.sum(axis=2) - dO_grp.sum(axis=2)) <= bound_v)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_attn_fwd_dv_workload3_shape(dk, dv):
    """attn_fwd_dv at the size the bench times it (B2 Hq32 Hkv8 T4096,
    causal): the last 64 rows of every head against the oracle (a row needs
    only its own query), and rows 0 (= v_0, bit for bit)."""
    w = wl.WORKLOADS[3]
    say("attn_fwd_dv full", dk, dv)
    q, k, _ = wl.random_qkv(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, dk, seed=3001)
    _, _, v = wl.random_qkv(w.B, w.Hq, w.Hkv, 1, w.Tk, dv, seed=3002)
    o = ra.attn_fwd_dv(*gpu(q, k, v), scale=dk ** -0.5)
    torch.cuda.synchronize()
    o = o.cpu()
    T = w.Tq
    want = oracle.attn(q[:, :, T - 64:], k, v, dk ** -0.5, q_offset=T - 64)
    err = float(np.max(np.abs(f64(o[:, :, T - 64:]) - want)))
    assert err <= TOL[torch.bfloat16], err
    rep = w.Hq // w.Hkv
    assert torch.equal(o[:, :, 0], v[:, :, 0].repeat_interleave(rep, dim=1))


def test_attn_fwd_rope_workload4_equals_unfused_bit_exact():
    """The fused RoPE prefill at the long-context size the bench steps it on
    (B1 Hq32 Hkv8 T16384 d128) gives the bits of rope_apply then attention
    (whose sampled rows the end-to-end test checks against the oracle)."""
    w = wl.WORKLOADS[4]
    say("attn_fwd_rope", w.name)
    q, k, v = gpu(*wl.inputs(w))
    k1 = k.clone()
    o1 = ra.attn_fwd_rope(q, k1, v, scale=w.scale, base=w.rope_base)
    q2, k2 = q.clone(), k.clone()
    ra.rope_apply(q2, k2, pos0=0, base=w.rope_base)
    o2 = ra.attn_fwd(q2, k2, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2)
    assert torch.equal(o1, o2)


# ---- long dense launches at head size 128 take 12-wave workgroups of 384
#      query rows (one per CU); these shapes cross that threshold (at least
#      1024 such workgroups) with a ragged last tile, GQA and a cache offset

@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,causal,qo", [
    (4, 128, 16, 400, 400, True, 0),      # 2 x 512 workgroups; the second tile holds 16 rows
    (2, 256, 32, 500, 900, True, 400),    # rows at 400.., more keys than rows
    (1, 512, 64, 390, 390, False, 0),     # no mask
    (8, 128, 128, 385, 385, True, 0),     # MHA; the last tile holds one row
    (3, 171, 57, 800, 1000, True, 200),   # B * Hkv not a multiple of 8 (no XCD grouping), 3 heads per K/V head
])
def test_wide_workgroups_match_oracle(B, Hq, Hkv, Tq, Tk, causal, qo):
    say("wide prefill", B, Hq, Hkv, Tq, Tk, causal, qo)
    assert ((Tq + 383) // 384) * B * Hq >= 1024   # the 12-wave path
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, 128, dtype=torch.bfloat16, seed=Tq + Tk + Hq)
    # output and log-sum-exp rows against one oracle pass
    qd, kd, vd = gpu(q, k, v)
    o = torch.empty_like(qd)
    lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    ra.attn_fwd_ws(qd, kd, vd, o, None, lse, scale=128 ** -0.5, causal=causal, q_offset=qo)
    torch.cuda.synchronize()
    want, want_lse = oracle.attn(q, k, v, 128 ** -0.5, causal=causal, q_offset=qo, return_lse=True)
    got = f64(o)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    lerr = float(np.max(np.abs(lse.cpu().double().numpy() - want_lse)))
    say("attn_fwd_ws max abs err", err, "lse", lerr)
    assert err <= TOL[torch.bfloat16], err
    assert lerr <= 4e-3, lerr
    # and the fused RoPE path on the same launch shape (k turned at 0.., query
    # row i at q_offset + i; every query position has a key angle here)
    if (qo if causal else 0) + Tq <= Tk:
        qd, kd, vd = gpu(q, k, v)
        o = ra.attn_fwd_rope(qd, kd, vd, scale=128 ** -0.5, causal=causal, q_offset=qo, base=10000.0)
        torch.cuda.synchronize()
        want = oracle.attn(oracle.rope(q, qo if causal else 0, 10000.0), oracle.rope(k, 0, 10000.0), v,
                           128 ** -0.5, causal=causal, q_offset=qo)
        err = float(np.max(np.abs(f64(o) - want)))
        say("attn_fwd_rope max abs err", err)
        assert err <= TOL[torch.bfloat16], err


# ---- small prefills split over the keys (a workspace of attn_workspace_bytes
#      lets a launch that would leave the chip idle use more workgroups)

@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal,qo", [
    (1, 32, 8, 512, 4096, 128, True, 3584),    # a chunk at the end of a cache
    (1, 8, 2, 300, 2000, 64, True, 1700),
    (1, 4, 4, 129, 1500, 128, False, 0),
    (2, 2, 1, 70, 3000, 64, True, 2930),
    (1, 4, 2, 1000, 1000, 128, True, 0),       # split ranges where early rows see nothing
])
def test_prefill_split_matches_oracle(B, Hq, Hkv, Tq, Tk, d, causal, qo):
    say("prefill split", B, Hq, Hkv, Tq, Tk, d, causal, qo)
    nb = ra.attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16)
    assert nb > 0   # these shapes take the split
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16, seed=500 + Tq)
    qd, kd, vd = gpu(q, k, v)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o1 = torch.empty_like(qd)
    lse1 = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    ra.attn_fwd_ws(qd, kd, vd, o1, ws, lse1, scale=d ** -0.5, causal=causal, q_offset=qo)
    o2 = torch.empty_like(qd)    # no workspace: one workgroup per query tile
    ra.attn_fwd_ws(qd, kd, vd, o2, None, None, scale=d ** -0.5, causal=causal, q_offset=qo)
    torch.cuda.synchronize()
    want, want_lse = oracle.attn(q, k, v, d ** -0.5, causal=causal, q_offset=qo, return_lse=True)
    for o in (o1, o2):
        err = float(np.max(np.abs(f64(o) - want)))
        assert err <= TOL[torch.bfloat16], err
    assert float(np.max(np.abs(f64(lse1) - want_lse))) <= 4.0e-3


# ---- RoPE with a position per token

@pytest.mark.parametrize("dtype,d,pairing", [(torch.bfloat16, 128, "split"), (torch.bfloat16, 64, "adjacent"),
                                             (torch.float32, 6, "split")])
def test_rope_apply_pos_matches_oracle(dtype, d, pairing):
    say("rope per token", dtype, d, pairing)
    B, Hq, Hkv, T = 3, 8, 2, 37
    q = _rand((B, Hq, T, d), dtype, 61)
    k = _rand((B, Hkv, T, d), dtype, 62)
    pos = torch.from_numpy(np.random.default_rng(63).integers(0, 20000, size=(B, T)).astype(np.int32))
    qd, kd, pd = gpu(q, k, pos)
    ra.rope_apply_pos(qd, kd, pd, pairing=pairing)
    torch.cuda.synchronize()
    for got, x in ((qd, q), (kd, k)):
        want = oracle.rope_positions(x, pos.numpy(), pairing=pairing)
        assert np.all(np.abs(f64(got) - want) <= rope_tol(want, dtype))


def test_rope_apply_pos_consecutive_is_rope_apply_bit_exact():
    """positions[b][t] = pos0_b + t gives rope_apply's bits, sequence by sequence."""
    say("rope per token vs scalar")
    B, Hq, Hkv, T, d = 4, 8, 2, 100, 128
    q = _rand((B, Hq, T, d), torch.bfloat16, 71).cuda()
    k = _rand((B, Hkv, T, d), torch.bfloat16, 72).cuda()
    starts = [0, 17, 4093, 123456]
    pos = torch.tensor([[s + t for t in range(T)] for s in starts], dtype=torch.int32, device=DEV)
    q1, k1 = q.clone(), k.clone()
    ra.rope_apply_pos(q1, k1, pos)
    for b, s in enumerate(starts):
        qb, kb = q[b:b + 1].clone(), k[b:b + 1].clone()
        ra.rope_apply(qb, kb, pos0=s)
        torch.cuda.synchronize()
        assert torch.equal(q1[b:b + 1], qb) and torch.equal(k1[b:b + 1], kb)
