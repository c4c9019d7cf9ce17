"""GPU parity over a seeded random sweep of small shapes: every bf16 and f32
attention entry point on shapes drawn from the edges of what the kernels
support (head counts and GQA ratios, ragged query and key counts, offsets
into a cache, causal or not), each against the fp64 oracle.  The sweep is
deterministic (fixed seed); a failure names its case.
"""
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


def draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = torch.bfloat16 if i % 4 else torch.float32
        d = int(rng.choice([64, 128])) if dtype == torch.bfloat16 else int(rng.choice([8, 36, 64, 100, 128]))
        Hkv = int(rng.integers(1, 4))
        R = int(rng.choice([1, 2, 3, 4, 8]))
        B = int(rng.integers(1, 3))
        causal = bool(rng.integers(0, 4) > 0)
        Tq = int(rng.choice([1, int(rng.integers(2, 40)), int(rng.integers(40, 400))]))
        if causal:
            qo = int(rng.choice([0, int(rng.integers(0, 600))]))
            # keys up to the last row's position, beyond it, or fewer (the
            # last rows then see every key)
            Tk = qo + Tq + int(rng.choice([0, 0, int(rng.integers(0, 50)),
                                           -int(rng.integers(0, qo + Tq))]))
        else:
            qo = 0
            Tk = int(rng.integers(1, 700))
        cases.append((i, dtype, B, Hkv * R, Hkv, Tq, Tk, d, causal, qo))
    return cases


CASES = draw_cases(100, 2024)


@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}" for c in CASES])
def test_sweep(case):
    i, dtype, B, Hq, Hkv, Tq, Tk, d, causal, qo = case
    say("sweep", i, dtype, B, Hq, Hkv, Tq, Tk, d, causal, qo)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=dtype, seed=3000 + i)
    scale = d ** -0.5
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    want, want_lse = oracle.attn(q, k, v, scale, causal=causal, q_offset=qo, return_lse=True)
    lse_tol = 1e-4 if dtype == torch.float32 else 4e-3
    nb = ra.attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, dtype)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    outs = []
    # with the workspace (decode and small prefills split), and for prefills
    # also without it (one workgroup per query tile)
    for use_ws in ([True, False] if Tq > 1 else [True]):
        o = torch.empty_like(qd)
        lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
        ra.attn_fwd_ws(qd, kd, vd, o, ws if (use_ws and nb) else None, lse, scale=scale,
                       causal=causal, q_offset=qo)
        outs.append((use_ws, o, lse))
    o_plain = ra.attn_fwd(qd, kd, vd, scale=scale, causal=causal, q_offset=qo)
    torch.cuda.synchronize()
    for use_ws, o, lse in outs:
        g = o.cpu().double().numpy()
        assert np.all(np.isfinite(g))
        err = float(np.max(np.abs(g - want)))
        assert err <= TOL[dtype], f"workspace={use_ws}: max abs err {err:.3e}"
        lerr = float(np.max(np.abs(lse.cpu().double().numpy() - want_lse)))
        assert lerr <= lse_tol, f"workspace={use_ws}: lse max abs err {lerr:.3e}"
    err = float(np.max(np.abs(o_plain.cpu().double().numpy() - want)))
    assert err <= TOL[dtype], f"attn_fwd: max abs err {err:.3e}"


BF16 = [c for c in CASES if c[1] == torch.bfloat16]


@pytest.mark.parametrize("case", [c for c in BF16 if c[5] > 1], ids=lambda c: f"c{c[0]}")
def test_sweep_fused_rope(case):
    """attn_fwd_rope: k turned in place at positions 0.., each query row at
    q_offset + i as it is loaded; the oracle turns both in fp64 first.
    Query positions past the last key's (q_offset + Tq > Tk) have no angle
    in the table the key pass writes: the call returns ERR_OFFSET."""
    i, dtype, B, Hq, Hkv, Tq, Tk, d, causal, qo = case
    say("sweep fused rope", i, B, Hq, Hkv, Tq, Tk, d, causal, qo)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=dtype, seed=4000 + i)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    if (qo if causal else 0) + Tq > Tk:
        with pytest.raises(ra.RocattnError, match="ERR_OFFSET"):
            ra.attn_fwd_rope(qd, kd, vd, scale=d ** -0.5, causal=causal, q_offset=qo)
        return
    o = ra.attn_fwd_rope(qd, kd, vd, scale=d ** -0.5, causal=causal, q_offset=qo, base=10000.0)
    torch.cuda.synchronize()
    want = oracle.attn(oracle.rope(q, qo, 10000.0), oracle.rope(k, 0, 10000.0), v, d ** -0.5,
                       causal=causal, q_offset=qo)
    err = float(np.max(np.abs(o.cpu().double().numpy() - want)))
    assert err <= TOL[dtype], f"max abs err {err:.3e}"


@pytest.mark.parametrize("case", BF16[::2], ids=lambda c: f"c{c[0]}")
def test_sweep_backward(case):
    """attn_bwd from the forward's own o and lse, against the oracle's
    gradients; bound relative to each gradient's largest entry (at least 1)."""
    i, dtype, B, Hq, Hkv, Tq, Tk, d, causal, qo = case
    say("sweep backward", i, B, Hq, Hkv, Tq, Tk, d, causal, qo)
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=dtype, seed=5000 + i)
    g = torch.Generator().manual_seed(5000 + i)
    dO = torch.randn(B, Hq, Tq, d, generator=g).to(dtype)
    scale = d ** -0.5
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dO))
    nb = ra.attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, dtype)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV) if nb else None
    o = torch.empty_like(qd)
    lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    ra.attn_fwd_ws(qd, kd, vd, o, ws, lse, scale=scale, causal=causal, q_offset=qo)
    dq, dk, dv = ra.attn_bwd(qd, kd, vd, o, gd, lse, scale=scale, causal=causal, q_offset=qo)
    torch.cuda.synchronize()
    want = oracle.attn_bwd(q, k, v, dO, scale, causal=causal, q_offset=qo)
    for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        gg = got.cpu().double().numpy()
        assert np.all(np.isfinite(gg))
        err = float(np.max(np.abs(gg - w))) / max(1.0, float(np.max(np.abs(w))))
        assert err <= TOL[dtype], f"{name}: relative max err {err:.3e}"
