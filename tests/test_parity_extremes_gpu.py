"""GPU parity on score distributions far from N(0, 1): keys whose magnitude
grows along the sequence, so that later key tiles lift a row's maximum far
above the earlier ones (the kernels' rescaling of the running sums), keys
whose magnitude shrinks (the later weights underflow to zero), and negative
scales.  Every case compares the HIP path, through the C ABI, with the fp64
oracle on the same bf16 / fp32 arrays.

The softmax of "Transformer" (ai-notes) -- Scaled dot-product attention is
invariant to a shift of a row's logits, so any reference maximum gives the
same result; these inputs make the kernels' choice of that reference matter
numerically.

Bounds.  Outputs: the stated 1e-5 (fp32) and 1.5e-2 (bf16), with values
drawn N(0, 1) -- the sigma of the workloads -- and N(0, 0.5^2) -- that of the
long-context workload.  Two roundings make up the bf16 error of a peaked
row: each bf16 weight carries a relative error of at most 2^-8, which moves
the output by at most 2^-8 times the spread of the values it mixes (about
4e-3 on these rows), and the output itself is rounded to bf16 (half a unit
in the last place: up to 7.8e-3 below 4 in magnitude and 1.56e-2 in [4, 8),
where N(0, 1) values of peaked rows land now and then).  In [4, 8) bf16
numbers are 2^-5 apart, so an exact output there can lie more than 1.5e-2
from every bf16 number (e.g. -4.10961 between -4.125 and -4.09375): no bf16
result meets the bound for it.  Such an element must instead be one of the
two bf16 numbers that bracket the exact value (a faithful rounding: error
below one unit in the last place); every element below 4 in magnitude is
held to 1.5e-2 without exception.  Log-sum-exp (bf16):
the row sum is a sum of the rounded weights, so when one weight dominates
it carries that weight's rounding whole: |error| <= ln(1 + 2^-8) = 3.9e-3,
plus float32 rounding; 4e-3.
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


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def graded(B, Hq, Hkv, Tq, Tk, d, dtype, seed, lo, hi, v_sigma=0.5):
    """q ~ N(0, 1), v ~ N(0, v_sigma^2); key j ~ N(0, 1) scaled by a factor
    running linearly from lo (first key) to hi (last key); cast to dtype."""
    q, k, v = wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, dtype=torch.float32, seed=seed)
    ramp = torch.linspace(lo, hi, Tk, dtype=torch.float32).view(1, 1, Tk, 1)
    return q.to(dtype), (k * ramp).to(dtype), (v_sigma * v).to(dtype)


V_SIGMAS = [0.5, 1.0]


def attn(q, k, v, scale, causal, qo, ws_bytes=None):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    od = torch.empty_like(qd)
    ws = None
    if ws_bytes:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    lse = torch.empty(q.shape[0], q.shape[1], q.shape[2], dtype=torch.float32, device=DEV)
    ra.attn_fwd_ws(qd, kd, vd, od, ws, lse, scale=scale, causal=causal, q_offset=qo)
    torch.cuda.synchronize()
    return od.cpu(), lse.cpu()


def bf16_ulp(x):
    """Distance between consecutive bf16 numbers around |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_within_contract(got, want, tol):
    """Every element within tol; for bf16 outputs of magnitude >= 4, where
    bf16 numbers are further apart than 2 * tol, a faithful rounding of the
    exact value (error below one bf16 unit in the last place) is accepted."""
    err = np.abs(got - want)
    ok = err <= tol
    if tol >= 1e-3:   # bf16 contract
        big = np.abs(want) >= 4.0
        ok |= big & (err < bf16_ulp(want))
        n_faithful = int(np.count_nonzero(big & (err > tol) & ok))
        if n_faithful:
            print(f"[case] {n_faithful} element(s) with |o| >= 4 held to faithful bf16 rounding "
                  f"(max err {float(err[big].max()):.3e})", flush=True)
    bad = ~ok
    assert not bad.any(), (f"{int(bad.sum())} element(s) outside the contract; max abs err "
                           f"{float(err.max()):.3e} at exact value {float(want[bad].flat[0]):.5f}")
    return float(err.max())


def compare(q, k, v, scale, causal, qo, ws_bytes=None, lse_tol=4e-3):
    got, lse = attn(q, k, v, scale, causal, qo, ws_bytes)
    want, want_lse = oracle.attn(q, k, v, scale, causal=causal, q_offset=qo, return_lse=True)
    g = f64(got)
    assert np.all(np.isfinite(g))
    err = assert_within_contract(g, want, TOL[q.dtype])
    lerr = float(np.max(np.abs(f64(lse) - want_lse)))
    assert lerr <= lse_tol, f"lse max abs err {lerr:.3e}"
    return err


# (B, Hq, Hkv, Tq, Tk, d, causal, q_offset, scale, key ramp lo, hi)
GROWING = [
    (1, 4, 2, 1000, 1000, 64, True, 0, 1.0, 0.2, 3.0),      # scaled logits up to ~24 sigma
    (1, 4, 2, 700, 700, 128, True, 0, 0.5, 0.2, 3.0),
    (1, 2, 2, 300, 900, 64, False, 0, 1.0, 0.1, 4.0),       # no mask
    (2, 4, 1, 257, 257, 128, True, 0, 1.0, 0.5, 2.5),
]


@pytest.mark.parametrize("vs", V_SIGMAS)
@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal,qo,scale,lo,hi", GROWING)
def test_prefill_growing_logits(B, Hq, Hkv, Tq, Tk, d, causal, qo, scale, lo, hi, vs):
    say("prefill growing", B, Hq, Hkv, Tq, Tk, d, causal, qo, scale, lo, hi, vs)
    q, k, v = graded(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16, 700 + Tk, lo, hi, vs)
    compare(q, k, v, scale, causal, qo)


@pytest.mark.parametrize("vs", V_SIGMAS)
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_shrinking_logits(d, vs):
    say("prefill shrinking", d, vs)
    q, k, v = graded(1, 4, 2, 600, 600, d, torch.bfloat16, 710 + d, 3.0, 0.1, vs)
    compare(q, k, v, 1.0, True, 0)


@pytest.mark.parametrize("vs", V_SIGMAS)
@pytest.mark.parametrize("d", [64, 128])
def test_split_prefill_growing_logits(d, vs):
    """A small chunk at the end of a long context, split over the keys
    (each split keeps its own reference maximum; the merge reconciles them)."""
    B, Hq, Hkv, Tq, Tk, qo = 1, 8, 2, 300, 2000, 1700
    nb = ra.attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16)
    assert nb > 0
    say("split prefill growing", d, nb, vs)
    q, k, v = graded(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16, 720 + d, 0.2, 3.0, vs)
    compare(q, k, v, 1.0, True, qo, ws_bytes=nb)


@pytest.mark.parametrize("vs", V_SIGMAS)
@pytest.mark.parametrize("lo,hi", [(0.2, 3.0), (3.0, 0.2)])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_graded_logits(d, lo, hi, vs):
    """One query row over a long cache, split into chunks whose maxima
    differ by tens of units."""
    B, Hq, Hkv, Tk = 2, 8, 2, 3000
    say("decode graded", d, lo, hi, vs)
    q, k, v = graded(B, Hq, Hkv, 1, Tk, d, torch.bfloat16, 730 + d, lo, hi, vs)
    nb = ra.attn_workspace_bytes(B, Hq, Hkv, 1, Tk, d, torch.bfloat16)
    compare(q, k, v, 1.0, True, Tk - 1, ws_bytes=nb)


def test_f32_growing_logits():
    say("f32 growing")
    q, k, v = graded(1, 2, 1, 300, 300, 64, torch.float32, 740, 0.2, 2.0)
    compare(q, k, v, 0.25, True, 0, lse_tol=1e-5)


@pytest.mark.parametrize("dtype,d,Tq", [(torch.bfloat16, 64, 500), (torch.bfloat16, 128, 500),
                                        (torch.float32, 64, 200), (torch.bfloat16, 128, 1)])
def test_negative_scale(dtype, d, Tq):
    """scale < 0 flips the sign of every logit; the pages put no sign on the
    scale, and the oracle applies it as given."""
    say("negative scale", dtype, d, Tq)
    Tk = 800 if Tq == 1 else Tq
    q, k, v = wl.random_qkv(1, 4, 2, Tq, Tk, d, dtype=dtype, seed=750 + d + Tq)
    nb = ra.attn_workspace_bytes(1, 4, 2, Tq, Tk, d, dtype) if Tq == 1 else None
    compare(q, k, v, -(d ** -0.5), True, Tk - Tq, ws_bytes=nb,
            lse_tol=1e-5 if dtype == torch.float32 else 4e-3)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_growing_logits(d):
    """Gradients when the forward rescaled its running sums: the backward
    recomputes the weights from the exported log-sum-exp alone."""
    B, Hq, Hkv, T = 1, 4, 2, 400
    say("bwd growing", d)
    q, k, v = graded(B, Hq, Hkv, T, T, d, torch.bfloat16, 760 + d, 0.2, 2.5, 1.0)
    g = torch.Generator().manual_seed(761 + d)
    dO = torch.randn(B, Hq, T, d, generator=g).to(torch.bfloat16)
    scale = 0.5
    o, lse = attn(q, k, v, scale, True, 0)
    qd, kd, vd, od, gd, lsed = (t.to(DEV) for t in (q, k, v, o, dO, lse))
    dq, dk, dv = ra.attn_bwd(qd, kd, vd, od, gd, lsed, scale=scale, causal=True, q_offset=0)
    torch.cuda.synchronize()
    want = oracle.attn_bwd(q, k, v, dO, scale, causal=True, q_offset=0)
    for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        gg = f64(got)
        assert np.all(np.isfinite(gg))
        err = float(np.max(np.abs(gg - w))) / max(1.0, float(np.max(np.abs(w))))
        assert err <= TOL[torch.bfloat16], f"{name}: relative max err {err:.3e}"
