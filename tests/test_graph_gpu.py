"""HIP-graph capture of the entry points that use a workspace or change
their inputs in place: one call captured into a graph (torch.cuda.graph on
the current stream), replayed three times with eager work and
synchronisation between the replays, must give the eager call's bits every
time.  None of these calls records a memset; the kernels write every
workspace byte they later read.
"""
import pytest
import torch

import transformer_causal_self_amd as ra
from transformer_causal_self_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def replay_matches_eager(fn, outputs, inputs_in_place=(), replays=3):
    saved = [x.clone() for x in inputs_in_place]

    def restore():
        for x, y in zip(inputs_in_place, saved):
            x.copy_(y)

    restore()
    fn()
    torch.cuda.synchronize()
    want = [x.clone() for x in outputs]
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=DEV)
    for r in range(replays):
        restore()
        for x in outputs:
            if not any(x is y for y in inputs_in_place):
                x.fill_(float("nan"))
        scratch.mul_(1.0001)          # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(outputs, want)):
            assert torch.equal(x, y), f"replay {r}: output {i} differs from the eager call"
    del g


def dev(*ts):
    return [t.to(DEV) for t in ts]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,qo", [
    (1, 8, 2, 300, 2000, 64, 1700),     # small prefill split over the keys
    (2, 8, 2, 1, 3000, 128, 2999),      # decode split-K and merge
])
def test_graph_attn_fwd_ws(B, Hq, Hkv, Tq, Tk, d, qo):
    say("graph attn_fwd_ws", B, Hq, Hkv, Tq, Tk, d, qo)
    q, k, v = dev(*wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16, seed=90 + Tq))
    nb = ra.attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    replay_matches_eager(
        lambda: ra.attn_fwd_ws(q, k, v, o, ws, lse, scale=d ** -0.5, causal=True, q_offset=qo),
        [o, lse])


def test_graph_attn_decode_step():
    """RoPE on the new rows, cache append and attention: q and both caches
    change in place, so they are restored before each run."""
    B, Hq, Hkv, Tn, Tmax, pos, d = 2, 8, 2, 1, 2048, 1500, 128
    say("graph attn_decode_step", B, Hq, Hkv, Tn, Tmax, pos, d)
    g = torch.Generator().manual_seed(91)
    q = torch.randn(B, Hq, Tn, d, generator=g).to(torch.bfloat16).to(DEV)
    kn = torch.randn(B, Hkv, Tn, d, generator=g).to(torch.bfloat16).to(DEV)
    vn = torch.randn(B, Hkv, Tn, d, generator=g).to(torch.bfloat16).to(DEV)
    kc = torch.randn(B, Hkv, Tmax, d, generator=g).to(torch.bfloat16).to(DEV)
    vc = torch.randn(B, Hkv, Tmax, d, generator=g).to(torch.bfloat16).to(DEV)
    ws = ra.decode_step_workspace(q, kc)   # zeroed once; every step leaves its counters zero
    o = torch.empty_like(q)
    replay_matches_eager(
        lambda: ra.attn_decode_step(q, kn, vn, kc, vc, pos, o=o, scale=d ** -0.5, workspace=ws),
        [o, q, kc, vc], inputs_in_place=[q, kc, vc])


def test_graph_attn_fwd_rope():
    B, Hq, Hkv, T, d = 1, 8, 2, 700, 128
    say("graph attn_fwd_rope", B, Hq, Hkv, T, d)
    q, k, v = dev(*wl.random_qkv(B, Hq, Hkv, T, T, d, torch.bfloat16, seed=92))
    tab = torch.empty(ra.attn_fwd_rope_workspace_bytes(T, d), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    replay_matches_eager(
        lambda: ra.attn_fwd_rope(q, k, v, o, scale=d ** -0.5, causal=True, workspace=tab),
        [o, k], inputs_in_place=[k])


@pytest.mark.parametrize("d", [64, 128])
def test_graph_attn_bwd(d):
    B, Hq, Hkv, T = 1, 4, 2, 600
    say("graph attn_bwd", d)
    q, k, v = dev(*wl.random_qkv(B, Hq, Hkv, T, T, d, torch.bfloat16, seed=93 + d))
    gen = torch.Generator().manual_seed(94)
    dO = torch.randn(B, Hq, T, d, generator=gen).to(torch.bfloat16).to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=DEV)
    ra.attn_fwd_ws(q, k, v, o, None, lse, scale=d ** -0.5, causal=True)
    nb = ra.attn_bwd_workspace_bytes(B, Hq, Hkv, T, T, d, torch.bfloat16)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    replay_matches_eager(
        lambda: ra.attn_bwd(q, k, v, o, dO, lse, scale=d ** -0.5, causal=True, dq=dq, dk=dk, dv=dv,
                            workspace=ws),
        [dq, dk, dv])


def test_two_streams_concurrently():
    """Calls on two streams at once, each with its own workspace (the split
    decode on one, the small-prefill split on the other), give the bits of
    the same calls made one after another: the library keeps no state shared
    between calls beyond read-only plans."""
    say("two streams")
    qa, ka, va = dev(*wl.random_qkv(2, 8, 2, 1, 3000, 128, torch.bfloat16, seed=95))
    qb, kb, vb = dev(*wl.random_qkv(1, 8, 2, 300, 2000, 64, torch.bfloat16, seed=96))
    na = ra.attn_workspace_bytes(2, 8, 2, 1, 3000, 128, torch.bfloat16)
    nb = ra.attn_workspace_bytes(1, 8, 2, 300, 2000, 64, torch.bfloat16)
    wsa = torch.empty(na, dtype=torch.uint8, device=DEV)
    wsb = torch.empty(nb, dtype=torch.uint8, device=DEV)
    oa, ob = torch.empty_like(qa), torch.empty_like(qb)
    lb = torch.empty(1, 8, 300, dtype=torch.float32, device=DEV)

    def run_a():
        ra.attn_fwd_ws(qa, ka, va, oa, wsa, None, scale=128 ** -0.5, causal=True, q_offset=2999)

    def run_b():
        ra.attn_fwd_ws(qb, kb, vb, ob, wsb, lb, scale=0.125, causal=True, q_offset=1700)

    run_a()
    run_b()
    torch.cuda.synchronize()
    want = [oa.clone(), ob.clone(), lb.clone()]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    for r in range(5):
        for x in (oa, ob, lb):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            for _ in range(3):
                run_a()
        with torch.cuda.stream(sb):
            for _ in range(3):
                run_b()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip((oa, ob, lb), want)):
            assert torch.equal(x, y), f"round {r}: output {i} differs"
