"""Pins that tie the CPU oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when that oracle disagrees with what the pages print or what mathematics
fixes.  They run against the real oracle (tests/test_oracle_pins.py) and
against deliberately broken copies of it (tests/test_oracle_mutants.py), so
each pin has to be sharp enough that a plausible slip in the oracle fails at
least one of them.

Sources (page title -- section):
  P1 "Transformer Math and Implementation Deep Dive" -- Attention Shapes,
     Attention Equation, Causal Masking, RoPE Intuition.
  P2 "The Transformer architecture" -- Scaled dot-product attention;
     Softmax is a differentiable allocation; Do the three projection
     matrices have any "actual meaning"? (Q -> QR, K -> K R^-T); Now: RoPE;
     What else the modern decoder-only model changed (GQA); Hands-on.
  P3 "Grasping Codes and Math 02" -- Flash Attention (library SDPA call).
  P4 "Transformer" (ai-notes) -- Scaled dot-product attention; RoPE.
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out.setdefault(key, []).append([float(x) for x in vals])
    return out


# --------------------------------------------------------------------------
# attention pins
# --------------------------------------------------------------------------

def pin_softmax_worked_example(orc):
    """P2 Softmax section: softmax([2,1,0]) ~ [0.665, 0.245, 0.090].

    With v_j = e_j the output row is the weight row itself.  Query row 2
    sees keys 0..2 with scores q.k_j = 2, 1, 0 (scale 1)."""
    g = _read_golden("softmax_worked_example.txt")
    scores = g["scores"][0]
    printed = np.array(g["weights"][0])
    tol = 0.5 * 10.0 ** (-g["decimals"][0][0])
    d, T = 8, 3
    q = np.zeros((1, 1, T, d)); k = np.zeros((1, 1, T, d)); v = np.zeros((1, 1, T, d))
    q[0, 0, 2, 0] = 1.0
    for j, s in enumerate(scores):
        k[0, 0, j, 0] = s
        v[0, 0, j, j] = 1.0
    o = orc.attn(q, k, v, 1.0, causal=True)
    w = o[0, 0, 2, :3]
    assert np.all(np.abs(w - printed) <= tol), (w, printed)
    assert np.all(o[0, 0, 2, 3:] == 0.0)


def pin_weights_rows_sum_to_one_and_mask_is_exact_zero(orc):
    """P2 Scaled dot-product attention: every weight row sums to 1.
    P3 Why Fill with Negative Infinity? / P2 (mask goes before the softmax):
    masked keys get exactly zero weight, visible keys positive weight."""
    r = _rng(1)
    d = Tk = 16
    for Tq, q_off, causal in ((16, 0, True), (8, 8, True), (5, 3, True), (7, 0, False)):
        q = r.standard_normal((1, 2, Tq, d)); k = r.standard_normal((1, 2, Tk, d))
        v = np.broadcast_to(np.eye(Tk, d), (1, 2, Tk, d)).copy()
        w = orc.attn(q, k, v, 0.7, causal=causal, q_offset=q_off)
        assert np.all(np.abs(w.sum(-1) - 1.0) < 1e-12)
        for i in range(Tq):
            lim = min(Tk - 1, q_off + i) if causal else Tk - 1
            assert np.all(w[..., i, lim + 1:] == 0.0), (i, lim)
            assert np.all(w[..., i, :lim + 1] > 0.0), (i, lim)


def pin_causal_row0_is_v0_bit_exact(orc):
    """P1 Causal Masking: row 0 sees only key 0, so its weight is exactly 1
    and o_0 = v_0 bit for bit; query head hq reads KV head hq // n_rep
    (P2 GQA: each group of n_rep query heads shares one K/V head)."""
    r = _rng(2)
    B, Hq, Hkv, T, d = 2, 6, 2, 5, 8
    q = r.standard_normal((B, Hq, T, d)); k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    o = orc.attn(q, k, v, 0.35, causal=True)
    for hq in range(Hq):
        assert np.array_equal(o[:, hq, 0, :], v[:, hq // (Hq // Hkv), 0, :]), hq


def pin_qr_invariance(orc):
    """P2 projection-matrix section: replacing Q, K by QR and K R^-T leaves
    the scores, hence the output, unchanged for any invertible R."""
    r = _rng(3)
    B, H, T, d = 1, 2, 12, 8
    q = r.standard_normal((B, H, T, d)); k = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, d))
    u1, _ = np.linalg.qr(r.standard_normal((d, d)))
    u2, _ = np.linalg.qr(r.standard_normal((d, d)))
    R = u1 @ np.diag(r.uniform(0.5, 2.0, d)) @ u2
    Rinv_T = np.linalg.inv(R).T
    o1 = orc.attn(q, k, v, 0.4, causal=True)
    o2 = orc.attn(q @ R, k @ Rinv_T, v, 0.4, causal=True)
    assert np.max(np.abs(o1 - o2)) < 1e-10
    # and the pin is not vacuous: changing K alone does change the output
    o3 = orc.attn(q, k @ R, v, 0.4, causal=True)
    assert np.max(np.abs(o1 - o3)) > 1e-3


def pin_closed_forms(orc):
    """Closed forms of softmax(QK^T scale + M) V (P4 Attn(Q,K,V;M)):
    T=1 gives v_0; T=2, d=1 gives o_1 = sig(s10-s11) v_0 + sig(s11-s10) v_1;
    scale 0 gives the prefix mean of v."""
    r = _rng(4)
    q = r.standard_normal((1, 1, 1, 4)); k = r.standard_normal((1, 1, 1, 4))
    v = r.standard_normal((1, 1, 1, 4))
    for causal in (True, False):
        assert np.array_equal(orc.attn(q, k, v, 0.9, causal=causal), v)
    q = r.standard_normal((1, 1, 2, 1)); k = r.standard_normal((1, 1, 2, 1))
    v = r.standard_normal((1, 1, 2, 1))
    sc = 0.8
    s10, s11 = sc * q[0, 0, 1, 0] * k[0, 0, 0, 0], sc * q[0, 0, 1, 0] * k[0, 0, 1, 0]
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    want = sig(s10 - s11) * v[0, 0, 0, 0] + sig(s11 - s10) * v[0, 0, 1, 0]
    got = orc.attn(q, k, v, sc, causal=True)[0, 0, 1, 0]
    assert abs(got - want) < 1e-14, (got, want)
    T = 9
    q = r.standard_normal((1, 2, T, 4)); k = r.standard_normal((1, 2, T, 4))
    v = r.standard_normal((1, 2, T, 4))
    o = orc.attn(q, k, v, 0.0, causal=True)
    mean = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    assert np.max(np.abs(o - mean)) < 1e-14


def pin_q_equals_k_scores_symmetric_weights_not(orc):
    """P2 (what Q = K does): the pre-softmax scores QQ^T are symmetric but the
    row-wise softmax weights are generally not."""
    r = _rng(5)
    T = d = 6
    x = r.standard_normal((1, 1, T, d))
    v = np.broadcast_to(np.eye(T, d), (1, 1, T, d)).copy()
    w = orc.attn(x, x, v, 0.5, causal=False)[0, 0]
    s = np.log(w) - np.log(w).mean(axis=1, keepdims=True)  # scores up to a row shift
    # row-shifted log weights: s_ij - s_ji = c_i - c_j (rank-one antisymmetry)
    anti = s - s.T
    c = anti[:, 0:1]
    assert np.max(np.abs(anti - (c - c.T))) < 1e-10
    assert np.max(np.abs(w - w.T)) > 1e-3


def pin_torch_sdpa_library(orc):
    """P3 Flash Attention section: the library call
    F.scaled_dot_product_attention computes the same attention.  Checked in
    float64 on the CPU with an explicit boolean mask (key j visible to row i
    iff j <= q_offset + i) and K/V heads expanded by repeat_interleave."""
    import torch
    import torch.nn.functional as F
    r = _rng(6)
    cases = [(2, 4, 2, 7, 7, 8, True, 0), (1, 6, 3, 4, 11, 5, True, 7),
             (2, 2, 1, 3, 9, 4, True, 2), (1, 4, 4, 5, 8, 3, False, 0),
             (1, 8, 2, 1, 13, 16, True, 12)]
    for B, Hq, Hkv, Tq, Tk, d, causal, qo in cases:
        q = r.standard_normal((B, Hq, Tq, d)); k = r.standard_normal((B, Hkv, Tk, d))
        v = r.standard_normal((B, Hkv, Tk, d))
        sc = 1.0 / math.sqrt(d)
        o = orc.attn(q, k, v, sc, causal=causal, q_offset=qo)
        tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
        rep = Hq // Hkv
        tk = tk.repeat_interleave(rep, dim=1); tv = tv.repeat_interleave(rep, dim=1)
        i = torch.arange(Tq)[:, None]; j = torch.arange(Tk)[None, :]
        mask = (j <= qo + i) if causal else torch.ones(Tq, Tk, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=sc)
        assert np.max(np.abs(o - ref.numpy())) < 1e-12, (B, Hq, Hkv, Tq, Tk, d)


def pin_value_width_differs_from_key_width(orc):
    """Values may have their own width d_v ("The Transformer architecture" --
    Scaled dot-product attention: queries and keys share d_k, values d_v).
    Against torch's float64 SDPA, which takes value rows of another width;
    T = 1 returns v_0 whatever d_v; and the output channels of V are
    independent: attention with V = [V1 | V2] is [attn(V1) | attn(V2)]."""
    import torch
    import torch.nn.functional as F
    r = _rng(17)
    for B, Hq, Hkv, Tq, Tk, dk, dv, causal, qo in [(2, 4, 2, 6, 9, 8, 12, True, 3),
                                                   (1, 2, 2, 5, 5, 16, 4, False, 0),
                                                   (1, 8, 2, 1, 13, 6, 10, True, 12)]:
        q = r.standard_normal((B, Hq, Tq, dk)); k = r.standard_normal((B, Hkv, Tk, dk))
        v = r.standard_normal((B, Hkv, Tk, dv))
        sc = 1.0 / math.sqrt(dk)
        o = orc.attn(q, k, v, sc, causal=causal, q_offset=qo)
        assert o.shape == (B, Hq, Tq, dv)
        rep = Hq // Hkv
        tk = torch.from_numpy(k).repeat_interleave(rep, dim=1)
        tv = torch.from_numpy(v).repeat_interleave(rep, dim=1)
        i = torch.arange(Tq)[:, None]; j = torch.arange(Tk)[None, :]
        mask = (j <= qo + i) if causal else torch.ones(Tq, Tk, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), tk, tv, attn_mask=mask, scale=sc)
        assert np.max(np.abs(o - ref.numpy())) < 1e-12
        split = dv // 2
        o1 = orc.attn(q, k, np.ascontiguousarray(v[..., :split]), sc, causal=causal, q_offset=qo)
        o2 = orc.attn(q, k, np.ascontiguousarray(v[..., split:]), sc, causal=causal, q_offset=qo)
        assert np.max(np.abs(np.concatenate([o1, o2], axis=-1) - o)) < 1e-14
    q = r.standard_normal((1, 2, 1, 8)); k = r.standard_normal((1, 1, 1, 8))
    v = r.standard_normal((1, 1, 1, 24))
    o = orc.attn(q, k, v, 0.3)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0]) and np.array_equal(o[0, 1, 0], v[0, 0, 0])


def pin_lse_matches_logsumexp(orc):
    """log of the softmax denominator equals torch.logsumexp of the masked,
    scaled scores (library routine)."""
    import torch
    r = _rng(7)
    B, Hq, Hkv, Tq, Tk, d, qo = 1, 4, 2, 6, 10, 8, 4
    q = r.standard_normal((B, Hq, Tq, d)); k = r.standard_normal((B, Hkv, Tk, d))
    v = r.standard_normal((B, Hkv, Tk, d))
    _, lse = orc.attn(q, k, v, 0.3, causal=True, q_offset=qo, return_lse=True)
    tk = torch.from_numpy(k).repeat_interleave(2, dim=1)
    s = 0.3 * torch.from_numpy(q) @ tk.transpose(-1, -2)
    i = torch.arange(Tq)[:, None]; j = torch.arange(Tk)[None, :]
    s = s.masked_fill(~(j <= qo + i), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


def pin_gqa_equals_mha_on_repeat_interleave(orc):
    """P1 Attention Shapes / P2 GQA: grouped heads equal MHA on K/V heads
    expanded group-wise (repeat_interleave); tiling the heads (repeat) is the
    wrong mapping and must differ (P1 Implementation Bugs: GQA head
    repetition wrong)."""
    r = _rng(8)
    B, Hq, Hkv, T, d = 2, 8, 2, 9, 4
    q = r.standard_normal((B, Hq, T, d)); k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    o = orc.attn(q, k, v, 0.5)
    o_rep = orc.attn(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), 0.5)
    assert np.max(np.abs(o - o_rep)) < 1e-13
    o_tile = orc.attn(q, np.tile(k, (1, Hq // Hkv, 1, 1)), np.tile(v, (1, Hq // Hkv, 1, 1)), 0.5)
    assert np.max(np.abs(o - o_tile)) > 1e-2


def pin_cached_rows_equal_prefill_rows(orc):
    """P2 Hands-on: with a cache, query row i of a step sits at cache.pos + i
    and sees keys 0 .. cache.pos + i; incremental decode equals the one-shot
    forward.  Every chunk of rows computed with q_offset equals the same rows
    of the full causal pass."""
    r = _rng(9)
    B, Hq, Hkv, T, d = 1, 4, 2, 12, 8
    q = r.standard_normal((B, Hq, T, d)); k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    full = orc.attn(q, k, v, 0.3)
    for t in range(T):  # one query at a time over the first t+1 keys
        step = orc.attn(q[:, :, t:t + 1], k[:, :, :t + 1], v[:, :, :t + 1], 0.3, q_offset=t)
        assert np.max(np.abs(step[:, :, 0] - full[:, :, t])) < 1e-14
    for c0, c1 in ((0, 4), (4, 9), (9, 12)):  # chunked prefill
        part = orc.attn(q[:, :, c0:c1], k[:, :, :c1], v[:, :, :c1], 0.3, q_offset=c0)
        assert np.max(np.abs(part - full[:, :, c0:c1])) < 1e-14
    # rows helper agrees with the full pass
    rows = np.array([[0, 0, 0], [0, 3, 11], [0, 2, 5]])
    got = orc.attn_rows(q, k, v, rows, 0.3)
    for n, (b, h, i) in enumerate(rows):
        assert np.array_equal(got[n], full[b, h, i])


def pin_decode_steps_replay_the_prefill(orc):
    """P2 Hands-on: with a cache, query positions start at cache.pos + i, keys
    at 0, RoPE is sliced from cache.pos, and incremental decode matches the
    one-shot forward (the page's kv-cache check).  Feeding a sequence to
    decode_step one token at a time, then a chunk of several, from an empty
    cache reproduces attention over the whole rotated sequence, and leaves
    the rotated keys and the values in the caches in token order (P1
    Implementation Bugs To Expect: the cache grows along the token axis)."""
    r = _rng(14)
    B, Hq, Hkv, T, d, Tmax = 2, 4, 2, 11, 8, 16
    q = r.standard_normal((B, Hq, T, d)); k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    qr, kr = orc.rope(q, 0, 500.0), orc.rope(k, 0, 500.0)
    full = orc.attn(qr, kr, v, 0.4)
    kc = np.full((B, Hkv, Tmax, d), np.nan); vc = np.full((B, Hkv, Tmax, d), np.nan)
    steps = [(t, t + 1) for t in range(7)] + [(7, 11)]   # one token at a time, then a chunk
    for c0, c1 in steps:
        o, q_rot, kc, vc = orc.decode_step(q[:, :, c0:c1], k[:, :, c0:c1], v[:, :, c0:c1],
                                           kc, vc, c0, 0.4, base=500.0)
        assert np.max(np.abs(q_rot - qr[:, :, c0:c1])) < 1e-14
        assert np.max(np.abs(o - full[:, :, c0:c1])) < 1e-13
    assert np.max(np.abs(kc[:, :, :T] - kr)) < 1e-14
    assert np.array_equal(vc[:, :, :T], v)
    assert np.all(np.isnan(kc[:, :, T:])) and np.all(np.isnan(vc[:, :, T:]))


# --------------------------------------------------------------------------
# gradient pins (the backward is the chain rule of the forward; nothing on
# the pages prints it, so it is tied to differences of the forward itself,
# to a library's automatic differentiation, and to two exact invariants)
# --------------------------------------------------------------------------

def _loss(orc, q, k, v, dO, scale, causal, q_offset):
    return float(np.sum(dO * orc.attn(q, k, v, scale, causal=causal, q_offset=q_offset)))


def pin_bwd_central_differences(orc):
    """dL/dx for L = sum(dO * attn(q, k, v)) equals the central difference
    (L(x + h) - L(x - h)) / 2h of the oracle's own forward, element by
    element, for a causal GQA chunk with q_offset and a non-causal case."""
    r = _rng(31)
    for causal, qo, Tq, Tk in ((True, 2, 3, 5), (False, 0, 4, 3)):
        B, Hq, Hkv, d = 1, 4, 2, 3
        q = r.standard_normal((B, Hq, Tq, d)); k = r.standard_normal((B, Hkv, Tk, d))
        v = r.standard_normal((B, Hkv, Tk, d)); dO = r.standard_normal((B, Hq, Tq, d))
        grads = orc.attn_bwd(q, k, v, dO, 0.7, causal=causal, q_offset=qo)
        h = 1e-5
        for x, gx in zip((q, k, v), grads):
            for idx in np.ndindex(x.shape):
                x0 = x[idx]
                x[idx] = x0 + h
                lp = _loss(orc, q, k, v, dO, 0.7, causal, qo)
                x[idx] = x0 - h
                lm = _loss(orc, q, k, v, dO, 0.7, causal, qo)
                x[idx] = x0
                assert abs((lp - lm) / (2 * h) - gx[idx]) < 1e-7, (idx, (lp - lm) / (2 * h), gx[idx])


def pin_bwd_torch_autograd(orc):
    """Automatic differentiation (torch, float64) of the explicit formula
    softmax(scale QK^T + M) V with K/V heads repeat_interleave'd."""
    import torch
    r = _rng(32)
    B, Hq, Hkv, Tq, Tk, d, qo = 2, 6, 2, 7, 12, 5, 5
    arrs = [r.standard_normal(s) for s in ((B, Hq, Tq, d), (B, Hkv, Tk, d), (B, Hkv, Tk, d),
                                           (B, Hq, Tq, d))]
    q, k, v, dO = (torch.tensor(a, requires_grad=i < 3) for i, a in enumerate(arrs))
    rep = Hq // Hkv
    s = 0.45 * q @ k.repeat_interleave(rep, 1).transpose(-1, -2)
    i = torch.arange(Tq)[:, None]
    j = torch.arange(Tk)[None, :]
    s = s.masked_fill(j > qo + i, float("-inf"))
    o = torch.softmax(s, -1) @ v.repeat_interleave(rep, 1)
    (o * dO).sum().backward()
    got = orc.attn_bwd(*arrs, 0.45, causal=True, q_offset=qo)
    for g, t in zip(got, (q, k, v)):
        assert np.max(np.abs(g - t.grad.numpy())) < 1e-12


def pin_bwd_invariants(orc):
    """Adding one vector to every key shifts each score row by a constant,
    which the softmax ignores: the dk of a K/V head sum to zero.  Every
    weight row sums to one: the dv of a K/V head sum to the dO rows of its
    query heads."""
    r = _rng(33)
    B, Hq, Hkv, Tq, Tk, d = 2, 4, 2, 9, 9, 6
    q = r.standard_normal((B, Hq, Tq, d)); k = r.standard_normal((B, Hkv, Tk, d))
    v = r.standard_normal((B, Hkv, Tk, d)); dO = r.standard_normal((B, Hq, Tq, d))
    dq, dk, dv = orc.attn_bwd(q, k, v, dO, 0.5)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
    want = dO.reshape(B, Hkv, Hq // Hkv, Tq, d).sum(axis=(2, 3))
    assert np.max(np.abs(dv.sum(axis=2) - want)) < 1e-12
    assert np.max(np.abs(dq)) > 1e-3 and np.max(np.abs(dk)) > 1e-3


# --------------------------------------------------------------------------
# RoPE pins
# --------------------------------------------------------------------------

def pin_rope_unit_rotation_and_sign(orc):
    """P2 Now: RoPE / P4 RoPE: each pair turns by [[cos, -sin], [sin, cos]];
    with d = 2 the only frequency is base^0 = 1, so at position 1
    (1,0) -> (cos 1, sin 1) and (0,1) -> (-sin 1, cos 1)."""
    x = np.zeros((1, 1, 2, 2)); x[0, 0, 0] = (1.0, 0.0); x[0, 0, 1] = (0.0, 1.0)
    y = orc.rope(x[:, :, :1], pos0=1)
    assert np.max(np.abs(y[0, 0, 0] - (math.cos(1), math.sin(1)))) < 1e-15
    y = orc.rope(x[:, :, 1:], pos0=1)
    assert np.max(np.abs(y[0, 0, 0] - (-math.sin(1), math.cos(1)))) < 1e-15


def pin_rope_frequency_schedule(orc):
    """P4 RoPE: theta_i(pos) = pos * 10000^(-2i/d_head).  For d = 4 pair 1
    (channels 1 and 3 in split-half pairing) turns by pos/100; pair 0 by pos."""
    for pos in (1, 7, 100, 12345):
        x = np.zeros((1, 1, 1, 4)); x[0, 0, 0, 1] = 1.0
        y = orc.rope(x, pos0=pos)[0, 0, 0]
        assert abs(y[1] - math.cos(pos / 100.0)) < 1e-12 and abs(y[3] - math.sin(pos / 100.0)) < 1e-12
        assert y[0] == 0.0 and y[2] == 0.0
        x = np.zeros((1, 1, 1, 4)); x[0, 0, 0, 0] = 1.0
        y = orc.rope(x, pos0=pos)[0, 0, 0]
        assert abs(y[0] - math.cos(pos)) < 1e-12 and abs(y[2] - math.sin(pos)) < 1e-12
    # another base scales every non-zero frequency
    x = np.zeros((1, 1, 1, 4)); x[0, 0, 0, 1] = 1.0
    y = orc.rope(x, pos0=3, base=500000.0)[0, 0, 0]
    assert abs(y[1] - math.cos(3 / math.sqrt(500000.0))) < 1e-12


def pin_rope_position_zero_identity_and_norms(orc):
    """Rotation by angle 0 is the identity (bit-exact) and every rotation
    keeps each channel pair's length (P2 Now: RoPE, R_m orthogonal)."""
    r = _rng(10)
    x = r.standard_normal((2, 3, 5, 16))
    y = orc.rope(x, pos0=0)
    assert np.array_equal(y[:, :, 0], x[:, :, 0])
    y = orc.rope(x, pos0=977)
    n_x = x[..., :8] ** 2 + x[..., 8:] ** 2
    n_y = y[..., :8] ** 2 + y[..., 8:] ** 2
    assert np.max(np.abs(n_x - n_y)) < 1e-12
    assert np.max(np.abs(x - y)) > 1e-2


def pin_rope_position_origin(orc):
    """P2 Hands-on: RoPE is sliced from cache.pos: token t of a step starting
    at pos0 is rotated exactly like token pos0 + t of a step starting at 0."""
    r = _rng(11)
    x = r.standard_normal((1, 2, 9, 8))
    full = orc.rope(x, pos0=0)
    part = orc.rope(x[:, :, 4:], pos0=4)
    assert np.array_equal(full[:, :, 4:], part)


def pin_rope_relative_position(orc):
    """P2 Now: RoPE and Hands-on (score(5,2) = score(20,17), score(20,10)
    different); P4 RoPE (the rotated dot product depends on pos_q - pos_k).
    Checked for offsets up to 16383 in double precision."""
    g = _read_golden("rope_relative_scores.txt")
    r = _rng(12)
    for d in (16, 128):
        q = r.standard_normal((1, 1, 1, d)); k = r.standard_normal((1, 1, 1, d))
        def score(m, n):
            return float(np.dot(orc.rope(q, pos0=m)[0, 0, 0], orc.rope(k, pos0=n)[0, 0, 0]))
        (m1, n1), (m2, n2) = g["pair"]
        (mo, no), = g["other"]
        s1, s2, so = score(m1, n1), score(m2, n2), score(mo, no)
        scale = np.linalg.norm(q) * np.linalg.norm(k)
        assert abs(s1 - s2) < 1e-12 * scale
        assert abs(s1 - so) > 1e-6 * scale
        for m, n, delta in ((0, 0, 16383), (100, 7, 9000), (16383, 0, 0), (3, 16000, 383)):
            a, b = score(m, n), score(m + delta, n + delta)
            assert abs(a - b) < 1e-9 * scale, (d, m, n, delta)


def pin_rope_pairings_differ_by_a_permutation(orc):
    """P2 Now: RoPE (warning): split-half and adjacent pairing differ by a
    channel permutation P: rope_adjacent(x) = P^-1 rope_split(P x)."""
    r = _rng(13)
    d = 12
    x = r.standard_normal((1, 2, 6, d))
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # adjacent -> split-half
    y_split = orc.rope(x[..., perm], pos0=3)
    back = np.empty_like(y_split); back[..., perm] = y_split
    y_adj = orc.rope(x, pos0=3, pairing="adjacent")
    assert np.max(np.abs(back - y_adj)) < 1e-14
    assert np.max(np.abs(orc.rope(x, pos0=3) - y_adj)) > 1e-3


def pin_rope_then_attention_relative(orc):
    """Attention on RoPE-rotated q/k (P1 Minimal Pseudocode: apply_rope then
    scores) depends only on relative positions: shifting every position by
    the same amount leaves the output unchanged."""
    r = _rng(14)
    B, Hq, Hkv, T, d = 1, 4, 2, 10, 16
    q = r.standard_normal((B, Hq, T, d)); k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    o1 = orc.attn(orc.rope(q, 0), orc.rope(k, 0), v, 0.25)
    o2 = orc.attn(orc.rope(q, 5000), orc.rope(k, 5000), v, 0.25)
    assert np.max(np.abs(o1 - o2)) < 1e-10


def pin_rope_table(orc):
    """The float32 angle table: position 0 turns nothing (cos 1, sin 0 for
    every pair); pair 0 turns by the position itself (base^0 = 1), so
    position 1 holds (cos 1, sin 1) and position 2 the double-angle values;
    every entry lies on the unit circle to float32 rounding; a table that
    starts at pos0 is the slice of one that starts at 0 (RoPE sliced from
    cache.pos, "The Transformer architecture" -- Hands-on); and turning
    vectors with the table's entries gives what the oracle's RoPE (its own
    double-precision angles) gives, to the table's float32 rounding."""
    d = 64
    tab = orc.rope_table(300, d, 0, 10000.0)
    assert np.all(tab[0, :, 0] == 1.0) and np.all(tab[0, :, 1] == 0.0)
    # cos 1 = 0.5403023058681398, sin 1 = 0.8414709848078965;
    # cos 2 = 2 cos^2 1 - 1, sin 2 = 2 sin 1 cos 1
    c1, s1 = 0.5403023058681398, 0.8414709848078965
    assert tab[1, 0, 0] == np.float32(c1) and tab[1, 0, 1] == np.float32(s1)
    assert abs(float(tab[2, 0, 0]) - (2 * c1 * c1 - 1)) < 1e-7
    assert abs(float(tab[2, 0, 1]) - 2 * s1 * c1) < 1e-7
    norm = tab[..., 0].astype(np.float64) ** 2 + tab[..., 1].astype(np.float64) ** 2
    assert np.max(np.abs(norm - 1.0)) < 3e-7
    assert np.array_equal(orc.rope_table(100, d, 200, 10000.0), tab[200:300])
    # rotation with the table against the oracle's RoPE
    x = np.random.default_rng(5).standard_normal((1, 1, 300, d))
    want = orc.rope(x, pos0=0)
    c = tab[..., 0].astype(np.float64)[None, None]
    sn = tab[..., 1].astype(np.float64)[None, None]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    got = np.concatenate([x1 * c - x2 * sn, x1 * sn + x2 * c], axis=-1)
    assert np.max(np.abs(got - want)) < 1e-6
    assert np.max(np.abs(got - want)) > 0.0   # the table is float32, the oracle's angles are not


def pin_rope_per_token_positions(orc):
    """RoPE at a position per token: consecutive positions pos0 + t give the
    scalar-offset rotation exactly; tokens are rotated independently
    (permuting tokens with their positions permutes the result); and two
    rotated vectors' dot product depends only on their position difference
    ("The Transformer architecture" -- Hands-on; "Transformer" (ai-notes) --
    RoPE)."""
    r = _rng(23)
    x = r.standard_normal((2, 3, 7, 16))
    pos = np.array([[40 + t for t in range(7)], [3 + t for t in range(7)]])
    y = orc.rope_positions(x, pos)
    assert np.array_equal(y[0:1], orc.rope(x[0:1], 40)) and np.array_equal(y[1:2], orc.rope(x[1:2], 3))
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    pos2 = r.integers(0, 5000, size=(2, 7))
    y2 = orc.rope_positions(x, pos2)
    y3 = orc.rope_positions(np.ascontiguousarray(x[:, :, perm]), pos2[:, perm])
    assert np.array_equal(y3, y2[:, :, perm])
    q = r.standard_normal((1, 1, 1, 32)); k = r.standard_normal((1, 1, 1, 32))
    qq = orc.rope_positions(np.repeat(q, 2, axis=2), [[5, 1005]])   # the same q at two positions
    kk = orc.rope_positions(np.repeat(k, 2, axis=2), [[2, 1002]])
    s0 = float(qq[0, 0, 0] @ kk[0, 0, 0]); s1 = float(qq[0, 0, 1] @ kk[0, 0, 1])
    assert abs(s0 - s1) < 1e-9


PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]


def run_all(orc):
    """{pin name: "ok" or the failure message} for one oracle copy."""
    out = {}
    for fn in PINS:
        try:
            fn(orc)
            out[fn.__name__] = "ok"
        except Exception as e:  # noqa: BLE001 -- report every kind of failure
            out[fn.__name__] = f"fail: {type(e).__name__}: {str(e)[:200]}"
    return out


if __name__ == "__main__":
    # python tests/oracle_pins.py <liboracle.so>  -> JSON of pin results
    here = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, os.path.dirname(here))
    from oracle import Oracle
    print(json.dumps(run_all(Oracle(sys.argv[1]))))
