"""attn_fwd_noalloc (the entry point that allocates nothing) against
attn_fwd_ws with a caller workspace of attn_workspace_bytes(): the same
kernels on the same inputs, so the outputs and log-sum-exps must be
bit-identical.  Two calls in a row on each path, the second with a smaller
input, so that the second reads a scratch buffer the first has filled."""
import pytest
import torch

import transformer_causal_self_amd as ra
from transformer_causal_self_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCRATCH = 64 << 20   # bytes of the library's fixed device scratch buffer


def say(*a):
    print("[case]", *a, flush=True)


def both(B, Hq, Hkv, Tq, Tk, d, causal, qo, seed):
    q, k, v = (t.to(DEV) for t in wl.random_qkv(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16, seed=seed))
    scale = d ** -0.5
    o1 = torch.empty_like(q)
    l1 = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    ra.attn_fwd_noalloc(q, k, v, o1, l1, scale=scale, causal=causal, q_offset=qo)
    nb = ra.attn_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, torch.bfloat16)
    assert nb <= SCRATCH   # within the fixed scratch: the same split as the workspace call
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV) if nb else None
    o2 = torch.empty_like(q)
    l2 = torch.empty(B, Hq, Tq, dtype=torch.float32, device=DEV)
    ra.attn_fwd_ws(q, k, v, o2, ws, l2, scale=scale, causal=causal, q_offset=qo)
    torch.cuda.synchronize()
    return nb, (o1, l1), (o2, l2)


# pairs of calls: (larger, then smaller) -- (B, Hq, Hkv, Tq, Tk, d, causal, q_offset)
CASES = [
    # split-K decode: the decode workload's shape, then a smaller cache
    ((32, 32, 8, 1, 8192, 128, True, 8191), (4, 16, 4, 1, 3000, 128, True, 2999)),
    ((2, 8, 2, 1, 20000, 64, True, 19999), (1, 4, 4, 1, 700, 64, True, 500)),
    # small prefills split over the keys, then a smaller chunk
    ((1, 32, 8, 512, 4096, 128, True, 3584), (1, 8, 2, 300, 2000, 128, True, 1700)),
    ((1, 8, 2, 300, 2000, 64, True, 1700), (2, 2, 1, 70, 3000, 64, True, 2930)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_call_twice(first, second):
    for shape in (first, second):
        say("noalloc", shape)
        nb, (o1, l1), (o2, l2) = both(*shape, seed=sum(shape[:6]))
        assert nb > 0   # every case here uses the scratch buffer
        assert torch.equal(o1, o2)
        assert torch.equal(l1, l2)


def test_noalloc_without_scratch_is_the_plain_call():
    """A prefill large enough to need no split uses no scratch."""
    shape = (8, 12, 12, 1024, 1024, 64, True, 0)   # the GPT-2-small shape: 768 workgroups
    say("noalloc no scratch", shape)
    nb, (o1, l1), (o2, l2) = both(*shape, seed=5)
    assert nb == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
