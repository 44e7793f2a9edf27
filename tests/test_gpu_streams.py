"""Calls enqueued on a stream other than torch's current one.

The binding allocates the backward's workspace (and copies a host sparse
plan) itself when the caller passes none. Those buffers must stay out of
reach of torch's caching allocator until the kernels on the caller's stream
have used them. Each test runs a call on a side stream, then at once
allocates and fills memory on the current stream (which would land in the
dropped buffer if it had been allocated there), and compares the results
with the same call on the current stream, bit for bit.
"""
import pytest
import torch

from exact_io_aware_07_amd import (attention_backward, attention_forward, fa_bwd, fa_bwd_workspace_bytes,
                                   fa_fwd_sparse_planned, fa_sparse_plan)
from exact_io_aware_07_amd import workloads as W
from tests.helpers import dev, say

pytestmark = pytest.mark.gpu


def _clobber(nbytes: int, rounds: int = 4):
    """Allocate and fill device memory on the current stream, several sizes."""
    keep = []
    for i in range(rounds):
        t = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        t.fill_(0x7f + i)
        keep.append(t)
    return keep


@pytest.mark.parametrize("d", [64, 128])
def test_backward_on_side_stream_equals_current_stream(d):
    B, H, N = 2, 4, 1000
    say(f"side-stream backward {B}x{H}x{N}x{d}")
    inp = W.random_case(B, H, N, d, "bf16", seed=5 + d, causal=True, backward=True)
    q, k, v, do = (dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = attention_forward(q, k, v, causal=True)
    ref = attention_backward(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
        fa_bwd(q, k, v, o, do, lse, dq, dk, dv, d ** -0.5, True, stream=side)
        keep = _clobber(fa_bwd_workspace_bytes(B, H, N, d))
        side.synchronize()
        torch.cuda.synchronize()
        for g, r in zip((dq, dk, dv), ref):
            assert torch.equal(g, r)
        del keep
    got = attention_backward(q, k, v, o, do, lse, causal=True, stream=side)
    keep = _clobber(q.numel() * 2)
    side.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    del keep


def test_planned_sparse_on_side_stream_equals_current_stream():
    B, H, N, d = 1, 4, 2048, 64
    say(f"side-stream planned sparse forward {B}x{H}x{N}x{d}")
    inp = W.random_case(B, H, N, d, "bf16", seed=9)
    q, k, v = (dev(inp[n]) for n in ("q", "k", "v"))
    mask = W.random_block_mask((H,), N, 0.5, seed=3)
    mask[:, :, 0] = 1
    plan = fa_sparse_plan(mask, B, H, N)
    dmask = mask.cuda()
    o_ref = torch.empty_like(q)
    lse_ref = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa_fwd_sparse_planned(q, k, v, o_ref, lse_ref, dmask, plan, d ** -0.5)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        o = torch.empty_like(q)
        lse = torch.empty_like(lse_ref)
        fa_fwd_sparse_planned(q, k, v, o, lse, dmask, plan, d ** -0.5, stream=side)
        keep = _clobber(plan["plan"].numel() * 4) + _clobber(64 << 20, rounds=1)
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        del keep
