"""The entry points under HIP graph capture: the library only enqueues
kernels on the caller's stream (no allocation, copy, memset or
synchronisation), so a step captured into a graph and replayed gives the
eager results bit for bit.

Each case captures a step on preallocated buffers, then replays it three
times with eager work between the replays (the outputs are overwritten with
NaN by a fill kernel, and the device is synchronised), and checks every
replay against the eager run. It then writes new inputs into the captured
buffers and checks a replay against an eager run on them, so the graph
reads its inputs live rather than baking them in.
"""
import pytest
import torch

from exact_io_aware_07_amd import (fa_bwd, fa_bwd_gqa, fa_bwd_gqa_workspace_bytes,
                                   fa_bwd_sparse_planned, fa_bwd_sparse_planned_workspace_bytes,
                                   fa_bwd_workspace_bytes, fa_fwd, fa_fwd_fp8_incoherent,
                                   fa_fwd_fp8_workspace_bytes, fa_fwd_gqa, fa_fwd_sparse_planned,
                                   fa_fwd_sparse_planned_workspace_bytes, fa_fwd_split,
                                   fa_fwd_split_workspace_bytes, fa_sparse_plan)
from exact_io_aware_07_amd import workloads as W
from helpers import say

pytestmark = pytest.mark.gpu

U8 = torch.uint8


def _inputs(B, H, N, d, dtype, seed, Hkv=None, kv=None, causal=False):
    inp = W.random_case(B, H, N, d, dtype, seed=seed, causal=causal, kv_len=kv, backward=True,
                        Hkv=Hkv)
    t = {n: inp[n].cuda() for n in ("q", "k", "v", "do")}
    t["kv"] = None if kv is None else inp["kv_len"].cuda()
    return t


def _dense_step(t, causal, out32):
    """Forward then one-call backward, all buffers allocated up front."""
    q, k, v, do, kv = t["q"], t["k"], t["v"], t["do"], t["kv"]
    B, H, N, d = q.shape
    sc = d ** -0.5
    o = torch.empty(q.shape, dtype=torch.float32 if out32 else q.dtype, device="cuda")
    ob = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    ws = torch.empty(fa_bwd_workspace_bytes(B, H, N, d), dtype=U8, device="cuda")

    def step():
        fa_fwd(q, k, v, o, lse, sc, causal, kv)
        ob.copy_(o)
        fa_bwd(q, k, v, ob, do, lse, dq, dk, dv, sc, causal, kv, ws)
    return step, [o, lse, dq, dk, dv]


def _gqa_step(t, causal, out32):
    q, k, v, do, kv = t["q"], t["k"], t["v"], t["do"], t["kv"]
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    sc = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    ws = torch.empty(fa_bwd_gqa_workspace_bytes(B, H, Hkv, N, d), dtype=U8, device="cuda")

    def step():
        fa_fwd_gqa(q, k, v, o, lse, sc, causal, kv)
        fa_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, sc, causal, kv, ws)
    return step, [o, lse, dq, dk, dv]


def _split_step(t, causal, out32):
    q, k, v, kv = t["q"], t["k"], t["v"], t["kv"]
    B, H, N, d = q.shape
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa_fwd_split_workspace_bytes(B, H, N, d, 3), dtype=U8, device="cuda")

    def step():
        fa_fwd_split(q, k, v, o, lse, d ** -0.5, causal, kv, 3, ws)
    return step, [o, lse]


def _sparse_step(t, causal, out32):
    q, k, v, do, kv = t["q"], t["k"], t["v"], t["do"], t["kv"]
    B, H, N, d = q.shape
    sc = d ** -0.5
    nb = (N + 127) // 128
    mask = W.random_block_mask((B, H), N, 0.5, seed=N)
    mask[0, 0, :, 0] = 1          # a long column and a long row: both get cut
    mask[-1, -1, nb - 1, :] = 1
    plan = fa_sparse_plan(mask, B, H, N, causal)
    assert int(plan["counts"][1]) > 0 and int(plan["counts"][4]) > 0
    # the plan on the device once: no host copy inside the captured step
    plan = dict(plan, plan=plan["plan"].cuda())
    m = mask.cuda()
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ob = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    wf = torch.empty(max(16, fa_fwd_sparse_planned_workspace_bytes(B, H, N, d, plan["counts"])),
                     dtype=U8, device="cuda")
    wb = torch.empty(fa_bwd_sparse_planned_workspace_bytes(B, H, N, d, plan["counts"]),
                     dtype=U8, device="cuda")

    def step():
        fa_fwd_sparse_planned(q, k, v, o, lse, m, plan, sc, causal, kv, wf)
        ob.copy_(o)
        fa_bwd_sparse_planned(q, k, v, ob, do, lse, dq, dk, dv, m, plan, sc, causal, kv, wb)
    return step, [o, lse, dq, dk, dv]


def _fp8_step(t, causal, out32):
    q, k, v, kv = t["q"], t["k"], t["v"], t["kv"]
    B, H, N, d = q.shape
    g = torch.Generator().manual_seed(d)
    signs = (torch.randint(0, 2, (d,), generator=g, dtype=torch.int8) * 2 - 1).cuda()
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa_fwd_fp8_workspace_bytes(B, H, N, d), dtype=U8, device="cuda")

    def step():
        fa_fwd_fp8_incoherent(q, k, v, signs, o, lse, d ** -0.5, causal, kv, ws)
    return step, [o, lse]


CASES = [  # (name, builder, B, H, Hkv, N, d, dtype, causal, kv_len, fp32 O)
    ("dense", _dense_step, 2, 3, None, 300, 64, "bf16", True, None, False),
    ("dense", _dense_step, 2, 2, None, 257, 128, "fp16", False, [200, 0], True),
    ("dense", _dense_step, 1, 2, None, 190, 64, "fp32", True, None, True),
    ("gqa", _gqa_step, 2, 4, 2, 333, 64, "bf16", True, [333, 100], False),
    ("split", _split_step, 1, 3, None, 700, 128, "bf16", True, None, True),
    ("sparse", _sparse_step, 2, 2, None, 1300, 64, "bf16", True, [1300, 900], True),
    ("fp8", _fp8_step, 1, 2, None, 513, 128, "bf16", False, None, True),
]


def _id(c):
    return f"{c[0]}-{c[2]}x{c[3]}x{c[5]}x{c[6]}-{c[7]}-c{int(c[8])}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_graph_replay_equals_eager(case):
    name, build, B, H, Hkv, N, d, dtype, causal, kv, out32 = case
    say(f"graph {_id(case)}")
    t = _inputs(B, H, N, d, dtype, seed=N + d, Hkv=Hkv, kv=kv, causal=causal)
    step, outs = build(t, causal, out32)

    def eager():
        step()
        torch.cuda.synchronize()
        return [x.clone() for x in outs]

    ref = eager()
    # capture on a side stream after a warm-up there, as torch's graphs want
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, r) in enumerate(zip(outs, ref)):
            assert torch.equal(x, r), f"replay {rep}, output {i}"
    # new inputs in the captured buffers
    g2 = torch.Generator().manual_seed(N + d + 1)
    for n in ("q", "k", "v", "do"):
        x = t[n]
        x.copy_(torch.randn(x.shape, generator=g2).to(x.dtype).cuda())
    ref2 = eager()
    assert any(not torch.equal(a, b) for a, b in zip(ref, ref2))
    for x in outs:
        x.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    for i, (x, r) in enumerate(zip(outs, ref2)):
        assert torch.equal(x, r), f"new inputs, output {i}"
