"""fa_bwd_noalloc through the C ABI: the backward with its D_i array in the
library's built-in device array, against fa_bwd (same kernels, caller's
workspace) and the fp64 oracle.

Two calls in a row, the second on a smaller problem, so that the second
reads none of the first call's leftovers; and no device allocation by the
call itself (torch's allocation counter does not move).
"""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import FA_ERR_TOO_LARGE, FA_NOALLOC_MAX_ROWS, FaError, fa_bwd, fa_bwd_noalloc
from exact_io_aware_07_amd import workloads as W
from oracle import attn_bwd64
from tests.helpers import F32_GRAD_REL_FRO, GRAD_REL_FRO, dev, np64, rel_fro, run_fwd, say

pytestmark = pytest.mark.gpu


def _case(B, H, N, d, dtype, causal, kv, seed):
    inp = W.random_case(B, H, N, d, dtype, seed=seed, causal=causal, kv_len=kv, backward=True)
    scale = d ** -0.5
    o, lse = run_fwd(inp, scale, causal)
    q, k, v, do = (dev(inp[n]) for n in ("q", "k", "v", "do"))
    kvd = dev(inp.get("kv_len"))
    return inp, scale, (q, k, v, o, do, lse, kvd)


def _run_both(args, scale, causal):
    q, k, v, o, do, lse, kvd = args
    ref = [torch.empty_like(t) for t in (q, k, v)]
    fa_bwd(q, k, v, o, do, lse, *ref, scale, causal, kvd)
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    torch.cuda.synchronize()
    n_alloc = torch.cuda.memory_stats()["allocation.all.allocated"]
    fa_bwd_noalloc(q, k, v, o, do, lse, *got, scale, causal, kvd)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == n_alloc
    return got, ref


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_noalloc_two_calls_second_smaller(dtype):
    tol = F32_GRAD_REL_FRO if dtype == "fp32" else GRAD_REL_FRO
    cases = [((2, 3, 700, 128), True, None, 1), ((1, 2, 333, 64), False, [200], 2)]
    if dtype == "fp32":
        cases = [((1, 2, 300, 128), True, None, 1), ((1, 1, 130, 64), False, [77], 2)]
    for (B, H, N, d), causal, kv, seed in cases:
        say(f"noalloc {dtype} {B}x{H}x{N}x{d} causal={causal} kv={kv}")
        inp, scale, args = _case(B, H, N, d, dtype, causal, kv, seed)
        got, ref = _run_both(args, scale, causal)
        for g, r in zip(got, ref):
            assert torch.equal(g, r)
        oracle = attn_bwd64(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, inp.get("kv_len"))
        for name, g, r in zip(("dq", "dk", "dv"), got, oracle):
            e = rel_fro(np64(g), r)
            print(f"  {name} rel-fro {e:.2e}", flush=True)
            assert e <= tol, (name, e)


def test_noalloc_at_a_workload_shape():
    w = W.GPT2
    say(f"noalloc {w.name}")
    inp = W.make_inputs(w)
    o, lse = run_fwd(inp, w.scale, w.causal)
    args = tuple(dev(inp[n]) for n in ("q", "k", "v")) + (o, dev(inp["do"]), lse, None)
    got, ref = _run_both(args, w.scale, w.causal)
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def test_noalloc_refuses_more_rows_than_its_scratch():
    N = FA_NOALLOC_MAX_ROWS // 2 + 64
    say(f"noalloc too large: 1x2x{N}x64 (refused before launch)")
    t = torch.zeros((1, 2, N, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 2, N), dtype=torch.float32, device="cuda")
    with pytest.raises(FaError) as ei:
        fa_bwd_noalloc(t, t, t, t, t, lse, t, t, t, 0.125, False)
    assert ei.value.status == FA_ERR_TOO_LARGE
