"""The longest sequences: sizes where every 32-bit byte offset inside a head
is large and the grid is long, checked where the fp64 oracle can follow.

  * forward at 1,048,576 tokens (causal, one head): O and LSE of sampled
    rows against the oracle, each row against all its keys;
  * backward at 262,144 tokens (causal, one head): dQ of sampled rows and
    dK, dV of the last keys (which only the last rows see) against the
    oracle, and for all of dV the identity that holds at any size:
    sum_j dV_j = sum_i dO_i (each row's probabilities sum to one);
  * planned block-sparse attention at the largest mask (4096 blocks);
  * multi-query attention at 65,536 tokens, where the grouped dK/dV stage
    adds the fp32 partials of two shares.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import workloads as W
from helpers import FWD_MAX_ABS, GRAD_REL_FRO, LSE_MAX_ABS, fwd_stats, np64, rel_fro, run_bwd, run_fwd, say
from oracle import attn_bwd64_sampled, attn_fwd64

pytestmark = pytest.mark.gpu


def test_forward_at_a_million_tokens():
    N, d = 1 << 20, 64
    say(f"long forward N={N}")
    inp = W.random_case(1, 1, N, d, "bf16", seed=50, causal=True)
    o, lse = run_fwd(inp, d ** -0.5, True, out_dtype=torch.float32)
    rows = [0, 1, 127, 128, 65535, 65536, 500000, N // 2, N - 129, N - 128, N - 2, N - 1]
    o_ref, lse_ref = attn_fwd64(inp["q"], inp["k"], inp["v"], d ** -0.5, True, rows=rows, row_chunk=4)
    st = fwd_stats(np64(o[:, :, rows]), np64(lse[:, :, rows]), o_ref, lse_ref)
    print(f"N={N} {st}", flush=True)
    assert st["max_abs"] <= FWD_MAX_ABS and st["lse_max_abs"] <= LSE_MAX_ABS, st


def test_backward_at_262144_tokens():
    N, d = 1 << 18, 64
    say(f"long backward N={N}")
    inp = W.random_case(1, 1, N, d, "bf16", seed=51, causal=True, backward=True)
    o, lse = run_fwd(inp, d ** -0.5, True)
    dq, dk, dv = run_bwd(inp, o, lse, d ** -0.5, True)
    rows = [0, 1, 127, 128, 100000, N // 2, N - 1]
    keys = [N - 1, N - 2, N - 64, N - 65, N - 128, N - 129, N - 200]
    sq, _, _ = attn_bwd64_sampled(inp["q"], inp["k"], inp["v"], inp["do"], d ** -0.5, True,
                                  heads=[(0, 0)], q_rows=rows, k_rows=[], row_chunk=4)
    _, sk, sv = attn_bwd64_sampled(inp["q"], inp["k"], inp["v"], inp["do"], d ** -0.5, True,
                                   heads=[(0, 0)], q_rows=[], k_rows=keys, row_chunk=64)
    errs = {"dq": rel_fro(np64(dq[0, 0, rows]), sq[0]), "dk": rel_fro(np64(dk[0, 0, keys]), sk[0]),
            "dv": rel_fro(np64(dv[0, 0, keys]), sv[0])}
    print(f"N={N} rel-fro {errs}", flush=True)
    for n, e in errs.items():
        assert e <= GRAD_REL_FRO, (n, e)
    # each row's probabilities sum to one: sum_j dV_j = sum_i dO_i, up to the
    # bf16 rounding of P (2^-9 of each row's sum) and of each dV row
    dv_sum = np64(dv[0, 0]).sum(axis=0)
    do_abs = np.abs(np64(inp["do"][0, 0])).sum(axis=0)
    dv_abs = np.abs(np64(dv[0, 0])).sum(axis=0)
    gap = np.abs(dv_sum - np64(inp["do"][0, 0]).sum(axis=0))
    assert np.all(gap <= 2 ** -8 * (do_abs + dv_abs)), gap.max()


def test_planned_sparse_at_the_largest_mask():
    """Block-sparse attention at 4096 mask blocks (N = 524,288), the most a
    mask row or column may hold: a band of three plus a global first block,
    so row 0 and column 0 keep all 4096 blocks (512 pieces each in the
    plan). O, LSE and dQ of sampled rows and dK, dV of keys that few rows
    see against the oracle; all of dV against sum_j dV_j = sum_i dO_i."""
    from exact_io_aware_07_amd import fa_bwd_sparse_planned, fa_fwd_sparse_planned, fa_sparse_plan
    from oracle import attn_bwd64_sparse_sampled, attn_fwd64_sparse
    N, d = 4096 * 128, 64
    w = W.SPARSE_GLOBAL.with_(H=1, N=N)
    say(f"planned sparse at the largest mask N={N}")
    inp = W.random_case(1, 1, N, d, "bf16", seed=52, backward=True)
    mask = W.block_mask(w)
    plan = fa_sparse_plan(mask, 1, 1, N, False)
    assert plan["counts"][2] == 512 and plan["counts"][5] == 512
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    m = mask.cuda()
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    fa_fwd_sparse_planned(q, k, v, o, lse, m, plan, d ** -0.5, False)
    grads = [torch.empty_like(q) for _ in range(3)]
    fa_bwd_sparse_planned(q, k, v, o.to(q.dtype), do, lse, *grads, m, plan, d ** -0.5, False)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 300000, N - 129, N - 1]
    o_ref, lse_ref = attn_fwd64_sparse(inp["q"], inp["k"], inp["v"], d ** -0.5, False, None,
                                       mask.numpy(), rows=rows, row_chunk=2)
    st = fwd_stats(np64(o[:, :, rows]), np64(lse[:, :, rows]), o_ref, lse_ref)
    print(f"N={N} {st}", flush=True)
    assert st["max_abs"] <= FWD_MAX_ABS and st["lse_max_abs"] <= LSE_MAX_ABS, st
    keys = [N - 1, N - 100, 300000, 300001]
    sq, sk, sv = attn_bwd64_sparse_sampled(inp["q"], inp["k"], inp["v"], inp["do"], d ** -0.5,
                                           False, None, mask.numpy(), [(0, 0)], rows[1:], keys,
                                           row_chunk=64)
    dq, dk, dv = grads
    errs = {"dq": rel_fro(np64(dq[0, 0, rows[1:]]), sq[0]), "dk": rel_fro(np64(dk[0, 0, keys]), sk[0]),
            "dv": rel_fro(np64(dv[0, 0, keys]), sv[0])}
    print(f"N={N} rel-fro {errs}", flush=True)
    for n, e in errs.items():
        assert e <= GRAD_REL_FRO, (n, e)
    dv_sum = np64(dv[0, 0]).sum(axis=0)
    do_abs = np.abs(np64(inp["do"][0, 0])).sum(axis=0)
    dv_abs = np.abs(np64(dv[0, 0])).sum(axis=0)
    gap = np.abs(dv_sum - np64(inp["do"][0, 0]).sum(axis=0))
    assert np.all(gap <= 2 ** -8 * (do_abs + dv_abs)), gap.max()


def test_multi_query_backward_at_65536_tokens():
    """Multi-query attention (4 query heads on one K/V head) at N = 65,536,
    causal, d = 64: the grid is small enough that the grouped dK/dV stage
    cuts the group into two shares and adds their fp32 partials. dQ of
    sampled rows of every query head, and dK, dV (summed over the group) of
    the last keys, against the oracle on K/V repeated over the group."""
    from exact_io_aware_07_amd import attention_backward, attention_forward
    N, d, H = 1 << 16, 64, 4
    say(f"long multi-query backward N={N}")
    inp = W.random_case(1, H, N, d, "bf16", seed=53, causal=True, backward=True, Hkv=1)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    sc = d ** -0.5
    o, lse = attention_forward(q, k, v, True, None, sc)
    dq, dk, dv = attention_backward(q, k, v, o, do, lse, True, None, sc)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 40000, N - 1]
    keys = [N - 1, N - 2, N - 64, N - 65, N - 130]
    kg, vg = inp["k"].repeat_interleave(H, dim=1), inp["v"].repeat_interleave(H, dim=1)
    heads = [(0, h) for h in range(H)]
    sq, _, _ = attn_bwd64_sampled(inp["q"], kg, vg, inp["do"], sc, True, heads=heads, q_rows=rows,
                                  k_rows=[], row_chunk=4)
    _, sk, sv = attn_bwd64_sampled(inp["q"], kg, vg, inp["do"], sc, True, heads=heads, q_rows=[],
                                   k_rows=keys, row_chunk=64)
    errs = {"dq": rel_fro(np64(dq[0][:, rows]), np.asarray(sq)),
            "dk": rel_fro(np64(dk[0, 0, keys]), np.asarray(sk).sum(axis=0)),
            "dv": rel_fro(np64(dv[0, 0, keys]), np.asarray(sv).sum(axis=0))}
    print(f"N={N} rel-fro {errs}", flush=True)
    for n, e in errs.items():
        assert e <= GRAD_REL_FRO, (n, e)
