"""Properties of exact attention checked on the HIP path at full size, and the
memory contract: no N x N buffer, no allocation by the library."""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import workloads as W
from oracle import score_matrix_bytes
from tests.helpers import np64, run_bwd, run_fwd, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_average_the_visible_values(causal, dtype):
    say(f"identical keys {dtype} causal={causal}")
    inp = W.random_case(1, 2, 777, 64, dtype, seed=2)
    inp["k"] = inp["k"][:, :, :1].expand_as(inp["k"]).contiguous()
    o, _ = run_fwd(inp, 0.125, causal, out_dtype=torch.float32)
    v = inp["v"].double()
    cnt = torch.arange(1, 778, dtype=torch.float64)[:, None]
    expect = (v.cumsum(dim=2) / cnt) if causal else v.mean(dim=2, keepdim=True).expand_as(v)
    tol = 1e-5 if dtype == "fp32" else 5e-3
    assert (o.double().cpu() - expect).abs().max().item() <= tol


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_single_key_and_causal_row_zero_return_first_value(dtype):
    say(f"single key {dtype}")
    one = W.random_case(2, 3, 1, 128, dtype, seed=4)
    o, lse = run_fwd(one, 128 ** -0.5, False)
    assert torch.equal(o.cpu(), one["v"])
    qk = (one["q"].double() * one["k"].double()).sum(-1) * 128 ** -0.5
    assert (lse.double().cpu() - qk).abs().max().item() <= 1e-5
    many = W.random_case(2, 3, 300, 64, dtype, seed=5)
    o, _ = run_fwd(many, 0.125, True)
    assert torch.equal(o[:, :, 0].cpu(), many["v"][:, :, 0])


def test_joint_permutation_of_keys_and_values():
    say("permutation")
    inp = W.random_case(1, 3, 1000, 128, "bf16", seed=6)
    perm = torch.randperm(1000, generator=torch.Generator().manual_seed(7))
    o1, l1 = run_fwd(inp, 128 ** -0.5, False, out_dtype=torch.float32)
    inp2 = dict(inp, k=inp["k"][:, :, perm].contiguous(), v=inp["v"][:, :, perm].contiguous())
    o2, l2 = run_fwd(inp2, 128 ** -0.5, False, out_dtype=torch.float32)
    assert (o1 - o2).abs().max().item() <= 2e-3
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_rows_of_p_sum_to_one_through_the_value_path():
    # V = ones: every output row with a visible key is exactly the row sum of P
    say("ones")
    inp = W.random_case(3, 2, 513, 64, "bf16", seed=8, kv_len=[513, 200, 1])
    inp["v"] = torch.ones_like(inp["v"])
    o, _ = run_fwd(inp, 0.125, True, out_dtype=torch.float32)
    assert (o - 1.0).abs().max().item() <= 5e-3


def _free_bytes():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


@pytest.mark.parametrize("wname", ["trading_day_bf16_causal_fwd", "long_context_bf16_fwd"])
def test_no_score_matrix_is_allocated(wname):
    w = W.CONFIGS[wname].with_(backward=True)
    say(f"memory {w.name}")
    inp = W.make_inputs(w)
    forbidden = score_matrix_bytes(w.B, w.H, w.N, w.elem_bytes)
    q, k, v, do = (x.cuda() for x in (inp["q"], inp["k"], inp["v"], inp["do"]))
    from exact_io_aware_07_amd import fa_bwd, fa_bwd_workspace_bytes, fa_fwd
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa_bwd_workspace_bytes(*q.shape), dtype=torch.uint8, device="cuda")
    fa_fwd(q, k, v, o, lse, w.scale, w.causal)          # warm-up: code objects load
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, w.scale, w.causal, None, ws)
    torch.cuda.reset_peak_memory_stats()
    before_alloc = torch.cuda.memory_allocated()
    free0 = _free_bytes()
    fa_fwd(q, k, v, o, lse, w.scale, w.causal)
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, w.scale, w.causal, None, ws)
    free1 = _free_bytes()
    assert torch.cuda.max_memory_allocated() == before_alloc
    assert free0 - free1 < forbidden // 64, (free0 - free1, forbidden)
    # the caller-owned workspace is O(N): one fp32 per row
    assert ws.numel() == w.B * w.H * w.N * 4 < forbidden


def test_every_other_entry_point_allocates_nothing():
    """The key-split, grouped-query, block-sparse and FP8 paths, each given
    its workspace: no torch allocation during the calls and no change in the
    device's free memory (the library never allocates)."""
    from exact_io_aware_07_amd import (fa_bwd_gqa, fa_bwd_gqa_workspace_bytes, fa_bwd_sparse,
                                       fa_bwd_sparse_planned, fa_bwd_sparse_planned_workspace_bytes,
                                       fa_bwd_workspace_bytes, fa_fwd_fp8_incoherent,
                                       fa_fwd_fp8_workspace_bytes, fa_fwd_gqa, fa_fwd_sparse,
                                       fa_fwd_sparse_planned, fa_fwd_sparse_planned_workspace_bytes,
                                       fa_fwd_split, fa_fwd_split_workspace_bytes, fa_sparse_plan)
    B, H, Hkv, N, d = 2, 8, 2, 2048, 128
    say("memory of the split, GQA, sparse, planned sparse and FP8 paths")
    inp = W.random_case(B, H, N, d, "bf16", seed=30, backward=True)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    kg, vg = k[:, :Hkv].contiguous(), v[:, :Hkv].contiguous()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dkg, dvg = torch.empty_like(kg), torch.empty_like(vg)
    mask_h = W.random_block_mask((), N, 0.7, seed=31)
    mask = mask_h.cuda()
    plan = fa_sparse_plan(mask_h, B, H, N, False)
    assert plan["counts"][2] > 0 and plan["counts"][5] > 0
    plan = {"plan": plan["plan"].cuda(), "counts": plan["counts"]}
    signs = W.random_signs(d, seed=32).cuda()
    ws_bytes = max(fa_fwd_split_workspace_bytes(B, H, N, d, 4), fa_bwd_gqa_workspace_bytes(B, H, Hkv, N, d),
                   fa_bwd_workspace_bytes(B, H, N, d), fa_fwd_fp8_workspace_bytes(B, H, N, d),
                   fa_fwd_sparse_planned_workspace_bytes(B, H, N, d, plan["counts"]),
                   fa_bwd_sparse_planned_workspace_bytes(B, H, N, d, plan["counts"]))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def calls():
        fa_fwd_split(q, k, v, o, lse, 0.1, True, None, 4, ws)
        fa_fwd_gqa(q, kg, vg, o, lse, 0.1, True)
        fa_bwd_gqa(q, kg, vg, o, do, lse, dq, dkg, dvg, 0.1, True, None, ws)
        fa_fwd_sparse(q, k, v, o, lse, mask, 0.1, False)
        fa_bwd_sparse(q, k, v, o, do, lse, dq, dk, dv, mask, 0.1, False, None, ws)
        fa_fwd_sparse_planned(q, k, v, o, lse, mask, plan, 0.1, False, None, ws)
        fa_bwd_sparse_planned(q, k, v, o, do, lse, dq, dk, dv, mask, plan, 0.1, False, None, ws)
        fa_fwd_fp8_incoherent(q, k, v, signs, o, lse, 0.1, False, None, ws)

    calls()  # code objects load
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    free0 = _free_bytes()
    calls()
    free1 = _free_bytes()
    assert torch.cuda.max_memory_allocated() == before
    # a score matrix of one call would take B*H*N^2*2 bytes (134 MB here)
    assert free0 - free1 < B * H * N * N * 2 // 64, (free0, free1)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_leaves_o_and_shifts_lse(causal):
    """Adding u to every key row adds scale * q_i . u to every score of row i:
    O is unchanged and LSE_i moves by that amount. fp16 keys on a 1/16 grid
    in [-4, 4] and u = 64 keep K + u exact in fp16; the scores become large,
    which drives the running maximum."""
    B, H, N, d = 2, 2, 300, 64
    say(f"key shift causal={causal}")
    g = torch.Generator().manual_seed(60)
    inp = W.random_case(B, H, N, d, "fp16", seed=61)
    inp["k"] = (torch.randint(-64, 65, (B, H, N, d), generator=g).float() / 16).to(torch.float16)
    u = 64.0
    shifted = dict(inp, k=(inp["k"].float() + u).to(torch.float16))
    assert torch.equal(shifted["k"].float(), inp["k"].float() + u)
    scale = d ** -0.5
    o1, l1 = run_fwd(inp, scale, causal, out_dtype=torch.float32)
    o2, l2 = run_fwd(shifted, scale, causal, out_dtype=torch.float32)
    shift = scale * u * inp["q"].double().sum(dim=-1).numpy()
    assert np.abs(np64(o2) - np64(o1)).max() <= 1e-2
    assert np.abs(np64(l2) - np64(l1) - shift).max() <= 1e-3 * max(1.0, np.abs(shift).max() / 64)
