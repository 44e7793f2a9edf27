"""GPU parity of the key-part entry points (fa_fwd_partial, fa_merge,
fa_fwd_split) against the fp64 oracle (oracle/split.py, oracle/attention.py),
through the C ABI. Partial results are fp32, judged at the forward's
tolerances; fa_fwd_split's bf16/fp16 output is judged like fa_fwd's."""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import fa_fwd, fa_fwd_partial, fa_fwd_split, fa_merge
from exact_io_aware_07_amd import workloads as W
from helpers import FWD_MAX_ABS, FWD_MEAN_ABS, LSE_MAX_ABS, dev, fwd_stats, np64, rounding_floor, say
from oracle import attn_fwd64, attn_part64, merge64

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def inputs(B, H, Nq, Nk, d, dtype, seed, kv_len=None):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g).to(TORCH[dtype])
    k = torch.randn(B, H, Nk, d, generator=g).to(TORCH[dtype])
    v = torch.randn(B, H, Nk, d, generator=g).to(TORCH[dtype])
    kv = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32)
    return q, k, v, kv


def run_partial(q, k, v, scale, causal, qp, kp, kv=None):
    B, H, Nq, d = q.shape
    o = torch.empty(B, H, Nq, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device="cuda")
    fa_fwd_partial(dev(q), dev(k), dev(v), o, lse, scale, causal, qp, kp, dev(kv))
    torch.cuda.synchronize()
    return o, lse


def check(o, lse, o_ref, lse_ref):
    st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
    assert st["max_abs"] <= FWD_MAX_ABS and st["mean_abs"] <= FWD_MEAN_ABS, st
    assert st["lse_max_abs"] <= LSE_MAX_ABS, st


# (B, H, Nq, Nk, d, q_pos0, k_pos0): short and long key blocks, ragged
# tails, query blocks before, after and straddling the key block
PARTIAL = [
    (1, 2, 128, 128, 64, 0, 0),
    (1, 2, 200, 333, 64, 333, 0),
    (2, 1, 77, 300, 128, 100, 50),
    (1, 3, 256, 64, 64, 0, 192),
    (1, 2, 130, 517, 128, -40, 0),
    (1, 1, 64, 1000, 64, 1000, 0),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", PARTIAL, ids=lambda c: "x".join(map(str, c)))
def test_partial_matches_oracle(case, causal, dtype):
    B, H, Nq, Nk, d, qp, kp = case
    say(f"fa_fwd_partial {case} causal={causal} {dtype}")
    q, k, v, _ = inputs(B, H, Nq, Nk, d, dtype, seed=Nq + Nk)
    o, lse = run_partial(q, k, v, d ** -0.5, causal, qp, kp)
    o_ref, lse_ref = attn_part64(q, k, v, d ** -0.5, causal, qp, kp)
    check(o, lse, o_ref, lse_ref)


def test_partial_key_padding_and_empty_parts():
    say("fa_fwd_partial kv_len, Nk = 0, keys all in the future")
    q, k, v, kv = inputs(3, 2, 150, 200, 64, "bf16", seed=5, kv_len=[0, 77, 500])
    o, lse = run_partial(q, k, v, 0.125, True, 300, 0, kv)
    o_ref, lse_ref = attn_part64(q, k, v, 0.125, True, 300, 0, kv)
    check(o, lse, o_ref, lse_ref)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    o, lse = run_partial(q, k[:, :, :0], v[:, :, :0], 0.125, False, 0, 0)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    o, lse = run_partial(q, k, v, 0.125, True, 0, 150)  # every key after every query
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("out", ["fp32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_merge_of_two_key_halves_is_full_attention(causal, out):
    say(f"fa_merge of key halves causal={causal} out={out}")
    B, H, N, d = 1, 3, 300, 128
    q, k, v, _ = inputs(B, H, N, N, d, "bf16", seed=11)
    cut = 128
    oa, la = run_partial(q, k[:, :, :cut], v[:, :, :cut], d ** -0.5, causal, 0, 0)
    ob, lb = run_partial(q, k[:, :, cut:], v[:, :, cut:], d ** -0.5, causal, 0, cut)
    o = torch.empty(B, H, N, d, dtype=torch.float32 if out == "fp32" else torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, N, device="cuda")
    fa_merge(oa, la, ob, lb, o, lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = attn_fwd64(q, k, v, d ** -0.5, causal)
    if out == "fp32":
        check(o, lse, o_ref, lse_ref)
    else:
        st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
        floor_max, floor_mean = rounding_floor(o_ref, torch.bfloat16)
        assert st["max_abs"] <= floor_max + FWD_MAX_ABS and st["mean_abs"] <= floor_mean + FWD_MEAN_ABS, st
        assert st["lse_max_abs"] <= LSE_MAX_ABS, st


def test_merge_in_place_against_oracle_merge():
    say("fa_merge in place on random parts, with empty rows")
    g = torch.Generator().manual_seed(3)
    rows, d = 1000, 64
    oa, ob = torch.randn(rows, d, generator=g), torch.randn(rows, d, generator=g)
    la, lb = 5 * torch.randn(rows, generator=g), 5 * torch.randn(rows, generator=g)
    la[::7] = -float("inf")
    lb[::7] = -float("inf")   # rows 0, 7, ... empty in both
    lb[3::11] = -float("inf")
    o_ref, l_ref = merge64([oa.numpy(), ob.numpy()], [la.numpy(), lb.numpy()])
    oa_d, la_d, ob_d, lb_d = dev(oa), dev(la), dev(ob), dev(lb)
    fa_merge(oa_d, la_d, ob_d, lb_d, oa_d, la_d)
    torch.cuda.synchronize()
    np.testing.assert_allclose(np64(oa_d), o_ref, rtol=0, atol=1e-5)
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(np64(la_d)))
    np.testing.assert_allclose(np64(la_d)[fin], l_ref[fin], rtol=0, atol=1e-5)
    assert torch.all(oa_d[::7] == 0)


def test_ring_schedule_matches_full_causal_forward():
    say("ring schedule: 4 query shards x 4 key shards, merged in place")
    B, H, N, d = 1, 2, 1024, 64
    q, k, v, _ = inputs(B, H, N, N, d, "bf16", seed=21)
    n = N // 4
    o_ref, lse_ref = attn_fwd64(q, k, v, 0.125, True)
    for r in range(4):
        qs = q[:, :, r * n:(r + 1) * n].contiguous()
        acc_o, acc_l = run_partial(qs, k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), 0.125, True, r * n, 0)
        for s in range(1, 4):
            po, pl = run_partial(qs, k[:, :, s * n:(s + 1) * n].contiguous(),
                                 v[:, :, s * n:(s + 1) * n].contiguous(), 0.125, True, r * n, s * n)
            fa_merge(acc_o, acc_l, po, pl, acc_o, acc_l)
        torch.cuda.synchronize()
        check(acc_o, acc_l, o_ref[:, :, r * n:(r + 1) * n], lse_ref[:, :, r * n:(r + 1) * n])


# (B, H, N, d, num_splits)
SPLIT = [(1, 2, 1000, 64, 4), (1, 1, 4096, 128, 8), (2, 2, 333, 64, 16), (1, 3, 65, 128, 2),
         (1, 2, 64, 64, 8), (1, 1, 2049, 64, 3)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SPLIT, ids=lambda c: "x".join(map(str, c)))
def test_split_forward_matches_oracle(case, causal, dtype):
    B, H, N, d, S = case
    say(f"fa_fwd_split {case} causal={causal} {dtype}")
    q, k, v, _ = inputs(B, H, N, N, d, dtype, seed=N + S)
    o32 = torch.empty(B, H, N, d, device="cuda")
    lse = torch.empty(B, H, N, device="cuda")
    fa_fwd_split(dev(q), dev(k), dev(v), o32, lse, d ** -0.5, causal, None, S)
    o16 = torch.empty(B, H, N, d, dtype=TORCH[dtype], device="cuda")
    lse16 = torch.empty(B, H, N, device="cuda")
    fa_fwd_split(dev(q), dev(k), dev(v), o16, lse16, d ** -0.5, causal, None, S)
    torch.cuda.synchronize()
    o_ref, lse_ref = attn_fwd64(q, k, v, d ** -0.5, causal)
    check(o32, lse, o_ref, lse_ref)
    st = fwd_stats(np64(o16), np64(lse16), o_ref, lse_ref)
    floor_max, floor_mean = rounding_floor(o_ref, TORCH[dtype])
    assert st["max_abs"] <= floor_max + FWD_MAX_ABS and st["mean_abs"] <= floor_mean + FWD_MEAN_ABS, st


def test_split_forward_key_padding():
    say("fa_fwd_split with kv_len, 5 parts")
    w = W.BERT
    inp = W.make_inputs(w)
    q, k, v, kv = (inp[n][:4] for n in ("q", "k", "v", "kv_len"))
    kv = kv.clone()
    kv[0] = 0
    o = torch.empty(q.shape, device="cuda")
    lse = torch.empty(q.shape[:3], device="cuda")
    fa_fwd_split(dev(q), dev(k), dev(v), o, lse, w.scale, False, dev(kv), 5)
    torch.cuda.synchronize()
    o_ref, lse_ref = attn_fwd64(q, k, v, w.scale, False, kv_len=kv)
    check(o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("parts", [2, 8])
def test_split_forward_agrees_with_forward_at_long_keys(parts):
    # the few-heads measurement shape, from the workload generator
    w = W.FEW_HEADS
    say(f"fa_fwd_split vs fa_fwd, {w.note}, {parts} parts")
    B, H, N, d = w.B, w.H, w.N, w.d
    inp = W.make_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    qd, kd, vd = dev(q), dev(k), dev(v)
    o1 = torch.empty(B, H, N, d, device="cuda")
    l1 = torch.empty(B, H, N, device="cuda")
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    fa_fwd(qd, kd, vd, o1, l1, d ** -0.5, True)
    fa_fwd_split(qd, kd, vd, o2, l2, d ** -0.5, True, None, parts)
    torch.cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 2e-3
    assert float((l1 - l2).abs().max()) <= 1e-4
    rows = np.array([0, 1, 4095, 4096, 9000, 16383])
    o_ref, lse_ref = attn_fwd64(q, k, v, d ** -0.5, True, rows=rows)
    check(o2[:, :, rows], l2[:, :, rows], o_ref, lse_ref)
