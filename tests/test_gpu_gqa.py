"""GPU parity of grouped-query attention (fa_fwd_gqa, fa_bwd_gqa) through the
C ABI, against the fp64 oracle (oracle/gqa.py, and oracle/attention.py on
one K/V head's group at full size).

Besides the oracle, two exact properties are checked: with Hkv = H the
entry points are fa_fwd / fa_bwd bit for bit, and the forward (and dQ) of a
grouped call equal, bit for bit, the plain call on K/V repeated over the
group, since each query head's arithmetic does not depend on which buffer
its K/V head is read from.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import fa_bwd, fa_bwd_gqa, fa_bwd_gqa_workspace_bytes, fa_fwd, fa_fwd_gqa
from exact_io_aware_07_amd import workloads as W
from helpers import (FWD_MAX_ABS, FWD_MEAN_ABS, GRAD_REL_FRO, LSE_MAX_ABS, dev, fwd_stats, np64,
                     rel_fro, say)
from oracle import attn_bwd64_gqa, attn_bwd64_sampled, attn_fwd64, attn_fwd64_gqa

pytestmark = pytest.mark.gpu


def fwd(q, k, v, scale, causal, kv=None, out_dtype=None):
    B, H, N, d = q.shape
    o = torch.empty(q.shape, dtype=out_dtype or q.dtype, device="cuda")
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    fa_fwd_gqa(q, k, v, o, lse, scale, causal, kv)
    torch.cuda.synchronize()
    return o, lse


def bwd(q, k, v, o, do, lse, scale, causal, kv=None):
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    fa_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, scale, causal, kv)
    torch.cuda.synchronize()
    return dq, dk, dv


def gpu_inputs(inp):
    return [dev(inp[n]) for n in ("q", "k", "v", "do", "kv_len")]


# (B, H, Hkv, N, d): groups of 2, 3, 4 and 8 (multi-query), ragged tails,
# several key blocks, both head dims
SHAPES = [
    (2, 4, 2, 129, 64),
    (1, 6, 2, 300, 128),
    (2, 6, 3, 77, 64),
    (1, 8, 1, 257, 64),
    (1, 8, 1, 200, 128),
    (3, 4, 1, 1, 64),
    (1, 16, 4, 520, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gqa_forward_and_backward_match_oracle(shape, causal, dtype):
    B, H, Hkv, N, d = shape
    say(f"gqa fwd+bwd {shape} causal={causal} {dtype}")
    inp = W.random_case(B, H, N, d, dtype, seed=N + 7 * Hkv, causal=causal, backward=True, Hkv=Hkv)
    q, k, v, do, _ = gpu_inputs(inp)
    scale = d ** -0.5
    o, lse = fwd(q, k, v, scale, causal)
    o_ref, lse_ref = attn_fwd64_gqa(inp["q"], inp["k"], inp["v"], scale, causal)
    st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
    assert st["max_abs"] <= FWD_MAX_ABS and st["mean_abs"] <= FWD_MEAN_ABS, st
    assert st["lse_max_abs"] <= LSE_MAX_ABS, st
    grads = bwd(q, k, v, o, do, lse, scale, causal)
    ref = attn_bwd64_gqa(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    errs = {n: rel_fro(np64(g), r) for n, g, r in zip(("dq", "dk", "dv"), grads, ref)}
    print(f"{shape} rel-fro {errs}", flush=True)
    for n, e in errs.items():
        assert e <= GRAD_REL_FRO, (n, e)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_key_padding(causal):
    kv_len = [0, 1, 150, 300]
    B, H, Hkv, N, d = 4, 4, 2, 300, 64
    say(f"gqa kv_len {kv_len} causal={causal}")
    inp = W.random_case(B, H, N, d, "bf16", seed=11, causal=causal, kv_len=kv_len,
                        backward=True, Hkv=Hkv)
    q, k, v, do, kv = gpu_inputs(inp)
    scale = d ** -0.5
    o, lse = fwd(q, k, v, scale, causal, kv)
    o_ref, lse_ref = attn_fwd64_gqa(inp["q"], inp["k"], inp["v"], scale, causal, inp["kv_len"])
    st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
    assert st["max_abs"] <= FWD_MAX_ABS and st["mean_abs"] <= FWD_MEAN_ABS, st
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    dq, dk, dv = bwd(q, k, v, o, do, lse, scale, causal, kv)
    ref = attn_bwd64_gqa(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, inp["kv_len"])
    for n, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        e = rel_fro(np64(g), r)
        assert e <= GRAD_REL_FRO, (n, e)
    for b, L in enumerate(kv_len):
        assert torch.all(dk[b, :, L:] == 0) and torch.all(dv[b, :, L:] == 0)
    assert torch.all(dq[0] == 0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_gqa_with_one_group_is_plain_attention_bit_for_bit(d, causal):
    B, H, N = 2, 3, 333
    say(f"gqa Hkv=H vs fa_fwd/fa_bwd d={d} causal={causal}")
    inp = W.random_case(B, H, N, d, "bf16", seed=d + causal, causal=causal, backward=True)
    q, k, v, do, _ = gpu_inputs(inp)
    scale = d ** -0.5
    o, lse = fwd(q, k, v, scale, causal)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    fa_fwd(q, k, v, o2, lse2, scale, causal)
    g1 = bwd(q, k, v, o, do, lse, scale, causal)
    g2 = [torch.empty_like(t) for t in (q, k, v)]
    fa_bwd(q, k, v, o, do, lse, *g2, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward_equals_plain_call_on_repeated_heads(causal):
    B, H, Hkv, N, d = 2, 8, 2, 400, 64
    G = H // Hkv
    say(f"gqa vs repeated K/V causal={causal}")
    inp = W.random_case(B, H, N, d, "bf16", seed=99, causal=causal, backward=True, Hkv=Hkv)
    q, k, v, do, _ = gpu_inputs(inp)
    kr = k.repeat_interleave(G, dim=1).contiguous()
    vr = v.repeat_interleave(G, dim=1).contiguous()
    scale = d ** -0.5
    o, lse = fwd(q, k, v, scale, causal)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    fa_fwd(q, kr, vr, o2, lse2, scale, causal)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    dq, dk, dv = bwd(q, k, v, o, do, lse, scale, causal)
    dq2, dk2, dv2 = (torch.empty_like(t) for t in (q, kr, vr))
    fa_bwd(q, kr, vr, o, do, lse, dq2, dk2, dv2, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2)
    # dK/dV: the grouped call sums the group in fp32 before one rounding; the
    # plain call rounds each head's share first. Both are near the fp64 sum.
    ref = attn_bwd64_gqa(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    sums = [np64(t).reshape(B, Hkv, G, N, d).sum(axis=2) for t in (dk2, dv2)]
    for got, plain, r in zip((dk, dv), sums, ref[1:]):
        assert rel_fro(np64(got), r) <= rel_fro(plain, r) * 1.5 + 1e-3


def shares(w) -> int:
    """Query-head shares the grouped dK/dV stage uses for ``w`` (read back
    from the workspace size: D per query row, then 2 fp32 tensors per share)."""
    extra = fa_bwd_gqa_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.d) - w.B * w.H * w.N * 4
    return max(extra // (2 * w.B * w.kv_heads * w.N * w.d * 4), 1)


# The measured shape (each group on one workgroup per key block), one
# sequence (groups in two shares) and groups of eight on one sequence (four
# shares): the reduction of fp32 shares is exercised at full size too.
FULL = [dict(), dict(B=1), dict(B=1, Hkv=4)]


@pytest.mark.parametrize("kw", FULL, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()) or "base")
def test_gqa_full_size_sampled_against_oracle(kw):
    """B=2 H=32 Hkv=8 N=4096 d=128 bf16 causal (and the variants above): O
    and LSE on sampled rows, dQ, dK, dV on sampled rows and keys of the first
    and last K/V head's group, whose dK/dV sum over the group's query heads."""
    w = W.GQA.with_(**kw)
    say(f"gqa full size {w.name} {kw} shares={shares(w)}")
    inp = W.make_inputs(w, seed=0)
    q, k, v, do, _ = gpu_inputs(inp)
    scale = w.scale
    o, lse = fwd(q, k, v, scale, w.causal)
    dq, dk, dv = bwd(q, k, v, o, do, lse, scale, w.causal)
    G = w.H // w.kv_heads
    rows = [0, 1, 63, 64, 1000, 2047, 2048, 3333, w.N - 2, w.N - 1]
    groups = [(0, 0), (w.B - 1, w.kv_heads - 1)] if not kw else [(w.B - 1, w.kv_heads - 1)]
    for b, hk in groups:
        hs = slice(hk * G, (hk + 1) * G)
        qg, dog = inp["q"][b:b + 1, hs], inp["do"][b:b + 1, hs]
        kg = inp["k"][b:b + 1, hk:hk + 1].repeat_interleave(G, dim=1)
        vg = inp["v"][b:b + 1, hk:hk + 1].repeat_interleave(G, dim=1)
        o_ref, lse_ref = attn_fwd64(qg, kg, vg, scale, w.causal, rows=rows)
        st = fwd_stats(np64(o[b:b + 1, hs, rows]), np64(lse[b:b + 1, hs, rows]), o_ref, lse_ref)
        assert st["max_abs"] <= FWD_MAX_ABS and st["lse_max_abs"] <= LSE_MAX_ABS, st
        heads = [(0, g) for g in range(G)]
        dq_ref, dk_ref, dv_ref = attn_bwd64_sampled(qg, kg, vg, dog, scale, w.causal, heads=heads,
                                                    q_rows=rows, k_rows=rows)
        e_q = rel_fro(np64(dq[b, hs][:, rows]), np.asarray(dq_ref))
        e_k = rel_fro(np64(dk[b, hk, rows]), np.asarray(dk_ref).sum(axis=0))
        e_v = rel_fro(np64(dv[b, hk, rows]), np.asarray(dv_ref).sum(axis=0))
        print(f"b={b} kv head {hk}: dq {e_q:.2e} dk {e_k:.2e} dv {e_v:.2e}", flush=True)
        assert max(e_q, e_k, e_v) <= GRAD_REL_FRO
