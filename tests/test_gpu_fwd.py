"""Forward parity of the HIP path (through the C ABI) against the fp64 oracle.

bf16/fp16: judged on the fp32-output mode (same kernel, fp32 store) at
max |err| <= 1e-2, mean |err| <= 1e-3, LSE <= 1e-3; the storage-dtype output
is held to the exact output's own rounding floor plus the same margins.
fp32: max |err| <= 1e-5 on O and LSE.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import workloads as W
from oracle import attn_fwd64
from tests.helpers import (F32_MAX_ABS, FWD_MAX_ABS, FWD_MEAN_ABS, LSE_MAX_ABS, fwd_stats, np64,
                           rounding_floor, run_fwd, say)

pytestmark = pytest.mark.gpu


def _check_16bit(inp, scale, causal, rows=None, heads=None, label=""):
    o32, lse = run_fwd(inp, scale, causal, out_dtype=torch.float32)
    o16, lse16 = run_fwd(inp, scale, causal)
    assert torch.equal(lse, lse16), "LSE must not depend on the output dtype"
    o_ref, lse_ref = attn_fwd64(inp["q"], inp["k"], inp["v"], scale, causal, inp.get("kv_len"),
                                rows=rows, heads=heads)
    g32, g16, gl = np64(o32), np64(o16), np64(lse)
    if heads is not None:
        g32 = np.stack([g32[b, h] for b, h in heads])
        g16 = np.stack([g16[b, h] for b, h in heads])
        gl = np.stack([gl[b, h] for b, h in heads])
    if rows is not None:
        g32, g16, gl = g32[..., rows, :], g16[..., rows, :], gl[..., rows]
    st = fwd_stats(g32, gl, o_ref, lse_ref)
    print(f"{label} fp32-out {st}", flush=True)
    assert st["max_abs"] <= FWD_MAX_ABS and st["mean_abs"] <= FWD_MEAN_ABS
    assert st["lse_max_abs"] <= LSE_MAX_ABS
    floor_max, floor_mean = rounding_floor(o_ref, inp["q"].dtype)
    st16 = fwd_stats(g16, gl, o_ref, lse_ref)
    print(f"{label} storage-out {st16} floor max {floor_max:.3g} mean {floor_mean:.3g}", flush=True)
    assert st16["max_abs"] <= floor_max + FWD_MAX_ABS
    assert st16["mean_abs"] <= floor_mean + FWD_MEAN_ABS
    return st, st16


SMALL = [(2, 3, n, d) for n in (1, 17, 127, 129, 200, 513) for d in (64, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_forward_small_shapes(shape, causal, dtype):
    B, H, N, d = shape
    say(f"fwd {shape} {dtype} causal={causal}")
    inp = W.random_case(B, H, N, d, dtype, seed=N * 7 + d, causal=causal)
    _check_16bit(inp, d ** -0.5, causal, label=str(shape))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_key_padding_with_empty_and_clamped_lengths(d, causal):
    N = 300
    kv = [0, 1, 129, 300, 1000]  # 0: no visible key; 1000 clamps to N
    say(f"fwd kv_len {kv} d={d} causal={causal}")
    inp = W.random_case(5, 2, N, d, "bf16", seed=11, causal=causal, kv_len=kv)
    _check_16bit(inp, d ** -0.5, causal, label="kv")
    o, lse = run_fwd(inp, d ** -0.5, causal, out_dtype=torch.float32)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.isfinite(o).all()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 64), (2, 1, 33, 64), (1, 2, 257, 128), (2, 2, 300, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forward_fp32_path(shape, causal):
    B, H, N, d = shape
    say(f"fwd fp32 {shape} causal={causal}")
    inp = W.random_case(B, H, N, d, "fp32", seed=5 + N, causal=causal,
                        kv_len=[max(1, N - 3)] + [N] * (B - 1))
    o, lse = run_fwd(inp, d ** -0.5, causal)
    o_ref, lse_ref = attn_fwd64(inp["q"], inp["k"], inp["v"], d ** -0.5, causal, inp["kv_len"])
    st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
    print(st, flush=True)
    assert st["max_abs"] <= F32_MAX_ABS and st["lse_max_abs"] <= F32_MAX_ABS


def test_config_tiny_fp32():
    w = W.TINY
    say(w.name)
    inp = W.make_inputs(w)
    o, lse = run_fwd(inp, w.scale, w.causal)
    o_ref, lse_ref = attn_fwd64(inp["q"], inp["k"], inp["v"], w.scale, w.causal)
    st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
    print(st, flush=True)
    assert st["max_abs"] <= F32_MAX_ABS and st["lse_max_abs"] <= F32_MAX_ABS


def test_config_bert_large_fp16_key_padding():
    w = W.BERT
    say(w.name)
    _check_16bit(W.make_inputs(w), w.scale, w.causal, label=w.name)


def test_config_long_context_bf16():
    w = W.LONG
    say(w.name)
    _check_16bit(W.make_inputs(w), w.scale, w.causal, label=w.name)


def test_config_trading_day_bf16_causal_sampled_rows():
    w = W.TRADE
    say(w.name)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 23295, 23296, 23399],
                                     rng.choice(w.N, 250, replace=False)]))
    heads = [(0, h) for h in range(w.H)]
    _check_16bit(W.make_inputs(w), w.scale, w.causal, rows=rows, heads=heads, label=w.name)


def test_config_gpt2_forward():
    w = W.GPT2
    say(w.name)
    _check_16bit(W.make_inputs(w), w.scale, w.causal, label=w.name)


def test_forward_is_deterministic():
    w = W.LONG.with_(H=4, N=1000)
    say("fwd determinism")
    inp = W.make_inputs(w)
    a = run_fwd(inp, w.scale, False)
    b = run_fwd(inp, w.scale, False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_large_logits_stress_running_max():
    # keys shifted far from zero and a few huge rows: the running max jumps
    # several times inside one row
    say("fwd large logits")
    inp = W.random_case(1, 4, 700, 128, "fp32", seed=3)
    k = inp["k"] + 6.0
    k[:, :, ::97] *= 12.0
    v = inp["v"]
    for dt in (torch.bfloat16, torch.float16):
        case = {"q": inp["q"].to(dt), "k": k.to(dt), "v": v.to(dt), "kv_len": None}
        _check_16bit(case, 128 ** -0.5, False, label=f"large-logits {dt}")
        _check_16bit(case, 128 ** -0.5, True, label=f"large-logits causal {dt}")
