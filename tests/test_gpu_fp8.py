"""GPU parity of the FP8 forward with incoherent processing through the C ABI,
against the oracle's step-by-step statement of it (oracle/fp8.py).

  * Quantisation is integer work: the codes of Q, K and V^T and the fp32
    block scales must equal the oracle's bit for bit (with and without the
    rotation, ragged N, both head dims).
  * Attention on those codes is compared with the oracle's tiled FP8
    attention on its own codes (equal to the GPU's, by the first test). The
    remaining differences come from the fp32 arithmetic of the kernel (the
    hardware exponential, and the FP8 matrix cores' accumulation, measured
    at up to 2e-4 of the sum of magnitudes on random codes) and from the
    rare P whose 256 p falls within that error of a rounding midpoint, which
    moves O by at most max|V| / 16 times that key's weight. Tolerance: O
    max |err| <= 2e-2 and mean <= 1e-3, LSE max |err| <= 1e-3. The seeded
    sweep also reaches short causal rows, where one key carries much of the
    weight. There a row may differ by 2e-2 plus the largest change one code
    left open by that accumulation error can make (the oracle's flip bound,
    S_ERR = 2e-4); every other code is unique.
  * End to end against exact attention: the error the method trades for
    speed, and the rotation lowering it on inputs with outlier channels.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import (fa_fp8_quantize, fa_fwd, fa_fwd_fp8, fa_fwd_fp8_incoherent,
                                   fp8_buffers)
from exact_io_aware_07_amd import workloads as W
from helpers import dev, fwd_stats, np64, say
from oracle import attn_fwd64, attn_fwd64_fp8, fp8_quantize

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 1e-3, 1e-3
S_ERR = 2e-4  # score accumulation error of the FP8 products, per sum of |products|


def gpu_quantize(inp, signs):
    q, k, v = (dev(inp[n]) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    bufs = fp8_buffers(B, H, N, d)
    fa_fp8_quantize(q, k, v, dev(signs), bufs)
    torch.cuda.synchronize()
    return bufs


SHAPES = [(1, 2, 300, 64), (2, 1, 129, 128), (1, 1, 64, 128), (1, 3, 1000, 64), (1, 1, 1, 64)]


@pytest.mark.parametrize("rot", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_quantisation_is_bit_exact(shape, dtype, rot):
    B, H, N, d = shape
    say(f"fp8 quantise {shape} {dtype} rot={rot}")
    inp = W.random_case(B, H, N, d, dtype, seed=N + d)
    signs = W.random_signs(d, seed=d) if rot else None
    bufs = gpu_quantize(inp, signs)
    ref = fp8_quantize(inp["q"], inp["k"], inp["v"], None if signs is None else signs.numpy())
    np.testing.assert_array_equal(bufs["q8"].cpu().numpy(), ref["q8"])
    np.testing.assert_array_equal(bufs["k8"].cpu().numpy(), ref["k8"])
    vt = bufs["vt8"].cpu().numpy()
    np.testing.assert_array_equal(np.swapaxes(vt[..., :N], -1, -2), ref["v8"])
    assert np.all(vt[..., N:] == 0)
    np.testing.assert_array_equal(bufs["q_scale"].cpu().numpy(), ref["sq"])
    np.testing.assert_array_equal(bufs["k_scale"].cpu().numpy(), ref["sk"])
    np.testing.assert_array_equal(bufs["v_scale"].cpu().numpy(), ref["sv"])


def test_quantisation_of_zero_blocks_and_outliers():
    say("fp8 quantise zero block, outlier channels")
    inp = W.random_case(1, 2, 200, 128, "bf16", seed=4)
    inp["q"][0, 0, 128:] = 0          # a zero query block
    inp["k"][0, 1, :64] = 0           # a zero key block
    inp["v"][0, 1] = 0                # a zero V head
    inp["k"][0, 0, :, 5] *= 64        # an outlier channel
    signs = W.random_signs(128, seed=5)
    bufs = gpu_quantize(inp, signs)
    ref = fp8_quantize(inp["q"], inp["k"], inp["v"], signs.numpy())
    for name, key in (("q8", "q8"), ("k8", "k8"), ("q_scale", "sq"), ("k_scale", "sk"), ("v_scale", "sv")):
        np.testing.assert_array_equal(bufs[name].cpu().numpy(), ref[key])
    assert bufs["q_scale"][0, 0, 1] == 0 and bufs["k_scale"][0, 1, 0] == 0 and bufs["v_scale"][0, 1] == 0


CASES = [(1, 2, 300, 64, False), (2, 1, 129, 128, True), (1, 2, 520, 128, False), (1, 2, 700, 64, True)]


@pytest.mark.parametrize("rot", [True, False])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_attention_on_codes_matches_oracle(case, rot):
    B, H, N, d, causal = case
    say(f"fp8 attention {case} rot={rot}")
    inp = W.random_case(B, H, N, d, "bf16", seed=3 * N + d)
    signs = W.random_signs(d, seed=d + 1) if rot else None
    bufs = gpu_quantize(inp, signs)
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa_fwd_fp8(bufs, rot, o, lse, d ** -0.5, causal)
    torch.cuda.synchronize()
    qz = fp8_quantize(inp["q"], inp["k"], inp["v"], None if signs is None else signs.numpy())
    o_ref, lse_ref = attn_fwd64_fp8(qz, d ** -0.5, causal)
    st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
    print(f"{case} rot={rot} {st}", flush=True)
    assert st["max_abs"] <= O_MAX and st["mean_abs"] <= O_MEAN and st["lse_max_abs"] <= LSE_MAX, st


@pytest.mark.parametrize("causal", [False, True])
def test_key_padding_and_empty_rows(causal):
    B, H, N, d = 3, 2, 300, 64
    kv = [0, 1, 250]
    say(f"fp8 kv_len {kv} causal={causal}")
    inp = W.random_case(B, H, N, d, "fp16", seed=9, kv_len=kv)
    signs = W.random_signs(d, seed=2)
    bufs = gpu_quantize(inp, signs)
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa_fwd_fp8(bufs, True, o, lse, 0.125, causal, dev(inp["kv_len"]))
    torch.cuda.synchronize()
    qz = fp8_quantize(inp["q"], inp["k"], inp["v"], signs.numpy())
    o_ref, lse_ref = attn_fwd64_fp8(qz, 0.125, causal, kv)
    st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
    assert st["max_abs"] <= O_MAX and st["mean_abs"] <= O_MEAN and st["lse_max_abs"] <= LSE_MAX, st
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_one_call_path_equals_the_two_steps(out):
    B, H, N, d = 1, 2, 333, 128
    say(f"fp8 one call vs two steps out={out}")
    inp = W.random_case(B, H, N, d, "bf16", seed=21)
    signs = W.random_signs(d, seed=22)
    q, k, v = (dev(inp[n]) for n in ("q", "k", "v"))
    dt = torch.float32 if out == "fp32" else torch.bfloat16
    o1, o2 = (torch.empty((B, H, N, d), dtype=dt, device="cuda") for _ in range(2))
    l1, l2 = (torch.empty((B, H, N), dtype=torch.float32, device="cuda") for _ in range(2))
    fa_fwd_fp8_incoherent(q, k, v, dev(signs), o1, l1, 0.1, True)
    bufs = gpu_quantize(inp, signs)
    fa_fwd_fp8(bufs, True, o2, l2, 0.1, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_end_to_end_error_and_the_rotation_on_outlier_channels():
    """FP8 against exact fp64 attention at the measurement shape (sampled
    rows of four heads): the error is bounded, and on these inputs with
    outlier channels the rotation lowers it (the claim of the pages)."""
    w = W.FP8
    say(f"fp8 end to end {w.name}")
    inp = W.make_inputs(w, seed=0)
    q, k, v = (dev(inp[n]) for n in ("q", "k", "v"))
    signs = dev(W.random_signs(w.d, seed=0))
    rows = list(range(0, w.N, 97))
    heads = [(0, h) for h in (0, 7, 19, 31)]
    o_ref, lse_ref = attn_fwd64(inp["q"], inp["k"], inp["v"], w.scale, w.causal, rows=rows, heads=heads)
    errs = {}
    for name, sg in (("rotated", signs), ("plain", None)):
        o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        fa_fwd_fp8_incoherent(q, k, v, sg, o, lse, w.scale, w.causal)
        torch.cuda.synchronize()
        got = np.stack([np64(o[b, h, rows]) for b, h in heads])
        errs[name] = float(np.sqrt(np.mean((got - o_ref) ** 2)))
    o16 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    l16 = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    fa_fwd(q, k, v, o16, l16, w.scale, w.causal)
    torch.cuda.synchronize()
    got16 = np.stack([np64(o16[b, h, rows]) for b, h in heads])
    errs["bf16"] = float(np.sqrt(np.mean((got16 - o_ref) ** 2)))
    print(f"rms error vs exact: {errs}, plain / rotated = {errs['plain'] / errs['rotated']:.2f}", flush=True)
    # The oracle's own FP8 steps on this input recipe (H=4, N=1024) give an
    # rms error of 0.076 rotated and 0.29 without the rotation (O has rms
    # 0.96; the outlier channels make the scores large, and e4m3 keeps 3
    # mantissa bits of each). Bounds: twice that, and a rotation that at
    # least halves the error.
    assert errs["rotated"] < 0.15
    assert errs["rotated"] < 0.5 * errs["plain"]


def test_long_sequence_codes_and_sampled_rows():
    """N = 131,072 at d = 128 (1,024 query blocks, 2,048 key scales, a V^T
    row of 131,072 codes): codes and scales bit for bit, and O, LSE of
    sampled rows against the oracle's FP8 attention on the same codes."""
    B, H, N, d = 1, 1, 1 << 17, 128
    say(f"fp8 long N={N}")
    inp = W.random_case(B, H, N, d, "bf16", seed=71)
    signs = W.random_signs(d, seed=72)
    bufs = gpu_quantize(inp, signs)
    ref = fp8_quantize(inp["q"], inp["k"], inp["v"], signs.numpy())
    np.testing.assert_array_equal(bufs["q8"].cpu().numpy(), ref["q8"])
    np.testing.assert_array_equal(bufs["k8"].cpu().numpy(), ref["k8"])
    np.testing.assert_array_equal(np.swapaxes(bufs["vt8"].cpu().numpy()[..., :N], -1, -2), ref["v8"])
    for name, key in (("q_scale", "sq"), ("k_scale", "sk"), ("v_scale", "sv")):
        np.testing.assert_array_equal(bufs[name].cpu().numpy(), ref[key])
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa_fwd_fp8(bufs, True, o, lse, d ** -0.5, True)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 65535, 65536, N - 65, N - 1]
    o_ref, lse_ref = attn_fwd64_fp8(ref, d ** -0.5, True, rows=rows)
    st = fwd_stats(np64(o[:, :, rows]), np64(lse[:, :, rows]), o_ref, lse_ref)
    print(f"N={N} {st}", flush=True)
    assert st["max_abs"] <= O_MAX and st["mean_abs"] <= O_MEAN and st["lse_max_abs"] <= LSE_MAX, st


def _fp8_draw(i: int) -> dict:
    """Case i of the FP8 sweep, from its own seeded generator."""
    import random
    r = random.Random(104729 * i + 3)
    N = r.choice([1, 16, 63, 64, 65, 127, 128, 129, 200, 257, 383, 500, 777, 1024, 1300, 2049])
    B = r.randint(1, 3)
    kv = None
    if r.random() < 0.4:
        kv = [r.choice([0, 1, N // 2, N - 1, N]) for _ in range(B)]
    return {"i": i, "B": B, "H": r.randint(1, 3), "N": N, "d": r.choice([64, 128]),
            "causal": r.random() < 0.5, "rot": r.random() < 0.7, "kv": kv,
            "dtype": r.choice(["bf16", "fp16"])}


FP8_SWEEP = [_fp8_draw(i) for i in range(60)]


@pytest.mark.parametrize("c", FP8_SWEEP, ids=lambda c: f"{c['i']}-{c['B']}x{c['H']}x{c['N']}x{c['d']}"
                         f"-{c['dtype']}-c{int(c['causal'])}-r{int(c['rot'])}")
def test_fp8_sweep_case(c):
    """Seeded random shapes, tails, key lengths, causal flags and rotations:
    codes and scales bit-exact, attention on them within the bounds above."""
    B, H, N, d, kv = c["B"], c["H"], c["N"], c["d"], c["kv"]
    say(f"fp8 sweep {c}")
    inp = W.random_case(B, H, N, d, c["dtype"], seed=7000 + c["i"], kv_len=kv)
    signs = W.random_signs(d, seed=7500 + c["i"]) if c["rot"] else None
    bufs = gpu_quantize(inp, signs)
    ref = fp8_quantize(inp["q"], inp["k"], inp["v"], None if signs is None else signs.numpy())
    np.testing.assert_array_equal(bufs["q8"].cpu().numpy(), ref["q8"])
    np.testing.assert_array_equal(bufs["k8"].cpu().numpy(), ref["k8"])
    np.testing.assert_array_equal(np.swapaxes(bufs["vt8"].cpu().numpy()[..., :N], -1, -2), ref["v8"])
    for name, key in (("q_scale", "sq"), ("k_scale", "sk"), ("v_scale", "sv")):
        np.testing.assert_array_equal(bufs[name].cpu().numpy(), ref[key])
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    kvt = None if kv is None else dev(inp["kv_len"])
    fa_fwd_fp8(bufs, c["rot"], o, lse, d ** -0.5, c["causal"], kvt)
    torch.cuda.synchronize()
    o_ref, lse_ref, flip = attn_fwd64_fp8(ref, d ** -0.5, c["causal"], kv, s_err=S_ERR)
    st = fwd_stats(np64(o), np64(lse), o_ref, lse_ref)
    err_row = np.abs(np64(o) - o_ref).max(axis=-1)
    worst = np.unravel_index(int(np.argmax(err_row - flip)), err_row.shape)
    print(f"{c} {st} worst row {worst}: err {err_row[worst]:.3e} flip bound {flip[worst]:.3e}",
          flush=True)
    assert np.all(err_row <= O_MAX + flip), (worst, err_row[worst], flip[worst])
    assert st["mean_abs"] <= O_MEAN and st["lse_max_abs"] <= LSE_MAX, st
    if kv is not None:
        for b, L in enumerate(kv):
            if L == 0:
                assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))
