"""GPU parity of the FP8 forward with incoherent processing through the C ABI,
against the oracle's step-by-step statement of it (oracle/fp8.py).

  * Quantisation is integer work: the codes of Q, K and V^T and the fp32
    block scales must equal the oracle's bit for bit (with and without the
    rotation, ragged N, both head dims).
  * Attention on those codes is compared with the oracle's tiled FP8
    attention on its own codes (equal to the GPU's, by the first test),
    element by element against the bound the oracle derives for an
    implementation of the same steps on the FP8 matrix cores with fp32
    arithmetic elsewhere (attn_fwd64_fp8 with trunc): the matrix cores add
    products in aligned groups of 8 and cut the smaller products of a group
    to a granularity of at most TRUNC times its largest; fp32 rounding of
    the scales, exponentials and rescales; and every P code whose 256 p lies
    within those errors of a rounding boundary (each may be decided either
    way; the bound sums their moves). On top of it: O mean |err| <= 1e-3 and
    LSE max |err| <= 1e-3.
  * That model of the matrix cores is pinned by three tests whose inputs
    isolate one product sum: the grouping itself (two large products among
    small ones), then the losses of scores (rows with one visible key, so
    LSE is the score) and of P V sums (all keys equal, so every P code is
    256) on random and crafted codes, each within the model's bound.
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
from oracle import attn_fwd64, attn_fwd64_fp8, e4m3_decode, fp8_quantize, mfma_loss_bound

pytestmark = pytest.mark.gpu

O_MEAN, LSE_MAX = 1e-3, 1e-3
# Alignment granularity of the FP8 matrix cores' grouped product sums,
# relative to a group's largest product (the three model tests below hold
# it: 448 x 448 = 200,704 cuts products of 4 to zero and keeps products of
# 16, a granularity of 8 or 16 = 2^-14.6 or 2^-13.6 of the largest).
TRUNC = 2.0 ** -12


def check_on_codes(o, lse, o_ref, lse_ref, bnd, label):
    """GPU O, LSE (device tensors, or arrays of the same rows) against the
    oracle's FP8 attention on the same codes and its derived bound."""
    o_gpu = o if isinstance(o, np.ndarray) else np64(o)
    lse_gpu = lse if isinstance(lse, np.ndarray) else np64(lse)
    st = fwd_stats(o_gpu, lse_gpu, o_ref, lse_ref)
    err = np.abs(o_gpu - o_ref)
    ratio = float((err / np.maximum(bnd["o"], 1e-300)).max()) if err.size else 0.0
    fin = np.isfinite(lse_ref)
    lerr = np.abs(lse_gpu[fin] - lse_ref[fin])
    lratio = float((lerr / bnd["lse"][fin]).max()) if lerr.size else 0.0
    open_rows = int(np.count_nonzero(bnd["flip"].max(axis=-1))) if err.size else 0
    print(f"{label} {st} err/bound max {ratio:.3f}, lse err/bound max {lratio:.3f}, "
          f"rows with open codes {open_rows}", flush=True)
    worst = np.unravel_index(int(np.argmax(err - bnd["o"])), err.shape) if err.size else None
    assert np.all(err <= bnd["o"]), (worst, err[worst], bnd["o"][worst])
    assert np.all(lerr <= bnd["lse"][fin]), lratio
    assert st["mean_abs"] <= O_MEAN and st["lse_max_abs"] <= LSE_MAX, st
    return st


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
    o_ref, lse_ref, bnd = attn_fwd64_fp8(qz, d ** -0.5, causal, trunc=TRUNC)
    check_on_codes(o, lse, o_ref, lse_ref, bnd, f"{case} rot={rot}")


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
    o_ref, lse_ref, bnd = attn_fwd64_fp8(qz, 0.125, causal, kv, trunc=TRUNC)
    check_on_codes(o, lse, o_ref, lse_ref, bnd, f"kv {kv} causal={causal}")
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
    o_ref, lse_ref, bnd = attn_fwd64_fp8(ref, d ** -0.5, True, rows=rows, trunc=TRUNC)
    check_on_codes(np64(o[:, :, rows]), np64(lse[:, :, rows]), o_ref, lse_ref, bnd, f"N={N}")


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
    o_ref, lse_ref, bnd = attn_fwd64_fp8(ref, d ** -0.5, c["causal"], kv, trunc=TRUNC)
    check_on_codes(o, lse, o_ref, lse_ref, bnd, str(c))
    if kv is not None:
        for b, L in enumerate(kv):
            if L == 0:
                assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))


def _outlier_inputs(B, H, N, d, seed):
    """The FP8 workload's recipe at a smaller size: N(0, 1) Q, K, V with four
    channels of Q and K (the same per head) scaled by 16."""
    return W.make_inputs(W.FP8.with_(B=B, H=H, N=N, d=d), seed=seed)


def _run_codes(q, k, v, d, scale, kv=None, rot=False, signs=None):
    B, H, N = q.shape[0], q.shape[1], q.shape[2]
    bufs = fp8_buffers(B, H, N, d)
    fa_fp8_quantize(dev(q), dev(k), dev(v), dev(signs), bufs)
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    kvt = None if kv is None else torch.full((B,), kv, dtype=torch.int32, device="cuda")
    fa_fwd_fp8(bufs, rot, o, lse, scale, False, kvt)
    torch.cuda.synchronize()
    return np64(o), np64(lse), bufs


@pytest.mark.parametrize("d", [64, 128])
def test_matrix_cores_add_products_in_aligned_groups_of_eight(d):
    """Two products of 448 x 448 at reduction indices a and b among small
    ones (2^-6 x 448 = 7, below the granularity): the small products of a
    group holding a large one are cut to zero, so 6 are lost when a and b
    share a group and 14 when they do not. Scores: one visible key (LSE is
    the score), b over every channel; P V: all keys equal (P codes 256), V
    column c large at keys a and c."""
    small = 2.0 ** -6
    for a in (0, 5, 33, d - 4):
        say(f"fp8 groups: scores d={d} a={a}")
        N = 128
        scale = 2.0 ** -12
        q = torch.full((1, 1, N, d), small)
        for r in range(N):
            q[0, 0, r, a] = 448.0
            q[0, 0, r, r % d] = 448.0
        k = torch.zeros((1, 1, N, d))
        k[0, 0, 0] = 448.0
        _, lse, bufs = _run_codes(q.to(torch.bfloat16), k.to(torch.bfloat16), torch.zeros_like(q).to(torch.bfloat16),
                                  d, scale, kv=1)
        qd = e4m3_decode(bufs["q8"].cpu().numpy()[0, 0]) * float(bufs["q_scale"][0, 0, 0])
        kd = e4m3_decode(bufs["k8"].cpu().numpy()[0, 0, 0]) * float(bufs["k_scale"][0, 0, 0])
        lost = np.rint(((qd * kd).sum(1) - lse[0, 0] / scale) / (small * 448.0)).astype(int)
        for b in range(d):
            expect = 7 if b == a else (6 if b // 8 == a // 8 else 14)
            assert lost[b] == expect, (a, b, lost[b])
    for a in (0, 5, 33, 60):
        say(f"fp8 groups: P V d={d} a={a}")
        N = 64
        q = torch.zeros((1, 1, N, d))
        q[..., 0] = 1.0
        k = q.clone()
        v = torch.full((1, 1, N, d), small)
        for c in range(d):
            v[0, 0, a, c] = 448.0
            v[0, 0, c % N, c] = 448.0
        o, _, bufs = _run_codes(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), d, 1.0)
        vd = e4m3_decode(bufs["vt8"].cpu().numpy()[0, 0][:, :N]) * float(bufs["v_scale"][0, 0])
        lost = np.rint((vd.sum(1) / N - o[0, 0, 0]) * N / small).astype(int)
        for c in range(d):
            b = c % N
            expect = 7 if b == a else (6 if b // 8 == a // 8 else 14)
            assert lost[c] == expect, (a, c, lost[c])


@pytest.mark.parametrize("rot", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_score_losses_are_within_the_matrix_core_model(d, rot):
    """Rows with one visible key (kv_len = 1): P = 1, so LSE is the scaled
    score q_i . k_0. Its difference from the oracle's stays within scale'
    times the model's grouped loss bound (mfma_loss_bound with TRUNC), plus
    2^-20 of the magnitude sum (fp32 addition of the group sums) and the
    fp32 rounding of the final LSE operations, 2^-20 (|LSE| + 32). 16,384
    dot products per case, with outlier channels; plus crafted rows with one
    product of 448 x 448 per group and seven small ones just below the
    granularity."""
    B, H, N = 2, 8, 1024
    say(f"fp8 score losses d={d} rot={rot}")
    inp = _outlier_inputs(B, H, N, d, seed=90 + d + rot)
    signs = W.random_signs(d, seed=91) if rot else None
    _, lse, bufs = _run_codes(inp["q"], inp["k"], inp["v"], d, d ** -0.5, kv=1, rot=rot, signs=signs)
    s_mul = d ** -0.5 / (d if rot else 1)
    ratios = []
    for b in range(B):
        for h in range(H):
            q8 = bufs["q8"].cpu().numpy()[b, h]
            qd = e4m3_decode(q8) * np.repeat(bufs["q_scale"].cpu().numpy()[b, h].astype(np.float64), 128)[:N, None]
            k0 = e4m3_decode(bufs["k8"].cpu().numpy()[b, h, :1]) * float(bufs["k_scale"][b, h, 0])
            exact = s_mul * (qd @ k0[0])
            allow = (s_mul * (mfma_loss_bound(np.abs(qd), np.abs(k0), TRUNC)[:, 0] +
                              2.0 ** -20 * (np.abs(qd) @ np.abs(k0[0]))) +
                     2.0 ** -20 * (np.abs(exact) + 32))
            ratios.append(np.abs(lse[b, h] - exact) / allow)
    r = np.concatenate(ratios)
    print(f"score loss / model bound: max {r.max():.3f}, 99.9% {np.quantile(r, 0.999):.3f}, "
          f"median {np.median(r):.3f}", flush=True)
    assert r.max() <= 1.0
    # crafted: per group of 8 channels one product 448 x 448 and seven of t
    # (q = t / 448 on the e4m3 grid against k = 448), t around the granularity
    say(f"fp8 score losses crafted d={d}")
    scale = 2.0 ** -12
    ts = [2.0 ** -9, 2.0 ** -7, 2.0 ** -5, 2.0 ** -4, 2.0 ** -3]  # q of the small products
    q = torch.tensor([ts[r_ % len(ts)] for r_ in range(128)])[:, None].repeat(1, d)[None, None]
    q[..., ::8] = 448.0
    k = torch.zeros((1, 1, 128, d))
    k[0, 0, 0] = 448.0
    _, lse, bufs = _run_codes(q.to(torch.bfloat16), k.to(torch.bfloat16), torch.zeros_like(q).to(torch.bfloat16),
                              d, scale, kv=1)
    qd = e4m3_decode(bufs["q8"].cpu().numpy()[0, 0]) * float(bufs["q_scale"][0, 0, 0])
    k0 = e4m3_decode(bufs["k8"].cpu().numpy()[0, 0, :1]) * float(bufs["k_scale"][0, 0, 0])
    exact = scale * (qd @ k0[0])
    allow = (scale * (mfma_loss_bound(np.abs(qd), np.abs(k0), TRUNC)[:, 0] + 2.0 ** -20 * (np.abs(qd) @ np.abs(k0[0]))) +
             2.0 ** -20 * (np.abs(exact) + 32))
    r = np.abs(lse[0, 0] - exact) / allow
    print(f"crafted score loss / model bound: max {r.max():.3f}", flush=True)
    assert r.max() <= 1.0


@pytest.mark.parametrize("d", [64, 128])
def test_p_v_losses_are_within_the_matrix_core_model(d):
    """Rows whose keys are all equal: every P code is 256, so O is the mean
    of V formed by the P V sums. Its difference from the oracle's stays
    within the model's grouped loss bound of those sums plus their fp32
    accumulation over tiles and the final scaling, (T + 8) 2^-24 of the
    magnitude sum. V has outlier columns, or one dominant key per group of
    8 keys."""
    B, H, N = 1, 8, 2048
    for case in ("outlier columns", "dominant keys"):
        say(f"fp8 P V losses d={d} {case}")
        inp = _outlier_inputs(B, H, N, d, seed=95 + d)
        inp["k"] = inp["k"][:, :, :1].expand(B, H, N, d).contiguous()
        if case == "outlier columns":
            inp["v"][..., :4] = inp["v"][..., :4] * 16
        else:
            inp["v"] = (inp["v"].float().abs() * 0.02).to(inp["v"].dtype)
            inp["v"][:, :, ::8] = 20.0
        o, _, bufs = _run_codes(inp["q"], inp["k"], inp["v"], d, d ** -0.5)
        ratios = []
        for b in range(B):
            for h in range(H):
                vd = e4m3_decode(bufs["vt8"].cpu().numpy()[b, h][:, :N]).T  # [N, d] codes
                sv = float(bufs["v_scale"][b, h])
                exact = vd.sum(0) * sv / N
                loss = np.zeros(d)
                for t0 in range(0, N, 64):
                    loss += mfma_loss_bound(np.ones((1, 64)), np.abs(vd[t0:t0 + 64]).T, TRUNC)[0]
                mag = np.abs(vd).sum(0)
                allow = (loss + (N / 64 + 8) * 2.0 ** -24 * mag) * sv / N + 2.0 ** -22 * np.abs(exact)
                ratios.append(np.abs(o[b, h] - exact[None, :]) / allow[None, :])
        r = np.concatenate([x.ravel() for x in ratios])
        print(f"P V loss / model bound ({case}): max {r.max():.3f}, 99.9% {np.quantile(r, 0.999):.3f}, "
              f"median {np.median(r):.3f}", flush=True)
        assert r.max() <= 1.0
