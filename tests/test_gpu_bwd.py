"""Backward parity of the HIP path (through the C ABI) against the fp64 oracle.

The GPU backward consumes the GPU forward's own O (in the input dtype) and
LSE; the oracle recomputes everything from the inputs in fp64. Each gradient
is held to relative Frobenius error <= 2e-2 (bf16/fp16) or <= 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import workloads as W
from oracle import attn_bwd64, attn_bwd64_sampled
from tests.helpers import F32_GRAD_REL_FRO, GRAD_REL_FRO, np64, rel_fro, run_bwd, run_fwd, say

pytestmark = pytest.mark.gpu


def _grads(inp, scale, causal):
    o, lse = run_fwd(inp, scale, causal)
    return run_bwd(inp, o, lse, scale, causal)


def _check_full(inp, scale, causal, tol, label, heads=None):
    dq, dk, dv = _grads(inp, scale, causal)
    ref = attn_bwd64(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, inp.get("kv_len"),
                     heads=heads)
    got = [np64(t) for t in (dq, dk, dv)]
    if heads is not None:
        got = [np.stack([g[b, h] for b, h in heads]) for g in got]
    errs = {n: rel_fro(g, r) for n, g, r in zip(("dq", "dk", "dv"), got, ref)}
    print(f"{label} rel-fro {errs}", flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
    return got, ref


SMALL = [(2, 2, n, d) for n in (1, 17, 129, 300) for d in (64, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_backward_small_shapes(shape, causal, dtype):
    B, H, N, d = shape
    say(f"bwd {shape} {dtype} causal={causal}")
    inp = W.random_case(B, H, N, d, dtype, seed=3 * N + d, causal=causal, backward=True)
    _check_full(inp, d ** -0.5, causal, GRAD_REL_FRO, str(shape))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_key_padding_masks_gradients(d, causal):
    N = 300
    kv = [0, 1, 150, 300]
    say(f"bwd kv_len {kv} d={d} causal={causal}")
    inp = W.random_case(4, 2, N, d, "bf16", seed=17, causal=causal, kv_len=kv, backward=True)
    got, _ = _check_full(inp, d ** -0.5, causal, GRAD_REL_FRO, "kv")
    dq, dk, dv = got
    for b, L in enumerate(kv):
        assert np.all(dk[b, :, L:] == 0.0) and np.all(dv[b, :, L:] == 0.0)
    assert np.all(dq[0] == 0.0)  # no visible key anywhere in batch 0
    assert all(np.isfinite(g).all() for g in got)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 64), (2, 1, 45, 64), (1, 2, 130, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_backward_fp32_path(shape, causal):
    B, H, N, d = shape
    say(f"bwd fp32 {shape} causal={causal}")
    inp = W.random_case(B, H, N, d, "fp32", seed=N, causal=causal, backward=True)
    _check_full(inp, d ** -0.5, causal, F32_GRAD_REL_FRO, f"fp32 {shape}")


def test_config_gpt2_backward():
    w = W.GPT2
    say(w.name)
    _check_full(W.make_inputs(w), w.scale, w.causal, GRAD_REL_FRO, w.name)


def test_long_context_backward_two_heads():
    w = W.LONG_BWD
    say(w.name)
    _check_full(W.make_inputs(w), w.scale, w.causal, GRAD_REL_FRO, w.name, heads=[(0, 0), (0, 31)])


def test_trading_day_backward_sampled():
    w = W.TRADE_BWD
    say(w.name)
    inp = W.make_inputs(w)
    dq, dk, dv = (np64(t) for t in _grads(inp, w.scale, w.causal))
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 23399], rng.choice(w.N, 120, replace=False)]))
    h = 5
    rq, rk, rv = attn_bwd64_sampled(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.causal,
                                    None, heads=[(0, h)], q_rows=rows, k_rows=rows)
    errs = {"dq": rel_fro(dq[0, h, rows], rq[0]), "dk": rel_fro(dk[0, h, rows], rk[0]),
            "dv": rel_fro(dv[0, h, rows], rv[0])}
    print(f"{w.name} sampled rel-fro {errs}", flush=True)
    for n, e in errs.items():
        assert e <= GRAD_REL_FRO, (n, e)


def test_backward_is_deterministic_and_satisfies_sum_rules():
    w = W.GPT2.with_(B=2, N=700, causal=False)
    say("bwd determinism")
    inp = W.make_inputs(w)
    a = _grads(inp, w.scale, False)
    b = _grads(inp, w.scale, False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    dk, dv = np64(a[1]), np64(a[2])
    do = inp["do"].double().numpy()
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, up to bf16 rounding of the
    # per-key gradients
    assert np.abs(dk.sum(axis=2)).max() <= 2e-2 * np.abs(dk).sum(axis=2).max()
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0,
                               atol=2e-2 * np.abs(dv).sum(axis=2).max())


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_stages_equal_the_one_call_backward(causal, d, dtype):
    """The exported stages give fa_bwd's results bit for bit: fa_bwd_dq then
    fa_bwd_dkdv (what fa_bwd enqueues). fa_bwd_dsum then fa_bwd_dkdv then
    fa_bwd_dq gives them too on every row that sees more than one 64-key
    tile (the D kernel sums in the dQ kernel's order); on rows that see one
    tile (here: queries 0-63 under the causal mask) fa_bwd_dq forms D_i from
    P and dP instead, so there only dQ and the final D match, and dK, dV of
    keys 0-63 come from the D of O (checked against the oracle)."""
    from exact_io_aware_07_amd import fa_bwd, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_dsum
    B, H, N = 2, 3, 333
    kv = [333, 200]
    say(f"backward stages vs one call d={d} causal={causal} {dtype}")
    inp = W.random_case(B, H, N, d, dtype, seed=90 + d, causal=causal, kv_len=kv, backward=True)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    kvt = inp["kv_len"].cuda()
    sc = d ** -0.5
    o, lse = run_fwd(inp, sc, causal)
    ws = torch.empty(B * H * N * 4 + 256, dtype=torch.uint8, device="cuda")
    g1 = [torch.empty_like(q) for _ in range(3)]
    fa_bwd(q, k, v, o, do, lse, *g1, sc, causal, kvt, ws)
    d1 = ws[:B * H * N * 4].view(torch.float32).view(B, H, N).clone()
    g2 = [torch.empty_like(q) for _ in range(3)]
    d2 = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa_bwd_dq(q, k, v, o, do, lse, d2, g2[0], sc, causal, kvt)
    fa_bwd_dkdv(q, k, v, do, lse, d2, g2[1], g2[2], sc, causal, kvt)
    g3 = [torch.empty_like(q) for _ in range(3)]
    d3 = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa_bwd_dsum(o, do, d3)
    fa_bwd_dkdv(q, k, v, do, lse, d3, g3[1], g3[2], sc, causal, kvt)
    fa_bwd_dq(q, k, v, o, do, lse, d3, g3[0], sc, causal, kvt)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2) and torch.equal(d1, d3)
    lo = 64 if causal else 0  # keys whose dK, dV see a one-tile row
    for i, (a, b, c) in enumerate(zip(g1, g2, g3)):
        assert torch.equal(a, b)
        assert torch.equal(a, c) if i == 0 else torch.equal(a[:, :, lo:], c[:, :, lo:])
    if causal:
        ref = attn_bwd64(inp["q"], inp["k"], inp["v"], inp["do"], sc, causal, kv)
        for g, r in zip(g3[1:], ref[1:]):
            assert rel_fro(np64(g), r) <= GRAD_REL_FRO


SHORT = [(2, 2, n, d) for n in (1, 2, 3) for d in (64, 128)]


@pytest.mark.parametrize("o32", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHORT, ids=lambda s: "x".join(map(str, s)))
def test_rows_of_one_to_three_keys(shape, causal, dtype, o32):
    """Rows of one, two or three keys, where dS = P (dP - D) is a difference
    of nearly equal terms: the dQ kernel forms D_i from its own P and dP on
    such one-tile rows, so the gradients meet the bound with the stored O in
    either dtype. D_i itself (the workspace) equals the oracle's sum_j P dP.
    A gradient whose exact value vanishes (N = 1: every row sees one key) is
    held to the bound relative to 1e-3 of the norm of dV."""
    from exact_io_aware_07_amd import fa_bwd
    B, H, N, d = shape
    say(f"bwd short rows {shape} causal={causal} {dtype} o32={o32}")
    inp = W.random_case(B, H, N, d, dtype, seed=700 + 7 * N + d, causal=causal, kv_len=[N, 1],
                        backward=True)
    sc = d ** -0.5
    o, lse = run_fwd(inp, sc, causal, out_dtype=torch.float32 if o32 else None)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    ws = torch.empty(B * H * N * 4 + 256, dtype=torch.uint8, device="cuda")
    g = [torch.empty_like(q) for _ in range(3)]
    fa_bwd(q, k, v, o, do, lse, *g, sc, causal, inp["kv_len"].cuda(), ws)
    torch.cuda.synchronize()
    ref = attn_bwd64(inp["q"], inp["k"], inp["v"], inp["do"], sc, causal, inp["kv_len"])
    floor = 1e-3 * float(np.linalg.norm(ref[2]))
    errs = [float(np.linalg.norm(np64(x) - r)) / max(float(np.linalg.norm(r)), floor) for x, r in zip(g, ref)]
    print(f"short rows {shape} errs {errs}", flush=True)
    assert all(e <= GRAD_REL_FRO for e in errs), errs
    from oracle import attn_probs64
    p = attn_probs64(inp["q"], inp["k"], sc, causal, inp["kv_len"])
    dp = np.einsum("bhic,bhjc->bhij", np64(inp["do"]), np64(inp["v"]))
    dref = (p * dp).sum(-1)
    dgpu = np64(ws[:B * H * N * 4].view(torch.float32).view(B, H, N))
    scale_d = np.abs(p * dp).sum(-1) + 1e-30
    assert np.all(np.abs(dgpu - dref) <= 1e-5 * scale_d + 1e-6), np.abs(dgpu - dref).max()


def test_fp32_o_forms_d_without_o_rounding():
    """On long rows the backward takes an fp32 O too: D_i = rowsum(dO * O)
    is then formed from the unrounded O (closer to the oracle's D than with
    the bf16 O), and the gradients meet the bound either way."""
    from exact_io_aware_07_amd import fa_bwd_dsum
    B, H, N, d = 2, 2, 300, 128
    say("bwd fp32 O long rows")
    inp = W.random_case(B, H, N, d, "bf16", seed=801, backward=True)
    sc = d ** -0.5
    o32, lse = run_fwd(inp, sc, False, out_dtype=torch.float32)
    do = inp["do"].cuda()
    d32 = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    d16 = torch.empty_like(d32)
    fa_bwd_dsum(o32, do, d32)
    fa_bwd_dsum(o32.to(torch.bfloat16), do, d16)
    torch.cuda.synchronize()
    from oracle import attn_probs64
    p = attn_probs64(inp["q"], inp["k"], sc)
    dref = (p * np.einsum("bhic,bhjc->bhij", np64(inp["do"]), np64(inp["v"]))).sum(-1)
    e32 = np.abs(np64(d32) - dref).max()
    e16 = np.abs(np64(d16) - dref).max()
    print(f"D error fp32 O {e32:.2e}, bf16 O {e16:.2e}", flush=True)
    assert e32 < e16
    dq, dk, dv = run_bwd(inp, o32, lse, sc, False)
    ref = attn_bwd64(inp["q"], inp["k"], inp["v"], inp["do"], sc, False)
    for x, r in zip((dq, dk, dv), ref):
        assert rel_fro(np64(x), r) <= GRAD_REL_FRO
