"""Backward with very negative log-sum-exp rows and key padding (HIP path
through the C ABI against the fp64 oracle).

Keys past kv_len read as zero rows in the kernels. Their score is then 0 and
their unmasked probability exp(0 - LSE), which is huge when every visible
score of the row is very negative (LSE about -20 here: e^20 = 4.9e8, past the
fp16 maximum 65504). Such keys must be masked, not only zeroed, or the dQ
product meets 0 * inf. The inputs put every query opposite the first key
(q_i = -c k_0 + small noise), so the visible scores sit near -20.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_07_amd import workloads as W
from oracle import attn_bwd64, attn_fwd64
from tests.helpers import GRAD_REL_FRO, np64, rel_fro, run_bwd, run_fwd, say

pytestmark = pytest.mark.gpu


def _negative_lse_case(N, d, dtype, kv, key_noise, seed):
    """Q rows opposite K row 0, so that scale * q_i . k_0 = -20 before noise;
    K rows are k_0 plus key_noise * N(0, 1)."""
    inp = W.random_case(1, 1, N, d, "fp32", seed=seed, backward=True)
    scale = d ** -0.5
    k0 = inp["k"][0, 0, 0].clone()
    c = 20.0 / (scale * float(k0 @ k0))
    k = k0[None, :] + key_noise * inp["k"][0, 0]
    k[0] = k0
    q = -c * k0[None, :] + 0.05 * inp["q"][0, 0]
    dt = W.DTYPES[dtype]
    out = {"q": q[None, None].to(dt).contiguous(), "k": k[None, None].to(dt).contiguous(),
           "v": inp["v"].to(dt).contiguous(), "do": inp["do"].to(dt).contiguous(),
           "kv_len": torch.tensor([kv], dtype=torch.int32)}
    return out, scale


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_one_visible_key_with_negative_lse(d, dtype):
    """kv_len = 1, N = 65, non-causal: one visible key per row, so P = 1, dS = 0
    and the exact dQ and dK are zero; dV_0 = sum_i dO_i."""
    N = 65
    say(f"negative LSE, one key: N={N} d={d} {dtype}")
    inp, scale = _negative_lse_case(N, d, dtype, 1, 0.0, seed=11 + d)
    o, lse = run_fwd(inp, scale, False)
    lse_ref = attn_fwd64(inp["q"], inp["k"], inp["v"], scale, False, inp["kv_len"])[1]
    assert float(lse_ref.max()) < -15.0  # the case really has very negative rows
    dq, dk, dv = run_bwd(inp, o, lse, scale, False)
    ref = attn_bwd64(inp["q"], inp["k"], inp["v"], inp["do"], scale, False, inp["kv_len"])
    got = [np64(t) for t in (dq, dk, dv)]
    for g in got:
        assert np.isfinite(g).all()
    # exact dQ, dK are zero; the GPU's come from fp32 differences dP - D of
    # order 1e-3 of |dO||V|, times scale |K| or |Q| (|Q| is about 20 here)
    print(f"max |dq| {np.abs(got[0]).max():.2e}, max |dk| {np.abs(got[1]).max():.2e}", flush=True)
    assert np.abs(got[0] - ref[0]).max() <= 5e-2
    assert np.abs(got[1] - ref[1]).max() <= 5e-1
    assert rel_fro(got[2], ref[2]) <= GRAD_REL_FRO
    assert np.all(got[1][0, 0, 1:] == 0) and np.all(got[2][0, 0, 1:] == 0)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("kv", [40, 64, 100])
def test_padded_keys_with_negative_lse(kv, dtype):
    """Rows of many visible keys, all scores near -20, the padded keys in the
    same tile: every gradient finite and within the bound."""
    N, d = 129, 64
    say(f"negative LSE, kv_len={kv}: N={N} d={d} {dtype}")
    inp, scale = _negative_lse_case(N, d, dtype, kv, 0.5, seed=kv)
    o, lse = run_fwd(inp, scale, False)
    dq, dk, dv = run_bwd(inp, o, lse, scale, False)
    ref = attn_bwd64(inp["q"], inp["k"], inp["v"], inp["do"], scale, False, inp["kv_len"])
    got = [np64(t) for t in (dq, dk, dv)]
    errs = {n: rel_fro(g, r) for n, g, r in zip(("dq", "dk", "dv"), got, ref)}
    print(f"kv {kv} rel-fro {errs}", flush=True)
    for n, g in zip(("dq", "dk", "dv"), got):
        assert np.isfinite(g).all(), n
    for n, e in errs.items():
        assert e <= GRAD_REL_FRO, (n, e)
