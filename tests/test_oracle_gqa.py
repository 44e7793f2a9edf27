"""Pins of the grouped-query oracle (oracle/gqa.py), CPU only.

  * brute force (pure-Python loops) per query head with the key/value head
    h // G, which fixes the head mapping;
  * G = 1 is plain attention;
  * the backward against central finite differences of the summed loss on a
    tiny problem: a shared key/value head receives the sum of its query
    heads' gradients, so a missing or wrong sum fails here.
"""
import math

import numpy as np
import pytest

from oracle import attn_bwd64, attn_bwd64_gqa, attn_fwd64, attn_fwd64_gqa, brute_head_forward, brute_loss


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 2), (4, 1), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward_matches_brute_force(H, Hkv, causal):
    B, N, d = 2, 5, 3
    q, k, v = rnd((B, H, N, d), 1), rnd((B, Hkv, N, d), 2), rnd((B, Hkv, N, d), 3)
    kv = [5, 3]
    o, lse = attn_fwd64_gqa(q, k, v, 0.6, causal, kv_len=np.array(kv))
    G = H // Hkv
    for b in range(B):
        for h in range(H):
            bo, bl = brute_head_forward(q[b, h], k[b, h // G], v[b, h // G], 0.6, causal, kv[b])
            np.testing.assert_allclose(o[b, h], np.array(bo), rtol=0, atol=1e-12)
            for x, y in zip(lse[b, h], bl):
                assert (x == y == -math.inf) or abs(x - y) < 1e-12


def test_gqa_with_one_query_head_per_group_is_plain_attention():
    q, k, v, do = (rnd((1, 3, 7, 4), s) for s in range(4, 8))
    o, lse = attn_fwd64_gqa(q, k, v, 0.5, True)
    o2, lse2 = attn_fwd64(q, k, v, 0.5, True)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    g1 = attn_bwd64_gqa(q, k, v, do, 0.5, True)
    g2 = attn_bwd64(q, k, v, do, 0.5, True)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_matches_finite_differences(causal):
    B, H, Hkv, N, d = 1, 4, 2, 4, 2
    G = H // Hkv
    q, k, v, do = rnd((B, H, N, d), 9), rnd((B, Hkv, N, d), 10), rnd((B, Hkv, N, d), 11), rnd((B, H, N, d), 12)
    dq, dk, dv = attn_bwd64_gqa(q, k, v, do, 0.7, causal)

    def loss(qq, kk, vv):
        return math.fsum(brute_loss(qq[0, h], kk[0, h // G], vv[0, h // G], do[0, h], 0.7, causal)
                         for h in range(H))

    step = 1e-5
    for name, x, g in (("k", k, dk), ("v", v, dv), ("q", q, dq)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += step
            xm[idx] -= step
            args_p = {"q": q, "k": k, "v": v, name: xp}
            args_m = {"q": q, "k": k, "v": v, name: xm}
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                       loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * step)
        np.testing.assert_allclose(g, fd, rtol=0, atol=1e-7, err_msg=name)
