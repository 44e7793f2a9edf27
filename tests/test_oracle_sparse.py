"""Pins of the block-sparse oracle (oracle/sparse.py), CPU only.

  * pure-Python brute force with the visibility table written out in loops
    here (mask entry of the (query block, key block) pair, key padding,
    causal), random masks, blocks of 2 on N <= 8;
  * a mask of all ones is plain attention; a causal mask that keeps the
    blocks on and below the diagonal is plain causal attention (the blocks
    it drops hold no visible key);
  * a block-diagonal mask is plain attention run on each block's slice of
    the sequence on its own;
  * an all-zero mask gives O = 0, LSE = -inf and zero gradients;
  * the backward against central finite differences of the brute-force loss;
  * the row subset of the forward and the sampled backward (for N too long
    for an N x N matrix) against the whole, pinned computation.
"""
import math

import numpy as np
import pytest

from oracle import (attn_bwd64, attn_bwd64_sparse, attn_bwd64_sparse_sampled, attn_fwd64,
                    attn_fwd64_sparse, brute_head_allowed, brute_loss_allowed)


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def table(N, blk, mask, causal, kv):
    return [[bool(mask[i // blk][j // blk]) and j < kv and (not causal or j <= i) for j in range(N)]
            for i in range(N)]


@pytest.mark.parametrize("N", [5, 7, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_sparse_forward_matches_brute_force(N, causal):
    B, H, d, blk = 2, 2, 3, 2
    nb = (N + blk - 1) // blk
    q, k, v = rnd((B, H, N, d), N), rnd((B, H, N, d), N + 1), rnd((B, H, N, d), N + 2)
    mask = (np.random.default_rng(N + causal).random((B, H, nb, nb)) < 0.6).astype(np.uint8)
    kv = [N, N - 2]
    o, lse = attn_fwd64_sparse(q, k, v, 0.7, causal, kv, mask, block=blk)
    for b in range(B):
        for h in range(H):
            bo, bl = brute_head_allowed(q[b, h], k[b, h], v[b, h], 0.7,
                                        table(N, blk, mask[b, h], causal, kv[b]))
            np.testing.assert_allclose(o[b, h], np.array(bo), rtol=0, atol=1e-12)
            for x, y in zip(lse[b, h], bl):
                assert (x == y == -math.inf) or abs(x - y) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_is_plain_attention(causal):
    B, H, N, d = 1, 2, 300, 8
    q, k, v, do = (rnd((B, H, N, d), s) for s in range(4))
    nb = (N + 127) // 128
    ones = np.ones((nb, nb), np.uint8)
    o, lse = attn_fwd64_sparse(q, k, v, 0.3, causal, [250], ones)
    o2, lse2 = attn_fwd64(q, k, v, 0.3, causal, [250])
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)
    for a, b in zip(attn_bwd64_sparse(q, k, v, do, 0.3, causal, [250], ones),
                    attn_bwd64(q, k, v, do, 0.3, causal, [250])):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_causal_lower_block_triangle_is_plain_causal_attention():
    B, H, N, d = 1, 1, 400, 8
    q, k, v = (rnd((B, H, N, d), s) for s in range(10, 13))
    nb = (N + 127) // 128
    tri = np.tril(np.ones((nb, nb), np.uint8))
    o, lse = attn_fwd64_sparse(q, k, v, 0.3, True, None, tri)
    o2, lse2 = attn_fwd64(q, k, v, 0.3, True)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_mask_is_attention_per_block(causal):
    B, H, N, d, blk = 2, 1, 300, 4, 128
    q, k, v, do = (rnd((B, H, N, d), s) for s in range(20, 24))
    nb = (N + blk - 1) // blk
    kv = [300, 170]
    eye = np.eye(nb, dtype=np.uint8)
    o, lse = attn_fwd64_sparse(q, k, v, 0.5, causal, kv, eye)
    dq, dk, dv = attn_bwd64_sparse(q, k, v, do, 0.5, causal, kv, eye)
    for s0 in range(0, N, blk):
        sl = slice(s0, min(s0 + blk, N))
        n = sl.stop - sl.start
        kv_loc = [min(max(x - s0, 0), n) for x in kv]
        o2, lse2 = attn_fwd64(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.5, causal, kv_loc)
        np.testing.assert_allclose(o[:, :, sl], o2, atol=1e-13)
        np.testing.assert_array_equal(np.isneginf(lse[:, :, sl]), np.isneginf(lse2))
        fin = np.isfinite(lse2)
        np.testing.assert_allclose(lse[:, :, sl][fin], lse2[fin], atol=1e-13)
        g2 = attn_bwd64(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], 0.5, causal, kv_loc)
        for a, b in zip((dq, dk, dv), g2):
            np.testing.assert_allclose(a[:, :, sl], b, atol=1e-12)


def test_empty_mask_gives_zero_output_and_gradients():
    B, H, N, d = 1, 2, 130, 4
    q, k, v, do = (rnd((B, H, N, d), s) for s in range(30, 34))
    zero = np.zeros((2, 2), np.uint8)
    o, lse = attn_fwd64_sparse(q, k, v, 0.5, False, None, zero)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    for g in attn_bwd64_sparse(q, k, v, do, 0.5, False, None, zero):
        assert np.all(g == 0)


def test_two_dimensional_mask_applies_to_every_head():
    B, H, N, d, blk = 2, 3, 9, 2, 4
    q, k, v = (rnd((B, H, N, d), s) for s in range(40, 43))
    m = (np.random.default_rng(4).random((3, 3)) < 0.5).astype(np.uint8)
    m[0, 0] = 1
    o, lse = attn_fwd64_sparse(q, k, v, 0.5, False, None, m, block=blk)
    o4, lse4 = attn_fwd64_sparse(q, k, v, 0.5, False, None, np.broadcast_to(m, (B, H, 3, 3)), block=blk)
    np.testing.assert_array_equal(o, o4)
    np.testing.assert_array_equal(lse, lse4)


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_backward_matches_finite_differences(causal):
    N, d, blk = 6, 2, 2
    q, k, v, do = rnd((1, 1, N, d), 50), rnd((1, 1, N, d), 51), rnd((1, 1, N, d), 52), rnd((1, 1, N, d), 53)
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8)
    allowed = table(N, blk, mask, causal, 5)
    dq, dk, dv = attn_bwd64_sparse(q, k, v, do, 0.8, causal, [5], mask, block=blk)
    step = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += step
            xm[idx] -= step
            args_p = {"q": q, "k": k, "v": v, name: xp}
            args_m = {"q": q, "k": k, "v": v, name: xm}
            lp = brute_loss_allowed(args_p["q"][0, 0], args_p["k"][0, 0], args_p["v"][0, 0], do[0, 0], 0.8, allowed)
            lm = brute_loss_allowed(args_m["q"][0, 0], args_m["k"][0, 0], args_m["v"][0, 0], do[0, 0], 0.8, allowed)
            fd[idx] = (lp - lm) / (2 * step)
        np.testing.assert_allclose(g, fd, rtol=0, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_keys_match_the_whole_backward(causal):
    B, H, N, d, blk = 2, 2, 37, 3, 4
    q, k, v, do = (rnd((B, H, N, d), s) for s in range(60, 64))
    nb = (N + blk - 1) // blk
    mask = (np.random.default_rng(9).random((B, H, nb, nb)) < 0.5).astype(np.uint8)
    kv = [37, 21]
    rows = [0, 3, 4, 20, 21, 36]
    o, lse = attn_fwd64_sparse(q, k, v, 0.6, causal, kv, mask, block=blk)
    o_r, lse_r = attn_fwd64_sparse(q, k, v, 0.6, causal, kv, mask, block=blk, rows=rows, row_chunk=4)
    np.testing.assert_allclose(o_r, o[:, :, rows], atol=1e-14)
    np.testing.assert_array_equal(lse_r, lse[:, :, rows])
    dq, dk, dv = attn_bwd64_sparse(q, k, v, do, 0.6, causal, kv, mask, block=blk)
    heads = [(0, 1), (1, 0)]
    sq, sk, sv = attn_bwd64_sparse_sampled(q, k, v, do, 0.6, causal, kv, mask, heads, rows, rows,
                                           block=blk, row_chunk=5)
    for t, (b, h) in enumerate(heads):
        np.testing.assert_allclose(sq[t], dq[b, h, rows], atol=1e-12)
        np.testing.assert_allclose(sk[t], dk[b, h, rows], atol=1e-12)
        np.testing.assert_allclose(sv[t], dv[b, h, rows], atol=1e-12)
    # rows alone and keys alone (each then forms LSE and D only where needed)
    keys = [1, 5, 30]
    sq2, _, _ = attn_bwd64_sparse_sampled(q, k, v, do, 0.6, causal, kv, mask, heads, rows, [],
                                          block=blk, row_chunk=3)
    _, sk2, sv2 = attn_bwd64_sparse_sampled(q, k, v, do, 0.6, causal, kv, mask, heads, [], keys,
                                            block=blk, row_chunk=3)
    for t, (b, h) in enumerate(heads):
        np.testing.assert_allclose(sq2[t], dq[b, h, rows], atol=1e-12)
        np.testing.assert_allclose(sk2[t], dk[b, h, keys], atol=1e-12)
        np.testing.assert_allclose(sv2[t], dv[b, h, keys], atol=1e-12)
