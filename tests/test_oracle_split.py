"""Pins of the partial-attention and merge oracle (oracle/split.py), CPU only.

What fixes each value, other than the functions themselves:
  * brute force (pure-Python loops) on tiny inputs, with position offsets;
  * the identity the merge exists for: attention over all keys equals the
    merge of attention over a partition of the keys (the online-softmax
    recurrence of the marketmaker.cc article, "在线softmax递归", holds for any
    split), checked against the pinned full-attention oracle;
  * ring attention's block schedule (Ultralytics glossary, "Flash Attention e
    termini correlati"): query shards merged over key shards with global
    positions give the full causal result;
  * closed forms: identical keys inside each part make O the mean of that
    part's values, so the merge must weight parts by their key counts;
  * merge identities: one part is unchanged, an empty part (LSE = -inf) is
    ignored, order does not matter, and merging is associative.
"""
import math

import numpy as np
import pytest

from oracle import attn_fwd64, attn_part64, brute_head_part, merge64


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("q_pos0,k_pos0", [(0, 0), (3, 0), (0, 3), (5, 2), (2, 9)])
def test_part_matches_brute_force(causal, q_pos0, k_pos0):
    q, k, v = rnd((1, 2, 4, 3), 1), rnd((1, 2, 6, 3), 2), rnd((1, 2, 6, 3), 3)
    o, lse = attn_part64(q, k, v, 0.7, causal, q_pos0, k_pos0)
    for h in range(2):
        bo, bl = brute_head_part(q[0, h], k[0, h], v[0, h], 0.7, causal, q_pos0, k_pos0)
        np.testing.assert_allclose(o[0, h], np.array(bo), rtol=0, atol=1e-12)
        for a, b in zip(lse[0, h], bl):
            assert (a == b == -math.inf) or abs(a - b) < 1e-12


def test_part_with_no_visible_key():
    # keys all after every query position: O = 0, LSE = -inf, no NaN
    q, k, v = rnd((1, 1, 3, 4), 4), rnd((1, 1, 5, 4), 5), rnd((1, 1, 5, 4), 6)
    o, lse = attn_part64(q, k, v, 0.5, True, q_pos0=0, k_pos0=10)
    assert np.all(o == 0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("causal", [False, True])
def test_part_is_full_attention_at_zero_offsets(causal):
    q, k, v = rnd((2, 2, 9, 5), 7), rnd((2, 2, 9, 5), 8), rnd((2, 2, 9, 5), 9)
    kv = np.array([9, 4])
    o, lse = attn_part64(q, k, v, 0.4, causal, kv_len=kv)
    o2, lse2 = attn_fwd64(q, k, v, 0.4, causal, kv_len=kv)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    fin = np.isfinite(lse2)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lse2[fin], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [[0, 7, 20], [0, 1, 2, 20], [0, 10, 10, 20], [0, 20]])
def test_merge_of_key_partition_is_full_attention(causal, cuts):
    q, k, v = rnd((1, 3, 20, 8), 10), rnd((1, 3, 20, 8), 11), rnd((1, 3, 20, 8), 12)
    parts = [attn_part64(q, k[:, :, a:b], v[:, :, a:b], 0.35, causal, 0, a)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = merge64([p[0] for p in parts], [p[1] for p in parts])
    o_ref, lse_ref = attn_fwd64(q, k, v, 0.35, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_ring_schedule_gives_full_causal_attention():
    N, shards = 24, 3
    q, k, v = rnd((1, 2, N, 4), 13), rnd((1, 2, N, 4), 14), rnd((1, 2, N, 4), 15)
    o_ref, lse_ref = attn_fwd64(q, k, v, 0.5, True)
    n = N // shards
    for r in range(shards):
        qs = q[:, :, r * n:(r + 1) * n]
        parts = [attn_part64(qs, k[:, :, s * n:(s + 1) * n], v[:, :, s * n:(s + 1) * n], 0.5, True,
                             r * n, s * n) for s in range(shards)]
        o, lse = merge64([p[0] for p in parts], [p[1] for p in parts])
        np.testing.assert_allclose(o, o_ref[:, :, r * n:(r + 1) * n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref[:, :, r * n:(r + 1) * n], rtol=0, atol=1e-12)


def test_merge_weights_parts_by_key_count():
    # part a: 3 identical keys with values va_j, part b: 5 identical keys (same
    # key vector) with values vb_j; every score is the same, so the merged O is
    # the mean over all 8 values and LSE = s + ln 8
    d = 4
    kvec = rnd((d,), 16)
    q = rnd((1, 1, 2, d), 17)
    ka, kb = np.tile(kvec, (1, 1, 3, 1)), np.tile(kvec, (1, 1, 5, 1))
    va, vb = rnd((1, 1, 3, d), 18), rnd((1, 1, 5, d), 19)
    oa, la = attn_part64(q, ka, va, 0.3)
    ob, lb = attn_part64(q, kb, vb, 0.3)
    o, lse = merge64([oa, ob], [la, lb])
    mean = np.concatenate([va, vb], axis=2).mean(axis=2)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(mean[0, 0], (2, d)), rtol=0, atol=1e-13)
    s = 0.3 * (q[0, 0] @ kvec)
    np.testing.assert_allclose(lse[0, 0], s + math.log(8), rtol=0, atol=1e-13)


def test_merge_identities():
    o1, l1 = rnd((2, 3, 5), 20), rnd((2, 3), 21)
    o2, l2 = rnd((2, 3, 5), 22), rnd((2, 3), 23)
    o3, l3 = rnd((2, 3, 5), 24), rnd((2, 3), 25)
    o, l = merge64([o1], [l1])
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(l, l1, atol=1e-15)
    empty_o, empty_l = rnd((2, 3, 5), 26), np.full((2, 3), -np.inf)
    o, l = merge64([o1, empty_o], [l1, empty_l])
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(l, l1, atol=1e-15)
    oa, la = merge64([o1, o2], [l1, l2])
    ob, lb = merge64([o2, o1], [l2, l1])
    np.testing.assert_allclose(oa, ob, atol=1e-14)
    np.testing.assert_allclose(la, lb, atol=1e-14)
    oc, lc = merge64([oa, o3], [la, l3])
    od, ld = merge64([o1, o2, o3], [l1, l2, l3])
    np.testing.assert_allclose(oc, od, atol=1e-13)
    np.testing.assert_allclose(lc, ld, atol=1e-13)
    o, l = merge64([empty_o, empty_o], [empty_l, empty_l])
    assert np.all(o == 0) and np.all(l == -np.inf)
