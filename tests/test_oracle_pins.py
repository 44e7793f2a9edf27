"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the
pure-Python brute force (a separate statement of the definition), closed
forms, invariants, finite differences, or numbers the pages print.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attn_bwd64, attn_fwd64, attn_probs64, brute_head_forward,
                    brute_head_grad_fd, score_matrix_bytes)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _kv_cases(N):
    return [None, [0, N], [1, N - 1 if N > 1 else 1], [N, (N + 1) // 2]]


# --- brute force on N <= 8, every mask combination -------------------------

@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("d", [1, 3, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_brute_force(N, d, causal):
    B, H = 2, 2
    for ci, kv in enumerate(_kv_cases(N)):
        q = _rand((B, H, N, d), 10 * N + d + ci)
        k = _rand((B, H, N, d), 20 * N + d + ci)
        v = _rand((B, H, N, d), 30 * N + d + ci)
        scale = 0.7
        o, lse = attn_fwd64(q, k, v, scale, causal, kv)
        for b in range(B):
            for h in range(H):
                lim = None if kv is None else kv[b]
                ob, lb = brute_head_forward(q[b, h], k[b, h], v[b, h], scale, causal, lim)
                np.testing.assert_allclose(o[b, h], np.array(ob), rtol=0, atol=1e-12)
                lb = np.array(lb)
                assert np.array_equal(np.isneginf(lse[b, h]), np.isneginf(lb))
                fin = np.isfinite(lb)
                np.testing.assert_allclose(lse[b, h][fin], lb[fin], rtol=0, atol=1e-12)


# --- closed forms -----------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    B, H, N, d = 1, 2, 37, 16
    q = _rand((B, H, N, d), 1)
    krow = _rand((1, H, 1, d), 2)
    k = np.broadcast_to(krow, (B, H, N, d)).copy()
    v = _rand((B, H, N, d), 3)
    scale = 0.25
    o, lse = attn_fwd64(q, k, v, scale, causal)
    for h in range(H):
        for i in range(N):
            cnt = i + 1 if causal else N
            expect = v[0, h, :cnt].mean(axis=0)
            np.testing.assert_allclose(o[0, h, i], expect, rtol=0, atol=1e-13)
            s = scale * float(q[0, h, i] @ krow[0, h, 0])
            assert abs(lse[0, h, i] - (s + math.log(cnt))) < 1e-12


def test_single_key_returns_that_value_row():
    q = _rand((1, 1, 1, 8), 4)
    k = _rand((1, 1, 1, 8), 5)
    v = _rand((1, 1, 1, 8), 6)
    o, lse = attn_fwd64(q, k, v, 0.3, False)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])
    assert abs(lse[0, 0, 0] - 0.3 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-15


def test_causal_row_zero_sees_only_first_key():
    q = _rand((2, 3, 19, 8), 7)
    k = _rand((2, 3, 19, 8), 8)
    v = _rand((2, 3, 19, 8), 9)
    o, lse = attn_fwd64(q, k, v, 0.5, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0],
                               0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-14)


def test_empty_rows_are_zero_with_neg_inf_lse():
    q = _rand((2, 1, 9, 4), 10)
    k = _rand((2, 1, 9, 4), 11)
    v = _rand((2, 1, 9, 4), 12)
    o, lse = attn_fwd64(q, k, v, 1.0, True, [0, 9])
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


# --- invariants ----------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    q = _rand((2, 2, 33, 8), 13)
    k = _rand((2, 2, 33, 8), 14)
    kv = [33, 20]
    p = attn_probs64(q, k, 0.4, causal, kv)
    assert np.all(p >= 0.0)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-13)
    i = np.arange(33)[:, None]
    j = np.arange(33)[None, :]
    for b, lim in enumerate(kv):
        hidden = np.broadcast_to((j >= lim) | ((j > i) if causal else False), (33, 33))
        assert np.all(p[b][:, hidden] == 0.0)


def test_joint_permutation_of_keys_and_values_non_causal():
    B, H, N, d = 1, 2, 64, 16
    q, k, v = (_rand((B, H, N, d), s) for s in (15, 16, 17))
    perm = np.random.default_rng(18).permutation(N)
    o1, l1 = attn_fwd64(q, k, v, 0.25)
    o2, l2 = attn_fwd64(q, k[:, :, perm], v[:, :, perm], 0.25)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_leaves_output_and_shifts_lse(causal):
    B, H, N, d = 1, 2, 50, 8
    q, k, v = (_rand((B, H, N, d), s) for s in (19, 20, 21))
    u = 30.0 * _rand((d,), 22)  # a large shift drives the row max far away
    o1, l1 = attn_fwd64(q, k, v, 0.35, causal)
    o2, l2 = attn_fwd64(q, k + u, v, 0.35, causal)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-11)
    np.testing.assert_allclose(l2 - l1, 0.35 * (q @ u), rtol=0, atol=1e-10)


def test_output_is_linear_in_values_and_ones_map_to_ones():
    B, H, N, d = 2, 1, 40, 8
    q, k, v1, v2 = (_rand((B, H, N, d), s) for s in (23, 24, 25, 26))
    a, c = 1.7, -0.3
    o1, _ = attn_fwd64(q, k, v1, 0.5, True, [40, 17])
    o2, _ = attn_fwd64(q, k, v2, 0.5, True, [40, 17])
    o3, _ = attn_fwd64(q, k, a * v1 + c * v2, 0.5, True, [40, 17])
    np.testing.assert_allclose(o3, a * o1 + c * o2, rtol=0, atol=1e-12)
    ones, _ = attn_fwd64(q, k, np.ones_like(v1), 0.5, True, [40, 17])
    np.testing.assert_allclose(ones, 1.0, rtol=0, atol=1e-13)


def test_row_and_head_subsets_match_full_computation():
    B, H, N, d = 2, 3, 70, 8
    q, k, v = (_rand((B, H, N, d), s) for s in (27, 28, 29))
    o, lse = attn_fwd64(q, k, v, 0.4, True, [70, 31], row_chunk=16)
    rows = [0, 5, 30, 31, 69]
    heads = [(1, 2), (0, 0)]
    os_, ls_ = attn_fwd64(q, k, v, 0.4, True, [70, 31], rows=rows, heads=heads)
    for t, (b, h) in enumerate(heads):
        np.testing.assert_allclose(os_[t], o[b, h, rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(ls_[t], lse[b, h, rows], rtol=0, atol=1e-14)


# --- backward ------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 3, 6])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(N, causal):
    B, H, d = 1, 1, 3
    for ci, kv in enumerate([None, [max(1, N - 2)]]):
        q, k, v, do = (_rand((B, H, N, d), 40 + s + 7 * ci) for s in range(4))
        scale = 0.8
        dq, dk, dv = attn_bwd64(q, k, v, do, scale, causal, kv)
        lim = None if kv is None else kv[0]
        fq, fk, fv = brute_head_grad_fd(q[0, 0], k[0, 0], v[0, 0], do[0, 0], scale,
                                        causal, lim)
        np.testing.assert_allclose(dq[0, 0], np.array(fq), rtol=0, atol=1e-8)
        np.testing.assert_allclose(dk[0, 0], np.array(fk), rtol=0, atol=1e-8)
        np.testing.assert_allclose(dv[0, 0], np.array(fv), rtol=0, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_autograd_of_the_definition(causal):
    B, H, N, d = 2, 2, 48, 16
    q, k, v, do = (_rand((B, H, N, d), 60 + s) for s in range(4))
    kv = [48, 29]
    scale = 0.25
    dq, dk, dv = attn_bwd64(q, k, v, do, scale, causal, kv)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    j = torch.arange(N)
    vis = (j[None, :] < torch.tensor(kv)[:, None])[:, None, None, :]
    if causal:
        vis = vis & (j[None, :] <= j[:, None])[None, None]
    s = scale * tq @ tk.transpose(-1, -2)
    s = s.masked_fill(~vis, float("-inf"))
    out = torch.softmax(s, dim=-1) @ tv
    (out * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    B, H, N, d = 2, 2, 41, 8
    q, k, v, do = (_rand((B, H, N, d), 70 + s) for s in range(4))
    kv = [41, 23]
    dq, dk, dv = attn_bwd64(q, k, v, do, 0.3, causal, kv)
    # sum over keys of dK is zero: each softmax row's dS sums to zero
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-11)
    # sum over keys of dV equals sum over query rows of dO (each P row sums to 1)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-11)
    # keys hidden by padding receive no gradient
    assert np.all(dk[1, :, 23:] == 0.0) and np.all(dv[1, :, 23:] == 0.0)


def test_identical_keys_give_zero_query_gradient():
    B, H, N, d = 1, 1, 30, 8
    q, v, do = (_rand((B, H, N, d), 80 + s) for s in range(3))
    k = np.broadcast_to(_rand((1, 1, 1, d), 84), (B, H, N, d)).copy()
    for causal in (False, True):
        dq, _, _ = attn_bwd64(q, k, v, do, 0.5, causal)
        np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-12)


def test_backward_head_subset_matches_full():
    B, H, N, d = 2, 2, 20, 4
    q, k, v, do = (_rand((B, H, N, d), 90 + s) for s in range(4))
    full = attn_bwd64(q, k, v, do, 0.5, True, [20, 9])
    part = attn_bwd64(q, k, v, do, 0.5, True, [20, 9], heads=[(1, 0)])
    for f, p in zip(full, part):
        np.testing.assert_array_equal(f[1, 0], p[0])


# --- numbers printed on the pages ----------------------------------------------

def test_worked_example_fp32_gap_is_rounding_sized():
    """The Ultralytics glossary page (section "Come funziona Flash Attention")
    prints a 4.3e-07 max gap between two fp32 computations of the same
    attention at n=4096, d=64 on a seed-0 normal draw. The oracle must sit
    within that fp32 rounding band of an fp32 evaluation of the definition
    on such a draw: a wrong scale, a transposed operand or a dropped term
    would be off by orders of magnitude more."""
    g = json.load(open(os.path.join(GOLDEN, "streaming_fp32_worked_example.json")))
    n, d = g["n"], g["d"]
    gen = torch.Generator().manual_seed(g["seed"])
    x = torch.randn((3, n, d), generator=gen)
    q, k, v = x[0], x[1], x[2]
    s32 = (q @ k.T) * (1.0 / math.sqrt(d))
    e32 = torch.exp(s32 - s32.max(dim=1, keepdim=True).values)
    ref32 = (e32 @ v) / e32.sum(dim=1, keepdim=True)
    o64, _ = attn_fwd64(q[None, None], k[None, None], v[None, None], 1.0 / math.sqrt(d))
    gap = float(np.abs(o64[0, 0] - ref32.double().numpy()).max())
    printed = g["printed_max_abs_diff_fp32"]
    assert printed / 20 < gap < printed * 10, gap
    assert g["printed_largest_tile"][0] * g["printed_largest_tile"][1] * 16 == n * n


def test_score_matrix_bytes_match_printed_examples():
    g = json.load(open(os.path.join(GOLDEN, "score_matrix_bytes.json")))
    for c in g["cases"]:
        got = score_matrix_bytes(c["batch"], c["heads"], c["seq"], c["elem_bytes"])
        if c["exact"]:
            assert got == c["printed_bytes"]
        else:
            assert abs(got / 1e9 - c["printed_gb_approx"]) <= c["rel_tol"] * c["printed_gb_approx"]


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_backward_matches_finite_differences_and_full(causal):
    from oracle import attn_bwd64_sampled
    # tiny: against central differences of the brute force directly
    B, H, N, d = 1, 1, 6, 3
    q, k, v, do = (_rand((B, H, N, d), 100 + s) for s in range(4))
    kv = [5]
    fq, fk, fv = brute_head_grad_fd(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.8, causal, kv[0])
    sq, sk, sv = attn_bwd64_sampled(q, k, v, do, 0.8, causal, kv, heads=[(0, 0)],
                                    q_rows=[0, 2, 5], k_rows=[1, 4, 5], row_chunk=2)
    np.testing.assert_allclose(sq[0], np.array(fq)[[0, 2, 5]], rtol=0, atol=1e-8)
    np.testing.assert_allclose(sk[0], np.array(fk)[[1, 4, 5]], rtol=0, atol=1e-8)
    np.testing.assert_allclose(sv[0], np.array(fv)[[1, 4, 5]], rtol=0, atol=1e-8)
    # larger: same numbers as the whole-matrix backward
    B, H, N, d = 2, 2, 90, 8
    q, k, v, do = (_rand((B, H, N, d), 110 + s) for s in range(4))
    kv = [90, 40]
    dq, dk, dv = attn_bwd64(q, k, v, do, 0.3, causal, kv)
    rows, keys = [0, 7, 39, 40, 89], [0, 3, 39, 40, 88]
    sq, sk, sv = attn_bwd64_sampled(q, k, v, do, 0.3, causal, kv, heads=[(1, 1), (0, 1)],
                                    q_rows=rows, k_rows=keys, row_chunk=32)
    for t, (b, h) in enumerate([(1, 1), (0, 1)]):
        np.testing.assert_allclose(sq[t], dq[b, h, rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sk[t], dk[b, h, keys], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sv[t], dv[b, h, keys], rtol=0, atol=1e-12)
    # dQ rows alone (no keys asked for): the same numbers without the pass over every row
    sq2, sk2, _ = attn_bwd64_sampled(q, k, v, do, 0.3, causal, kv, heads=[(1, 1), (0, 1)],
                                     q_rows=rows, k_rows=[], row_chunk=32)
    assert sk2.shape == (2, 0, d)
    for t, (b, h) in enumerate([(1, 1), (0, 1)]):
        np.testing.assert_allclose(sq2[t], dq[b, h, rows], rtol=0, atol=1e-12)


def test_sampled_backward_of_late_keys_under_the_causal_mask():
    """Keys near the end (causal): only the rows from the first such key on
    are passed over; the result is the whole backward's."""
    from oracle import attn_bwd64_sampled
    B, H, N, d = 1, 1, 70, 4
    q, k, v, do = (_rand((B, H, N, d), 120 + s) for s in range(4))
    dq, dk, dv = attn_bwd64(q, k, v, do, 0.5, True)
    keys = [69, 60, 55]
    _, sk, sv = attn_bwd64_sampled(q, k, v, do, 0.5, True, heads=[(0, 0)], q_rows=[], k_rows=keys,
                                   row_chunk=8)
    np.testing.assert_allclose(sk[0], dk[0, 0, keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sv[0], dv[0, 0, keys], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_magnitudes_by_explicit_loops_and_as_bounds(causal):
    """attn_bwd64_magnitudes against the same formulas written as loops with
    math.exp (N = 5), as elementwise bounds of the gradients on random
    inputs, and equal to dV where dO >= 0."""
    from oracle import attn_bwd64_magnitudes
    rng = np.random.default_rng(21 + causal)
    B, H, N, d, scale = 1, 1, 5, 3, 0.7
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    mq, mk, mv = attn_bwd64_magnitudes(q, k, v, do, scale, causal)
    Q, K, V, G = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    P = [[0.0] * N for _ in range(N)]
    for i in range(N):
        keys = [j for j in range(N) if not (causal and j > i)]
        s = {j: scale * sum(Q[i][c] * K[j][c] for c in range(d)) for j in keys}
        mx = max(s.values())
        z = math.fsum(math.exp(s[j] - mx) for j in keys)
        for j in keys:
            P[i][j] = math.exp(s[j] - mx) / z
    dP = [[sum(G[i][c] * V[j][c] for c in range(d)) for j in range(N)] for i in range(N)]
    D = [math.fsum(P[i][j] * dP[i][j] for j in range(N)) for i in range(N)]
    W = [[P[i][j] * (abs(dP[i][j]) + abs(D[i])) for j in range(N)] for i in range(N)]
    for i in range(N):
        for c in range(d):
            assert abs(mq[0, 0, i, c] - scale * math.fsum(W[i][j] * abs(K[j][c]) for j in range(N))) < 1e-12
            assert abs(mk[0, 0, i, c] - scale * math.fsum(W[j][i] * abs(Q[j][c]) for j in range(N))) < 1e-12
            assert abs(mv[0, 0, i, c] - math.fsum(P[j][i] * abs(G[j][c]) for j in range(N))) < 1e-12
    q, k, v, do = (rng.standard_normal((2, 2, 40, 8)) for _ in range(4))
    grads = attn_bwd64(q, k, v, do, 0.3, causal, [40, 17])
    mags = attn_bwd64_magnitudes(q, k, v, do, 0.3, causal, [40, 17])
    for g, m in zip(grads, mags):
        assert np.all(np.abs(g) <= m + 1e-12)
    dv = attn_bwd64(q, k, v, np.abs(do), 0.3, causal)[2]
    np.testing.assert_allclose(attn_bwd64_magnitudes(q, k, v, np.abs(do), 0.3, causal)[2], dv,
                               rtol=0, atol=1e-12)
