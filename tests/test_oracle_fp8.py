"""Pins of the FP8 oracle (oracle/fp8.py), CPU only.

  * the e4m3 codec: values fixed by the format (1.0, 448, the smallest
    normal and subnormal, signed zero, NaN codes), every finite code round
    trips, and encoding agrees with a pure-Python nearest search (ties to the
    even code) on random values and on every midpoint;
  * the transform: equal to multiplication by the Sylvester Hadamard matrix
    (exactly, on integer inputs), applying it twice gives d x, and the
    rotated dot products are d times the originals;
  * block quantisation: the block maximum maps to the code of 448, every
    value is within half a step of the e4m3 grid after scaling, an all-zero
    block gives scale 0;
  * attention: on inputs the quantiser represents exactly and with P left
    unquantised, the tiled loop equals the plain fp64 oracle (masks, scale,
    the 1/d of the rotation, the V scale); identical keys give the mean of V
    exactly even with P quantised; the quantisation of P moves O by at most
    1/16 of max|V|.
"""
import math

import numpy as np
import pytest

from oracle import (E4M3_MAX, attn_fwd64, attn_fwd64_fp8, e4m3_decode, e4m3_encode, fp8_quantize,
                    fp8_quantize_rows, fwht32)


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def py_decode(c):
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if s else v


POS = [(py_decode(c), c) for c in range(127)]  # codes 0..126: 0 .. 448, increasing


def py_encode(x):
    """Nearest e4m3 value by exhaustive search, ties to the even code."""
    a = abs(x)
    best = min(abs(v - a) for v, _ in POS)
    codes = [c for v, c in POS if abs(v - a) == best]
    c = codes[0] if len(codes) == 1 else [c for c in codes if c % 2 == 0][0]
    return c | (0x80 if math.copysign(1.0, x) < 0 else 0)


def test_decode_fixed_values():
    assert e4m3_decode(0x38) == 1.0 and e4m3_decode(0xB8) == -1.0
    assert e4m3_decode(0x7E) == 448.0 and e4m3_decode(0x01) == 2.0 ** -9
    assert e4m3_decode(0x08) == 2.0 ** -6 and e4m3_decode(0x07) == 7 * 2.0 ** -9
    z = e4m3_decode(0x80)
    assert z == 0.0 and math.copysign(1.0, z) < 0
    assert np.isnan(e4m3_decode(0x7F)) and np.isnan(e4m3_decode(0xFF))
    vals = e4m3_decode(np.arange(127))
    assert np.all(np.diff(vals) > 0)
    for c in range(256):
        a, b = e4m3_decode(c), py_decode(c)
        assert (np.isnan(a) and math.isnan(b)) or a == b


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_matches_exhaustive_search():
    rng = np.random.default_rng(1)
    xs = list(rng.uniform(-448, 448, 400)) + list(rng.standard_normal(300) * 0.01)
    xs += [0.5 * (py_decode(c) + py_decode(c + 1)) for c in range(126)]       # every midpoint
    xs += [-0.5 * (py_decode(c) + py_decode(c + 1)) for c in range(126)]
    xs += [448.0, -448.0, 2.0 ** -10, 2.0 ** -10 * 3, 1e-9]
    got = e4m3_encode(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == py_encode(x), (x, int(g), py_encode(x))
    with pytest.raises(ValueError):
        e4m3_encode(np.array([449.0]))


def hadamard(d):
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_fwht_is_the_hadamard_matrix(d):
    x = np.random.default_rng(d).integers(-50, 50, (7, d)).astype(np.float32)
    np.testing.assert_array_equal(fwht32(x), (x.astype(np.float64) @ hadamard(d)).astype(np.float32))
    np.testing.assert_array_equal(fwht32(fwht32(x)), d * x)
    y = rnd((5, d), d + 1).astype(np.float32)
    np.testing.assert_allclose(fwht32(y), y.astype(np.float64) @ hadamard(d), rtol=0, atol=1e-4 * d)


def test_rotation_preserves_dot_products_up_to_d():
    d = 128
    q, k = rnd((6, d), 2).astype(np.float32), rnd((9, d), 3).astype(np.float32)
    s = np.where(np.random.default_rng(4).random(d) < 0.5, -1.0, 1.0).astype(np.float32)
    qr, kr = fwht32(q * s), fwht32(k * s)
    np.testing.assert_allclose(qr.astype(np.float64) @ kr.T.astype(np.float64) / d,
                               q.astype(np.float64) @ k.T, atol=1e-4)


def test_block_quantisation():
    x = (rnd((2, 300, 16), 5) * np.array([1.0, 30.0])[:, None, None]).astype(np.float32)
    x[1, 64:128] = 0.0
    codes, scales = fp8_quantize_rows(x, 64)
    assert scales.shape == (2, 5) and scales[1, 1] == 0 and np.all(codes[1, 64:128] == 0)
    for b in range(2):
        for i in range(5):
            blk = x[b, i * 64:(i + 1) * 64]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            assert scales[b, i] == np.float32(amax) / np.float32(448)
            c = codes[b, i * 64:(i + 1) * 64]
            at = np.abs(blk) == amax
            assert np.all((c[at] & 0x7F) == 0x7E)
            t = np.abs(blk.astype(np.float64) * 448 / amax)
            deq = np.abs(e4m3_decode(c))
            step = np.where(t >= 2 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(t, 2 ** -6))) - 3), 2.0 ** -9)
            assert np.all(np.abs(deq - t) <= 0.5 * step * (1 + 1e-6))


def exact_inputs(B, H, N, d, seed):
    """Values on the e4m3 grid with a 448 in every 64-row block (every
    128-row block too) and in every head of V, so that quantisation is
    lossless with scale 1."""
    rng = np.random.default_rng(seed)
    grid = e4m3_decode(np.arange(0x30, 0x48))           # 0.5 .. 4, exactly representable
    def make():
        x = rng.choice(grid, (B, H, N, d)) * rng.choice([-1.0, 1.0], (B, H, N, d))
        x[..., ::64, 0] = 448.0
        return x.astype(np.float32)
    return make(), make(), make()


@pytest.mark.parametrize("causal", [False, True])
def test_lossless_quantisation_and_exact_p_is_plain_attention(causal):
    B, H, N, d = 2, 2, 200, 16
    q, k, v = exact_inputs(B, H, N, d, 7)
    qz = fp8_quantize(q, k, v, None)
    assert np.all(qz["sq"] == 1) and np.all(qz["sk"] == 1) and np.all(qz["sv"] == 1)
    np.testing.assert_array_equal(e4m3_decode(qz["q8"]), q)
    kv = [200, 77]
    o, lse = attn_fwd64_fp8(qz, 0.01, causal, kv, quantize_p=False)
    o2, lse2 = attn_fwd64(q, k, v, 0.01, causal, kv)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)


def test_rotation_factor_and_scales_are_undone():
    B, H, N, d = 1, 2, 150, 64
    q, k, v = (rnd((B, H, N, d), s) for s in (8, 9, 10))
    s = np.where(np.random.default_rng(11).random(d) < 0.5, -1.0, 1.0)
    qz = fp8_quantize(q, k, v, s)
    o, lse = attn_fwd64_fp8(qz, 0.125, True, None, quantize_p=False)
    o2, lse2 = attn_fwd64(q, k, v, 0.125, True)
    # only the e4m3 rounding of Q, K and V separates the two
    assert np.abs(o - o2).max() < 0.15 and np.abs(lse - lse2).max() < 0.1
    assert np.abs(o - o2).mean() < 0.02


def test_identical_keys_give_the_mean_of_v_with_p_quantised():
    B, H, N, d = 1, 1, 130, 16
    q = rnd((B, H, N, d), 12)
    k = np.repeat(rnd((1, 1, 1, d), 13), N, axis=2)
    _, _, v = exact_inputs(B, H, N, d, 14)
    qz = fp8_quantize(q, k, v, None)
    o, _ = attn_fwd64_fp8(qz, 0.3, True, None)
    vd = e4m3_decode(qz["v8"][0, 0]) * qz["sv"][0, 0]
    np.testing.assert_allclose(o[0, 0], np.cumsum(vd, axis=0) / np.arange(1, N + 1)[:, None], atol=1e-12)


def test_quantised_p_moves_o_by_at_most_a_sixteenth_of_v():
    B, H, N, d = 1, 2, 300, 32
    q, k, v = (rnd((B, H, N, d), s) for s in (15, 16, 17))
    qz = fp8_quantize(q, k, v, None)
    o, _ = attn_fwd64_fp8(qz, 0.2, False, None)
    o_exact_p, _ = attn_fwd64_fp8(qz, 0.2, False, None, quantize_p=False)
    vmax = np.abs(e4m3_decode(qz["v8"]) * qz["sv"][..., None, None]).max()
    assert np.abs(o - o_exact_p).max() <= vmax / 16
    assert np.abs(o - o_exact_p).max() > 0  # P quantisation does change O


def one_row_case(scores, seed):
    """Query row 0 against N keys whose scores are ``scores`` exactly: q = e_0,
    k_j = scores_j e_0 / scale (values on the e4m3 grid, one block each, a
    448 placed in an unused column so that every scale is 1); V on the grid."""
    N, d = len(scores), 16
    q = np.zeros((1, 1, N, d), np.float32)
    k = np.zeros((1, 1, N, d), np.float32)
    q[0, 0, :, 0] = 1.0
    q[0, 0, ::128, d - 1] = 448.0
    k[0, 0, :, 0] = scores
    k[0, 0, ::64, d - 2] = 448.0
    _, _, v = exact_inputs(1, 1, N, d, seed)
    return q, k, v


def test_two_keys_closed_form_sum_of_unquantised_p():
    q, k, v = one_row_case([0.0, -1.0], 20)
    qz = fp8_quantize(q, k, v, None)
    o, lse = attn_fwd64_fp8(qz, 1.0, False, None)
    p1 = math.exp(-1.0)
    q1 = py_decode(py_encode(256 * p1)) / 256  # 94 / 256
    vd = e4m3_decode(qz["v8"][0, 0]).astype(np.float64)
    expect = (vd[0] + q1 * vd[1]) / (1.0 + p1)
    np.testing.assert_allclose(o[0, 0, 0], expect, atol=1e-13)
    assert abs(lse[0, 0, 0] - math.log(1 + p1)) < 1e-13


def test_p_is_quantised_against_the_running_max():
    # 64 keys of score 0 fill the first tile, then one key of score c: the
    # first tile's p are quantised as 1 (exact), then rescaled by e^-c
    c = 2.0
    q, k, v = one_row_case([0.0] * 64 + [c], 21)
    qz = fp8_quantize(q, k, v, None)
    o, lse = attn_fwd64_fp8(qz, 1.0, False, None)
    vd = e4m3_decode(qz["v8"][0, 0]).astype(np.float64)
    a = math.exp(-c)
    expect = (a * vd[:64].sum(axis=0) + vd[64]) / (64 * a + 1)
    np.testing.assert_allclose(o[0, 0, 0], expect, atol=1e-12)
    assert abs(lse[0, 0, 0] - (c + math.log(64 * a + 1))) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_row_subset_equals_the_whole(causal):
    """``rows`` only selects outputs: each selected row is the same as in the
    whole computation (the row's own query block scale, all its keys)."""
    rng = np.random.default_rng(11)
    B, H, N, d = 2, 1, 300, 64
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    qz = fp8_quantize(q, k, v, np.where(rng.random(d) < 0.5, -1, 1))
    o, lse = attn_fwd64_fp8(qz, 0.125, causal, [300, 170])
    rows = [0, 5, 127, 128, 169, 170, 299]
    o_r, lse_r = attn_fwd64_fp8(qz, 0.125, causal, [300, 170], rows=rows)
    # equal up to fp64 rounding (the products are blocked differently)
    np.testing.assert_allclose(o_r, o[:, :, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_r, lse[:, :, rows], rtol=0, atol=1e-12)


TRUNC = 2.0 ** -12  # the matrix cores' alignment granularity the GPU tests use


def test_error_bound_leaves_o_and_lse_unchanged():
    rng = np.random.default_rng(31)
    q, k, v = (rng.standard_normal((1, 2, 200, 64)) for _ in range(3))
    qz = fp8_quantize(q, k, v, np.where(rng.random(64) < 0.5, -1, 1))
    o, lse = attn_fwd64_fp8(qz, 0.125, True, None)
    o2, lse2, bnd = attn_fwd64_fp8(qz, 0.125, True, None, trunc=TRUNC)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    assert bnd["o"].shape == o.shape and bnd["flip"].shape == o.shape and bnd["lse"].shape == lse.shape
    assert np.all(bnd["flip"] >= 0) and bnd["flip"].max() > 0
    assert np.all(bnd["o"] >= bnd["flip"]) and np.all(bnd["lse"] > 0)
    # with (almost) no alignment loss only codes within a few fp32 ulps of a
    # rounding boundary stay open
    _, _, tiny = attn_fwd64_fp8(qz, 0.125, True, None, trunc=1e-14)
    rows_open = np.count_nonzero(bnd["flip"].max(axis=-1))
    assert np.count_nonzero(tiny["flip"].max(axis=-1)) <= 0.1 * rows_open


def _group_loss(qrow, krow, trunc):
    """The model's bound on what one product sum loses, by explicit loops:
    per aligned group of 8, min(sum |q_c k_c|, 7 trunc max|q_c| max|k_c|)."""
    total = 0.0
    for g0 in range(0, len(qrow), 8):
        pg = [abs(float(qrow[c]) * float(krow[c])) for c in range(g0, min(g0 + 8, len(qrow)))]
        qm = max(abs(float(x)) for x in qrow[g0:g0 + 8])
        km = max(abs(float(x)) for x in krow[g0:g0 + 8])
        total += min(sum(pg), 7 * trunc * qm * km)
    return total


def test_group_loss_bound_against_explicit_loops():
    from oracle import mfma_loss_bound
    rng = np.random.default_rng(7)
    a = rng.standard_normal((5, 70)) * np.where(rng.random(70) < 0.1, 30, 1)
    b = rng.standard_normal((6, 70))
    got = mfma_loss_bound(np.abs(a), np.abs(b), 1e-3)
    for r in range(5):
        for j in range(6):
            assert abs(got[r, j] - _group_loss(a[r], b[j], 1e-3)) <= 1e-12 * (1 + got[r, j])


def test_group_loss_bound_covers_truncating_groups():
    """Sums computed as the model says (per aligned group of 8, every product
    but the group's largest cut toward zero to a multiple of trunc x that
    largest product) lose no more than the bound: random products, random
    ones with a dominant product per group, and a case the bound nearly
    meets (one product of 90,000 per group and seven of 21.2, each just under
    the granularity 90,000 / 4096 = 22.0, so all seven are lost)."""
    from oracle import mfma_loss_bound
    rng = np.random.default_rng(8)
    trunc = 2.0 ** -12
    for case in ("random", "dominant", "tight"):
        a = rng.standard_normal((40, 64))
        b = rng.standard_normal((30, 64))
        if case == "dominant":
            a[:, ::8] *= 300.0
            b[:, ::8] *= 300.0
        if case == "tight":
            a[:] = 4.6
            b[:] = 4.6
            a[:, ::8] = 300.0
            b[:, ::8] = 300.0
        exact = a @ b.T
        cut = np.zeros_like(exact)
        for g0 in range(0, 64, 8):
            prod = a[:, None, g0:g0 + 8] * b[None, :, g0:g0 + 8]
            mx = np.abs(prod).max(axis=-1, keepdims=True)
            G = trunc * mx
            t = np.trunc(prod / G) * G
            top = np.abs(prod) == mx
            cut += np.where(top, prod, t).sum(axis=-1)
        loss = np.abs(cut - exact)
        bound = mfma_loss_bound(np.abs(a), np.abs(b), trunc)
        assert np.all(loss <= bound * (1 + 1e-12))
        if case == "tight":
            assert (loss / bound).min() > 0.9


def test_flip_bound_of_one_open_code_closed_form():
    # scores 0 and c = -0.625 (on the e4m3 grid): 256 e^c = 137.03 lies 0.76%
    # above the rounding boundary 136 between the codes 128 and 144. Key 1's
    # product sum has one nonzero product, c, in the group of channels 0-7,
    # so its loss bound is 7 trunc |c|, and its exponent error about twice
    # that (its own score and the row max): open for trunc = 2e-3, closed for
    # trunc = 2e-4.
    c = -0.625
    q, k, v = one_row_case([0.0, c], 22)
    qz = fp8_quantize(q, k, v, None)
    p1 = math.exp(c)
    assert py_decode(py_encode(256 * p1)) == 144
    vd = e4m3_decode(qz["v8"][0, 0]).astype(np.float64)
    _, _, b_open = attn_fwd64_fp8(qz, 1.0, False, None, trunc=2e-3)
    expect = (16 / 256) * np.abs(vd[1]) * float(qz["sv"][0, 0]) / (1 + p1)
    np.testing.assert_allclose(b_open["flip"][0, 0, 0], expect, rtol=0, atol=1e-13)
    _, _, b_closed = attn_fwd64_fp8(qz, 1.0, False, None, trunc=2e-4)
    assert np.all(b_closed["flip"][0, 0, 0] == 0)


def _exponent_error(qrow, krows, s, a, scale, trunc):
    """The model's exponent error bound for one row inside one tile, by
    explicit loops: s, a the row's visible scores and magnitude sums
    (natural-log units)."""
    u = 2.0 ** -24
    loss = np.array([_group_loss(qrow, kr, trunc) for kr in krows])
    delta = scale * loss + 16 * u * a + 4 * u * np.abs(s)
    return delta + delta.max() + 8 * u * (np.abs(s) + abs(s.max()) + 8)


@pytest.mark.parametrize("causal", [False, True])
def test_flip_bound_covers_every_combination_of_code_moves(causal):
    """Brute force over one tile: for each row, every subset of its open
    codes moved to their other candidates changes O by no more than the
    flip bound, element by element; and the bound (a sum over the open
    codes) is within a factor two of the largest such change."""
    rng = np.random.default_rng(40 + causal)
    N, d, scale, trunc = 48, 64, 0.125, 2.0 ** -14
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    qz = fp8_quantize(q, k, v, None)
    o, _, bnd = attn_fwd64_fp8(qz, scale, causal, None, trunc=trunc)
    flip = bnd["flip"][0, 0]
    qd = e4m3_decode(qz["q8"][0, 0]) * float(qz["sq"][0, 0, 0])
    kd = e4m3_decode(qz["k8"][0, 0]) * float(qz["sk"][0, 0, 0])
    vd = e4m3_decode(qz["v8"][0, 0])
    sv = float(qz["sv"][0, 0])
    most = 0
    for i in range(N):
        keys = np.arange(i + 1 if causal else N)
        s = scale * (kd[keys] @ qd[i])
        a = scale * (np.abs(kd[keys]) @ np.abs(qd[i]))
        p = np.exp(s - s.max())
        x = 256 * p
        codes = e4m3_decode(e4m3_encode(x))
        o_i = (codes / 256) @ vd[keys] * sv / p.sum()
        np.testing.assert_allclose(o_i, o[0, 0, i], rtol=0, atol=1e-12)
        e = _exponent_error(qd[i], kd[keys], s, a, scale, trunc)
        alts = []
        for j in range(len(keys)):
            for alt in (e4m3_decode(e4m3_encode(x[j] * np.exp(e[j]))),
                        e4m3_decode(e4m3_encode(x[j] * np.exp(-e[j])))):
                if alt != codes[j]:
                    alts.append((j, alt))
        assert len(alts) <= 12
        most = max(most, len(alts))
        worst = np.zeros(d)
        for mask in range(1 << len(alts)):
            c2 = codes.copy()
            for bit, (j, alt) in enumerate(alts):
                if mask >> bit & 1:
                    c2[j] = alt
            diff = np.abs((c2 / 256) @ vd[keys] * sv / p.sum() - o_i)
            assert np.all(diff <= flip[i] + 1e-12), (i, mask)
            worst = np.maximum(worst, diff)
        assert np.all(worst >= 0.5 * flip[i] - 1e-12), i
    assert most >= 3  # rows with several open codes at once were exercised


def _grouped_sum(a, b, trunc, mode, rng):
    """Product sums a_r . b_j the way the model lets the matrix cores form
    them: per aligned group of 8, every product but the group's largest cut
    toward zero to a multiple of trunc x that largest product ("extreme"), or
    by a random part of that cut ("random")."""
    out = np.zeros((a.shape[0], b.shape[0]))
    for g0 in range(0, a.shape[1], 8):
        prod = a[:, None, g0:g0 + 8] * b[None, :, g0:g0 + 8]
        mx = np.abs(prod).max(axis=-1, keepdims=True)
        G = np.where(mx > 0, trunc * mx, 1.0)
        t = np.trunc(prod / G) * G
        if mode == "random":
            t = prod + rng.uniform(0, 1, prod.shape) * (t - prod)
        out += np.where(np.abs(prod) == mx, prod, t).sum(axis=-1)
    return out


def _fp32_like(qz, scale, causal, trunc, rng, extreme):
    """One implementation of the FP8 attention steps as the error model
    allows them to err: the scores and the P V sums formed by grouped
    truncation (_grouped_sum), every score also off by up to 2^-20 of its
    magnitude sum plus 2^-22 of itself, each exponential and rescale by up
    to its fp32 error; the P codes decided from these values (so open codes
    may go either way). ``extreme`` draws the perturbations at the ends of
    their ranges."""
    q8, k8, v8 = qz["q8"], qz["k8"], qz["v8"]
    B, H, N, d = q8.shape
    u = 2.0 ** -24
    s_mul = scale / (d if qz["rotated"] else 1)
    out = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    mode = "extreme" if extreme else "random"

    def draw(shape):
        r = rng.uniform(-1, 1, shape)
        return np.sign(r) if extreme else r

    for b in range(B):
        for h in range(H):
            qd = e4m3_decode(q8[b, h]) * qz["sq"][b, h].astype(np.float64)[np.arange(N) // 128][:, None]
            kd = e4m3_decode(k8[b, h]) * np.repeat(qz["sk"][b, h].astype(np.float64), 64)[:N, None]
            vd = e4m3_decode(v8[b, h])
            s_all = s_mul * _grouped_sum(qd, kd, trunc, mode, rng)
            a_all = s_mul * (np.abs(qd) @ np.abs(kd).T)
            s_all = s_all + draw(s_all.shape) * (16 * u * a_all + 4 * u * np.abs(s_all))
            for i in range(N):
                m, l, acc = -np.inf, 0.0, np.zeros(d)
                for t0 in range(0, N, 64):
                    cols = np.arange(t0, min(t0 + 64, N))
                    if causal:
                        cols = cols[cols <= i]
                    if len(cols) == 0:
                        break
                    s = s_all[i, cols]
                    m_new = max(m, s.max())
                    if m_new > m:
                        alpha = np.exp(m - m_new) * (1 + draw(()) * 8 * u * (abs(m_new) + 8)) if m > -np.inf else 1.0
                        l *= alpha
                        acc = acc * alpha
                        m = m_new
                    p = np.exp(s - m) * (1 + draw(len(cols)) * 8 * u * (np.abs(s) + abs(m) + 8))
                    l += p.sum()
                    pq = e4m3_decode(e4m3_encode(256 * p)) / 256
                    # the tile's P V sums: keys grouped by 8 from the tile start
                    pv = np.zeros(64)
                    pv[cols - t0] = pq
                    vt = np.zeros((64, d))
                    vt[cols - t0] = vd[cols]
                    acc = acc + _grouped_sum(pv[None, :], vt.T, trunc, mode, rng)[0]
                out[b, h, i] = acc * float(qz["sv"][b, h]) / l
                lse[b, h, i] = m + math.log(l)
    return out, lse


@pytest.mark.parametrize("extreme", [False, True])
@pytest.mark.parametrize("causal,rot", [(False, True), (True, False)])
def test_error_bound_covers_perturbed_implementations(causal, rot, extreme):
    """Implementations that err as the model allows, over several tiles with
    rescales (random and extreme truncation, outlier channels so that
    products differ widely): every element of O and every LSE stays within
    the bounds, and the bound is not vacuous for them."""
    rng = np.random.default_rng(60 + 2 * causal + rot + 4 * extreme)
    B, H, N, d, scale = 1, 2, 200, 64, 0.125
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    q[..., 3] *= 16
    k[..., 3] *= 16
    qz = fp8_quantize(q, k, v, np.where(rng.random(d) < 0.5, -1, 1) if rot else None)
    o, lse, bnd = attn_fwd64_fp8(qz, scale, causal, None, trunc=TRUNC)
    used = 0.0
    for _ in range(2):
        o2, lse2 = _fp32_like(qz, scale, causal, TRUNC, rng, extreme)
        assert np.all(np.abs(o2 - o) <= bnd["o"]), np.abs(o2 - o).max()
        assert np.all(np.abs(lse2 - lse) <= bnd["lse"]), np.abs(lse2 - lse).max()
        used = max(used, float((np.abs(o2 - o) / bnd["o"]).max()))
    assert used > 0.05


@pytest.mark.parametrize("extreme", [False, True])
def test_error_bound_covers_p_v_truncation(extreme):
    """Identical keys with small scores: every P code is 256 and unique, and
    the score errors are tiny, so what the bound must cover is the grouped
    truncation of the P V sums alone. V has one dominant key (code 448) in
    every group of 8 keys and seven keys of code 0.1015625, just under the
    granularity 448 / 4096 = 0.109, the case where truncation loses most."""
    rng = np.random.default_rng(70 + extreme)
    B, H, N, d = 1, 1, 192, 64
    q = 0.01 * rng.standard_normal((B, H, N, d))
    k = np.repeat(rng.standard_normal((B, H, 1, d)), N, axis=2)
    v = np.full((B, H, N, d), 0.1015625 * 300.0 / 448.0)
    v[:, :, ::8] = 300.0
    qz = fp8_quantize(q, k, v, None)
    o, lse, bnd = attn_fwd64_fp8(qz, 0.125, False, None, trunc=TRUNC)
    assert np.all(bnd["flip"] == 0)
    o2, _ = _fp32_like(qz, 0.125, False, TRUNC, rng, extreme)
    err = np.abs(o2 - o)
    assert np.all(err <= bnd["o"]), (err / bnd["o"]).max()
    if extreme:
        assert (err / bnd["o"]).max() > 0.3
