"""FP8 attention forward with incoherent processing, step by step.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The marketmaker.cc article (section "FA3：料斗力学", item 3) says that plain
FP8 attention is spoiled by outliers and that the FP8 path of FlashAttention-3
rotates the vectors at random before quantising them block by block, which
spreads an outlier over all coordinates; the Ultralytics glossary page
("FlashAttention-2, -3 e -4") adds that FlashAttention-3 supports FP8. The
pages give no formulas. This is an approximation, so the oracle follows the
steps of the method in order, with these readings:

  * rotation: y = FWHT(x * s) for every row x of Q and of K, where s is a
    random +-1 vector of length d (an input) and FWHT the unnormalised
    Walsh-Hadamard transform, in fp32, stage by stage (h = 1, 2, ..., d/2;
    elements i and i + h with bit h of i clear become a + b and a - b). The
    rotation is orthogonal up to the factor d: (Q R)(K R)^T = d Q K^T, so the
    scores carry an extra 1/d. V is not rotated;
  * quantisation to OCP FP8 e4m3 (bias 7, max 448, no infinities), block by
    block: one fp32 scale per block of 128 query rows, per block of 64 key
    rows, and per head for V; scale = amax / 448 and code =
    e4m3_rne(clamp(x * (448 / amax), -448, 448)), every product and quotient
    in fp32 (the precision in which the codes are decided); an all-zero block
    has scale 0 and codes 0;
  * attention over the dequantised Q and K in fp64, tile by tile over 64
    keys with the running row max and running sum of the online softmax
    (marketmaker.cc article, section "在线softmax递归"); in each tile the
    probabilities p = exp(S - m) (m the running max after the tile) are
    quantised as e4m3_rne(256 p) before the P V product; the running sum adds
    the unquantised p; the output is acc * scale_v / l and LSE = m + ln l.
"""
from __future__ import annotations

import numpy as np

from .attention import _kv_lens

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "fwht32", "fp8_quantize_rows",
           "fp8_quantize", "mfma_loss_bound", "attn_fwd64_fp8"]

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values (fp64) of OCP e4m3 codes: sign, 4-bit exponent (bias 7), 3-bit
    mantissa; exponent 0 is subnormal (m * 2^-9); 0x7f / 0xff are NaN."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even of each value to the e4m3 grid, as uint8 codes.
    |x| must not exceed 448 (the caller clamps); -0 keeps its sign bit."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: |x| > 448, clamp first")
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    # subnormal range: steps of 2^-9 below 2^-6 (a step count of 8 is 2^-6,
    # which is the code of the smallest normal number, so no special case)
    sub = np.rint(a / 2.0 ** -9).astype(np.int64)
    mant, ex = np.frexp(np.where(a > 0, a, 1.0))       # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                                          # a = (2 mant) * 2^e, 2 mant in [1, 2)
    m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    e = np.where(m == 8, e + 1, e)
    m = np.where(m == 8, 0, m)
    norm = ((e + 7) << 3) | m
    code = np.where(a < 2.0 ** -6, sub, norm)
    return (sign | code).astype(np.uint8)


def fwht32(x) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of the last axis (a power of
    two) in fp32, stage by stage: h = 1, 2, 4, ...; indices i and i + h with
    bit h of i clear become (a + b, a - b)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(lead + (d,))
        h *= 2
    return y


def fp8_quantize_rows(x32: np.ndarray, block: int):
    """Quantise fp32 rows [..., N, d] in blocks of ``block`` rows (the last
    block may be short). Returns (codes uint8 [..., N, d], scales fp32
    [..., ceil(N / block)])."""
    x32 = np.asarray(x32, dtype=np.float32)
    N = x32.shape[-2]
    nb = (N + block - 1) // block
    codes = np.zeros(x32.shape, dtype=np.uint8)
    scales = np.zeros(x32.shape[:-2] + (nb,), dtype=np.float32)
    for i in range(nb):
        blk = x32[..., i * block:(i + 1) * block, :]
        amax = np.abs(blk).max(axis=(-2, -1)).astype(np.float32)
        safe = np.where(amax > 0, amax, np.float32(1))
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / safe, np.float32(0)).astype(np.float32)
        scales[..., i] = np.where(amax > 0, safe / np.float32(E4M3_MAX), np.float32(0))
        t = (blk * inv[..., None, None]).astype(np.float32)
        t = np.clip(t, -np.float32(E4M3_MAX), np.float32(E4M3_MAX))
        codes[..., i * block:(i + 1) * block, :] = e4m3_encode(t)
    return codes, scales


def _to32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to(device="cpu", dtype=torch.float32).numpy()
    return np.asarray(x, dtype=np.float32)


def fp8_quantize(q, k, v, signs=None, block_q: int = 128, block_k: int = 64):
    """The quantisation step. q, k, v: [B, H, N, d] (any float type, exactly
    widened to fp32); signs: +-1 vector of length d, or None for no rotation.
    Returns a dict: q8, k8, v8 (uint8 [B, H, N, d], row-major), sq [B, H,
    ceil(N / block_q)], sk [B, H, ceil(N / block_k)], sv [B, H] (fp32)."""
    q32, k32, v32 = _to32(q), _to32(k), _to32(v)
    if signs is not None:
        s = np.asarray(signs, dtype=np.float32)
        q32 = fwht32(q32 * s)
        k32 = fwht32(k32 * s)
    q8, sq = fp8_quantize_rows(q32, block_q)
    k8, sk = fp8_quantize_rows(k32, block_k)
    N = v32.shape[-2]
    v8, sv = fp8_quantize_rows(v32, max(N, 1))
    return {"q8": q8, "k8": k8, "v8": v8, "sq": sq, "sk": sk, "sv": sv[..., 0],
            "rotated": signs is not None}


def mfma_loss_bound(a_abs: np.ndarray, b_abs: np.ndarray, trunc: float, group: int = 8) -> np.ndarray:
    """Upper bound of what grouped alignment can lose in the product sums
    a_r . b_j (rows of a against rows of b, the reduction over the last
    axis), for a matrix core that adds the products of each aligned group of
    ``group`` reduction indices after cutting every product to a multiple of
    a granularity G <= trunc * (the group's largest |product|), toward zero,
    then adds the group sums exactly enough to ignore (their fp32 rounding is
    counted elsewhere). A group then loses at most its largest product's
    (group - 1) neighbours' share below G each, and never more than the sum
    of its |products|: min(sum |products|, (group - 1) trunc max|a| max|b|),
    where max|a| max|b| (over the group) bounds the largest product."""
    n = a_abs.shape[-1]
    out = np.zeros((a_abs.shape[0], b_abs.shape[0]))
    for g0 in range(0, n, group):
        ag = a_abs[:, g0:g0 + group]
        bg = b_abs[:, g0:g0 + group]
        out += np.minimum(ag @ bg.T, (group - 1) * trunc * np.outer(ag.max(axis=1), bg.max(axis=1)))
    return out


def attn_fwd64_fp8(qz: dict, scale: float, causal: bool = False, kv_len=None, tile: int = 64,
                   block_q: int = 128, block_k: int = 64, p_scale: float = 256.0,
                   quantize_p: bool = True, rows=None, trunc: float = 0.0, group: int = 8):
    """Attention over the quantised inputs of ``fp8_quantize`` (tile by tile,
    P quantised per tile; see the module text). ``quantize_p=False`` skips
    the quantisation of P (for pinning the rest); ``rows`` restricts the
    output to those query rows (each still against all its keys). Returns
    (O [B, H, R, d], LSE [B, H, R]) in fp64.

    ``trunc > 0`` also returns a third item, the bounds within which an
    implementation of the same steps on FP8 matrix cores with fp32
    arithmetic elsewhere may differ from this result (a dict of fp64
    arrays): "o" [B, H, R, d] and "lse" [B, H, R], and "flip" [B, H, R, d],
    the part of "o" due to P codes that such an implementation may decide
    either way. The model of that implementation:

      * the matrix cores add products in aligned groups of ``group`` along
        the reduction axis (channels for Q K^T, the keys of a tile for P V),
        losing at most what mfma_loss_bound gives with granularity ``trunc``
        relative to the group's largest product; the group sums and the
        running accumulator add in fp32, and every other fp32 operation
        errs by a relative 2^-24;
      * so score j of a row is off by at most delta_j = scale' L_j + 2^-20
        A_j + 2^-22 |s_j| (L_j the loss bound of its product sum, A_j =
        scale' sum_c |q_c k_jc|, natural-log units), the running max by at
        most delta_max (the largest delta_j of the row's visible keys), and
        the exponent of p_j = exp(s_j - m) by e_j = delta_j + delta_max +
        eta_j, eta_j = 2^-21 (|s_j| + |m| + 8) covering the fp32 multiply-add,
        the exponential and the rescale factors;
      * a P code is open when rounding 256 p e^(-e_j) and 256 p e^(e_j) gives
        different codes; each open code can move O_c by its gap times |V_jc|
        (weighted and normalised as O is), and the codes are decided
        independently, so "flip" is the sum of those moves over every open
        code of the row (every other code is unique);
      * the numerator of O (the P V sums) is off by the grouped loss of each
        tile's P V product sums, plus a relative 2 delta_max + (T + 2)
        eta_max + (T + 8) 2^-24 of sum_j w_j |P_j| |V_jc| (the running
        maxima, the T rescales, fp32 accumulation); the row sum of
        unquantised p (the denominator) by eps_l = e_max + (T + 1) eta_max
        + (n + 4) 2^-24 relative (n visible keys);
      * LSE = m + ln l is off by at most delta_max + eta_max (T + 2) + (n + 4)
        2^-24 + 2^-20 (|LSE| + 32) (the last for the logarithm and the
        final fp32 operations, a few ulps of numbers up to |LSE| + 32).
    The O and LSE bounds are first-order sums of these terms, widened by the
    factor 1 + 4 e_max. (A quantised value decided by floating point admits
    more than one correct result near a rounding boundary.)"""
    q8, k8, v8 = qz["q8"], qz["k8"], qz["v8"]
    B, H, N, d = q8.shape
    lens = _kv_lens(kv_len, B, N)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    s_mul = scale / (d if qz["rotated"] else 1)
    bound = trunc > 0 and quantize_p
    o = np.zeros((B, H, R, d))
    lse = np.zeros((B, H, R))
    o_bnd = np.zeros((B, H, R, d))
    flip_out = np.zeros((B, H, R, d))
    lse_bnd = np.zeros((B, H, R))
    u = 2.0 ** -24
    for b in range(B):
        for h in range(H):
            qd = (e4m3_decode(q8[b, h][rows]) *
                  qz["sq"][b, h].astype(np.float64)[rows // block_q][:, None])
            kd = e4m3_decode(k8[b, h]) * np.repeat(qz["sk"][b, h].astype(np.float64), block_k)[:N, None]
            vd = e4m3_decode(v8[b, h])
            qa, ka, vabs = np.abs(qd), np.abs(kd), np.abs(vd)
            m = np.full(R, -np.inf)
            l = np.zeros(R)
            acc = np.zeros((R, d))
            flip = np.zeros((R, d))   # sum over open codes of w |gap| |V|
            mag = np.zeros((R, d))    # sum over keys of w |P| |V|
            pvl = np.zeros((R, d))    # grouped loss of the P V sums, weighted
            e_max = np.zeros(R)
            eta_max = np.zeros(R)
            n_vis = np.zeros(R)
            n_tiles = np.zeros(R)
            dmax = np.zeros(R)

            def score_err(cols, s_fin):
                return (s_mul * (mfma_loss_bound(qa, ka[cols], trunc, group) + u * 16 * (qa @ ka[cols].T)) +
                        4 * u * np.abs(s_fin))

            if bound and N:
                # delta_max: the largest score error bound over the row's visible keys
                keys = np.arange(N)[None, :]
                vis_all = keys < lens[b]
                if causal:
                    vis_all = vis_all & (keys <= rows[:, None])
                for t0 in range(0, N, tile):
                    cols = np.arange(t0, min(t0 + tile, N))
                    dl = score_err(cols, s_mul * (qd @ kd[cols].T))
                    dmax = np.maximum(dmax, np.where(vis_all[:, cols], dl, 0.0).max(axis=1))
            for t0 in range(0, N, tile):
                cols = np.arange(t0, min(t0 + tile, N))
                s = s_mul * (qd @ kd[cols].T)
                vis = cols[None, :] < lens[b]
                if causal:
                    vis = vis & (cols[None, :] <= rows[:, None])
                s = np.where(vis, s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                grow = m_new > m
                # m - m_new only where the max grew (elsewhere both may be -inf)
                alpha = np.where(grow, np.exp(np.subtract(m, m_new, out=np.zeros_like(m), where=grow)), 1.0)
                l *= alpha
                acc *= alpha[:, None]
                flip *= alpha[:, None]
                mag *= alpha[:, None]
                pvl *= alpha[:, None]
                m_safe = np.where(np.isfinite(m_new), m_new, 0.0)
                p = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
                l += p.sum(axis=1)
                pq = e4m3_decode(e4m3_encode(p * p_scale)) / p_scale if quantize_p else p
                acc += pq @ vd[cols]
                if bound:
                    s_fin = np.where(vis, s, 0.0)
                    delta = score_err(cols, s_fin)
                    eta = 8 * u * (np.abs(s_fin) + np.abs(m_safe)[:, None] + 8.0)
                    e = np.where(vis, delta + dmax[:, None] + eta, 0.0)
                    x = p * p_scale
                    hi = np.minimum(x * np.exp(e), E4M3_MAX)
                    gap = (e4m3_decode(e4m3_encode(hi)) - e4m3_decode(e4m3_encode(x * np.exp(-e)))) / p_scale
                    flip += np.abs(gap) @ vabs[cols]
                    mag += np.abs(pq) @ vabs[cols]
                    pvl += mfma_loss_bound(np.abs(pq), vabs[cols].T, trunc, group)
                    e_max = np.maximum(e_max, e.max(axis=1))
                    eta_max = np.maximum(eta_max, np.where(vis, eta, 0.0).max(axis=1))
                    nv = vis.sum(axis=1)
                    n_vis += nv
                    n_tiles += nv > 0
                m = m_new
            has = l > 0
            inv_l = np.where(has, 1.0 / np.where(has, l, 1.0), 0.0)
            sv = float(qz["sv"][b, h])
            o[b, h] = np.where(has[:, None], acc * sv / np.where(has, l, 1.0)[:, None], 0.0)
            lse[b, h] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
            if bound:
                T = np.maximum(n_tiles, 1.0)
                w_num = 2 * dmax + (T + 2) * eta_max + (T + 8) * u
                eps_l = e_max + (T + 1) * eta_max + (n_vis + 4) * u
                widen = (1 + 4 * e_max)[:, None]
                fl = flip * sv * inv_l[:, None]
                flip_out[b, h] = fl
                o_bnd[b, h] = widen * (fl + (pvl + mag * w_num[:, None]) * sv * inv_l[:, None] +
                                       np.abs(o[b, h]) * (eps_l + 4 * u)[:, None])
                fin = np.where(has, lse[b, h], 0.0)
                lse_bnd[b, h] = np.where(has, (1 + 4 * e_max) * (dmax + (T + 2) * eta_max + (n_vis + 4) * u +
                                                                 16 * u * (np.abs(fin) + 32.0)), 0.0)
    if bound:
        return o, lse, {"o": o_bnd, "lse": lse_bnd, "flip": flip_out}
    return o, lse
