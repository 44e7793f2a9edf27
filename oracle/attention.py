"""Plain fp64 CPU attention: the oracle the HIP path is checked against.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this package; only
the test suite, the smoke check and the CPU-baseline leg of the benchmark
may call it. It shares no code with the HIP kernels.

What it computes is the plain definition of scaled dot-product attention,
softmax(Q K^T * scale) V, with the full score matrix S materialised and a
two-pass softmax (max, then exp and sum). The pages state the tiled method
reaches this same result in exact arithmetic and differs only in rounding
order (marketmaker.cc article, section "在线softmax递归" / online softmax
recurrence; Ultralytics glossary page, opening definition; delect.ru
glossary, section "Что подтверждено"), so the definition itself is the
oracle. The definition is the one given in the marketmaker.cc article,
sections "为什么注意力是受记忆限制的" (why attention is memory-bound) and
"集成是八行" (the three-line materialised path it replaces).

Readings of points the pages leave open:
  * causal means key j is hidden from query i when j > i, top-left aligned
    (marketmaker.cc article, section "因果掩盖..." / causal masking: tiles whose
    keys lie wholly in the future of their queries are skipped);
  * key padding hides keys j >= kv_len[b] from every query row and head;
    every query row is still computed;
  * a query row with no visible key has O = 0 and LSE = -inf;
  * LSE is the natural log of the sum of exp over the scaled, masked scores,
    i.e. the one number per row that stands for the pair (m, l) the
    marketmaker.cc article keeps for the backward (section "向后传递");
  * the backward is the textbook softmax-Jacobian chain rule, since the pages
    only say the backward recomputes P from Q, K and the stored statistics.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = ["attn_fwd64", "attn_probs64", "attn_bwd64", "attn_bwd64_magnitudes", "attn_bwd64_sampled",
           "visible_mask"]


def _f64(x) -> np.ndarray:
    """Exact upcast of a float array (numpy or torch CPU) to fp64."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no numpy dtype
        import torch  # local: the oracle does not otherwise depend on torch
        x = x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _kv_lens(kv_len, B: int, N: int) -> np.ndarray:
    if kv_len is None:
        return np.full(B, N, dtype=np.int64)
    if hasattr(kv_len, "detach"):
        kv_len = kv_len.detach().cpu().numpy()
    out = np.asarray(kv_len, dtype=np.int64).reshape(B)
    return np.clip(out, 0, N)


def visible_mask(rows: np.ndarray, N: int, causal: bool, kv_len_b: int) -> np.ndarray:
    """Boolean [R, N]: True where key j is visible to query row rows[r]."""
    j = np.arange(N)[None, :]
    vis = j < kv_len_b
    if causal:
        vis = vis & (j <= rows[:, None])
    return np.broadcast_to(vis, (len(rows), N))


def _rows_forward(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
                  scale: float, causal: bool, kv_len_b: int):
    """Definition for one head and a set of query rows: (O, LSE, P)."""
    N = k.shape[0]
    s = scale * (q_rows @ k.T)                              # [R, N], materialised
    vis = visible_mask(rows, N, causal, kv_len_b)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)                        # pass 1: row max
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    p = np.where(vis, np.exp(s - m_safe), 0.0)              # pass 2: exp
    l = p.sum(axis=1, keepdims=True)                        # and row sum
    l_safe = np.where(has_key, l, 1.0)
    probs = p / l_safe                                      # softmax rows
    o = probs @ v
    lse = np.where(has_key[:, 0], m_safe[:, 0] + np.log(l_safe[:, 0]), -np.inf)
    return o, lse, probs


def attn_fwd64(q, k, v, scale: float, causal: bool = False, kv_len=None,
               rows: Optional[Sequence[int]] = None,
               heads: Optional[Sequence[Tuple[int, int]]] = None,
               row_chunk: int = 1024):
    """Forward attention in fp64.

    q, k, v: [B, H, N, d] arrays (numpy or torch CPU, any float dtype; upcast
    exactly to fp64). kv_len: None or [B] ints. ``rows`` restricts the output
    to those query rows (the full K and V are still used); ``heads`` restricts
    it to a list of (b, h) pairs. Returns (O, LSE) as fp64 arrays of shape
    [B, H, R, d] and [B, H, R] (or [len(heads), R, d] / [len(heads), R] when
    ``heads`` is given). Rows are processed ``row_chunk`` at a time; each chunk
    still sees whole rows of S, so the softmax is the two-pass one.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    rows_arr = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    R = len(rows_arr)
    o_out = np.zeros((len(pairs), R, d))
    lse_out = np.zeros((len(pairs), R))
    for t, (b, h) in enumerate(pairs):
        for c0 in range(0, R, row_chunk):
            rr = rows_arr[c0:c0 + row_chunk]
            o, lse, _ = _rows_forward(q[b, h, rr], k[b, h], v[b, h], rr,
                                      scale, causal, int(lens[b]))
            o_out[t, c0:c0 + len(rr)] = o
            lse_out[t, c0:c0 + len(rr)] = lse
    if heads is None:
        return o_out.reshape(B, H, R, d), lse_out.reshape(B, H, R)
    return o_out, lse_out


def attn_probs64(q, k, scale: float, causal: bool = False, kv_len=None) -> np.ndarray:
    """The softmax matrix P [B, H, N, N] in fp64 (small N only)."""
    q, k = _f64(q), _f64(k)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    out = np.zeros((B, H, N, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            _, _, p = _rows_forward(q[b, h], k[b, h], np.zeros((N, 1)), rows,
                                    scale, causal, int(lens[b]))
            out[b, h] = p
    return out


def attn_bwd64(q, k, v, dout, scale: float, causal: bool = False, kv_len=None,
               heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Gradients (dQ, dK, dV) of L = sum(dO * O) in fp64.

    Chain rule through O = P V and P = softmax(S), S = scale * Q K^T:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
      dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
    P is this oracle's own fp64 softmax of the materialised S. Returns arrays
    of shape [B, H, N, d] (or [len(heads), N, d] when ``heads`` is given).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    dq = np.zeros((len(pairs), N, d))
    dk = np.zeros((len(pairs), N, d))
    dv = np.zeros((len(pairs), N, d))
    rows = np.arange(N)
    for t, (b, h) in enumerate(pairs):
        _, _, p = _rows_forward(q[b, h], k[b, h], v[b, h], rows, scale, causal, int(lens[b]))
        do = dout[b, h]
        dv[t] = p.T @ do
        dp = do @ v[b, h].T
        dsum = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - dsum)
        dq[t] = scale * (ds @ k[b, h])
        dk[t] = scale * (ds.T @ q[b, h])
    if heads is None:
        return (dq.reshape(B, H, N, d), dk.reshape(B, H, N, d), dv.reshape(B, H, N, d))
    return dq, dk, dv


def attn_bwd64_magnitudes(q, k, v, dout, scale: float, causal: bool = False, kv_len=None):
    """The gradient formulas of ``attn_bwd64`` with every term in absolute
    value, the scale of rounding in a floating-point evaluation of them:
      M_dQ = scale (P * (|dP| + |D|)) |K|,  M_dK = scale (P * (|dP| + |D|))^T |Q|,
      M_dV = P^T |dO|.
    Each bounds its gradient elementwise (|dQ| <= M_dQ, ...). Where the terms
    nearly cancel (a row of one or two keys with nearly equal dP), the
    gradient is far smaller than M and a relative error bound on it alone is
    out of reach of any fp32 evaluation. Returns three [B, H, N, d] arrays."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    mq, mk, mv = (np.zeros((B, H, N, d)) for _ in range(3))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            _, _, p = _rows_forward(q[b, h], k[b, h], v[b, h], rows, scale, causal, int(lens[b]))
            do = dout[b, h]
            dp = do @ v[b, h].T
            dsum = (p * dp).sum(axis=1, keepdims=True)
            w = p * (np.abs(dp) + np.abs(dsum))
            mq[b, h] = scale * (w @ np.abs(k[b, h]))
            mk[b, h] = scale * (w.T @ np.abs(q[b, h]))
            mv[b, h] = p.T @ np.abs(do)
    return mq, mk, mv


def attn_bwd64_sampled(q, k, v, dout, scale: float, causal: bool = False, kv_len=None,
                       heads: Sequence[Tuple[int, int]] = ((0, 0),),
                       q_rows: Sequence[int] = (), k_rows: Sequence[int] = (),
                       row_chunk: int = 1024):
    """The same gradients as ``attn_bwd64``, evaluated only for sampled query
    rows (dQ) and sampled keys (dK, dV) of the listed heads, for sequences too
    long for a full N x N fp64 matrix.

    Per head: LSE_i and D_i = sum_j P_ij dP_ij come from whole rows of S (rows
    are independent, so they are taken ``row_chunk`` at a time); then
      dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j    for i in q_rows (whole rows)
      dK_j = scale * sum_i P_ij (dP_ij - D_i) Q_i    for j in k_rows (whole columns)
      dV_j = sum_i P_ij dO_i                         for j in k_rows
    with P_ij = exp(S_ij - LSE_i) on visible entries and 0 elsewhere.
    Returns (dQ [len(heads), R, d], dK [len(heads), C, d], dV [len(heads), C, d]).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    qr = np.asarray(q_rows, dtype=np.int64)
    kr = np.asarray(k_rows, dtype=np.int64)
    pairs = list(heads)
    dq = np.zeros((len(pairs), len(qr), d))
    dk = np.zeros((len(pairs), len(kr), d))
    dv = np.zeros((len(pairs), len(kr), d))
    all_rows = np.arange(N)
    for t, (b, h) in enumerate(pairs):
        lim = int(lens[b])
        lse = np.full(N, -np.inf)
        dsum = np.zeros(N)
        # D_i of every row is needed only for dK / dV (columns); dQ rows
        # need their own D_i, which their own P rows give. Under the causal
        # mask a row before the first requested key sees none of them
        # (P = 0 there), so the pass starts at that key.
        row0 = int(kr.min()) if (causal and len(kr)) else 0
        for c0 in range(row0, N if len(kr) else row0, row_chunk):
            rr = all_rows[c0:c0 + row_chunk]
            _, l_c, p_c = _rows_forward(q[b, h, rr], k[b, h], v[b, h], rr, scale, causal, lim)
            dp_c = dout[b, h, rr] @ v[b, h].T
            lse[rr] = l_c
            dsum[rr] = (p_c * dp_c).sum(axis=1)
        if len(qr):
            _, _, p_r = _rows_forward(q[b, h, qr], k[b, h], v[b, h], qr, scale, causal, lim)
            dp_r = dout[b, h, qr] @ v[b, h].T
            d_r = (p_r * dp_r).sum(axis=1)
            dq[t] = scale * ((p_r * (dp_r - d_r[:, None])) @ k[b, h])
        if len(kr):
            s_c = scale * (q[b, h] @ k[b, h, kr].T)                  # [N, C] columns of S
            vis = (kr[None, :] < lim) & ((kr[None, :] <= all_rows[:, None]) if causal else True)
            has_key = np.isfinite(lse)
            lse_safe = np.where(has_key, lse, 0.0)
            p_c = np.where(vis & has_key[:, None], np.exp(s_c - lse_safe[:, None]), 0.0)
            dp_c = dout[b, h] @ v[b, h, kr].T
            ds_c = p_c * (dp_c - dsum[:, None])
            dk[t] = scale * (ds_c.T @ q[b, h])
            dv[t] = p_c.T @ dout[b, h]
    return dq, dk, dv
