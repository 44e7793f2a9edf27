"""Block-sparse attention in fp64: attention restricted to the (query block,
key block) pairs a block mask keeps.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The pages describe a block-sparse variant of the tiled method that skips
the tiles a mask leaves empty, and call it an approximation of full
attention that is specified separately from the exact algorithm
(Ultralytics glossary page "Flash Attention", section "Flash Attention e
termini correlati"; delect.ru glossary page "FlashAttention", section
"Что подтверждено"). They give no formula; the reading used here is the
plain one: with blocks of ``block`` queries by ``block`` keys and a 0/1 mask
M of ceil(N/block) x ceil(N/block) entries per head, key j is visible to
query i when M[i // block, j // block] != 0 and the usual masks allow it
(j < kv_len[b]; j <= i when causal). On that visible set the result is
exact softmax attention, computed as in ``attention.py``: S materialised,
two-pass softmax, a row with no visible key gives O = 0 and LSE = -inf, and
the backward is the same chain rule with P zero off the visible set.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, _kv_lens

__all__ = ["sparse_visible", "attn_fwd64_sparse", "attn_bwd64_sparse", "attn_bwd64_sparse_sampled"]


def sparse_visible(N: int, causal: bool, kv_len_b: int, mask_bh, block: int,
                   rows=None, cols=None) -> np.ndarray:
    """Boolean [R, C]: True where key j is visible to query i for one head
    whose block mask is ``mask_bh`` ([ceil(N/block), ceil(N/block)]); rows
    and cols (default: all N) pick the queries i and keys j."""
    i = (np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = (np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64))[None, :]
    m = np.asarray(mask_bh) != 0
    vis = m[i // block, j // block] & (j < kv_len_b)
    if causal:
        vis = vis & (j <= i)
    return vis


def _probs(q, k, vis, scale):
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    mx = s.max(axis=1, keepdims=True)
    has_key = np.isfinite(mx)
    mx0 = np.where(has_key, mx, 0.0)
    e = np.where(vis, np.exp(s - mx0), 0.0)
    tot = e.sum(axis=1, keepdims=True)
    tot1 = np.where(has_key, tot, 1.0)
    lse = np.where(has_key[:, 0], mx0[:, 0] + np.log(tot1[:, 0]), -np.inf)
    return e / tot1, lse


def _mask_of(block_mask, b: int, h: int):
    m = np.asarray(block_mask)
    return m[b, h] if m.ndim == 4 else m


def attn_fwd64_sparse(q, k, v, scale: float, causal: bool, kv_len, block_mask, block: int = 128,
                      rows=None, row_chunk: int = 1024):
    """q, k, v: [B, H, N, d]; block_mask: [B, H, nb, nb] or [nb, nb] (one mask
    for every head), nb = ceil(N / block). ``rows`` restricts the output to
    those query rows (all keys still used), taken ``row_chunk`` at a time.
    Returns (O [B, H, R, d], LSE [B, H, R])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    rr = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, H, len(rr), d))
    lse = np.zeros((B, H, len(rr)))
    for b in range(B):
        for h in range(H):
            for c0 in range(0, len(rr), row_chunk):
                part = rr[c0:c0 + row_chunk]
                vis = sparse_visible(N, causal, int(lens[b]), _mask_of(block_mask, b, h), block,
                                     rows=part)
                p, lse[b, h, c0:c0 + len(part)] = _probs(q[b, h, part], k[b, h], vis, scale)
                o[b, h, c0:c0 + len(part)] = p @ v[b, h]
    return o, lse


def attn_bwd64_sparse(q, k, v, dout, scale: float, causal: bool, kv_len, block_mask,
                      block: int = 128):
    """Gradients (dQ, dK, dV) of L = sum(dO * O) for ``attn_fwd64_sparse``:
    dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P (dP - D),
    dQ = scale dS K, dK = scale dS^T Q, with P zero off the visible set."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    dq, dk, dv = (np.zeros((B, H, N, d)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            vis = sparse_visible(N, causal, int(lens[b]), _mask_of(block_mask, b, h), block)
            p, _ = _probs(q[b, h], k[b, h], vis, scale)
            dv[b, h] = p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, h].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def attn_bwd64_sparse_sampled(q, k, v, dout, scale: float, causal: bool, kv_len, block_mask,
                              heads, q_rows, k_rows, block: int = 128, row_chunk: int = 1024):
    """The gradients of ``attn_bwd64_sparse`` on sampled query rows (dQ) and
    keys (dK, dV) of the listed (b, h) heads, for N too long for an N x N
    matrix. Per head, LSE_i and D_i = sum_j P_ij dP_ij come from whole rows
    taken ``row_chunk`` at a time (only the rows that a sampled row or key
    needs); then
      dQ_i = scale sum_j P_ij (dP_ij - D_i) K_j   (whole rows i in q_rows)
      dK_j = scale sum_i P_ij (dP_ij - D_i) Q_i   (whole columns j in k_rows)
      dV_j = sum_i P_ij dO_i
    with P_ij = exp(S_ij - LSE_i) on the visible set and 0 elsewhere.
    Returns (dQ [len(heads), R, d], dK [len(heads), C, d], dV [len(heads), C, d])."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    qr = np.asarray(q_rows, dtype=np.int64)
    kr = np.asarray(k_rows, dtype=np.int64)
    dq = np.zeros((len(heads), len(qr), d))
    dk = np.zeros((len(heads), len(kr), d))
    dv = np.zeros((len(heads), len(kr), d))
    for t, (b, h) in enumerate(heads):
        m = _mask_of(block_mask, b, h)
        lim = int(lens[b])
        # LSE_i and D_i are needed for the sampled rows and for every row whose
        # mask row keeps the block of a sampled key; the other rows see none
        # of those keys, so they stay at -inf / 0 and give P = 0 below.
        need = np.zeros(N, dtype=bool)
        need[qr] = True
        if len(kr):
            kept = (np.asarray(m) != 0)[:, np.unique(kr // block)].any(axis=1)
            need |= np.repeat(kept, block)[:N]
        lse = np.full(N, -np.inf)
        dsum = np.zeros(N)
        rows_needed = np.nonzero(need)[0]
        for c0 in range(0, len(rows_needed), row_chunk):
            part = rows_needed[c0:c0 + row_chunk]
            vis = sparse_visible(N, causal, lim, m, block, rows=part)
            p, lse[part] = _probs(q[b, h, part], k[b, h], vis, scale)
            dsum[part] = (p * (dout[b, h, part] @ v[b, h].T)).sum(axis=1)
        if len(qr):
            vis = sparse_visible(N, causal, lim, m, block, rows=qr)
            p, _ = _probs(q[b, h, qr], k[b, h], vis, scale)
            dp = dout[b, h, qr] @ v[b, h].T
            dq[t] = scale * ((p * (dp - dsum[qr, None])) @ k[b, h])
        if len(kr):
            vis = sparse_visible(N, causal, lim, m, block, cols=kr)
            has = np.isfinite(lse)
            s_c = scale * (q[b, h] @ k[b, h, kr].T)
            p = np.where(vis & has[:, None], np.exp(s_c - np.where(has, lse, 0.0)[:, None]), 0.0)
            ds = p * (dout[b, h] @ v[b, h, kr].T - dsum[:, None])
            dk[t] = scale * (ds.T @ q[b, h])
            dv[t] = p.T @ dout[b, h]
    return dq, dk, dv
