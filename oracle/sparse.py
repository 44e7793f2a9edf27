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

__all__ = ["sparse_visible", "attn_fwd64_sparse", "attn_bwd64_sparse"]


def sparse_visible(N: int, causal: bool, kv_len_b: int, mask_bh, block: int) -> np.ndarray:
    """Boolean [N, N]: True where key j is visible to query i for one head
    whose block mask is ``mask_bh`` ([ceil(N/block), ceil(N/block)])."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
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


def attn_fwd64_sparse(q, k, v, scale: float, causal: bool, kv_len, block_mask, block: int = 128):
    """q, k, v: [B, H, N, d]; block_mask: [B, H, nb, nb] or [nb, nb] (one mask
    for every head), nb = ceil(N / block). Returns (O [B, H, N, d], LSE [B, H, N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    lens = _kv_lens(kv_len, B, N)
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            vis = sparse_visible(N, causal, int(lens[b]), _mask_of(block_mask, b, h), block)
            p, lse[b, h] = _probs(q[b, h], k[b, h], vis, scale)
            o[b, h] = p @ v[b, h]
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
