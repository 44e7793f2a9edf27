"""Grouped-query attention in fp64: query heads share key/value heads.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The delect.ru glossary page ("FlashAttention", section "Что подтверждено")
notes that the tiled method changes how attention is computed for given Q,
K, V and not how many K/V heads there are, so grouped-query attention is the
same operation with K/V heads shared. The definition used (a reading, since
the pages give no formula): with H query heads and H_kv key/value heads,
G = H / H_kv, query head h attends with key/value head h // G, exactly as in
plain attention. In the backward, a key/value head's gradient is the sum of
the gradients its G query heads send it (it is one parameter used G times).
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, attn_bwd64, attn_fwd64

__all__ = ["attn_fwd64_gqa", "attn_bwd64_gqa"]


def _repeat(x, G: int) -> np.ndarray:
    return np.repeat(_f64(x), G, axis=1)


def attn_fwd64_gqa(q, k, v, scale: float, causal: bool = False, kv_len=None, rows=None):
    """q: [B, H, N, d]; k, v: [B, H_kv, N, d] with H % H_kv == 0."""
    q = _f64(q)
    G = q.shape[1] // _f64(k).shape[1]
    return attn_fwd64(q, _repeat(k, G), _repeat(v, G), scale, causal, kv_len, rows=rows)


def attn_bwd64_gqa(q, k, v, dout, scale: float, causal: bool = False, kv_len=None):
    """Returns (dQ [B, H, N, d], dK [B, H_kv, N, d], dV [B, H_kv, N, d])."""
    q = _f64(q)
    B, H, N, d = q.shape
    Hkv = _f64(k).shape[1]
    G = H // Hkv
    dq, dk, dv = attn_bwd64(q, _repeat(k, G), _repeat(v, G), dout, scale, causal, kv_len)
    return dq, dk.reshape(B, Hkv, G, N, d).sum(axis=2), dv.reshape(B, Hkv, G, N, d).sum(axis=2)
