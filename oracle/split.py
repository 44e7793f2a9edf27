"""Attention over part of the keys, and the merge of partial results (fp64).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may call it.

Ring attention (Ultralytics glossary page, section "Flash Attention e
termini correlati") keeps a block of queries on each device, visits the
other devices' key/value blocks and combines what each visit returns. One
visit is plain attention of the query block over one key block; the
combination is the online-softmax recurrence (marketmaker.cc article,
section "在线softmax递归") applied to two finished partial results, where a
row's LSE stands for its pair (m, l):

    m = max(LSE_a, LSE_b),   w_a = exp(LSE_a - m),   w_b = exp(LSE_b - m),
    O = (w_a O_a + w_b O_b) / (w_a + w_b),   LSE = m + ln(w_a + w_b).

Readings of points the pages leave open:
  * a partial step attends queries at global positions q_pos0 + i to keys
    at global positions k_pos0 + j; causal hides a key whose position is
    after the query's; key padding hides local keys j >= kv_len[b];
  * a row with no visible key in the part has O = 0 and LSE = -inf, and the
    merge treats it as an empty part (weight 0); a row empty in every part
    stays O = 0, LSE = -inf.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .attention import _f64

__all__ = ["attn_part64", "merge64"]


def attn_part64(q, k, v, scale: float, causal: bool = False, q_pos0: int = 0, k_pos0: int = 0,
                kv_len=None):
    """q: [B, H, Nq, d]; k, v: [B, H, Nk, d]. Returns (O [B, H, Nq, d], LSE
    [B, H, Nq]) of softmax(scale q k^T) v over the visible keys, with the full
    Nq x Nk score matrix materialised and a two-pass softmax."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if kv_len is None:
        lens = np.full(B, Nk, dtype=np.int64)
    else:
        if hasattr(kv_len, "detach"):
            kv_len = kv_len.detach().cpu().numpy()
        lens = np.clip(np.asarray(kv_len, dtype=np.int64).reshape(B), 0, Nk)
    qpos = q_pos0 + np.arange(Nq)[:, None]
    kpos = k_pos0 + np.arange(Nk)[None, :]
    o_out = np.zeros((B, H, Nq, d))
    lse_out = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        vis = np.arange(Nk)[None, :] < lens[b]
        if causal:
            vis = vis & (kpos <= qpos)
        vis = np.broadcast_to(vis, (Nq, Nk))
        for h in range(H):
            s = np.where(vis, scale * (q[b, h] @ k[b, h].T), -np.inf)
            m = s.max(axis=1) if Nk else np.full(Nq, -np.inf)
            has = np.isfinite(m)
            m0 = np.where(has, m, 0.0)
            p = np.where(vis, np.exp(s - m0[:, None]), 0.0)
            l = p.sum(axis=1)
            l1 = np.where(has, l, 1.0)
            o_out[b, h] = np.where(has[:, None], (p / l1[:, None]) @ v[b, h], 0.0)
            lse_out[b, h] = np.where(has, m0 + np.log(l1), -np.inf)
    return o_out, lse_out


def merge64(o_parts: Sequence, lse_parts: Sequence):
    """Combine partial results over disjoint key sets. o_parts: P arrays
    [..., d]; lse_parts: P arrays [...]. Returns (O [..., d], LSE [...])."""
    o = np.stack([_f64(x) for x in o_parts])
    lse = np.stack([_f64(x) for x in lse_parts])
    m = lse.max(axis=0)
    has = np.isfinite(m)
    m0 = np.where(has, m, 0.0)
    w = np.where(np.isfinite(lse), np.exp(lse - m0), 0.0)
    den = w.sum(axis=0)
    den1 = np.where(has, den, 1.0)
    out = (w[..., None] * o).sum(axis=0) / den1[..., None]
    out = np.where(has[..., None], out, 0.0)
    return out, np.where(has, m0 + np.log(den1), -np.inf)
