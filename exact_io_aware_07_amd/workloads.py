"""Seeded synthetic workloads for exact attention.

This module only draws random inputs and describes shapes. It holds none of
the attention arithmetic, so both the HIP path and the fp64 oracle can be fed
from it without sharing any computation.

Recipe (applies to every workload):
  * one ``torch.Generator`` on the CPU, seeded (default seed 0);
  * fp32 standard-normal draws in the order Q, K, V, then dO (only for
    workloads with a backward pass), each of shape [B, H, N, d] (K and V
    [B, Hkv, N, d] for a workload with grouped K/V heads);
  * then the per-workload extras, in this order: the key-padding lengths
    (``randint(lo, hi + 1, (B,))``), then the outlier key rows (for each
    (b, h) in row-major order, ``randperm(N)[:round(frac * N)]`` and those K
    rows multiplied by the factor), then the outlier channels (for each
    (b, h), ``randperm(d)[:count]`` and those columns of Q and K multiplied
    by the factor);
  * finally a round-to-nearest-even cast of Q, K, V, dO to the workload dtype.

The workloads are named after the shapes the pages discuss: BERT-large at
sequence 512 and GPT-2 at 1K (the end-to-end results quoted on the Ultralytics
glossary page, section "Impatto sull'addestramento e sui contesti lunghi"), the
32-head 4096-token example of the onecalc.app attention-memory calculator
(section "計算例"), and the 23,400-step, 12-head trading day of the
marketmaker.cc article (its opening section). Standard-normal synthetic data
stands in for every dataset; no real model, weight or text is used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool = False
    kv_len_range: Optional[Tuple[int, int]] = None  # inclusive (lo, hi)
    k_outlier_frac: float = 0.0
    k_outlier_scale: float = 1.0
    backward: bool = False
    measurement_only: bool = False
    Hkv: Optional[int] = None  # K/V heads (grouped-query attention); None means H
    block_pattern: Optional[str] = None  # block-sparse mask (see block_mask); None means dense
    ch_outliers: int = 0               # channels of Q and K scaled per (b, h), FP8 workload
    ch_outlier_scale: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload("tiny_fp32_fwd", 1, 1, 256, 64, "fp32",
                note="B=1 H=1 N=256 d=64 fp32, no mask")
BERT = Workload("bert_large_fp16_fwd", 32, 16, 512, 64, "fp16",
                kv_len_range=(128, 512),
                note="B=32 H=16 N=512 d=64 fp16, key padding U[128,512]")
LONG = Workload("long_context_bf16_fwd", 1, 32, 4096, 128, "bf16",
                k_outlier_frac=0.01, k_outlier_scale=8.0,
                note="B=1 H=32 N=4096 d=128 bf16, 1% of K rows x8")
TRADE = Workload("trading_day_bf16_causal_fwd", 1, 12, 23400, 64, "bf16",
                 causal=True,
                 note="B=1 H=12 N=23400 d=64 bf16 causal")
GPT2 = Workload("gpt2_bf16_causal_fwd_bwd", 8, 12, 1024, 64, "bf16",
                causal=True, backward=True,
                note="B=8 H=12 N=1024 d=64 bf16 causal, forward + backward")

# Backward at N >= 4096: the same generator on the long-context and
# trading-day shapes, used for timing the backward at long sequence length.
LONG_BWD = LONG.with_(name="long_context_bf16_bwd", backward=True,
                      measurement_only=True)
TRADE_BWD = TRADE.with_(name="trading_day_bf16_causal_bwd", backward=True,
                        measurement_only=True)

# Few heads, long causal sequence: too few query blocks to fill the chip, the
# shape a key-split forward (the one-GPU half of ring attention) is for.
FEW_HEADS = Workload("few_heads_long_causal_bf16_split", 1, 2, 32768, 64, "bf16", causal=True,
                     measurement_only=True,
                     note="B=1 H=2 N=32768 d=64 bf16 causal, forward plain and key-split")

# Grouped-query attention: the 32 query heads and 4096 tokens of the
# long-context shape sharing 8 K/V heads (groups of 4), causal, forward and
# backward, two sequences.
GQA = Workload("long_context_gqa_bf16_causal_fwd_bwd", 2, 32, 4096, 128, "bf16", causal=True,
               backward=True, measurement_only=True, Hkv=8,
               note="B=2 H=32 Hkv=8 N=4096 d=128 bf16 causal, forward + backward")

# Block-sparse: 16 heads of 16,384 tokens where each 128-token query block
# keeps its own key block, its two neighbours and the first key block (the
# "band_sink" pattern of block_mask), 4 of 128 blocks per row.
SPARSE = Workload("long_block_sparse_band_bf16_fwd_bwd", 1, 16, 16384, 64, "bf16",
                  backward=True, measurement_only=True, block_pattern="band_sink",
                  note="B=1 H=16 N=16384 d=64 bf16, 128x128 block mask: band of 3 + first block")

# The same shape with a global first block: it keeps every key block and
# every query block keeps it, so one mask row and one mask column hold 128
# kept blocks while the others hold four (the load the plan's pieces spread).
SPARSE_GLOBAL = Workload("long_block_sparse_global_bf16_fwd_bwd", 1, 16, 16384, 64, "bf16",
                         backward=True, measurement_only=True, block_pattern="band_global",
                         note="B=1 H=16 N=16384 d=64 bf16, 128x128 block mask: band of 3 + "
                              "global first block (its row and column kept)")

# FP8 forward: the long-context shape with four outlier channels of Q and K
# (x16, the same channels in Q and K of a head), the case the rotation of
# the FP8 path is for.
FP8 = Workload("long_context_fp8_outlier_channels_fwd", 1, 32, 4096, 128, "bf16",
               measurement_only=True, ch_outliers=4, ch_outlier_scale=16.0,
               note="B=1 H=32 N=4096 d=128 bf16, 4 channels of Q and K x16; FP8 forward")

CONFIGS: Dict[str, Workload] = {w.name: w for w in (TINY, BERT, LONG, TRADE, GPT2)}
MEASUREMENT: Dict[str, Workload] = {w.name: w for w in (LONG_BWD, TRADE_BWD, FEW_HEADS, GQA, SPARSE,
                                                        SPARSE_GLOBAL, FP8)}
ALL: Dict[str, Workload] = {**CONFIGS, **MEASUREMENT}


def make_inputs(w: Workload, seed: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    """Draw the seeded inputs of ``w`` on the CPU, already cast to its dtype.

    Returns a dict with ``q`` (and ``do`` when ``w.backward``) as contiguous
    [B, H, N, d] tensors, ``k, v`` as [B, Hkv, N, d] (Hkv = H unless the
    workload groups its K/V heads) and ``kv_len`` as an int32 [B] tensor or
    ``None``. The same seed always yields bit-identical tensors.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (w.B, w.H, w.N, w.d)
    kv_shape = (w.B, w.kv_heads, w.N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(kv_shape, generator=g, dtype=torch.float32)
    v = torch.randn(kv_shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32) if w.backward else None
    kv_len = None
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        kv_len = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64)
        kv_len = kv_len.to(torch.int32)
    if w.k_outlier_frac > 0.0:
        count = int(round(w.k_outlier_frac * w.N))
        for b in range(w.B):
            for h in range(w.kv_heads):
                idx = torch.randperm(w.N, generator=g)[:count]
                k[b, h, idx] *= w.k_outlier_scale
    if w.ch_outliers > 0:
        for b in range(w.B):
            for h in range(w.H):
                ch = torch.randperm(w.d, generator=g)[:w.ch_outliers]
                q[b, h][:, ch] *= w.ch_outlier_scale
                if h < w.kv_heads:
                    k[b, h][:, ch] *= w.ch_outlier_scale
    dt = w.torch_dtype
    out = {
        "q": q.to(dt).contiguous(),
        "k": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "do": do.to(dt).contiguous() if do is not None else None,
        "kv_len": kv_len,
    }
    return out


def outlier_rows(w: Workload, seed: int = 0) -> Optional[torch.Tensor]:
    """The [B, Hkv, count] indices of the scaled K rows drawn by ``make_inputs``."""
    if w.k_outlier_frac <= 0.0:
        return None
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (w.B, w.H, w.N, w.d)
    kv_shape = (w.B, w.kv_heads, w.N, w.d)
    for s in (shape, kv_shape, kv_shape) + ((shape,) if w.backward else ()):
        torch.randn(s, generator=g, dtype=torch.float32)
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64)
    count = int(round(w.k_outlier_frac * w.N))
    rows = torch.empty((w.B, w.kv_heads, count), dtype=torch.int64)
    for b in range(w.B):
        for h in range(w.kv_heads):
            rows[b, h] = torch.randperm(w.N, generator=g)[:count]
    return rows


def random_case(B: int, H: int, N: int, d: int, dtype: str, seed: int,
                causal: bool = False, kv_len: Optional[list] = None,
                backward: bool = False, Hkv: Optional[int] = None
                ) -> Dict[str, Optional[torch.Tensor]]:
    """Seeded inputs for an ad-hoc shape (tails, edge cases), same recipe."""
    w = Workload(f"case_{B}x{H}x{N}x{d}_{dtype}", B, H, N, d, dtype,
                 causal=causal, backward=backward, Hkv=Hkv)
    out = make_inputs(w, seed)
    if kv_len is not None:
        out["kv_len"] = torch.tensor(kv_len, dtype=torch.int32)
    return out


MASK_BLOCK = 128  # queries (and keys) per block of a block-sparse mask


def block_mask(w: Workload) -> Optional[torch.Tensor]:
    """The uint8 [nb, nb] block mask of a block-sparse workload (nb =
    ceil(N / 128)), shared by every batch and head, or None for a dense one.

    "band_sink": query block i keeps key blocks i - 1, i, i + 1 and 0.
    "band_global": the same, and query block 0 keeps every key block.
    """
    if w.block_pattern is None:
        return None
    nb = (w.N + MASK_BLOCK - 1) // MASK_BLOCK
    i = torch.arange(nb)[:, None]
    j = torch.arange(nb)[None, :]
    if w.block_pattern == "band_sink":
        return (((i - j).abs() <= 1) | (j == 0)).to(torch.uint8)
    if w.block_pattern == "band_global":
        return (((i - j).abs() <= 1) | (j == 0) | (i == 0)).to(torch.uint8)
    raise ValueError(f"unknown block pattern {w.block_pattern!r}")


def random_block_mask(lead: Tuple[int, ...], N: int, keep: float, seed: int) -> torch.Tensor:
    """A seeded uint8 block mask of shape lead + (nb, nb): each block pair
    kept with probability ``keep`` (one ``torch.rand`` draw per entry)."""
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.rand(tuple(lead) + (nb, nb), generator=g) < keep).to(torch.uint8)


def random_signs(d: int, seed: int) -> torch.Tensor:
    """The +-1 vector (int8 [d]) of the FP8 path's rotation: one seeded
    ``torch.randint(0, 2, (d,))`` draw mapped to -1 / +1."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randint(0, 2, (d,), generator=g) * 2 - 1).to(torch.int8)
