"""Bytes of the materialised score matrix: the allocation exact tiled
attention must never make.

TEST INFRASTRUCTURE ONLY.

The onecalc.app attention-memory calculator (section "計算式", formula) sizes
the score matrix of plain attention as batch x heads x seq^2 x bytes-per-score;
its worked example (section "計算例") is one 4096-token sequence with 32 heads
at 2 bytes per score. The marketmaker.cc article (opening section) sizes the
same matrix for a 23,400-step day with 12 heads in fp16.
"""
from __future__ import annotations


def score_matrix_bytes(batch: int, heads: int, seq: int, elem_bytes: int) -> int:
    """Exact integer byte count of one layer's B x H x N x N score matrix."""
    return int(batch) * int(heads) * int(seq) * int(seq) * int(elem_bytes)
