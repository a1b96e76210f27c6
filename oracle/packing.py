"""Ragged packing and block arithmetic — oracle side (test infrastructure only).

Sources:
  * "Continuous batching in transformers" (ai-infrastructure.net), section "Why use it":
    a rectangular batch pads every row to the longest one; when an n-token prompt joins
    B-1 one-token decodes the rectangle wastes (n-1)(B-1) slots, while ragged packing
    stores only the real tokens; a zero-length row is an error, not a row to pad.
  * Same page, section "The paged cache, its two reserved blocks, and the block-size
    trade": a sequence of L tokens occupies ceil(L / block_size) blocks and wastes the
    unused tail of its last block; block_size below 4 is rejected.
  * "3.3 Batching & Memory Management", section "PagedAttention: block tables" and
    "Check your understanding": the same ceil-div count (1000 tokens at 16 per block
    -> 63 blocks, 8 slots unused).
"""
from __future__ import annotations

import numpy as np

MIN_BLOCK_SIZE = 4


def _check_rows(row_lengths):
    lens = [int(x) for x in row_lengths]
    if not lens:
        raise ValueError("a batch needs at least one row")
    if min(lens) <= 0:
        raise ValueError("every row of a batch must hold at least one token")
    return lens


def padded_slots(row_lengths) -> int:
    """Slots of the rectangle a padded batch allocates: number of rows times the longest row."""
    lens = _check_rows(row_lengths)
    return len(lens) * max(lens)


def useful_slots(row_lengths) -> int:
    """Slots a ragged (packed) batch stores: exactly the real tokens."""
    lens = _check_rows(row_lengths)
    return sum(lens)


def padding_waste(B: int, n: int) -> int:
    """Padded-minus-ragged slots when one n-token prompt joins B-1 single-token decodes."""
    rows = [n] + [1] * (B - 1)
    return padded_slots(rows) - useful_slots(rows)


def blocks_for(seq_len: int, block_size: int) -> int:
    """Blocks a sequence of ``seq_len`` tokens occupies (ceil-div)."""
    if block_size < MIN_BLOCK_SIZE:
        raise ValueError(f"block_size must be at least {MIN_BLOCK_SIZE}, got {block_size}")
    if seq_len < 0:
        raise ValueError("negative sequence length")
    return -(-int(seq_len) // int(block_size))


def internal_waste(seq_len: int, block_size: int) -> int:
    """Unused slots in the last block of a sequence."""
    return blocks_for(seq_len, block_size) * block_size - int(seq_len)


def pack_ragged(rows):
    """Concatenate per-sequence token arrays along axis 0; return (packed, cu_seqlens).

    cu_seqlens[i] is where sequence i starts in the packed array; cu_seqlens[-1] is the
    total. No batch axis, no padding.
    """
    rows = [np.asarray(r) for r in rows]
    _check_rows([r.shape[0] for r in rows])
    cu = np.zeros(len(rows) + 1, dtype=np.int64)
    for i, r in enumerate(rows):
        cu[i + 1] = cu[i] + r.shape[0]
    return np.concatenate(rows, axis=0), cu
