"""Ragged packing and block arithmetic — oracle side (test infrastructure only).

What is counted, and where the pages define it:
  * A padded batch is a rectangle: every row is stretched to the longest row. A ragged batch
    keeps only the real tokens, one after another with no batch axis, and every row must hold
    at least one token ("Continuous batching in transformers", section "Why use it").
  * A sequence of L tokens is stored in blocks of block_size token slots; position p sits in
    the sequence's block p // block_size, so the last block may have unused slots. Block sizes
    below 4 are rejected ("Continuous batching in transformers", section "The paged cache, its
    two reserved blocks, and the block-size trade"; "3.3 Batching & Memory Management",
    sections "PagedAttention: block tables" and "Check your understanding").

The counts are taken from explicit layouts: the padded rectangle as a boolean occupancy grid,
and a sequence's blocks as the block index of each of its positions.
"""
from __future__ import annotations

import numpy as np

SMALLEST_BLOCK = 4


def occupancy(row_lengths) -> np.ndarray:
    """Boolean grid [rows, longest row] of a padded batch: cell (r, j) is True when row r has
    a real token at column j, False where the rectangle holds padding."""
    lens = np.asarray([int(x) for x in row_lengths], dtype=np.int64)
    if lens.size == 0:
        raise ValueError("a batch needs at least one row")
    if (lens <= 0).any():
        raise ValueError("every row of a batch must hold at least one token")
    return np.arange(int(lens.max()))[None, :] < lens[:, None]


def rectangle_count(row_lengths) -> dict:
    """Cells of the padded rectangle, real tokens (what ragged packing stores) and the padding
    in between, counted on the occupancy grid."""
    grid = occupancy(row_lengths)
    real = int(grid.sum())
    return {"padded": int(grid.size), "ragged": real, "wasted": int(grid.size) - real}


def prompt_among_decodes(B: int, n: int) -> dict:
    """rectangle_count of a batch of B rows: one n-token prompt and B - 1 one-token decodes."""
    return rectangle_count(np.where(np.arange(int(B)) == 0, int(n), 1))


def block_layout(seq_len: int, block_size: int) -> dict:
    """Blocks a sequence of seq_len tokens occupies and the unused slots of its last block, from
    the block index of every position."""
    if block_size < SMALLEST_BLOCK:
        raise ValueError(f"block_size must be at least {SMALLEST_BLOCK}, got {block_size}")
    if seq_len < 0:
        raise ValueError("negative sequence length")
    block_of_position = np.arange(int(seq_len)) // int(block_size)
    blocks = int(np.unique(block_of_position).size)
    return {"blocks": blocks, "unused_tail": blocks * int(block_size) - int(seq_len)}


def pack_ragged(rows):
    """Concatenate per-sequence token arrays along axis 0; return (packed, cu_seqlens).

    cu_seqlens[i] is where sequence i starts in the packed array; cu_seqlens[-1] is the
    total. No batch axis, no padding.
    """
    rows = [np.asarray(r) for r in rows]
    occupancy([r.shape[0] for r in rows])  # the same row rules
    starts = [0]
    for r in rows:
        starts.append(starts[-1] + r.shape[0])
    return np.concatenate(rows, axis=0), np.asarray(starts, dtype=np.int64)
