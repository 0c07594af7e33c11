"""CPU oracle: paged cache layout (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library.

Paged, append-only caches ("FP8 KV Cache Quantization: Why Keys Break Before
Values", section "Should you quantize keys pre-RoPE or post-RoPE?") keep the
cache in fixed-size blocks; per-channel key groups are formed within them.
Reading taken: a page holds P consecutive tokens of one sequence for every kv
head, and block_table[b][j] names the page of tokens [j P, (j + 1) P) of
sequence b.  A token section of the arena is then [pages][H][rows per page]
[...] where a page holds P token rows, P / G per-channel key-group rows, or
P / 32 value blocks.  The oracle does not model pages in its arithmetic: it
quantizes every sequence as the contiguous cache it is (oracle.cache, at that
sequence's own length) and gathers a paged section back into that layout, so
paged and contiguous caches are compared byte for byte.
"""
from __future__ import annotations

import numpy as np


def blocks_of(T: int, P: int) -> int:
    """Pages a sequence of T tokens occupies."""
    return -(-int(T) // int(P))


def gather_pages(section: np.ndarray, block_table: np.ndarray, b: int, P: int, T: int) -> np.ndarray:
    """The rows of sequence b's first T tokens from a paged section
    [pages][H][rows per page][...], in contiguous order: [H][blocks * rows per
    page][...] with the pages block_table[b][0], block_table[b][1], ... laid
    end to end (rows past T in the last page included)."""
    n = blocks_of(T, P)
    if n == 0:
        return section[:0].reshape((section.shape[1], 0) + section.shape[3:])
    return np.concatenate([section[int(block_table[b, j])] for j in range(n)], axis=1)


def scatter_pages(rows: np.ndarray, block_table: np.ndarray, b: int, out: np.ndarray) -> np.ndarray:
    """Inverse of gather_pages for whole pages: rows [H][n * rows per page][...]
    of sequence b written into the section out [pages][H][rows per page][...]."""
    per = out.shape[2]
    assert rows.shape[1] % per == 0
    for j in range(rows.shape[1] // per):
        out[int(block_table[b, j])] = rows[:, j * per:(j + 1) * per]
    return out
