"""KV-cache waste accounting (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

LESSON, "The Concept: PagedAttention as a virtual memory system": reserving a
fixed maximum number of slots per request wastes the reserved-but-unused
share (its worked example: 8192 slots reserved, about 1500 used, roughly 82%
of the reservation wasted), while 16-token blocks waste only the unused tail
of each sequence's last block.  The LESSON's exercises (item 4) pose the
comparison for a trace of requests of a given mean and spread.

Definitions used here:
  paged internal waste  = 1 - (tokens held) / (block_size * blocks held)
  contiguous waste      = 1 - (tokens held) / (reservation * requests)
Both are ratios of unused to reserved KV slots over a set of sequences.
"""
from __future__ import annotations

import numpy as np


def paged_blocks(lengths, block_size: int = 16) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    return -(-lengths // block_size)


def paged_waste(lengths, block_size: int = 16) -> float:
    lengths = np.asarray(lengths, dtype=np.int64)
    held = int(paged_blocks(lengths, block_size).sum()) * block_size
    return 0.0 if held == 0 else 1.0 - float(lengths.sum()) / held


def contiguous_waste(lengths, reservation: int = 8192) -> float:
    lengths = np.minimum(np.asarray(lengths, dtype=np.int64), reservation)
    total = reservation * len(lengths)
    return 0.0 if total == 0 else 1.0 - float(lengths.sum()) / total

