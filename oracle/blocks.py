"""Block-granular H2O eviction on a paged cache (oracle).

THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT (see oracle/__init__.py).

Eviction-and-reuse survey, section 4: the blocks are sorted by their mean
attention score (Python's stable sort, lowest first) and the first
int(n * (1 - retention)) of them are evicted; evicted blocks release their
reference ("KV Cache optimization techniques" tutorial, section 3.2: a block
is free again when its count reaches zero). A block's score is the mean H2O
score over its filled slots and all KV heads of the sequence; the kept
blocks keep their order, and so do their tokens.
"""
import numpy as np


def block_evict(table_row, length: int, scores: np.ndarray, retention: float, block_size: int = 16):
    """One sequence. table_row: physical block ids by logical block;
    scores: [H][capacity] H2O scores by logical slot.

    Returns (new_row, new_length, freed, kept): the rewritten table row
    (kept physical blocks in order, then -1), the new length, the evicted
    physical blocks in block order, and the kept logical blocks in order."""
    if not 0.0 <= retention <= 1.0:
        raise ValueError("retention must lie in [0, 1]")
    n = (length + block_size - 1) // block_size
    fills = [min(block_size, length - block_size * j) for j in range(n)]
    means = [float(np.mean(np.asarray(scores, dtype=np.float64)[:, block_size * j:block_size * j + fills[j]]))
             for j in range(n)]
    order = sorted(range(n), key=lambda j: means[j])   # stable: equal means keep block order
    n_evict = int(n * (1 - retention))
    evicted = set(order[:n_evict])
    kept = [j for j in range(n) if j not in evicted]
    new_row = [int(table_row[j]) for j in kept] + [-1] * (len(table_row) - len(kept))
    freed = [int(table_row[j]) for j in range(n) if j in evicted]
    new_length = sum(fills[j] for j in kept)
    return new_row, new_length, freed, kept


def move_block_scores(scores: np.ndarray, kept, length: int, block_size: int = 16) -> np.ndarray:
    """Scores of the kept blocks at their new slots: new block i takes old
    block kept[i] (its filled slots only); other slots are zero."""
    out = np.zeros_like(scores)
    for i, j in enumerate(kept):
        fill = min(block_size, length - block_size * j)
        out[:, block_size * i:block_size * i + fill] = scores[:, block_size * j:block_size * j + fill]
    return out
