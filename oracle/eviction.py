"""Oracle: H2O score accumulation, sink + recent + heavy-hitter keep-set, compaction.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* "KV Cache Compression Report", §3.4 (L3: H2O 驱逐): a token's heavy-hitter
  score is its accumulated attention; the cache keeps the top-scoring tokens
  plus the most recent ones, and the kept indices are sorted.
* Eviction-and-reuse survey, §3.3 (驱逐策略的信息损失下界): a token's score is
  the attention it receives from all later tokens, summed; greedy top-k on that
  score approximates the best subset.
* "KV Cache optimization techniques" tutorial, §2.2 (H2O): append first, evict
  when the length exceeds the limit, keep indices in ascending order, and move
  the scores along with the kept K/V.
* Same tutorial, §2.4, and the report's §3.3 (L2: StreamingLLM 滑窗): the first
  tokens are permanent attention sinks; the window holds the most recent tokens;
  a token is a sink or in the window, not both.

Readings:
* Scores are kept per (sequence, KV head); a KV head's score sums the
  probabilities of the query heads that read it.
* Keep-set = sinks [0, n_sink) + recent [L - n_recent, L) + the k = budget -
  n_sink - n_recent highest-scoring slots among the rest, so the set has exactly
  ``budget`` slots. Equal scores go to the lower slot.
* If L <= budget every slot is kept.
* Compaction is stable: kept slots keep their relative order.
"""
from __future__ import annotations

import numpy as np


def h2o_accumulate(score_row_group: np.ndarray, p_group: np.ndarray) -> np.ndarray:
    """score[i] + sum over the group's query heads of p[h, i].

    score_row_group [L] (fp64); p_group [G][L] (fp64). Returns a new array.
    """
    return np.asarray(score_row_group, dtype=np.float64) + p_group.sum(axis=0)


def select_keep(score_row: np.ndarray, length: int, budget: int, n_sink: int,
                n_recent: int) -> np.ndarray:
    """Boolean keep mask over slots [0, length) of one (sequence, KV head) row."""
    if budget < 1 or n_sink < 0 or n_recent < 0 or n_sink + n_recent > budget:
        raise ValueError("need 1 <= budget and n_sink + n_recent <= budget")
    keep = np.zeros(length, dtype=bool)
    if length <= budget:
        keep[:] = True
        return keep
    keep[:n_sink] = True
    keep[length - n_recent:] = True
    cand = np.arange(n_sink, length - n_recent)
    k = budget - n_sink - n_recent
    sc = np.asarray(score_row, dtype=np.float64)[cand]
    # Primary key: higher score; secondary: lower slot.
    order = np.lexsort((cand, -sc))
    keep[cand[order[:k]]] = True
    return keep


def kth_threshold(score_row: np.ndarray, length: int, budget: int, n_sink: int,
                  n_recent: int):
    """Score of the k-th kept candidate (None when nothing is selected by score)."""
    if length <= budget:
        return None
    k = budget - n_sink - n_recent
    if k <= 0:
        return None
    cand = np.asarray(score_row, dtype=np.float64)[n_sink:length - n_recent]
    return float(np.sort(cand)[::-1][k - 1])


def compact_row(keep: np.ndarray, *arrays):
    """Stable gather of the kept slots (ascending) of each array along axis 0."""
    idx = np.nonzero(keep)[0]
    return [np.asarray(a)[idx] for a in arrays]
