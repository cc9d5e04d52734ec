"""Oracle: attention with K and V stored apart (scoring on K, top-k V).

Test infrastructure only (see ``oracle/__init__.py``).

Source: "KV Cache Compression Report", §3.5 (L4: K/V 分离存储): the quantized
K of every token stays on the GPU and is used to score the query; the full
V is kept in fp16, hot rows on the GPU and cold rows in host memory, and only
the V rows of the top-k scored tokens are fetched to form the output.

Readings:
* The scores are the cache's ordinary attention logits, s_i = q . K_i /
  sqrt(D) for every cached token, with K_i the key as that attention reads it:
  code_i * scale_i, or the fp16 row on a cache's fp16 tiers.
* The top-k is taken per KV head, by the attention probability the group's
  query heads give each token in this step (softmax over all tokens, summed
  over the group) -- the H2O mass of one step, the same granularity as the
  keep-set. Ties go to the lower slot; k = min(top_k, L).
* The page's ``softmax(scores[idx])`` (a softmax of one score) is read as the
  softmax over the selected tokens' scores: out = sum over the selection of
  e^{s_i} / sum_j e^{s_j} * v_i.
* V values are the tokens' fp16 rows; where a row lives (GPU or host) does
  not change its value.
"""
from __future__ import annotations

import math

import numpy as np

from .eviction import select_keep


def kv_separated_attention(q16: np.ndarray, K: np.ndarray, v16: np.ndarray, length: int, top_k: int):
    """One KV head and the G query heads that read it.

    q16 [G][D] fp16; K [>= L][D] the keys as the cache's attention reads them
    (``dequantize`` of the codes, or ``tier_values`` on a tiered cache);
    v16 [>= L][D] the fp16 V rows. Returns (out [G][D] fp64, keep [L] bool).
    """
    if top_k < 1:
        raise ValueError("top_k must be >= 1")
    L = int(length)
    D = q16.shape[-1]
    K = np.asarray(K[:L], dtype=np.float64)
    q = q16.astype(np.float64)
    s = (q @ K.T) / math.sqrt(D)                     # [G][L]
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    keep = select_keep(p.sum(axis=0), L, top_k, 0, 0)
    idx = np.nonzero(keep)[0]
    sk = s[:, idx]
    w = np.exp(sk - sk.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return w @ v16[idx].astype(np.float64), keep
