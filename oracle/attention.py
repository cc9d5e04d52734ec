"""Oracle: single-query decode attention over a quantized KV cache.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* "KV Cache Compression Report", §1.1 (KV 缓存是什么): attention is
  softmax(Q K^T / sqrt(d)) V.
* Same report, §3.2 (L1: INT8 量化): attention reads the dequantized cache,
  K_q * scale_k and V_q * scale_v, dequantized inside the attention kernel.
  The oracle writes that product out in fp64; the product is exact there.
* "KV Cache optimization techniques" tutorial, §3.2 (PagedAttention与vLLM缓存):
  a sequence's tokens live in fixed-size blocks named by a per-sequence block
  list; logical token t sits in block list[t // block_size] at offset
  t % block_size.
* Eviction-and-reuse survey (大模型推理 KV 缓存智能驱逐与复用策略), §6: with GQA
  several query heads share one KV head.

Readings: every cached token is attended (the query is
the newest token, so no mask applies); no positional transform is applied to
the cached keys; query head h reads KV head h // (Hq / Hkv).

The plain definition is computed: all logits, a max-shifted exp, a division
by the sum, and a probability-weighted sum of V. Split-K with an online
softmax reaches the same result up to rounding.
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

from .quant import dequantize


def attend_head_group(q16: np.ndarray, kc: np.ndarray, ks: np.ndarray,
                      vc: np.ndarray, vs: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """One KV head and the G query heads that read it.

    q16 [G][D] fp16; kc, vc [L][D] integer codes (unpacked); ks, vs [L] fp32.
    Returns (out [G][D] fp64, p [G][L] fp64).
    """
    return attend_values(q16, dequantize(kc, ks), dequantize(vc, vs))


def attend_values(q16: np.ndarray, K: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(q K^T / sqrt(D)) V for the G query heads of one KV head, given
    the key and value rows as numbers: K, V [L][D] (any real dtype, taken in
    fp64). Returns (out [G][D] fp64, p [G][L] fp64).
    """
    D = q16.shape[-1]
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    q = q16.astype(np.float64)               # [G][D]
    s = (q @ K.T) / math.sqrt(D)             # [G][L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ V, p


def decode_attention(q16: np.ndarray, kc: np.ndarray, ks: np.ndarray,
                     vc: np.ndarray, vs: np.ndarray, lengths) -> Tuple[np.ndarray, List[np.ndarray]]:
    """Contiguous cache. q16 [B][Hq][D]; kc, vc [B][Hkv][cap][D] unpacked codes;
    ks, vs [B][Hkv][cap]; lengths [B].

    Returns out [B][Hq][D] fp64 and, per sequence, p [Hq][L_b] fp64.
    """
    B, Hq, D = q16.shape
    Hkv = kc.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    probs = []
    for b in range(B):
        L = int(lengths[b])
        pb = np.zeros((Hq, L))
        for g in range(Hkv):
            o, p = attend_head_group(q16[b, g * G:(g + 1) * G], kc[b, g, :L], ks[b, g, :L],
                                     vc[b, g, :L], vs[b, g, :L])
            out[b, g * G:(g + 1) * G] = o
            pb[g * G:(g + 1) * G] = p
        probs.append(pb)
    return out, probs


def paged_gather(pool: np.ndarray, table_row: np.ndarray, length: int, block_size: int) -> np.ndarray:
    """Gather one sequence's tokens out of a block pool.

    pool [NB][Hkv][block_size][...] -> [Hkv][length][...]; logical token t is
    slot t % block_size of physical block table_row[t // block_size].
    """
    t = np.arange(length)
    blocks = np.asarray(table_row)[t // block_size]
    if np.any(blocks < 0) or np.any(blocks >= pool.shape[0]):
        raise ValueError("block table names a block outside the pool")
    g = pool[blocks, :, t % block_size]      # [length][Hkv][...]
    return np.moveaxis(g, 0, 1)


def paged_decode_attention(q16, k_pool, k_scale_pool, v_pool, v_scale_pool,
                           table, lengths, block_size):
    """Paged cache: gather each sequence through its block table, then attend."""
    B, Hq, D = q16.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lengths[b])
        kc = paged_gather(k_pool, table[b], L, block_size)
        vc = paged_gather(v_pool, table[b], L, block_size)
        ks = paged_gather(k_scale_pool, table[b], L, block_size)
        vs = paged_gather(v_scale_pool, table[b], L, block_size)
        for g in range(Hkv):
            o, _ = attend_head_group(q16[b, g * G:(g + 1) * G], kc[g], ks[g], vc[g], vs[g])
            out[b, g * G:(g + 1) * G] = o
    return out
