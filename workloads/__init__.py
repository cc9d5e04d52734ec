"""Seeded synthetic inputs for compressed-KV decode attention.

This module only draws random numbers and arranges them into the shapes of the
five workloads below. It holds none of the method's arithmetic: no
quantization, attention, scoring or selection. The oracle-based tests and the
HIP path both consume exactly the fp16 arrays produced here.

Draw order per workload is fixed: q, then K (one chunk per sequence, b = 0..B-1),
then V (same), then structure (outlier channels or tokens, lengths, block
permutation), then per-step draws. Normal values are drawn in float32 with
``numpy.random.default_rng(seed)`` and cast to float16 with round-to-nearest-even.

Shapes follow the workloads the pages discuss: an 8192-token context ("7 models @
8192 tokens" in the checklist table of "KV Cache 推理效率自查"), LLaMA-7B
dimensions of 32 layers x 32 heads x 128 (the memory analysis of the KV cache
optimization tutorial, and §1.2 of the KV cache compression report), and GQA
with fewer KV heads (§6 of the eviction-and-reuse survey). No dataset or trained
model is used; none is available.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "draw"]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    bits: int
    context: int                 # L attended at the measured step, appended token included
    budget: Optional[int]        # keep budget after eviction; None = no eviction
    n_sink: int = 0
    n_recent: int = 0
    prior_queries: int = 0       # decode queries that seed H2O scores before the measured one
    steps: int = 1               # decode steps (streaming loop)
    outlier_channels: int = 0    # per KV head, channels scaled by outlier_scale (K and V)
    outlier_token_frac: float = 0.0  # fraction of token positions scaled by outlier_scale
    outlier_scale: float = 1.0
    paged_block: int = 0         # 0 = contiguous cache, else tokens per block
    len_lo: int = 0              # paged: per-sequence lengths uniform in [len_lo, len_hi]
    len_hi: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, **kw) -> "Workload":
        """Same workload with some fields changed (e.g. a shorter context for tests)."""
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # Tiny MHA decode step: budget 128 = 4 sinks + 64 recent + 60 heavy hitters,
    # scores seeded by 8 prior decode queries.
    "tiny_mha": Workload("tiny_mha", 1001, 1, 4, 4, 64, 8, 512, 128, 4, 64,
                         prior_queries=8),
    # LLaMA-7B-shaped layer at 8192 tokens, 4 outlier channels per head x10,
    # keep ratio 0.3 -> budget floor(0.3 * 8192) = 2457 = 4 + 1024 + 1429.
    "llama7b_8k": Workload("llama7b_8k", 1002, 1, 32, 32, 128, 8, 8192, 2457, 4, 1024,
                           outlier_channels=4, outlier_scale=10.0),
    # Batched paged decode: 32 sequences, lengths uniform in [1024, 4096],
    # 16-token INT8 blocks placed by a seeded permutation, no eviction.
    "paged_b32": Workload("paged_b32", 1003, 32, 32, 32, 128, 8, 4096, None,
                          paged_block=16, len_lo=1024, len_hi=4096),
    # Qwen2.5-7B-shaped GQA streaming: 28 q heads / 4 KV heads, 32768-token
    # context, 64 decode steps each evicting back to floor(0.25 * 32768) = 8192
    # = 4 sinks + 2048 recent + 6140 heavy.
    "qwen_gqa_stream": Workload("qwen_gqa_stream", 1004, 8, 28, 4, 128, 8, 32768, 8192,
                                4, 2048, steps=64),
    # 70B-shaped GQA with an INT4 cache: 64 q heads / 8 KV heads, 131072 tokens,
    # 1% of token positions x8, keep ratio 0.2 -> floor(0.2 * 131072) = 26214
    # = 4 + 2048 + 24162.
    "llama70b_int4": Workload("llama70b_int4", 1005, 4, 64, 8, 128, 4, 131072, 26214,
                              4, 2048, outlier_token_frac=0.01, outlier_scale=8.0),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _to_f16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16, round to nearest even (IEEE). torch's conversion is
    the same rounding and runs on every core; numpy's is the fallback."""
    try:
        import torch
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float16).numpy()
    except ImportError:
        return x.astype(np.float16)


def _normal16(rng: np.random.Generator, shape) -> np.ndarray:
    return _to_f16(rng.standard_normal(size=shape, dtype=np.float32))


def _kv_chunk(rng, shape, chans: Optional[np.ndarray], toks: Optional[np.ndarray], scale: float) -> np.ndarray:
    """One sequence's K or V, [Hkv][L][D]: N(0, 1), with the outlier channels
    (per KV head) or outlier token positions multiplied by `scale` in float32
    before the cast."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    s = np.float32(scale)
    if chans is not None:
        for g in range(shape[0]):
            x[g][:, chans[g]] *= s
    if toks is not None:
        x[:, toks, :] *= s
    return _to_f16(x)


def draw(w: Workload) -> Dict[str, np.ndarray]:
    """Draw every input of workload ``w``.

    Returns a dict of numpy arrays (fp16 values, int32 structure):

    * ``q``        [B][Hq][D]          the measured query
    * ``k``, ``v`` [B][Hkv][L][D]      contiguous: all tokens attended at the
      measured step; the last one is the token appended by that step
    * ``k_seq``/``v_seq`` (paged)      list of [Hkv][L_b][D] per sequence
    * ``lengths``  [B]                 tokens per sequence at the measured step
    * ``prior_q``  [P][B][Hq][D]       queries that seed H2O scores (if P > 0)
    * ``block_table`` [B][max_blocks]  paged: physical block per logical block, -1 pad
    * ``num_blocks`` scalar            paged: blocks in the pool
    * ``step_q`` [S][B][Hq][D], ``step_k``/``step_v`` [S][B][Hkv][1][D]
      streaming: per decode step (the first step's token is also ``k[:, :, -1]``)
    """
    rng = np.random.default_rng(w.seed)
    B, Hq, Hkv, D = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    out: Dict[str, np.ndarray] = {}
    out["q"] = _normal16(rng, (B, Hq, D))

    if w.paged_block:
        # Lengths first would change the K/V draw shapes, so they come from a
        # child generator seeded by the same workload seed.
        lrng = np.random.default_rng([w.seed, 1])
        lengths = lrng.integers(w.len_lo, w.len_hi, endpoint=True, size=B).astype(np.int32)
        out["lengths"] = lengths
        out["k_seq"] = [_normal16(rng, (Hkv, int(lengths[b]), D)) for b in range(B)]
        out["v_seq"] = [_normal16(rng, (Hkv, int(lengths[b]), D)) for b in range(B)]
        bs = w.paged_block
        nblk = [(int(n) + bs - 1) // bs for n in lengths]
        nb_total = int(sum(nblk))
        perm = rng.permutation(nb_total).astype(np.int32)
        max_blocks = max(nblk)
        table = np.full((B, max_blocks), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            table[b, : nblk[b]] = perm[off: off + nblk[b]]
            off += nblk[b]
        out["block_table"] = table
        out["num_blocks"] = np.int32(nb_total)
        return out

    L = w.context
    # Structure is drawn from a child generator so that K and V chunks can be
    # produced in one pass with the outlier mask already known.
    srng = np.random.default_rng([w.seed, 2])
    chans = None
    if w.outlier_channels:
        # per KV head, distinct channels in ascending order
        chans = np.stack([np.sort(srng.choice(D, size=w.outlier_channels, replace=False))
                          for _ in range(Hkv)]).astype(np.int32)
        out["outlier_channels"] = chans
    toks = None
    if w.outlier_token_frac:
        n_out = int(round(w.outlier_token_frac * L))
        toks = np.stack([np.sort(srng.choice(L, size=n_out, replace=False)) for _ in range(B)]).astype(np.int32)
        out["outlier_tokens"] = toks

    k = np.empty((B, Hkv, L, D), dtype=np.float16)
    v = np.empty((B, Hkv, L, D), dtype=np.float16)
    for b in range(B):
        k[b] = _kv_chunk(rng, (Hkv, L, D), chans, None if toks is None else toks[b], w.outlier_scale)
    for b in range(B):
        v[b] = _kv_chunk(rng, (Hkv, L, D), chans, None if toks is None else toks[b], w.outlier_scale)
    out["k"], out["v"] = k, v
    out["lengths"] = np.full(B, L, dtype=np.int32)

    if w.prior_queries:
        out["prior_q"] = _normal16(rng, (w.prior_queries, B, Hq, D))
    if w.steps > 1:
        S = w.steps
        out["step_q"] = np.concatenate([out["q"][None], _normal16(rng, (S - 1, B, Hq, D))])
        sk = _normal16(rng, (S - 1, B, Hkv, 1, D))
        sv = _normal16(rng, (S - 1, B, Hkv, 1, D))
        out["step_k"] = np.concatenate([k[None, :, :, L - 1: L], sk])
        out["step_v"] = np.concatenate([v[None, :, :, L - 1: L], sv])
    return out
