"""Oracle: a reference compressed KV cache and the decode-step schedule.

Test infrastructure only (see ``oracle/__init__.py``).

A decode step runs the four parts in the order the pages give them:
quantize-on-write of the new token ("KV Cache Compression Report", §3.2: the
cache is quantized when written and never recomputed), attention over the whole
cache with H2O accumulation (§3.4 of the report), then, when the length exceeds
the budget, selection and compaction ("KV Cache optimization techniques"
tutorial, §2.2: append, then evict when over the limit).

Readings: a freshly appended slot starts with score 0 and
receives the current query's probability in the same step; a slot's position
is the running count of tokens the sequence has seen.
"""
from __future__ import annotations

import numpy as np

from .attention import attend_values, decode_attention
from .eviction import compact_row, h2o_accumulate, select_keep
from .quant import quantize_rows
from .tiers import tier_values


class RefCache:
    """Contiguous per-(sequence, KV head) cache with unpacked integer codes."""

    def __init__(self, batch: int, num_kv_heads: int, head_dim: int, capacity: int, bits: int,
                 v_bits: int | None = None, fp16_sinks: int = 0, fp16_recent: int = 0):
        B, H, D, C = batch, num_kv_heads, head_dim, capacity
        self.bits = bits
        # Keys and values may use different widths ("KV Cache optimization
        # techniques" tutorial, section 1.1: the quantizer's K-V mode).
        self.v_bits = v_bits or bits
        self.capacity = C
        self.k_codes = np.zeros((B, H, C, D), dtype=np.int8)
        self.v_codes = np.zeros((B, H, C, D), dtype=np.int8)
        self.k_scale = np.zeros((B, H, C), dtype=np.float32)
        self.v_scale = np.zeros((B, H, C), dtype=np.float32)
        self.positions = np.zeros((B, H, C), dtype=np.int64)
        self.score = np.zeros((B, H, C), dtype=np.float64)
        self.lengths = np.zeros(B, dtype=np.int64)
        self.num_seen = np.zeros(B, dtype=np.int64)
        # fp16 tiers ("KV Cache Compression Report", section 3.2: sinks in fp16;
        # tutorial section 1.3: recent tokens in fp16). Every slot keeps the
        # fp16 row it was written with; attention reads it on the tiers.
        self.fp16_sinks, self.fp16_recent = fp16_sinks, fp16_recent
        self.tiered = fp16_sinks > 0 or fp16_recent > 0
        if self.tiered:
            self.k_raw = np.zeros((B, H, C, D), dtype=np.float16)
            self.v_raw = np.zeros((B, H, C, D), dtype=np.float16)

    # -- quantize-on-write ------------------------------------------------
    def append(self, k16: np.ndarray, v16: np.ndarray) -> None:
        """Append n tokens per sequence: k16, v16 [B][Hkv][n][D] fp16."""
        n = k16.shape[2]
        ck, sk = quantize_rows(k16, self.bits)
        cv, sv = quantize_rows(v16, self.v_bits)
        for b in range(k16.shape[0]):
            L = int(self.lengths[b])
            if L + n > self.capacity:
                raise ValueError("append beyond capacity")
            sl = slice(L, L + n)
            self.k_codes[b, :, sl] = ck[b]
            self.v_codes[b, :, sl] = cv[b]
            self.k_scale[b, :, sl] = sk[b]
            self.v_scale[b, :, sl] = sv[b]
            self.positions[b, :, sl] = self.num_seen[b] + np.arange(n)
            if self.tiered:
                self.k_raw[b, :, sl] = k16[b]
                self.v_raw[b, :, sl] = v16[b]
            self.score[b, :, sl] = 0.0
            self.lengths[b] += n
            self.num_seen[b] += n

    # -- attention + H2O --------------------------------------------------
    def attend(self, q16: np.ndarray, h2o: bool = True):
        if self.tiered:
            out, probs = self._attend_tiered(q16)
        else:
            out, probs = decode_attention(q16, self.k_codes, self.k_scale, self.v_codes,
                                          self.v_scale, self.lengths)
        if h2o:
            Hkv = self.k_codes.shape[1]
            G = q16.shape[1] // Hkv
            for b, p in enumerate(probs):
                L = int(self.lengths[b])
                for g in range(Hkv):
                    self.score[b, g, :L] = h2o_accumulate(self.score[b, g, :L],
                                                          p[g * G:(g + 1) * G])
        return out, probs

    def _attend_tiered(self, q16: np.ndarray):
        B, Hq, D = q16.shape
        Hkv = self.k_codes.shape[1]
        G = Hq // Hkv
        out = np.zeros((B, Hq, D))
        probs = []
        for b in range(B):
            L = int(self.lengths[b])
            pb = np.zeros((Hq, L))
            for g in range(Hkv):
                K = tier_values(self.k_codes[b, g], self.k_scale[b, g], self.k_raw[b, g], L,
                                self.fp16_sinks, self.fp16_recent)
                V = tier_values(self.v_codes[b, g], self.v_scale[b, g], self.v_raw[b, g], L,
                                self.fp16_sinks, self.fp16_recent)
                o, p = attend_values(q16[b, g * G:(g + 1) * G], K, V)
                out[b, g * G:(g + 1) * G] = o
                pb[g * G:(g + 1) * G] = p
            probs.append(pb)
        return out, probs

    # -- eviction ---------------------------------------------------------
    def select(self, budget: int, n_sink: int, n_recent: int) -> np.ndarray:
        if self.tiered and (n_sink < self.fp16_sinks or n_recent < self.fp16_recent):
            # Eviction must keep both tiers whole: the sink tier is slots
            # [0, fp16_sinks) and the recent tier the newest fp16_recent slots.
            raise ValueError("eviction must keep the fp16 tiers: n_sink >= fp16_sinks, "
                             "n_recent >= fp16_recent")
        B, H, C = self.score.shape
        keep = np.zeros((B, H, C), dtype=bool)
        for b in range(B):
            L = int(self.lengths[b])
            for g in range(H):
                keep[b, g, :L] = select_keep(self.score[b, g, :L], L, budget, n_sink, n_recent)
        return keep

    def compact(self, keep: np.ndarray) -> None:
        B, H, C = self.score.shape
        new_len = None
        for b in range(B):
            L = int(self.lengths[b])
            counts = {int(keep[b, g, :L].sum()) for g in range(H)}
            if len(counts) != 1:
                raise ValueError("every KV head of a sequence must keep the same count")
            cnt = counts.pop()
            for g in range(H):
                arrs = compact_row(keep[b, g, :L], self.k_codes[b, g, :L], self.v_codes[b, g, :L],
                                   self.k_scale[b, g, :L], self.v_scale[b, g, :L],
                                   self.positions[b, g, :L], self.score[b, g, :L])
                for dst, a in zip((self.k_codes, self.v_codes, self.k_scale, self.v_scale,
                                   self.positions, self.score), arrs):
                    dst[b, g, :cnt] = a
                if self.tiered:  # the fp16 rows travel with their slots
                    kr, vr = compact_row(keep[b, g, :L], self.k_raw[b, g, :L], self.v_raw[b, g, :L])
                    self.k_raw[b, g, :cnt] = kr
                    self.v_raw[b, g, :cnt] = vr
            self.lengths[b] = cnt
            new_len = cnt
        return new_len

    def step(self, q16, k16, v16, budget=None, n_sink=0, n_recent=0, h2o=True):
        """One decode step: append, attend (+H2O), and evict when over budget."""
        self.append(k16, v16)
        out, probs = self.attend(q16, h2o=h2o)
        keep = None
        if budget is not None and int(self.lengths.max()) > budget:
            keep = self.select(budget, n_sink, n_recent)
            self.compact(keep)
        return out, probs, keep


def paged_append(k_pool, k_scale_pool, v_pool, v_scale_pool, table, lengths,
                 k16, v16, bits, block_size):
    """Quantize n new tokens per sequence into a block pool.

    Pools are [NB][Hkv][block_size][D] (unpacked codes) and [NB][Hkv][block_size];
    ``lengths`` [B] is the length before the append and is advanced in place.
    Logical token t of sequence b goes to slot t % block_size of block
    table[b][t // block_size] (tutorial §3.2, with the length tracked per sequence).
    """
    n = k16.shape[2]
    ck, sk = quantize_rows(k16, bits)
    cv, sv = quantize_rows(v16, bits)
    for b in range(k16.shape[0]):
        for j in range(n):
            t = int(lengths[b]) + j
            blk = int(table[b][t // block_size])
            if blk < 0:
                raise ValueError("append into an unreserved block")
            off = t % block_size
            k_pool[blk, :, off] = ck[b, :, j]
            v_pool[blk, :, off] = cv[b, :, j]
            k_scale_pool[blk, :, off] = sk[b, :, j]
            v_scale_pool[blk, :, off] = sv[b, :, j]
        lengths[b] += n
