"""Oracle: fp16 precision tiers at both ends of a quantized cache.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* "KV Cache Compression Report", §3.2 (L1: INT8 量化), design notes: the K and
  V of the attention-sink tokens stay in fp16, to avoid losing precision where
  the model keeps putting attention.
* "KV Cache optimization techniques" tutorial, §1.3 (混合精度KV Cache): recent
  tokens at a higher precision (fp16), older tokens at a lower one (INT4); the
  same page's strategy table names this mode "int4_hybrid" (recent fp16,
  distant INT4).

Readings:
* The sink tier is the first ``n_sink16`` slots of a row, the recent tier the
  last ``n_recent16`` slots; a slot in both (a row shorter than the two
  together) belongs to the sink tier, so the recent tier takes the last
  min(n_recent16, L - min(n_sink16, L)) slots.
* A tier slot is attended at its exact fp16 value; every other slot at its
  dequantized codes. The tutorial's code slices the *first* recent_len tokens
  as "recent", against its own docstring; the docstring is taken (the newest
  tokens are the recent ones), and the window is a fixed token count.
* Codes are written for every token, tier or not (quantize on write, never
  recompute): a token that leaves the recent tier is attended from the codes
  written when it arrived.
"""
from __future__ import annotations

import numpy as np

from .quant import dequantize


def tier_bounds(length: int, n_sink16: int, n_recent16: int):
    """(ns, lo) for a row of ``length`` slots: slots [0, ns) form the sink
    tier and [lo, length) the recent tier; [ns, lo) is read from the codes."""
    ns = min(n_sink16, length)
    nr = min(n_recent16, length - ns)
    return ns, length - nr


def tier_values(codes: np.ndarray, scale: np.ndarray, raw16: np.ndarray, length: int,
                n_sink16: int, n_recent16: int) -> np.ndarray:
    """The first ``length`` rows of one (sequence, KV head) as attention reads
    them: fp16 values on the tiers, code * scale elsewhere (fp64 [length][D]).

    codes [>= length][D] unpacked; scale [>= length] fp32; raw16 [>= length][D]
    the fp16 rows as they were written.
    """
    vals = dequantize(codes[:length], scale[:length])
    ns, lo = tier_bounds(length, n_sink16, n_recent16)
    vals[:ns] = raw16[:ns].astype(np.float64)
    vals[lo:length] = raw16[lo:length].astype(np.float64)
    return vals
