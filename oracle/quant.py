"""Oracle: per-token symmetric quantization of K and V, and KV byte accounting.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* "KV Cache optimization techniques" tutorial (metaphor-xennon), §1.2 逐Token量化
  (per-token quantizer): one scale per (batch, head, token), taken as the
  max-abs over head_dim divided by the largest code, then round and clamp.
  Dequantization multiplies the code by its scale.
* Same tutorial, §1.1 量化基础: the INT4 constants (divide by 7, clamp to
  [-8, 7]) and symmetric dequantization.
* "KV Cache Compression Report" (纯文本大语言模型 KV 缓存压缩 — 完整技术报告),
  §3.2 (L1: INT8 量化): the same max-abs/127 rule applied at write time
  to K and V, with codes clamped to [-127, 127].
* Same tutorial, section "KV Cache的挑战": bytes per token of KV cache are
  2 x layers x heads x head_dim x bytes per element.

Readings taken where the pages leave a step open:
* No epsilon is added to the scale; an all-zero row gets scale 0 and codes 0.
* The scale is an fp32 number: the correctly rounded fp32 quotient amax/qmax.
* Each code is round-half-to-even of the correctly rounded fp32 quotient
  x/scale (a true division, not a multiply by a reciprocal).
* INT4 stores two two's-complement nibbles per byte, element 2j in the low
  nibble and element 2j+1 in the high nibble.

Precision note: amax and qmax are exact in fp32, so the fp64 quotient rounded
once to fp32 equals the correctly rounded fp32 quotient (double rounding is
innocuous because 53 >= 2*24 + 2). The same holds for x/scale, because x is an
fp16 value and scale an fp32 value.
"""
from __future__ import annotations

import numpy as np

QMAX = {8: 127, 4: 7}
QMIN = {8: -127, 4: -8}


def quantize_rows(x16: np.ndarray, bits: int):
    """Quantize the last axis of ``x16`` (fp16 values) row by row.

    Returns ``(codes, scale)``: ``codes`` int8 with the shape of ``x16`` (INT4
    codes unpacked, one per element) and ``scale`` float32 with the last axis
    dropped.
    """
    if bits not in QMAX:
        raise ValueError("bits must be 8 or 4")
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    qmax = QMAX[bits]
    # Step 1: amax over head_dim (exact).
    amax = np.max(np.abs(x), axis=-1)
    # Step 2: fp32 scale = amax / qmax, correctly rounded.
    scale = (amax / qmax).astype(np.float32)
    s = scale.astype(np.float64)[..., None]
    nz = s > 0
    # Step 3: fp32 quotient x / scale, correctly rounded.
    t = (x / np.where(nz, s, 1.0)).astype(np.float32).astype(np.float64)
    # Step 4: round half to even, clamp to the code range.
    code = np.clip(np.rint(t), QMIN[bits], qmax)
    code = np.where(nz, code, 0.0)
    return code.astype(np.int8), scale


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x_hat = code * scale in fp64 (exact: an 8-bit integer times an fp32)."""
    return codes.astype(np.float64) * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Pack int4 codes (last axis even) two per byte: low nibble = element 2j."""
    c = np.asarray(codes, dtype=np.int16)
    if c.shape[-1] % 2:
        raise ValueError("head_dim must be even for INT4")
    if c.min(initial=0) < -8 or c.max(initial=0) > 7:
        raise ValueError("int4 code out of range")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_int4`, sign-extending each nibble."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def kv_bytes_per_token(num_layers: int, num_heads: int, head_dim: int,
                       bytes_per_element: float) -> float:
    """KV-cache bytes for one token: K and V, every layer and head."""
    return 2 * num_layers * num_heads * head_dim * bytes_per_element


def compressed_bytes_per_token_head(head_dim: int, bits: int, with_scales: bool = True) -> int:
    """Stored bytes for one token of one KV head, K and V together:
    the codes (head_dim * bits / 8 each) plus one fp32 scale each."""
    codes = head_dim * bits // 8
    return 2 * (codes + (4 if with_scales else 0))
