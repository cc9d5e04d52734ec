"""Pins for the oracle's quantization and byte accounting (CPU only).

Each check is independent of the oracle's own code path: constructed halfway
cases whose answer is known by hand, numpy's native IEEE fp32 division as a
second route to the correctly rounded quotient, the dequantization error bound,
an exhaustive nibble round trip, and the byte figures the pages print.
"""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(path):
    rows = []
    with open(os.path.join(GOLDEN, path)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _all_finite_fp16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    return x[np.isfinite(x)]


def _native_fp32_codes(x16, amax16, bits):
    """Second route: fp32 arithmetic done by numpy in fp32 (IEEE division)."""
    qmax = np.float32(oracle.QMAX[bits])
    s = np.float32(amax16) / qmax
    if s == 0:
        return np.zeros(x16.shape, np.int8), s
    t = x16.astype(np.float32) / s
    return np.clip(np.rint(t), oracle.QMIN[bits], oracle.QMAX[bits]).astype(np.int8), s


@pytest.mark.parametrize("row", _rows("quant_halfway.txt"))
def test_golden_halfway_cases(row):
    bits, amax, x, code = int(row[0]), float(row[1]), float(row[2]), int(row[3])
    c, s = oracle.quantize_rows(np.array([[x, amax]], np.float16), bits)
    assert s[0] == np.float32(1.0)
    assert int(c[0, 0]) == code
    assert int(c[0, 1]) == oracle.QMAX[bits]


@pytest.mark.parametrize("bits", [8, 4])
def test_extremes_map_to_qmax(bits):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((256, 128)).astype(np.float16)
    c, s = oracle.quantize_rows(x, bits)
    am = np.abs(x.astype(np.float64)).argmax(axis=1)
    got = c[np.arange(256), am].astype(int)
    want = np.sign(x[np.arange(256), am].astype(np.float64)).astype(int) * oracle.QMAX[bits]
    assert np.array_equal(got, want)
    assert c.min() >= -oracle.QMAX[bits]  # -128 / -8 are never produced


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("amax", [127.0, 1.0, 3.140625, 0.0999755859375, 6.103515625e-05,
                                  1000.0, 65504.0, 5.960464477539063e-08, 2.5, 37.3125])
def test_exhaustive_fp16_against_native_fp32_division(bits, amax):
    """Every finite fp16 x with |x| <= amax: the oracle's fp64-then-round route
    equals numpy's fp32 division followed by round-half-to-even."""
    a16 = np.float16(amax)
    xs = _all_finite_fp16()
    xs = xs[np.abs(xs.astype(np.float64)) <= float(a16)]
    rows = np.stack([xs, np.full_like(xs, a16)], axis=1)
    c, s = oracle.quantize_rows(rows, bits)
    want, s_native = _native_fp32_codes(xs, a16, bits)
    assert np.all(s == s_native)
    assert np.array_equal(c[:, 0], want)


def test_zero_row():
    c, s = oracle.quantize_rows(np.zeros((3, 64), np.float16), 8)
    assert np.all(s == 0) and np.all(c == 0)


@settings(max_examples=200, deadline=None)
@given(st.integers(0, 2 ** 32 - 1), st.sampled_from([8, 4]), st.sampled_from([1.0, 1e-3, 30.0]))
def test_dequant_error_bound(seed, bits, mag):
    """|x - code*scale| <= scale/2 (+ the fp32 rounding of the quotient)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((8, 64)) * mag).astype(np.float16)
    c, s = oracle.quantize_rows(x, bits)
    xh = oracle.dequantize(c, s)
    x64 = x.astype(np.float64)
    bound = s.astype(np.float64)[:, None] / 2 + np.abs(x64) * 2.0 ** -23
    assert np.all(np.abs(x64 - xh) <= bound * (1 + 1e-12))


def test_int4_pack_roundtrip_all_bytes():
    allb = np.arange(256, dtype=np.uint8)[None]
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(allb)), allb)
    u = oracle.unpack_int4(np.array([[0x08, 0x80, 0xF7, 0x7F]], np.uint8))
    assert u.tolist() == [[-8, 0, 0, -8, 7, -1, -1, 7]]


def test_int4_pack_layout():
    codes = np.array([[1, -2, 7, -8]], np.int8)
    assert oracle.pack_int4(codes).tolist() == [[0xE1, 0x87]]


# -- planted mistakes: each must be caught by the pins above -------------------

def _quant_round_half_away(x16, bits):
    x = x16.astype(np.float64)
    s = (np.abs(x).max(-1) / oracle.QMAX[bits]).astype(np.float32)
    t = (x / s.astype(np.float64)[..., None]).astype(np.float32).astype(np.float64)
    return np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), oracle.QMIN[bits], oracle.QMAX[bits]), s


def _quant_reciprocal(x16, bits):
    x = x16.astype(np.float32)
    s = np.abs(x).max(-1) / np.float32(oracle.QMAX[bits])
    r = np.float32(1.0) / s
    return np.clip(np.rint(x * r[..., None]), oracle.QMIN[bits], oracle.QMAX[bits]), s


def _quant_eps(x16, bits):
    x = x16.astype(np.float64)
    s = (np.abs(x).max(-1) / oracle.QMAX[bits] + 1e-8).astype(np.float32)
    t = (x / s.astype(np.float64)[..., None]).astype(np.float32)
    return np.clip(np.rint(t), oracle.QMIN[bits], oracle.QMAX[bits]), s


def test_planted_round_half_away_is_caught():
    c, _ = _quant_round_half_away(np.array([[2.5, 127.0]], np.float16), 8)
    assert c[0, 0] != 2  # the golden table says 2


def test_planted_reciprocal_multiply_is_caught():
    xs = _all_finite_fp16()
    a16 = np.float16(37.3125)
    xs = xs[np.abs(xs.astype(np.float64)) <= float(a16)]
    rows = np.stack([xs, np.full_like(xs, a16)], axis=1)
    bad, _ = _quant_reciprocal(rows, 8)
    good, _ = oracle.quantize_rows(rows, 8)
    assert not np.array_equal(bad[:, 0], good[:, 0])


def test_planted_epsilon_is_caught():
    rows = np.array([[1.0, 3.140625]], np.float16)
    _, s_bad = _quant_eps(rows, 8)
    _, s = oracle.quantize_rows(rows, 8)
    _, s_native = _native_fp32_codes(rows[0], rows[0, 1], 8)
    assert s[0] == s_native and s_bad[0] != s_native


# -- byte accounting ----------------------------------------------------------

def test_kv_bytes_printed_examples():
    for tag, seq, gb, bpe in _rows("kv_bytes.txt"):
        total = oracle.kv_bytes_per_token(32, 32, 128, int(bpe)) * int(seq) / 1024 ** 3
        assert abs(total - float(gb)) < 5e-3 * max(1.0, float(gb)), (tag, seq)
    assert oracle.kv_bytes_per_token(32, 32, 128, 2) == 524288


def test_compression_ratio_printed():
    for bits, ratio in _rows("compression_ratio.txt"):
        codes = oracle.compressed_bytes_per_token_head(128, int(bits), with_scales=False)
        assert codes / (2 * 128 * 2) == float(ratio)


def test_llama7b_int8_layer_bytes():
    per_tok = oracle.compressed_bytes_per_token_head(128, 8)
    assert per_tok == 264
    assert 32 * 8192 * per_tok == 69_206_016
    # 70B-shaped INT4 layer: B=4 sequences x 8 KV heads x 131072 tokens.
    assert 4 * 8 * 131072 * oracle.compressed_bytes_per_token_head(128, 4) == 570_425_344


def test_mixed_widths_are_the_two_uniform_halves():
    """A cache with INT8 keys and INT4 values (the tutorial's K-V mode, section
    1.1) holds the K half of an all-INT8 cache and the V half of an all-INT4
    cache, and its attention is that over those dequantized halves."""
    rng = np.random.default_rng(41)
    B, H, D, L = 2, 2, 64, 40
    k = rng.standard_normal((B, H, L, D)).astype(np.float16)
    v = rng.standard_normal((B, H, L, D)).astype(np.float16)
    mixed = oracle.RefCache(B, H, D, L, 8, v_bits=4)
    k8, v4 = oracle.RefCache(B, H, D, L, 8), oracle.RefCache(B, H, D, L, 4)
    for c in (mixed, k8, v4):
        c.append(k, v)
    assert np.array_equal(mixed.k_codes, k8.k_codes) and np.array_equal(mixed.k_scale, k8.k_scale)
    assert np.array_equal(mixed.v_codes, v4.v_codes) and np.array_equal(mixed.v_scale, v4.v_scale)
    assert mixed.v_codes.min() >= -8 and mixed.v_codes.max() <= 7
    q = rng.standard_normal((B, 4, D)).astype(np.float16)
    out, _ = mixed.attend(q, h2o=False)
    want, _ = oracle.decode_attention(q, k8.k_codes, k8.k_scale, v4.v_codes, v4.v_scale, mixed.lengths)
    assert np.array_equal(out, want)
