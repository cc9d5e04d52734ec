"""Pins for the oracle's decode attention (CPU only).

Closed forms and invariants that fix the result independently of how the
oracle computes it: rows of p sum to 1, one token returns its V row, equal keys
average V, a dominant key selects its V row, two tokens follow the logistic
function of the logit gap, the 1/sqrt(D) factor fixes p1/p0 for a known key
difference, the GQA mapping sends query head h to KV head h // G, token order
does not matter, and paged storage gives the result of contiguous storage.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def _cache(rng, Hkv, L, D, bits=8, scale=1.0):
    k = (rng.standard_normal((Hkv, L, D)) * scale).astype(np.float16)
    v = (rng.standard_normal((Hkv, L, D)) * scale).astype(np.float16)
    kc, ks = oracle.quantize_rows(k, bits)
    vc, vs = oracle.quantize_rows(v, bits)
    return kc, ks, vc, vs


@settings(max_examples=50, deadline=None)
@given(st.integers(0, 2 ** 32 - 1), st.sampled_from([1, 2, 4]), st.integers(1, 300))
def test_rows_sum_to_one(seed, G, L):
    rng = np.random.default_rng(seed)
    kc, ks, vc, vs = _cache(rng, 2, L, 32)
    q = rng.standard_normal((1, 2 * G, 32)).astype(np.float16)
    _, probs = oracle.decode_attention(q, kc[None], ks[None], vc[None], vs[None], [L])
    assert np.all(np.abs(probs[0].sum(axis=1) - 1) <= 1e-12)
    assert np.all(probs[0] >= 0)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    kc, ks, vc, vs = _cache(rng, 1, 1, 64)
    q = rng.standard_normal((1, 1, 64)).astype(np.float16)
    out, _ = oracle.decode_attention(q, kc[None], ks[None], vc[None], vs[None], [1])
    assert np.array_equal(out[0, 0], vc[0, 0].astype(np.float64) * float(vs[0, 0]))


def test_equal_keys_average_values():
    rng = np.random.default_rng(2)
    _, _, vc, vs = _cache(rng, 1, 37, 64)
    kc = np.zeros((1, 37, 64), np.int8)
    ks = np.zeros((1, 37), np.float32)
    q = rng.standard_normal((1, 1, 64)).astype(np.float16)
    out, _ = oracle.decode_attention(q, kc[None], ks[None], vc[None], vs[None], [37])
    mean = (vc[0].astype(np.float64) * vs[0].astype(np.float64)[:, None]).mean(axis=0)
    assert np.allclose(out[0, 0], mean, rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(3)
    L, D = 50, 64
    _, _, vc, vs = _cache(rng, 1, L, D)
    kc = np.zeros((1, L, D), np.int8)
    ks = np.ones((1, L), np.float32)
    kc[0, 17, :] = 127          # logit 127*sum(q)/8 with q = 1 -> 127*64/8 = 1016
    q = np.ones((1, 1, D), np.float16)
    out, probs = oracle.decode_attention(q, kc[None], ks[None], vc[None], vs[None], [L])
    assert probs[0][0, 17] == 1.0
    assert np.abs(out[0, 0] - vc[0, 17].astype(np.float64) * float(vs[0, 17])).max() < 1e-20


def test_two_tokens_logistic_and_sqrt_d():
    """p1 = 1 / (1 + exp(-(s1 - s0))) with s_i = q.k_i / sqrt(D)."""
    for D in (16, 64, 128):
        kc = np.zeros((1, 2, D), np.int8)
        kc[0, 1, 0] = 3                     # q.k1 - q.k0 = 3 * 0.5 * 2 = 3
        ks = np.full((1, 2), 0.5, np.float32)
        vc = np.zeros((1, 2, D), np.int8)
        vc[0, 1, :] = 1
        vs = np.ones((1, 2), np.float32)
        q = np.zeros((1, 1, D), np.float16)
        q[0, 0, 0] = 2.0
        out, probs = oracle.decode_attention(q, kc[None], ks[None], vc[None], vs[None], [2])
        gap = 3.0 / math.sqrt(D)
        want = 1.0 / (1.0 + math.exp(-gap))
        assert abs(probs[0][0, 1] - want) < 1e-15
        assert abs(out[0, 0, 5] - want) < 1e-15


def test_gqa_head_mapping():
    """Each KV head carries a constant V row; query head h must read h // G."""
    Hkv, G, L, D = 4, 3, 20, 32
    rng = np.random.default_rng(4)
    kc, ks, _, _ = _cache(rng, Hkv, L, D)
    vc = np.zeros((Hkv, L, D), np.int8)
    for g in range(Hkv):
        vc[g] = g + 1
    vs = np.ones((Hkv, L), np.float32)
    q = rng.standard_normal((1, Hkv * G, D)).astype(np.float16)
    out, _ = oracle.decode_attention(q, kc[None], ks[None], vc[None], vs[None], [L])
    for h in range(Hkv * G):
        assert np.allclose(out[0, h], h // G + 1, rtol=0, atol=1e-13)


def test_token_permutation_invariance():
    rng = np.random.default_rng(5)
    kc, ks, vc, vs = _cache(rng, 2, 64, 32)
    q = rng.standard_normal((1, 2, 32)).astype(np.float16)
    perm = rng.permutation(64)
    a, _ = oracle.decode_attention(q, kc[None], ks[None], vc[None], vs[None], [64])
    b, _ = oracle.decode_attention(q, kc[None][:, :, perm], ks[None][:, :, perm],
                                   vc[None][:, :, perm], vs[None][:, :, perm], [64])
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_length_limits_the_attended_set():
    rng = np.random.default_rng(6)
    kc, ks, vc, vs = _cache(rng, 1, 40, 32)
    q = rng.standard_normal((1, 1, 32)).astype(np.float16)
    a, _ = oracle.decode_attention(q, kc[None], ks[None], vc[None], vs[None], [25])
    junk = kc.copy()
    junk[:, 25:] = 127
    b, _ = oracle.decode_attention(q, junk[None], ks[None], vc[None], vs[None], [25])
    assert np.array_equal(a, b)


def test_paged_equals_contiguous():
    rng = np.random.default_rng(7)
    B, Hkv, D, bs = 3, 2, 32, 16
    lens = [33, 16, 50]
    nblk = [(n + bs - 1) // bs for n in lens]
    NB = sum(nblk) + 2
    perm = rng.permutation(NB)
    table = np.full((B, max(nblk)), -1, np.int64)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    kp = np.zeros((NB, Hkv, bs, D), np.int8)
    vp = np.zeros((NB, Hkv, bs, D), np.int8)
    ksp = np.zeros((NB, Hkv, bs), np.float32)
    vsp = np.zeros((NB, Hkv, bs), np.float32)
    q = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    cap = max(lens)
    kc = np.zeros((B, Hkv, cap, D), np.int8)
    vc = np.zeros((B, Hkv, cap, D), np.int8)
    ks = np.zeros((B, Hkv, cap), np.float32)
    vs = np.zeros((B, Hkv, cap), np.float32)
    for b in range(B):
        k16 = rng.standard_normal((Hkv, lens[b], D)).astype(np.float16)
        v16 = rng.standard_normal((Hkv, lens[b], D)).astype(np.float16)
        c1, s1 = oracle.quantize_rows(k16, 8)
        c2, s2 = oracle.quantize_rows(v16, 8)
        kc[b, :, :lens[b]], ks[b, :, :lens[b]] = c1, s1
        vc[b, :, :lens[b]], vs[b, :, :lens[b]] = c2, s2
        for t in range(lens[b]):
            blk, off_ = table[b, t // bs], t % bs
            kp[blk, :, off_], ksp[blk, :, off_] = c1[:, t], s1[:, t]
            vp[blk, :, off_], vsp[blk, :, off_] = c2[:, t], s2[:, t]
    a, _ = oracle.decode_attention(q, kc, ks, vc, vs, lens)
    b_ = oracle.paged_decode_attention(q, kp, ksp, vp, vsp, table, lens, bs)
    assert np.array_equal(a, b_)


# -- planted mistakes ----------------------------------------------------------

def _attend_no_sqrt(q16, kc, ks, vc, vs):
    K = oracle.dequantize(kc, ks)
    V = oracle.dequantize(vc, vs)
    s = q16.astype(np.float64) @ K.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p @ V, p


def test_planted_missing_sqrt_is_caught():
    D = 64
    kc = np.zeros((2, D), np.int8)
    kc[1, 0] = 3
    ks = np.full(2, 0.5, np.float32)
    vc = np.zeros((2, D), np.int8)
    vc[1] = 1
    vs = np.ones(2, np.float32)
    q = np.zeros((1, D), np.float16)
    q[0, 0] = 2.0
    _, p = _attend_no_sqrt(q, kc, ks, vc, vs)
    want = 1.0 / (1.0 + math.exp(-3.0 / math.sqrt(D)))
    assert abs(p[0, 1] - want) > 1e-3
