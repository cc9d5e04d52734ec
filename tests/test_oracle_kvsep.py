"""Pins for the oracle's K/V-separated attention (top-k V over K scores).

Closed forms and brute force, not the oracle's own formula: with top_k >= L
it is full attention over the dequantized keys and the fp16 values, computed
here by plain Python loops; top_k = 1 returns the V row of the token with the
largest group mass; a constant V returns that constant (the weights over the
selection sum to 1 -- a planted version that keeps the full-softmax weights
without renormalizing fails this); a dominant key returns its own V row; and
the selection is the top-k of the group mass found by sorting all slots.
"""
import math

import numpy as np
import pytest

import oracle


def _rand16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def _head(rng, G, L, D, bits=8):
    k = _rand16(rng, (1, 1, L, D))
    kc, ks = oracle.quantize_rows(k, bits)
    return _rand16(rng, (G, D)), kc[0, 0], ks[0, 0], _rand16(rng, (L, D))


def _loop_attention(q, K, V):
    D = len(q)
    s = [sum(float(q[d]) * float(K[i][d]) for d in range(D)) / math.sqrt(D) for i in range(len(K))]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    return [sum(e[i] / z * float(V[i][d]) for i in range(len(K))) for d in range(D)]


@pytest.mark.parametrize("top_k", [9, 50])
def test_top_k_covering_every_token_is_full_attention(top_k):
    rng = np.random.default_rng(31)
    G, L, D = 2, 9, 16
    q, kc, ks, v = _head(rng, G, L, D, bits=4)
    out, keep = oracle.kv_separated_attention(q, oracle.dequantize(kc, ks), v, L, top_k)
    assert keep.all()
    K = oracle.dequantize(kc, ks)
    for h in range(G):
        assert np.allclose(out[h], _loop_attention(q[h], K, v), rtol=0, atol=1e-12)


def test_top_one_returns_the_heaviest_tokens_row():
    rng = np.random.default_rng(32)
    G, L, D = 3, 40, 32
    q, kc, ks, v = _head(rng, G, L, D)
    out, keep = oracle.kv_separated_attention(q, oracle.dequantize(kc, ks), v, L, 1)
    K = oracle.dequantize(kc, ks)
    s = q.astype(np.float64) @ K.T / math.sqrt(D)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    best = int(np.argmax(p.sum(axis=0)))
    assert np.nonzero(keep)[0].tolist() == [best]
    assert np.array_equal(out, np.repeat(v[best][None].astype(np.float64), G, axis=0))


def test_constant_values_come_back_exactly():
    rng = np.random.default_rng(33)
    G, L, D = 2, 60, 32
    q, kc, ks, _ = _head(rng, G, L, D)
    v = np.full((L, D), 1.5, np.float16)
    for top_k in (1, 7, 30, 60):
        out, _ = oracle.kv_separated_attention(q, oracle.dequantize(kc, ks), v, L, top_k)
        assert np.allclose(out, 1.5, rtol=0, atol=1e-14), top_k

    # planted: the full-softmax weights of the kept tokens, not renormalized
    K = oracle.dequantize(kc, ks)
    s = q.astype(np.float64) @ K.T / math.sqrt(D)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    _, keep = oracle.kv_separated_attention(q, oracle.dequantize(kc, ks), v, L, 7)
    planted = p[:, keep] @ v[keep].astype(np.float64)
    assert not np.allclose(planted, 1.5, rtol=0, atol=1e-6)


def test_dominant_key_returns_its_row():
    rng = np.random.default_rng(34)
    L, D = 30, 64
    q, kc, ks, v = _head(rng, 1, L, D)
    q[:] = 0
    q[0, 0] = 64.0
    k = _rand16(rng, (1, 1, L, D), 0.01)
    k[0, 0, 17, 0] = 64.0
    kc, ks = oracle.quantize_rows(k, 8)
    for top_k in (1, 5, 30):
        out, keep = oracle.kv_separated_attention(q, oracle.dequantize(kc[0, 0], ks[0, 0]), v, L, top_k)
        assert keep[17]
        assert np.allclose(out[0], v[17].astype(np.float64), rtol=0, atol=1e-20)


@pytest.mark.parametrize("seed", range(5))
def test_selection_is_the_top_k_of_group_mass(seed):
    rng = np.random.default_rng(100 + seed)
    G, L, D, top_k = 4, 50, 16, 12
    q, kc, ks, v = _head(rng, G, L, D)
    _, keep = oracle.kv_separated_attention(q, oracle.dequantize(kc, ks), v, L, top_k)
    K = oracle.dequantize(kc, ks)
    s = q.astype(np.float64) @ K.T / math.sqrt(D)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    mass = p.sum(axis=0)
    order = sorted(range(L), key=lambda i: (-mass[i], i))
    assert set(np.nonzero(keep)[0].tolist()) == set(order[:top_k])
