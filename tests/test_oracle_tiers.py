"""Pins for the oracle's fp16 precision tiers (sinks and recent window).

What fixes the result without the oracle's own arithmetic: hand-worked tier
bounds; one token attends to exactly its fp16 value row (not the dequantized
one); a dominant key returns its own value row, fp16 on a tier and
dequantized off it, which also fixes *which* end of the row the recent tier is
(the newest slots, not the first ones); a cache whose tiers cover every token
gives the attention over the unquantized fp16 rows, computed here by plain
Python loops; empty tiers change nothing; and after appends and evictions the
fp16 rows on the tiers are the inputs of the positions they hold, with the
sink tier at positions 0..S-1 and the recent tier ending at the newest token.
A planted mistake (the tutorial's code, which slices the first tokens as the
recent ones) must fail.
"""
import math

import numpy as np
import pytest

import oracle


def _rand16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


@pytest.mark.parametrize("L,S,R,want", [
    (10, 4, 3, (4, 7)),    # sinks 0..3, codes 4..6, recent 7..9
    (5, 4, 3, (4, 4)),     # only one slot left for the recent tier
    (3, 4, 3, (3, 3)),     # shorter than the sink tier: all sinks
    (10, 0, 0, (0, 10)),   # no tiers
    (10, 0, 10, (0, 0)),   # all recent
    (0, 4, 4, (0, 0)),     # empty row
])
def test_tier_bounds_hand_worked(L, S, R, want):
    assert oracle.tier_bounds(L, S, R) == want


def _cache_with(rng, B, H, D, C, bits, S16, R16, n, scale=1.0, v_bits=None):
    c = oracle.RefCache(B, H, D, C, bits, v_bits=v_bits, fp16_sinks=S16, fp16_recent=R16)
    k = _rand16(rng, (B, H, n, D), scale)
    v = _rand16(rng, (B, H, n, D), scale)
    c.append(k, v)
    return c, k, v


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("S16,R16", [(1, 0), (0, 1)])
def test_single_token_returns_its_fp16_value(bits, S16, R16):
    rng = np.random.default_rng(11)
    c, k, v = _cache_with(rng, 1, 1, 64, 4, bits, S16, R16, 1)
    q = _rand16(rng, (1, 1, 64))
    out, _ = c.attend(q, h2o=False)
    assert np.array_equal(out[0, 0], v[0, 0, 0].astype(np.float64))
    # ...and not its dequantized row, which differs at this width
    plain, _, _ = _cache_with(np.random.default_rng(11), 1, 1, 64, 4, bits, 0, 0, 1)
    pout, _ = plain.attend(q, h2o=False)
    assert not np.array_equal(pout[0, 0], out[0, 0])


def _dominant(rng, D, L, slot, bits, S16, R16):
    """A cache whose key at `slot` has logit >= 60 above every other key."""
    c = oracle.RefCache(1, 1, D, L, bits, fp16_sinks=S16, fp16_recent=R16)
    k = _rand16(rng, (1, 1, L, D), 0.01)
    q = np.zeros((1, 1, D), np.float16)
    q[0, 0, 0] = 64.0
    k[0, 0, slot, 0] = 64.0    # logit 64*64/sqrt(D) >= 362 vs |others| < 3
    v = _rand16(rng, (1, 1, L, D), 3.0)
    c.append(k, v)
    return c, q, v


@pytest.mark.parametrize("bits", [8, 4])
def test_dominant_key_selects_fp16_row_on_tiers_and_codes_elsewhere(bits):
    rng = np.random.default_rng(12)
    D, L, S16, R16 = 64, 12, 2, 3
    for slot in range(L):
        c, q, v = _dominant(rng, D, L, slot, bits, S16, R16)
        out, _ = c.attend(q, h2o=False)
        if slot < S16 or slot >= L - R16:
            want = v[0, 0, slot].astype(np.float64)
        else:
            want = oracle.dequantize(c.v_codes[0, 0, slot], c.v_scale[0, 0, slot])
        assert np.allclose(out[0, 0], want, rtol=0, atol=1e-20), slot


def test_recent_tier_is_the_newest_slots_not_the_first():
    """The tutorial's code slices the first recent_len tokens; a tier built
    that way would read slot 0 at fp16 and the newest slot from its codes."""
    rng = np.random.default_rng(13)
    D, L = 64, 8
    for slot, on_tier in ((0, False), (L - 1, True)):
        c, q, v = _dominant(rng, D, L, slot, 8, 0, 2)
        out, _ = c.attend(q, h2o=False)
        fp16 = v[0, 0, slot].astype(np.float64)
        deq = oracle.dequantize(c.v_codes[0, 0, slot], c.v_scale[0, 0, slot])
        assert not np.array_equal(fp16, deq)
        assert np.array_equal(out[0, 0], fp16) == on_tier

    # the planted mistake: tiers taken from the front fail the same pin
    def tier_values_front(codes, scale, raw16, length, s16, r16):
        vals = oracle.dequantize(codes[:length], scale[:length])
        vals[:s16 + r16] = raw16[:s16 + r16].astype(np.float64)
        return vals
    c, q, v = _dominant(rng, D, L, L - 1, 8, 0, 2)
    V = tier_values_front(c.v_codes[0, 0], c.v_scale[0, 0], c.v_raw[0, 0], L, 0, 2)
    assert not np.array_equal(V[L - 1], v[0, 0, L - 1].astype(np.float64))


def _loop_attention(q, K, V):
    """softmax(q K^T / sqrt(D)) V by plain Python loops (one query head)."""
    D = len(q)
    s = [sum(float(q[d]) * float(K[i][d]) for d in range(D)) / math.sqrt(D) for i in range(len(K))]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    return [sum(e[i] / z * float(V[i][d]) for i in range(len(K))) for d in range(D)]


@pytest.mark.parametrize("S16,R16", [(3, 4), (7, 0), (0, 7), (5, 5)])
def test_tiers_covering_every_token_give_fp16_attention(S16, R16):
    rng = np.random.default_rng(14)
    B, H, G, D, L = 1, 2, 2, 16, 7
    c, k, v = _cache_with(rng, B, H, D, 8, 4, S16, R16, L, scale=2.0)
    q = _rand16(rng, (B, H * G, D))
    out, _ = c.attend(q, h2o=False)
    for h in range(H * G):
        g = h // G
        want = _loop_attention(q[0, h], k[0, g], v[0, g])
        assert np.allclose(out[0, h], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bits,v_bits", [(8, None), (4, None), (8, 4)])
def test_empty_tiers_change_nothing(bits, v_bits):
    rng = np.random.default_rng(15)
    B, H, D, C, n = 2, 2, 32, 40, 33
    k = _rand16(rng, (B, H, n, D))
    v = _rand16(rng, (B, H, n, D))
    q = _rand16(rng, (B, 2 * H, D))
    a = oracle.RefCache(B, H, D, C, bits, v_bits=v_bits)
    t = oracle.RefCache(B, H, D, C, bits, v_bits=v_bits, fp16_sinks=0, fp16_recent=0)
    a.append(k, v)
    t.append(k, v)
    oa, pa = a.attend(q)
    ot, pt = t.attend(q)
    assert np.array_equal(oa, ot)
    assert all(np.array_equal(x, y) for x, y in zip(pa, pt))


def test_tier_rows_follow_their_positions_through_eviction():
    rng = np.random.default_rng(16)
    B, H, D, S16, R16 = 2, 2, 32, 2, 5
    budget, n_sink, n_recent = 16, 3, 6
    c = oracle.RefCache(B, H, D, 64, 8, fp16_sinks=S16, fp16_recent=R16)
    ks, vs = [], []
    pre_k, pre_v = _rand16(rng, (B, H, 20, D)), _rand16(rng, (B, H, 20, D))
    c.append(pre_k, pre_v)
    ks.append(pre_k)
    vs.append(pre_v)
    for step in range(30):
        k, v = _rand16(rng, (B, H, 1, D)), _rand16(rng, (B, H, 1, D))
        ks.append(k)
        vs.append(v)
        q = _rand16(rng, (B, H, D))
        c.step(q, k, v, budget=budget, n_sink=n_sink, n_recent=n_recent)
    allk = np.concatenate(ks, axis=2)
    allv = np.concatenate(vs, axis=2)
    for b in range(B):
        L, seen = int(c.lengths[b]), int(c.num_seen[b])
        ns, lo = oracle.tier_bounds(L, S16, R16)
        for g in range(H):
            pos = c.positions[b, g, :L]
            assert list(pos[:ns]) == list(range(ns))
            assert list(pos[lo:]) == list(range(seen - (L - lo), seen))
            for i in list(range(ns)) + list(range(lo, L)):
                assert np.array_equal(c.k_raw[b, g, i], allk[b, g, pos[i]])
                assert np.array_equal(c.v_raw[b, g, i], allv[b, g, pos[i]])


def test_h2o_mass_invariant_with_tiers():
    rng = np.random.default_rng(17)
    B, H, G, D = 1, 2, 3, 32
    c, _, _ = _cache_with(rng, B, H, D, 64, 4, 3, 9, 40)
    steps = 5
    for _ in range(steps):
        c.attend(_rand16(rng, (B, H * G, D)))
    for g in range(H):
        assert abs(c.score[0, g, :40].sum() - steps * G) <= 1e-12


def test_eviction_must_keep_the_tiers():
    c = oracle.RefCache(1, 1, 16, 32, 8, fp16_sinks=4, fp16_recent=8)
    with pytest.raises(ValueError):
        c.select(16, 3, 8)
    with pytest.raises(ValueError):
        c.select(16, 4, 7)
    c.select(16, 4, 8)
