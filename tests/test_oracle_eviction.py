"""Pins for the oracle's H2O accumulation, keep-set selection and compaction.

Brute force over every subset on tiny rows, hand-made edge cases, the H2O mass
invariant (before eviction each KV head's scores sum to steps x G, because
every softmax row sums to 1), and the structural facts compaction must leave
behind.
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import draw, get


def _brute_force_keep(score, L, budget, S, R):
    if L <= budget:
        return set(range(L))
    cand = list(range(S, L - R))
    k = budget - S - R
    best, best_set = None, None
    for sub in itertools.combinations(cand, k):
        val = sum(score[i] for i in sub)
        if best is None or val > best:
            best, best_set = val, set(sub)
    return set(range(S)) | set(range(L - R, L)) | best_set


@settings(max_examples=120, deadline=None)
@given(st.integers(0, 2 ** 32 - 1), st.integers(3, 12), st.integers(0, 2), st.integers(0, 3),
       st.integers(1, 12))
def test_select_matches_brute_force(seed, L, S, R, budget):
    if S + R > budget:
        return
    rng = np.random.default_rng(seed)
    score = rng.permutation(L).astype(np.float64) + rng.random(L)   # distinct scores
    keep = oracle.select_keep(score, L, budget, S, R)
    assert set(np.nonzero(keep)[0]) == _brute_force_keep(score, L, budget, S, R)
    assert keep.sum() == min(L, budget)


def test_select_edge_cases():
    s = np.array([5, 1, 9, 3, 7, 2, 8, 0.5], np.float64)
    assert oracle.select_keep(s, 8, 8, 2, 2).all()                  # L <= budget
    k0 = oracle.select_keep(s, 8, 4, 2, 2)                           # k = 0
    assert np.nonzero(k0)[0].tolist() == [0, 1, 6, 7]
    eq = oracle.select_keep(np.ones(10), 10, 5, 1, 1)                 # ties -> lower slots
    assert np.nonzero(eq)[0].tolist() == [0, 1, 2, 3, 9]
    top = oracle.select_keep(s, 8, 5, 1, 1)                           # heavy from [1, 7)
    assert np.nonzero(top)[0].tolist() == [0, 2, 4, 6, 7]
    with pytest.raises(ValueError):
        oracle.select_keep(s, 8, 3, 2, 2)


def test_h2o_mass_invariant_tiny_schedule():
    """tiny_mha: 8 prior queries + the measured one, G = 1 -> each head sums to 9."""
    w = get("tiny_mha")
    d = draw(w)
    c = oracle.RefCache(w.batch, w.num_kv_heads, w.head_dim, w.context, w.bits)
    c.append(d["k"][:, :, :-1], d["v"][:, :, :-1])
    c.append(d["k"][:, :, -1:], d["v"][:, :, -1:])
    for j in range(w.prior_queries):
        c.attend(d["prior_q"][j])
    c.attend(d["q"])
    sums = c.score[:, :, :w.context].sum(axis=2)
    assert np.allclose(sums, 9.0 * w.group, rtol=0, atol=1e-11)


def test_h2o_mass_invariant_gqa():
    rng = np.random.default_rng(11)
    B, Hkv, G, D, L = 2, 3, 4, 32, 40
    c = oracle.RefCache(B, Hkv, D, L + 5, 8)
    c.append(rng.standard_normal((B, Hkv, L, D)).astype(np.float16),
             rng.standard_normal((B, Hkv, L, D)).astype(np.float16))
    for _ in range(5):
        c.attend(rng.standard_normal((B, Hkv * G, D)).astype(np.float16))
    assert np.allclose(c.score[:, :, :L].sum(axis=2), 5.0 * G, rtol=0, atol=1e-11)


def test_compaction_invariants_and_consistency():
    w = get("tiny_mha")
    d = draw(w)
    c = oracle.RefCache(w.batch, w.num_kv_heads, w.head_dim, w.context, w.bits)
    c.append(d["k"][:, :, :-1], d["v"][:, :, :-1])
    for j in range(w.prior_queries):
        c.attend(d["prior_q"][j])
    src = {n: getattr(c, n).copy() for n in ("k_codes", "v_codes", "k_scale", "v_scale",
                                                "positions", "score")}
    c.append(d["k"][:, :, -1:], d["v"][:, :, -1:])
    out_before, _ = c.attend(d["q"])
    mass_before = c.score[:, :, :w.context].sum()
    full = {n: getattr(c, n).copy() for n in src}
    keep = c.select(w.budget, w.n_sink, w.n_recent)
    c.compact(keep)
    B, H = w.batch, w.num_kv_heads
    assert np.all(c.lengths == w.budget)
    assert c.score[:, :, :w.budget].sum() <= mass_before + 1e-12
    for b in range(B):
        for g in range(H):
            pos = c.positions[b, g, :w.budget]
            assert np.all(np.diff(pos) > 0)
            assert pos[:w.n_sink].tolist() == list(range(w.n_sink))
            assert pos[-w.n_recent:].tolist() == list(range(w.context - w.n_recent, w.context))
            idx = np.nonzero(keep[b, g, :w.context])[0]
            assert np.array_equal(c.k_codes[b, g, :w.budget], full["k_codes"][b, g, idx])
            assert np.array_equal(c.v_scale[b, g, :w.budget], full["v_scale"][b, g, idx])
            assert np.array_equal(c.score[b, g, :w.budget], full["score"][b, g, idx])
    # Attention over the compacted cache equals attention over the kept subset.
    q = d["prior_q"][0]
    o1, _ = oracle.decode_attention(q, c.k_codes, c.k_scale, c.v_codes, c.v_scale, c.lengths)
    sub_k = np.zeros_like(full["k_codes"][:, :, :w.budget])
    sub_v, sub_ks, sub_vs = sub_k.copy(), np.zeros((B, H, w.budget), np.float32), np.zeros((B, H, w.budget), np.float32)
    for b in range(B):
        for g in range(H):
            idx = np.nonzero(keep[b, g, :w.context])[0]
            sub_k[b, g], sub_v[b, g] = full["k_codes"][b, g, idx], full["v_codes"][b, g, idx]
            sub_ks[b, g], sub_vs[b, g] = full["k_scale"][b, g, idx], full["v_scale"][b, g, idx]
    o2, _ = oracle.decode_attention(q, sub_k, sub_ks, sub_v, sub_vs, [w.budget] * B)
    assert np.array_equal(o1, o2)


def test_new_slot_score_starts_at_zero():
    rng = np.random.default_rng(12)
    c = oracle.RefCache(1, 1, 16, 8, 8)
    c.append(rng.standard_normal((1, 1, 4, 16)).astype(np.float16),
             rng.standard_normal((1, 1, 4, 16)).astype(np.float16))
    c.score[0, 0, 4] = 123.0          # stale value in the next free slot
    c.append(rng.standard_normal((1, 1, 1, 16)).astype(np.float16),
             rng.standard_normal((1, 1, 1, 16)).astype(np.float16))
    assert c.score[0, 0, 4] == 0.0
    assert c.positions[0, 0, :5].tolist() == [0, 1, 2, 3, 4]


def test_kth_threshold():
    s = np.array([0, 5, 1, 9, 3, 7, 0], np.float64)
    assert oracle.kth_threshold(s, 7, 4, 1, 1) == 7.0
    assert oracle.kth_threshold(s, 7, 7, 1, 1) is None


def test_planted_highest_index_tiebreak_is_caught():
    scores = np.ones(10)
    bad = np.zeros(10, bool)
    bad[[0, 9]] = True
    cand = np.arange(1, 9)
    bad[cand[np.lexsort((-cand, -scores[cand]))[:3]]] = True
    assert not np.array_equal(bad, oracle.select_keep(scores, 10, 5, 1, 1))
