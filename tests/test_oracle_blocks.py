"""Pins of the block-granular eviction oracle (oracle/blocks.py) and host
tests of the pool's refcounted release (no GPU needed)."""
import itertools

import numpy as np
import pytest

import oracle
from oracle.blocks import block_evict, move_block_scores


def _scores(means_per_block, H=2, bs=16, length=None):
    n = len(means_per_block)
    s = np.zeros((H, n * bs))
    for j, m in enumerate(means_per_block):
        s[:, j * bs:(j + 1) * bs] = m
    return s


def test_retention_one_keeps_all_and_zero_evicts_all():
    s = _scores([3.0, 1.0, 2.0])
    row = [7, 5, 9, -1]
    assert block_evict(row, 40, s, 1.0) == (row, 40, [], [0, 1, 2])
    assert block_evict(row, 40, s, 0.0) == ([-1, -1, -1, -1], 0, [7, 5, 9], [])


def test_stable_tie_order_hand_example():
    # Means 1, 1, 0.5, 2 and retention 0.5: n_evict = int(4 * 0.5) = 2. The
    # stable ascending order is blocks 2, 0, 1, 3 (equal means keep block
    # order), so blocks 2 and 0 go and 1, 3 stay.
    s = _scores([1.0, 1.0, 0.5, 2.0])
    new_row, new_len, freed, kept = block_evict([10, 11, 12, 13], 64, s, 0.5)
    assert kept == [1, 3] and new_row == [11, 13, -1, -1] and freed == [10, 12] and new_len == 32


def test_evict_count_is_truncated_in_double():
    # 5 blocks, retention 0.3: 5 * (1 - 0.3) is 3.4999999999999996 in double -> 3.
    s = _scores([5.0, 4.0, 3.0, 2.0, 1.0])
    _, _, freed, kept = block_evict(list(range(5)), 80, s, 0.3)
    assert len(freed) == 3 and kept == [0, 1]


def test_partial_last_block_length():
    s = _scores([1.0, 2.0, 3.0])
    assert block_evict([4, 5, 6], 37, s, 0.5)[1] == 16 + 5       # last (5 slots) kept with block 1
    s2 = _scores([3.0, 2.0, 1.0])
    assert block_evict([4, 5, 6], 37, s2, 0.5)[1] == 32           # the partial last block goes


def test_mean_over_filled_slots_only():
    s = np.zeros((1, 48))
    s[0, :16] = 1.0
    s[0, 16:32] = 0.9
    s[0, 32:34] = 5.0            # partial block of 2 filled slots, mean 5
    s[0, 34:48] = -100.0         # past the length: must not count
    assert block_evict([0, 1, 2], 34, s, 2 / 3)[3] == [0, 2]


@pytest.mark.parametrize("seed", range(20))
def test_brute_force_subset(seed):
    """The evicted set is the only set of size n_evict whose members all come
    before every kept block in (mean, index) order."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 7))
    vals = rng.integers(0, 3, size=n).astype(float)            # many exact ties
    r = float(rng.choice([0.0, 0.25, 0.5, 0.6, 1.0]))
    length = 16 * (n - 1) + int(rng.integers(1, 17))
    s = _scores(list(vals), length=length)
    _, _, _, kept = block_evict(list(range(n)), length, s, r)
    n_evict = int(n * (1 - r))
    means = [float(np.mean(s[:, 16 * j:16 * j + min(16, length - 16 * j)])) for j in range(n)]
    ok = [set(c) for c in itertools.combinations(range(n), n_evict)
          if all((means[e], e) < (means[k], k) for e in c for k in set(range(n)) - set(c))]
    assert ok == [set(range(n)) - set(kept)]


def test_attention_over_rewritten_table_equals_kept_tokens():
    """The table rewrite moves no code: paged attention through the new table
    equals contiguous attention over the kept tokens."""
    rng = np.random.default_rng(3)
    H, G, D, bs, nblk, L = 2, 2, 16, 16, 6, 85
    k = rng.standard_normal((nblk, H, bs, D)).astype(np.float16)
    v = rng.standard_normal((nblk, H, bs, D)).astype(np.float16)
    kp, vp = np.zeros((nblk, H, bs, D), np.int8), np.zeros((nblk, H, bs, D), np.int8)
    ks, vs = np.zeros((nblk, H, bs), np.float32), np.zeros((nblk, H, bs), np.float32)
    table = np.array([[4, 1, 5, 0, 3, 2]], np.int32)
    seq_k = np.concatenate([k[table[0, j]] for j in range(nblk)], axis=1)[None, :, :L]
    seq_v = np.concatenate([v[table[0, j]] for j in range(nblk)], axis=1)[None, :, :L]
    oracle.paged_append(kp, ks, vp, vs, table, np.zeros(1, np.int64), seq_k, seq_v, 8, bs)
    scores = rng.random((H, nblk * bs))
    new_row, new_len, freed, kept = block_evict(list(table[0]), L, scores, 0.5)
    q = rng.standard_normal((1, H * G, D)).astype(np.float16)
    out_new = oracle.paged_decode_attention(q, kp, ks, vp, vs, np.array([new_row], np.int32),
                                            np.array([new_len]), bs)
    tok = [bs * j + t for j in kept for t in range(min(bs, L - bs * j))]
    kk = np.stack([kp[table[0, i // bs], :, i % bs] for i in tok], axis=1)[None]
    ksk = np.stack([ks[table[0, i // bs], :, i % bs] for i in tok], axis=1)[None]
    vv = np.stack([vp[table[0, i // bs], :, i % bs] for i in tok], axis=1)[None]
    vsk = np.stack([vs[table[0, i // bs], :, i % bs] for i in tok], axis=1)[None]
    out_ref, _ = oracle.decode_attention(q, kk, ksk, vv, vsk, np.array([len(tok)]))
    np.testing.assert_allclose(out_new, out_ref, rtol=0, atol=1e-12)
    moved = move_block_scores(scores, kept, L)
    assert np.array_equal(moved[:, :new_len], scores[:, tok])


kvc = pytest.importorskip("compressed_kv_cache_kvc_amd")


def test_pool_release_refcounts_and_order():
    p = kvc.BlockPool(10, 16, shuffle_seed=0)
    p.reserve(1, 16 * 5)                     # blocks 0..4
    t = p.block_table([1], 6)
    assert t.tolist() == [[0, 1, 2, 3, 4, -1]]
    p.release(1, [3, 1])
    assert p.num_free == 7 and p.num_blocks_of(1) == 3
    assert p.block_table([1], 6).tolist() == [[0, 2, 4, -1, -1, -1]]   # the rest keep their order
    with pytest.raises(kvc.KvcError):
        p.release(1, [1])                    # no longer held
    with pytest.raises(kvc.KvcError):
        p.release(1, [0, 0])                 # listed twice
    with pytest.raises(kvc.KvcError):
        p.release(9, [0])                    # unknown sequence
    assert p.num_free == 7 and p.num_blocks_of(1) == 3   # failed calls change nothing
    p.reserve(2, 16)                          # a freed block is handed out again
    assert p.num_free == 6
