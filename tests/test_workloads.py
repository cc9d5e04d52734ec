"""The seeded generators: determinism and the structure each workload promises."""
import numpy as np

from workloads import draw, get


def test_deterministic_and_fp16():
    w = get("tiny_mha")
    a, b = draw(w), draw(w)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["k"].dtype == np.float16 and a["q"].dtype == np.float16


def test_outlier_channels_are_scaled():
    w = get("llama7b_8k").scaled(context=512)
    d = draw(w)
    ch = d["outlier_channels"]
    assert ch.shape == (32, 4)
    for g in range(32):
        std = d["k"][0, g].astype(np.float64).std(axis=0)
        assert set(np.argsort(std)[-4:]) == set(ch[g].tolist())


def test_outlier_tokens_are_scaled():
    w = get("llama70b_int4").scaled(context=4096, batch=1)
    d = draw(w)
    toks = d["outlier_tokens"][0]
    assert len(toks) == round(0.01 * 4096)
    amax = np.abs(d["k"][0].astype(np.float64)).max(axis=(0, 2))
    assert amax[toks].min() > np.delete(amax, toks).max() * 0.9 or amax[toks].mean() > 5 * np.delete(amax, toks).mean()


def test_paged_table_is_a_permutation():
    w = get("paged_b32").scaled(batch=4, num_q_heads=2, num_kv_heads=2)
    d = draw(w)
    t = d["block_table"]
    used = t[t >= 0]
    assert sorted(used.tolist()) == list(range(int(d["num_blocks"])))
    for b in range(4):
        n = (int(d["lengths"][b]) + 15) // 16
        assert np.all(t[b, :n] >= 0) and np.all(t[b, n:] == -1)
        assert 1024 <= d["lengths"][b] <= 4096


def test_streaming_first_step_is_last_context_token():
    w = get("qwen_gqa_stream").scaled(context=64, steps=3, batch=2)
    d = draw(w)
    assert np.array_equal(d["step_k"][0][:, :, 0], d["k"][:, :, -1])
    assert d["step_q"].shape == (3, 2, 28, 128)
