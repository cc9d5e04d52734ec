"""GPU parity of K/V-separated attention (top-k V over quantized-K scores).

The cache holds the quantized K and V as usual (optionally with fp16 tiers,
the hot V rows); the cold V rows sit in a pinned host tensor that the kernel
reads directly. Each (sequence, KV head) is checked against
``oracle.kv_separated_attention`` on the same fp16 inputs: outputs within the
attention tolerance wherever the oracle's top-k has no candidate within the
score tolerance of its threshold (such a row has more than one correct
selection; the test reports how many were skipped and requires it to be rare).
"""
import numpy as np
import pytest

import oracle
from workloads import draw, get

from kvc_testlib import OUT_ATOL, SCORE_FLOOR, SCORE_RTOL, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
kvc = pytest.importorskip("compressed_kv_cache_kvc_amd")


def _mass(q16, K, L):
    s = q16.astype(np.float64) @ K[:L].T / np.sqrt(q16.shape[-1])
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


CASES = [
    # bits, hq, hkv, D, B, L, top_k, fp16_sinks, fp16_recent
    (8, 4, 4, 128, 2, 600, 100, 0, 0),       # every V row from host memory
    (4, 8, 2, 128, 2, 1000, 300, 4, 64),     # INT4, GQA 4, hot rows from the fp16 tiers
    (8, 16, 2, 64, 2, 333, 333, 0, 40),      # GQA 8, D = 64, top_k = L (all kept)
    (8, 8, 8, 128, 2, 257, 1, 4, 0),         # top_k = 1
    (8, 32, 2, 128, 2, 900, 512, 2, 100),    # GQA 16
    (4, 4, 4, 128, 2, 40, 50, 0, 0),         # L < top_k <= capacity: all kept
    (8, 32, 32, 128, 1, 8192, 2457, 0, 0),   # the benchmarked layer: every kept row cold
    (8, 32, 32, 128, 1, 8192, 2457, 4, 1024),  # the benchmarked layer with the hot window
]


@pytest.mark.parametrize("bits,hq,hkv,D,B,L,top_k,S16,R16", CASES)
def test_kvsep_matches_oracle(bits, hq, hkv, D, B, L, top_k, S16, R16):
    print(f"[kvsep] bits={bits} hq={hq} hkv={hkv} D={D} L={L} top_k={top_k} tiers={S16}/{R16}", flush=True)
    w = get("qwen_gqa_stream").scaled(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, bits=bits, context=L,
                                      steps=1)
    d = draw(w)
    cap = L + 16
    gc = kvc.KVCache(B, hkv, D, cap, bits, fp16_sinks=S16, fp16_recent=R16)
    kvc.kvc_quant_append(gc, dev(d["k"]), dev(d["v"]))
    v_host = torch.zeros((B, hkv, cap, D), dtype=torch.float16).pin_memory()
    v_host[:, :, :L] = torch.from_numpy(d["v"])
    out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn_kvsep(gc, dev(d["q"]), top_k, v_host, out)
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(np.isfinite(got))
    kc, ks = oracle.quantize_rows(d["k"], bits)
    G = hq // hkv
    checked = skipped = 0
    for b in range(B):
        for g in range(hkv):
            q = d["q"][b, g * G:(g + 1) * G]
            # keys as the cache's attention reads them (fp16 rows on the tiers)
            K = oracle.tier_values(kc[b, g], ks[b, g], d["k"][b, g], L, S16, R16)
            ro, keep = oracle.kv_separated_attention(q, K, d["v"][b, g], L, top_k)
            k = min(top_k, L)
            if k < L:
                mass = _mass(q, K, L)
                T = np.sort(mass)[::-1][k - 1]
                if np.sum(np.abs(mass - T) <= SCORE_RTOL * T + SCORE_FLOOR) > 1:
                    skipped += 1
                    continue
            err = np.abs(got[b, g * G:(g + 1) * G] - ro).max()
            assert err <= OUT_ATOL, (b, g, err)
            checked += 1
    assert skipped <= max(1, checked // 8), (checked, skipped)


def test_kvsep_with_all_tokens_kept_equals_fp16_value_attention():
    """top_k >= L keeps every token: the output is ordinary attention over the
    quantized keys with the exact fp16 values, on both hot and cold rows."""
    B, hq, hkv, D, L = 2, 8, 4, 128, 700
    w = get("qwen_gqa_stream").scaled(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, bits=8, context=L,
                                      steps=1)
    d = draw(w)
    gc = kvc.KVCache(B, hkv, D, L, 8, fp16_sinks=4, fp16_recent=128)
    kvc.kvc_quant_append(gc, dev(d["k"]), dev(d["v"]))
    v_host = torch.from_numpy(np.ascontiguousarray(d["v"])).pin_memory()
    out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn_kvsep(gc, dev(d["q"]), L, v_host, out)
    torch.cuda.synchronize()
    kc, ks = oracle.quantize_rows(d["k"], 8)
    G = hq // hkv
    for b in range(B):
        for g in range(hkv):
            K = oracle.tier_values(kc[b, g], ks[b, g], d["k"][b, g], L, 4, 128)
            ro, _ = oracle.attend_values(d["q"][b, g * G:(g + 1) * G], K, d["v"][b, g])
            assert np.abs(host(out)[b, g * G:(g + 1) * G] - ro).max() <= OUT_ATOL


def test_kvsep_paged_equals_contiguous():
    """On a paged cache (blocks in a seeded random order, fp16 tiers) the call
    gives the contiguous cache's output bit for bit; the contiguous side is
    the one checked against the oracle above."""
    B, hq, hkv, D, L, bs, top_k = 2, 8, 2, 128, 900, 16, 200
    w = get("qwen_gqa_stream").scaled(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, bits=8, context=L,
                                      steps=1)
    d = draw(w)
    cap = 912
    mb = cap // bs
    table = np.random.default_rng(9).permutation(B * mb).astype(np.int32).reshape(B, mb)
    pg = kvc.KVCache(B, hkv, D, 0, 8, block_size=bs, num_blocks=B * mb, max_blocks_per_seq=mb, fp16_sinks=4,
                     fp16_recent=64)
    pg.block_table.copy_(dev(table))
    ct = kvc.KVCache(B, hkv, D, cap, 8, fp16_sinks=4, fp16_recent=64)
    v_host = torch.zeros((B, hkv, cap, D), dtype=torch.float16).pin_memory()
    v_host[:, :, :L] = torch.from_numpy(d["v"])
    outs = []
    for c in (pg, ct):
        kvc.kvc_quant_append(c, dev(d["k"]), dev(d["v"]))
        out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
        kvc.kvc_decode_attn_kvsep(c, dev(d["q"]), top_k, v_host, out)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
