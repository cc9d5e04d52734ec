"""GPU parity of the fp16 tiers (sinks and recent window) against the oracle.

A decode loop on a tiered cache: prefill (the tier rows of a many-token
append), then steps of append, attention with H2O and eviction, so the recent
ring wraps many times and the tiers survive compactions. Each step's output
and scores are checked against ``oracle.RefCache`` with the same tiers, the
keep-set against the oracle's, and both sides then compact with the oracle's
mask. The fused calls (append inside the attention; the one-call decode
step) must equal the separate calls bit for bit.
"""
import numpy as np
import pytest

import oracle
from workloads import draw, get

from kvc_testlib import assert_codes_equal, assert_keep_equivalent, assert_out_close, assert_scores_close, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
kvc = pytest.importorskip("compressed_kv_cache_kvc_amd")


def _workload(bits, hq, hkv, D, P, steps):
    return get("qwen_gqa_stream").scaled(batch=2, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, bits=bits,
                                        context=P + 1, steps=steps)


def _tiered(w, cap, v_bits, S16, R16, like=None):
    return kvc.KVCache(w.batch, w.num_kv_heads, w.head_dim, cap, w.bits, v_bits=v_bits, fp16_sinks=S16,
                       fp16_recent=R16, share_tiers_with=like)


def _check_tier_rows(gc, ref, S16, R16):
    """The GPU's tier buffers hold the fp16 rows of the tier slots: the sink
    rows by slot, the ring by position."""
    ks, vs = (host(gc.k_sink16), host(gc.v_sink16)) if S16 else (None, None)
    kr, vr = (host(gc.k_recent16), host(gc.v_recent16)) if R16 else (None, None)
    for b in range(ref.k_raw.shape[0]):
        L, seen = int(ref.lengths[b]), int(ref.num_seen[b])
        ns, lo = oracle.tier_bounds(L, S16, R16)
        for g in range(ref.k_raw.shape[1]):
            for i in range(ns):
                assert np.array_equal(ks[b, g, i], ref.k_raw[b, g, i]) and np.array_equal(vs[b, g, i],
                                                                                          ref.v_raw[b, g, i])
            for i in range(lo, L):
                p = (seen - L + i) % R16
                assert np.array_equal(kr[b, g, p], ref.k_raw[b, g, i]) and np.array_equal(vr[b, g, p],
                                                                                          ref.v_raw[b, g, i])


LOOPS = [
    # bits, v_bits, hq, hkv, D, S16, R16
    (8, 0, 4, 4, 128, 4, 0),       # fp16 sinks only (Report 3.2)
    (4, 0, 8, 2, 128, 4, 64),      # INT4 with fp16 sinks and recent window, GQA 4
    (4, 0, 4, 4, 64, 0, 100),      # recent window only, D = 64, two tier parts
    (8, 4, 16, 2, 128, 2, 37),     # K INT8 / V INT4, GQA 8
    (8, 0, 32, 2, 128, 4, 70),     # GQA 16
    (8, 0, 8, 4, 64, 4, 50),       # D = 64, GQA 2
]


@pytest.mark.parametrize("bits,v_bits,hq,hkv,D,S16,R16", LOOPS)
@pytest.mark.parametrize("path", ["separate", "fused"])
def test_tier_decode_loop(bits, v_bits, hq, hkv, D, S16, R16, path):
    P, steps, budget = 500, 12, 420
    n_sink, n_recent = max(S16, 4), max(R16, 64)
    print(f"[tiers] bits={bits}/{v_bits} hq={hq} hkv={hkv} D={D} S16={S16} R16={R16} path={path}", flush=True)
    w = _workload(bits, hq, hkv, D, P, steps)
    d = draw(w)
    cap = P + steps + 8
    gc = _tiered(w, cap, v_bits, S16, R16)
    score = gc.score_buffer()
    ref = oracle.RefCache(w.batch, hkv, D, cap, bits, v_bits=v_bits or None, fp16_sinks=S16, fp16_recent=R16)
    kvc.kvc_quant_append(gc, dev(d["k"][:, :, :P]), dev(d["v"][:, :, :P]), h2o_score=score)
    ref.append(d["k"][:, :, :P], d["v"][:, :, :P])
    torch.cuda.synchronize()
    _check_tier_rows(gc, ref, S16, R16)
    for i in range(steps):
        q, k, v = d["step_q"][i], d["step_k"][i], d["step_v"][i]
        out = torch.empty((w.batch, hq, D), dtype=torch.float32, device="cuda")
        if path == "separate":
            kvc.kvc_quant_append(gc, dev(k), dev(v), h2o_score=score)
            kvc.kvc_decode_attn(gc, dev(q), out, h2o_score=score)
        else:
            kvc.kvc_append_decode_attn(gc, dev(k), dev(v), dev(q), out, h2o_score=score)
        ref.append(k, v)
        ro, _ = ref.attend(q)
        torch.cuda.synchronize()
        assert_codes_equal(gc, ref)
        _check_tier_rows(gc, ref, S16, R16)
        assert_out_close(host(out), ro)
        assert_scores_close(host(score), ref.score, ref.lengths)
        if int(ref.lengths.max()) > budget:
            mask = torch.zeros((w.batch, hkv, cap), dtype=torch.uint8, device="cuda")
            kvc.kvc_h2o_select(gc, score, budget, n_sink, n_recent, mask)
            torch.cuda.synchronize()
            assert_keep_equivalent(host(mask), ref.score, ref.lengths, budget, n_sink, n_recent)
            keep = ref.select(budget, n_sink, n_recent)
            ref.compact(keep)
            dst = _tiered(w, cap, v_bits, S16, R16, like=gc)
            dsc = dst.score_buffer()
            kvc.kvc_compact(gc, score, dev(keep.astype(np.uint8)), dst, dsc)
            gc, score = dst, dsc
            torch.cuda.synchronize()
            assert_codes_equal(gc, ref)


@pytest.mark.parametrize("L", [1, 3, 5, 60, 68, 70, 131])
def test_tier_short_rows(L):
    """Rows shorter than, equal to and just past the two tiers together
    (fp16_sinks 4 + fp16_recent 64): every slot a sink, all slots on a tier, one
    coded slot, several tier parts."""
    w = _workload(8, 8, 4, 128, L, 1)
    d = draw(w)
    gc = _tiered(w, L + 4, 0, 4, 64)
    score = gc.score_buffer()
    ref = oracle.RefCache(w.batch, 4, 128, L + 4, 8, fp16_sinks=4, fp16_recent=64)
    kvc.kvc_quant_append(gc, dev(d["k"][:, :, :L]), dev(d["v"][:, :, :L]), h2o_score=score)
    ref.append(d["k"][:, :, :L], d["v"][:, :, :L])
    out = torch.empty((w.batch, 8, 128), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn(gc, dev(d["q"]), out, h2o_score=score)
    ro, _ = ref.attend(d["q"])
    torch.cuda.synchronize()
    _check_tier_rows(gc, ref, 4, 64)
    assert_out_close(host(out), ro)
    assert_scores_close(host(score), ref.score, ref.lengths)


@pytest.mark.parametrize("hq,hkv,bits", [(4, 4, 8), (8, 2, 4), (16, 2, 8)])  # G = 8: the step's separate launches
def test_tier_decode_step_equals_separate_calls(hq, hkv, bits):
    """kvc_decode_step on a tiered cache equals kvc_append_decode_attn +
    kvc_h2o_evict bit for bit (output, keep list, compacted cache, kept
    scores, tier buffers), and its output equals the oracle's."""
    P, S16, R16, budget = 900, 4, 96, 600
    w = _workload(bits, hq, hkv, 128, P, 2)
    d = draw(w)
    cap = P + 8
    res = []
    for path in ("calls", "step"):
        gc = _tiered(w, cap, 0, S16, R16)
        score = gc.score_buffer()
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :P]), dev(d["v"][:, :, :P]), h2o_score=score)
        dst = _tiered(w, cap, 0, S16, R16, like=gc)
        dsc = dst.score_buffer()
        kidx = torch.full((w.batch, hkv, budget), -5, dtype=torch.int32, device="cuda")
        out = torch.empty((w.batch, hq, 128), dtype=torch.float32, device="cuda")
        knew, vnew, q = dev(d["step_k"][0]), dev(d["step_v"][0]), dev(d["step_q"][0])
        if path == "calls":
            kvc.kvc_append_decode_attn(gc, knew, vnew, q, out, h2o_score=score)
            kvc.kvc_h2o_evict(gc, score, budget, S16, R16, kidx, dst, dsc)
        else:
            kvc.kvc_decode_step(gc, knew, vnew, q, out, score, budget, S16, R16, kidx, dst, dsc)
        torch.cuda.synchronize()
        res.append((gc, dst, dsc, kidx, out))
    (gA, dA, sA, kA, oA), (gB, dB, sB, kB, oB) = res
    assert torch.equal(oA, oB) and torch.equal(kA, kB) and torch.equal(sA, sB)
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "positions", "lengths", "num_seen"):
        assert torch.equal(getattr(dA, name), getattr(dB, name)), name
    for name in ("k_sink16", "v_sink16", "k_recent16", "v_recent16"):
        assert torch.equal(getattr(gA, name), getattr(gB, name)), name
    ref = oracle.RefCache(w.batch, hkv, 128, cap, bits, fp16_sinks=S16, fp16_recent=R16)
    ref.append(d["k"][:, :, :P + 1], d["v"][:, :, :P + 1])
    ro, _ = ref.attend(d["step_q"][0])
    assert_out_close(host(oB), ro)


@pytest.mark.parametrize("bits,hq,hkv", [(8, 8, 4), (4, 16, 2)])
def test_tier_paged_equals_contiguous(bits, hq, hkv):
    """A paged tiered cache (blocks in a seeded random order) attends exactly
    as a contiguous tiered cache holding the same tokens: output and H2O
    scores bit for bit, on the separate calls and on the fused append; the
    contiguous side is the one the oracle checks above."""
    L, D, S16, R16, bs = 700, 128, 4, 80, 16
    print(f"[tiers paged] bits={bits} hq={hq} hkv={hkv}", flush=True)
    w = _workload(bits, hq, hkv, D, L, 2)
    d = draw(w)
    B, cap = w.batch, 736
    mb = cap // bs
    table = np.random.default_rng(7).permutation(B * mb).astype(np.int32).reshape(B, mb)
    pg = kvc.KVCache(B, hkv, D, 0, bits, block_size=bs, num_blocks=B * mb, max_blocks_per_seq=mb, fp16_sinks=S16,
                     fp16_recent=R16)
    pg.block_table.copy_(dev(table))
    ct = _tiered(w, cap, 0, S16, R16)
    res = []
    for c in (pg, ct):
        score = c.score_buffer()
        kvc.kvc_quant_append(c, dev(d["k"][:, :, :L]), dev(d["v"][:, :, :L]), h2o_score=score)
        out1 = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
        kvc.kvc_decode_attn(c, dev(d["q"]), out1, h2o_score=score)
        out2 = torch.empty_like(out1)
        kvc.kvc_append_decode_attn(c, dev(d["step_k"][1]), dev(d["step_v"][1]), dev(d["step_q"][1]), out2,
                                   h2o_score=score)
        torch.cuda.synchronize()
        res.append((out1, out2, score))
    (a1, a2, sa), (b1, b2, sb) = res
    assert torch.equal(a1, b1) and torch.equal(a2, b2) and torch.equal(sa, sb)
    for name in ("k_sink16", "v_sink16", "k_recent16", "v_recent16", "lengths", "num_seen"):
        assert torch.equal(getattr(pg, name), getattr(ct, name)), name


@pytest.mark.parametrize("path", ["separate", "fused"])
def test_int4_hybrid_llama7b_full_size(path):
    """The benchmarked hybrid layer at full size: INT4 codes, 32 heads,
    D = 128, 8192 tokens, 4 fp16 sinks and the newest int(0.3 L) = 2457 tokens
    at fp16 (39 tier parts per row), one attention call with H2O (the
    benchmark's call and length hint on the separate path); every head
    checked. "fused" appends the 8192nd token inside the attention call (its
    rows go to the ring there)."""
    w = get("llama7b_8k").scaled(bits=4)
    d = draw(w)
    L, S16, R16 = w.context, 4, int(0.3 * w.context)
    print(f"[tiers] INT4 hybrid full size, path={path}", flush=True)
    gc = _tiered(w, L, 0, S16, R16)
    score = gc.score_buffer()
    ref = oracle.RefCache(w.batch, w.num_kv_heads, w.head_dim, L, 4, fp16_sinks=S16, fp16_recent=R16)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    if path == "separate":
        kvc.kvc_quant_append(gc, dev(d["k"]), dev(d["v"]), h2o_score=score)
        kvc.kvc_decode_attn(gc, dev(d["q"]), out, h2o_score=score, max_len_hint=L)
    else:
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :L - 1]), dev(d["v"][:, :, :L - 1]), h2o_score=score)
        kvc.kvc_append_decode_attn(gc, dev(d["k"][:, :, L - 1:]), dev(d["v"][:, :, L - 1:]), dev(d["q"]), out,
                                   h2o_score=score)
    ref.append(d["k"], d["v"])
    ro, _ = ref.attend(d["q"])
    torch.cuda.synchronize()
    assert_codes_equal(gc, ref)
    _check_tier_rows(gc, ref, S16, R16)
    err = assert_out_close(host(out), ro)
    rel = assert_scores_close(host(score), ref.score, ref.lengths)
    print(f"max-abs out err {err:.2e}, worst score rel err {rel:.2e}", flush=True)


@pytest.mark.parametrize("hq,R16", [(8, 64), (4, 0)])  # (4, 0): one head per KV head, sinks only (folded tier)
@pytest.mark.parametrize("L", [1, 3, 4, 5, 66])
def test_tier_short_rows_fused_append(L, hq, R16):
    """The fused append + attention when the appended token is itself a sink
    (L <= fp16_sinks = 4) or the row is just past the sinks: the new token's
    rows come from k_new / v_new and go to the tiers in the same call. With
    one query head per KV head and the sinks alone, the tier is a single part
    that the split kernel computes itself."""
    print(f"[tier short fused] L={L} hq={hq} R16={R16}", flush=True)
    w = _workload(8, hq, 4, 128, L, 2)
    d = draw(w)
    gc = _tiered(w, L + 4, 0, 4, R16)
    score = gc.score_buffer()
    ref = oracle.RefCache(w.batch, 4, 128, L + 4, 8, fp16_sinks=4, fp16_recent=R16)
    if L > 1:
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :L - 1]), dev(d["v"][:, :, :L - 1]), h2o_score=score)
        ref.append(d["k"][:, :, :L - 1], d["v"][:, :, :L - 1])
    out = torch.empty((w.batch, hq, 128), dtype=torch.float32, device="cuda")
    kvc.kvc_append_decode_attn(gc, dev(d["k"][:, :, L - 1:L]), dev(d["v"][:, :, L - 1:L]), dev(d["q"]), out,
                               h2o_score=score)
    ref.append(d["k"][:, :, L - 1:L], d["v"][:, :, L - 1:L])
    ro, _ = ref.attend(d["q"])
    torch.cuda.synchronize()
    _check_tier_rows(gc, ref, 4, R16)
    assert_out_close(host(out), ro)
    assert_scores_close(host(score), ref.score, ref.lengths)
