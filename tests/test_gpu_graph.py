"""Captured-graph replays of the benchmarked calls equal their eager results.

``bench.py`` times the calls as HIP graph replays. Here each call is captured
once, its inputs restored by ordinary (eager) copies before every replay, and
each of three replays must reproduce the eager call's outputs and cache
state bit for bit: the one-call decode step (split kernel, then the
eviction kernel with the merge), the fused append + attention on a tiered
INT4 cache (split, tier and merge kernels) and on a plain INT8 cache (also
replayed three times in a row), and on a paged cache the attention with H2O
and the block eviction.
"""
import numpy as np
import pytest

from workloads import draw, get

from kvc_testlib import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
kvc = pytest.importorskip("compressed_kv_cache_kvc_amd")

STATE = ("k_codes", "v_codes", "k_scale", "v_scale", "positions", "lengths", "num_seen",
         "k_sink16", "v_sink16", "k_recent16", "v_recent16")


def _state(c):
    return {n: getattr(c, n) for n in STATE if getattr(c, n, None) is not None and getattr(c, n).numel() > 0}


def _replays_match(call, restore, outputs, n=3):
    """Eager call, capture, then n replays, each after restore(); every
    replay's outputs (a dict of tensors) must equal the eager ones."""
    restore()
    call()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in outputs.items()}
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for r in range(n):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in outputs.items():
            assert torch.equal(t, ref[k]), f"replay {r}: {k} differs from the eager call"
    del g


def _workload(bits, hq, hkv, P):
    return get("qwen_gqa_stream").scaled(batch=2, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, bits=bits,
                                        context=P + 1, steps=2)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2)])
def test_decode_step_graph_replays(hq, hkv):
    P, budget, S, R = 900, 600, 4, 96
    print(f"[graph] decode step hq={hq} hkv={hkv}", flush=True)
    w = _workload(8, hq, hkv, P)
    d = draw(w)
    B, D, cap = w.batch, 128, P + 8
    gc = kvc.KVCache(B, hkv, D, cap, 8)
    score = gc.score_buffer()
    kvc.kvc_quant_append(gc, dev(d["k"][:, :, :P]), dev(d["v"][:, :, :P]), h2o_score=score)
    torch.cuda.synchronize()
    saved = {n: t.clone() for n, t in _state(gc).items()}
    saved_score = score.clone()
    dst = kvc.KVCache(B, hkv, D, cap, 8)
    dsc = dst.score_buffer()
    kidx = torch.zeros((B, hkv, budget), dtype=torch.int32, device="cuda")
    out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    knew, vnew, q = dev(d["step_k"][0]), dev(d["step_v"][0]), dev(d["step_q"][0])
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(gc, hq, P + 1, True), dtype=torch.uint8, device="cuda")

    def call():
        kvc.kvc_decode_step(gc, knew, vnew, q, out, score, budget, S, R, kidx, dst, dsc, max_len_hint=P,
                            workspace=ws)

    def restore():
        for n, t in _state(gc).items():
            t.copy_(saved[n])
        score.copy_(saved_score)
        for t in _state(dst).values():
            t.zero_()
        dsc.zero_()
        kidx.fill_(-1)
        out.zero_()

    outputs = {"out": out, "keep_index": kidx, "dst_score": dsc, "score": score,
               **{"src." + n: t for n, t in _state(gc).items()}, **{"dst." + n: t for n, t in _state(dst).items()}}
    _replays_match(call, restore, outputs)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 2)])
def test_tiered_append_attention_graph_replays(hq, hkv):
    P, S16, R16 = 700, 4, 100
    print(f"[graph] tiered INT4 append + attention hq={hq} hkv={hkv}", flush=True)
    w = _workload(4, hq, hkv, P)
    d = draw(w)
    B, D, cap = w.batch, 128, P + 8
    gc = kvc.KVCache(B, hkv, D, cap, 4, fp16_sinks=S16, fp16_recent=R16)
    score = gc.score_buffer()
    kvc.kvc_quant_append(gc, dev(d["k"][:, :, :P]), dev(d["v"][:, :, :P]), h2o_score=score)
    torch.cuda.synchronize()
    saved = {n: t.clone() for n, t in _state(gc).items()}
    saved_score = score.clone()
    out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    knew, vnew, q = dev(d["step_k"][0]), dev(d["step_v"][0]), dev(d["step_q"][0])
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(gc, hq, P + 1, True), dtype=torch.uint8, device="cuda")

    def call():
        kvc.kvc_append_decode_attn(gc, knew, vnew, q, out, h2o_score=score, max_len_hint=P, workspace=ws)

    def restore():
        for n, t in _state(gc).items():
            t.copy_(saved[n])
        score.copy_(saved_score)
        out.zero_()

    outputs = {"out": out, "score": score, **{"cache." + n: t for n, t in _state(gc).items()}}
    _replays_match(call, restore, outputs)
    assert np.isfinite(out.cpu().numpy()).all()


def test_append_attention_graph_replays_in_a_row():
    """The append + attention at one query head per KV head captured once:
    replays after a restore equal the eager call, and three replays in a row
    equal three eager calls (the lengths advance once per replay)."""
    P, hq = 900, 8
    print("[graph] append + attention, replays in a row", flush=True)
    w = _workload(8, hq, hq, P)
    d = draw(w)
    B, D, cap = w.batch, 128, P + 8
    gc = kvc.KVCache(B, hq, D, cap, 8)
    score = gc.score_buffer()
    kvc.kvc_quant_append(gc, dev(d["k"][:, :, :P]), dev(d["v"][:, :, :P]), h2o_score=score)
    torch.cuda.synchronize()
    saved = {n: t.clone() for n, t in _state(gc).items()}
    saved_score = score.clone()
    out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    knew, vnew, q = dev(d["step_k"][0]), dev(d["step_v"][0]), dev(d["step_q"][0])
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(gc, hq, P + 4, True), dtype=torch.uint8, device="cuda")

    def call():
        kvc.kvc_append_decode_attn(gc, knew, vnew, q, out, h2o_score=score, max_len_hint=P + 2, workspace=ws)

    def restore():
        for n, t in _state(gc).items():
            t.copy_(saved[n])
        score.copy_(saved_score)
        out.zero_()

    outputs = {"out": out, "score": score, **{"cache." + n: t for n, t in _state(gc).items()}}
    _replays_match(call, restore, outputs)

    # Three in a row, eager, then as replays of one captured call.
    restore()
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in outputs.items()}
    assert ref["cache.lengths"].tolist() == [P + 3] * B
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    restore()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    for k, t in outputs.items():
        assert torch.equal(t, ref[k]), f"three replays: {k} differs from three eager calls"
    del g


def test_paged_attention_and_block_evict_graph_replays():
    """The paged cache's attention with H2O (split kernel on the page table,
    then the merge) and its block eviction (block means, then the table
    rewrite and score move), each captured and replayed."""
    B, hq, hkv, D, L, bs = 4, 8, 4, 128, 600, 16
    print("[graph] paged attention and block eviction", flush=True)
    w = _workload(8, hq, hkv, L).scaled(batch=B)
    d = draw(w)
    mb = (L + 8 + bs - 1) // bs
    table = np.random.default_rng(5).permutation(B * mb).astype(np.int32).reshape(B, mb)
    pg = kvc.KVCache(B, hkv, D, 0, 8, block_size=bs, num_blocks=B * mb, max_blocks_per_seq=mb)
    pg.block_table.copy_(dev(table))
    score = pg.score_buffer()
    kvc.kvc_quant_append(pg, dev(d["k"][:, :, :L]), dev(d["v"][:, :, :L]), h2o_score=score)
    torch.cuda.synchronize()
    saved_score = score.clone()
    out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    q = dev(d["step_q"][0])
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(pg, hq, L, True), dtype=torch.uint8, device="cuda")

    def attend():
        kvc.kvc_decode_attn(pg, q, out, h2o_score=score, max_len_hint=L, workspace=ws)

    def restore_attend():
        score.copy_(saved_score)
        out.zero_()

    _replays_match(attend, restore_attend, {"out": out, "score": score})

    # Block eviction on scores with spread (one attention step's mass is
    # nearly flat): seeded random scores.
    score.copy_(torch.from_numpy(np.random.default_rng(6).random((B, hkv, pg.capacity)).astype(np.float32)))
    dst = pg.table_view()
    dsc = torch.zeros_like(score)
    freed = torch.zeros((B, mb), dtype=torch.int32, device="cuda")
    fcount = torch.zeros((B,), dtype=torch.int32, device="cuda")
    wsb = torch.empty(kvc.kvc_paged_block_evict_workspace_bytes(pg), dtype=torch.uint8, device="cuda")

    def evict():
        kvc.kvc_paged_block_evict(pg, score, 0.6, dst, dsc, freed, fcount, max_len_hint=L, workspace=wsb)

    def restore_evict():
        dst.block_table.fill_(-1)
        dst.lengths.zero_()
        dst.num_seen.zero_()
        dsc.fill_(-3.0)
        freed.fill_(-9)
        fcount.fill_(-1)

    _replays_match(evict, restore_evict, {"table": dst.block_table, "lengths": dst.lengths, "num_seen": dst.num_seen,
                                          "dst_score": dsc, "freed": freed, "freed_count": fcount})
    assert int(fcount.min()) > 0
