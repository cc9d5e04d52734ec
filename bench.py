"""Benchmark: one decode step of compressed-KV attention on one MI355X.

A step is one pass of the whole hot path over one layer of the LLaMA-7B-shaped
workload (B=1, 32 query/KV heads, D=128, 8192 tokens, INT8 per-token cache,
H2O keep 0.3 = 4 sinks + 1024 recent + 1429 heavy hitters):

  1. quantize-append the new token's K and V,
  2. attention over all 8192 tokens + H2O accumulation,
  3. eviction: keep-set selection down to 2457 slots (a mask and an
     ascending keep list) and compaction of the kept slots into the other
     buffer.

Steps rotate over 32 distinct layer caches (2.1 GiB, like the 32 layers of the
model), so every launch streams its 66 MiB from HBM rather than from the
256 MB Infinity Cache. Inputs are resident in HBM before timing starts.

Exactly --warmup untimed steps, then exactly --steps timed steps, in decode
order (layer 0, 1, ..., 31, 0, ...), twice:

  * as the one-call step (kvc_decode_step: the split attention kernel with
    the append, then the eviction kernel that also merges the splits):
    `ms_per_step` and `tokens_per_s`;
  * as the separate calls (kvc_decode_attn_split with the append,
    kvc_decode_attn_merge with H2O, kvc_h2o_evict), with HIP events between
    the phases: `value` is decode attention's KV GB/s, the attention's
    algorithmic bytes (KV codes and scales, q, out) over the split and merge
    phases' time; `phases` gives each phase; `roofline` is the split kernel,
    the step's dominant HBM kernel, alone.

Steps are replayed from HIP graphs of up to 32 layer-steps each (a block of
fewer layers covers a step count that is not a multiple of 32).

Prints one JSON line. Run ``python bench.py --help`` for options.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s & tokens/s (fraction of HBM peak), INT8, L=8192, 1 GPU"

# HBM bytes one launch of the split attention kernel moves on this workload,
# from rocprofv3 FETCH_SIZE and WRITE_SIZE passes scaled by the same counters
# on a plain 64 MiB device copy. The figure holds only for the attention
# sources it was taken on; any change to them reports null.
TRAFFIC_SOURCES = ("compressed_kv_cache_kvc_amd/csrc/decode_attn.hip",
                   "compressed_kv_cache_kvc_amd/csrc/kvc_internal.h",
                   "compressed_kv_cache_kvc_amd/csrc/quant_row.h",
                   "compressed_kv_cache_kvc_amd/csrc/merge.h",
                   "compressed_kv_cache_kvc_amd/csrc/tiers.h",
                   "compressed_kv_cache_kvc_amd/csrc/api.hip")
# FETCH_SIZE 33,915.7 KiB x 1.9993 + WRITE_SIZE 1,308.09 KiB per launch
# on the LLaMA-7B layer, with the copy calibration above.
TRAFFIC_SHA256 = "5807953937d734d32ac098c75ee72e66f4ecd0b5b2b23c1981bfdca1919e3702"
TRAFFIC_BYTES = 70774469


def attention_traffic():
    return TRAFFIC_BYTES if TRAFFIC_SHA256 is not None and traffic_sources_sha256() == TRAFFIC_SHA256 else None


def traffic_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


HBM_PEAK_GBPS = 8000.0
LAYERS = 32


def step_bytes(B, Hq, H, D, bits, L, budget):
    """Algorithmic bytes of one step, by part (what the method must move)."""
    rb = D * bits // 8
    kv = B * H * L * 2 * (rb + 4)                        # codes + fp32 scales, K and V
    parts = {
        "append": B * H * (2 * D * 2 + 2 * (rb + 4) + 4 + 4),   # fp16 in; codes, scales, position, score out
        "attention": kv + B * Hq * D * 2,                       # KV + q (fp16)
        "out": B * Hq * D * 4,                                  # out (fp32)
        "h2o": 2 * B * H * L * 4,                                # score read-modify-write
        # scores in; mask and keep list out; kept rows (codes, scales, position, score) in and out
        "evict": B * H * (L * 4 + L + budget * 4) + 2 * B * H * budget * (2 * (rb + 4) + 8),
    }
    # The split kernel's own algorithmic bytes (KV + q), and decode
    # attention's (KV + q + out: what the split and merge kernels must move).
    return parts, kv + B * Hq * D * 2, kv + B * Hq * D * 2 + B * Hq * D * 4


def phase_table(phase_ms, steps, parts, attn_alg):
    """Per-phase time and HBM roofline fraction of one step. Each phase is one
    replayed graph (one launch per layer buffer) timed with events on the
    replay stream; bytes are the phase's algorithmic bytes: the split kernel
    moves the append's inputs and cache writes, the KV stream and q (the
    roofline entry's bytes); the merge the H2O score read-modify-write and the
    output; eviction the selection's score reads, mask and keep-list writes
    and the compaction's kept rows in and out."""
    names = ("attention_split", "attention_merge", "evict")
    alg = (parts["append"] + attn_alg, parts["h2o"] + parts["out"], parts["evict"])
    table = {}
    for name, ms, b in zip(names, phase_ms, alg):
        us = ms * 1e3 / steps
        gbps = b / (us * 1e-6) / 1e9
        table[name] = {"us": round(us, 3), "bytes": int(b), "gbps": round(gbps, 1),
                       "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    return table


def cpu_baseline(w, d, budget_s=12.0):
    """Time the fp64 oracle (unchanged) on the host on the same workload: one
    full step (append, attention + H2O, select, compact), repeated until about
    ``budget_s`` seconds have passed, then the attention alone (with H2O) on
    the same cache for about a third of that."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    B, H, D, L = w.batch, w.num_kv_heads, w.head_dim, w.context
    ref = oracle.RefCache(B, H, D, L, w.bits)
    ref.append(d["k"][:, :, :L - 1], d["v"][:, :, :L - 1])
    snap = (ref.k_codes.copy(), ref.v_codes.copy(), ref.k_scale.copy(), ref.v_scale.copy(),
            ref.positions.copy(), ref.lengths.copy(), ref.num_seen.copy())
    times = []
    t_total = time.perf_counter()
    while True:
        (ref.k_codes[:], ref.v_codes[:], ref.k_scale[:], ref.v_scale[:], ref.positions[:],
         ref.lengths[:], ref.num_seen[:]) = snap
        ref.score[:] = 0
        t0 = time.perf_counter()
        ref.step(d["q"], d["k"][:, :, L - 1:], d["v"][:, :, L - 1:], budget=w.budget, n_sink=w.n_sink,
                 n_recent=w.n_recent)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_total > budget_s or len(times) >= 20:
            break
    # Attention alone: the cache with the new token appended, no eviction.
    (ref.k_codes[:], ref.v_codes[:], ref.k_scale[:], ref.v_scale[:], ref.positions[:],
     ref.lengths[:], ref.num_seen[:]) = snap
    ref.append(d["k"][:, :, L - 1:], d["v"][:, :, L - 1:])
    attn = []
    t_total = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        ref.attend(d["q"], h2o=True)
        attn.append(time.perf_counter() - t0)
        if time.perf_counter() - t_total > budget_s / 3 or len(attn) >= 20:
            break
    return min(times), len(times), min(attn), len(attn), cores


def copy_calibration(torch, mib):
    """Eight copies of ``mib`` MiB between two device buffers: each launch
    reads and writes exactly ``mib`` MiB, so per-dispatch FETCH_SIZE and
    WRITE_SIZE of this kernel give the counters' scale in bytes."""
    torch.cuda.set_device(0)
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(8):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / 8
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "us_per_copy": round(us, 2),
                      "gbps_read_plus_write": round(2 * n / (us * 1e-6) / 1e9, 1)}))
    return 0


def layer_schedules(kvc, torch, caches, scores, lengths_all, k_new, v_new, q, out, dst, dst_score, ws, L, S, R,
                    stream, blocks):
    """The decode-order step with per-layer budgets from the pyramid schedules
    (kvc_layer_budgets, base = the context, floor = sinks + window): layer i
    of the 32 keeps budgets[i] tokens. Time per layer-step over the same
    number of 32-layer blocks as the headline."""
    B, H = caches[0].batch, caches[0].num_kv_heads
    lists = [torch.zeros((B, H, L), dtype=torch.int32, device="cuda") for _ in range(LAYERS)]
    res = {}
    for name, sched, ratio in (("linear", kvc.KVC_SCHEDULE_LINEAR, 0.0), ("quadratic", kvc.KVC_SCHEDULE_QUADRATIC, 0.2)):
        budgets = kvc.kvc_layer_budgets(sched, LAYERS, L, ratio, S + R)

        def block():
            lengths_all.fill_(L - 1)
            for i in range(LAYERS):
                kvc.kvc_decode_step(caches[i], k_new, v_new, q, out, scores[i], budgets[i], S, R, lists[i], dst,
                                    dst_score, max_len_hint=L - 1, workspace=ws)

        with torch.cuda.stream(stream):
            block()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            block()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(blocks):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        res[name] = {"ratio": ratio if sched == kvc.KVC_SCHEDULE_QUADRATIC else None,
                     "budget_first_layer": budgets[0], "budget_last_layer": budgets[-1],
                     "mean_budget": round(sum(budgets) / LAYERS, 1),
                     "us_per_step": round(e0.elapsed_time(e1) * 1e3 / (blocks * LAYERS), 3)}
        del g
    return res


def read_probe(kvc, torch, nbytes, blocks=4):
    """HBM read ceiling of one launch: kvc_bw_probe over 32 buffers of the
    attention's KV size in turn (so every launch reads from HBM, as the
    attention does), replayed as one graph per 32 launches."""
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(LAYERS)]
    sink = torch.empty(kvc.kvc_bw_probe_sink_bytes(), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for buf in bufs:
            kvc.kvc_bw_probe(buf, sink)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for buf in bufs:
            kvc.kvc_bw_probe(buf, sink)
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(blocks):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (blocks * LAYERS)
    del bufs, g
    torch.cuda.empty_cache()
    return {"kernel": "bw_probe_kernel (kvc_bw_probe)", "bytes_per_launch": nbytes, "us": round(us, 3),
            "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}


def secondary_attention(kvc, torch, reps=16):
    """Decode-attention throughput of the other workloads at full size, as KV
    GB/s of algorithmic bytes (codes + scales + q) and the fraction of the
    8 TB/s peak. Cache contents are random device data quantized by the library
    (timing does not depend on the values); the paged lengths follow the
    paged workload's seeded lengths, its block table a seeded permutation.
    Caches that fit the 256 MB Infinity Cache are rotated. Launches are timed
    as replays of a captured graph."""
    from workloads import get
    res = {}

    def timed(launch, n_bufs, n=None):
        # n launches (buffers in turn) captured as one graph and replayed
        # twice, so host launch cost does not enter the device time.
        n = n or reps
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for i in range(3):
                launch(i % n_bufs)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                launch(i % n_bufs)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / (2 * n)

    def report(name, w, kv_bytes, us, extra):
        gbps = kv_bytes / (us * 1e-6) / 1e9
        res[name] = {"workload": name, "us_per_launch": round(us, 2), "kv_bytes": int(kv_bytes),
                     "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4), **extra}

    # Paged batch: 32 sequences, 16-token INT8 blocks, no H2O.
    w = get("paged_b32")
    B, H, D, bs = w.batch, w.num_kv_heads, w.head_dim, w.paged_block
    lengths = np.random.default_rng([w.seed, 1]).integers(w.len_lo, w.len_hi, endpoint=True, size=B)
    nblk = [(int(n) + bs - 1) // bs for n in lengths]
    perm = np.random.default_rng(w.seed).permutation(sum(nblk)).astype(np.int32)
    table = np.full((B, max(nblk)), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    gc = kvc.KVCache(B, H, D, 0, 8, block_size=bs, num_blocks=int(sum(nblk)), max_blocks_per_seq=table.shape[1])
    gc.block_table.copy_(torch.from_numpy(table).cuda())
    for b in range(B):
        one = kvc.KvcCacheDesc.from_buffer_copy(gc.desc)
        one.batch = 1
        one.block_table = gc.block_table[b].data_ptr()
        one.lengths = gc.lengths[b:b + 1].data_ptr()
        one.num_seen = gc.num_seen[b:b + 1].data_ptr()
        kv = torch.randn((2, 1, H, int(lengths[b]), D), device="cuda").half()
        kvc.kvc_quant_append(one, kv[0], kv[1], max_len_hint=0)
    q = torch.randn((B, w.num_q_heads, D), device="cuda").half()
    out = torch.empty((B, w.num_q_heads, D), dtype=torch.float32, device="cuda")
    hint = int(lengths.max())
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(gc, w.num_q_heads, hint, False), dtype=torch.uint8,
                     device="cuda")
    us = timed(lambda i: kvc.kvc_decode_attn(gc, q, out, max_len_hint=hint, workspace=ws), 1)
    report("paged_b32", w, int(lengths.sum()) * H * 2 * (D + 4) + q.numel() * 2, us,
           {"tokens": int(lengths.sum()), "h2o": False})
    # Block-granular eviction of the same batch (retention 0.5): one launch
    # over random scores, the table rewritten into a view of the same pools.
    sc = torch.rand((B, H, gc.capacity), device="cuda")
    dv, dsc = gc.table_view(), torch.empty((B, H, gc.capacity), device="cuda")
    freed = torch.empty((B, gc.max_blocks_per_seq), dtype=torch.int32, device="cuda")
    fcount = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws_be = torch.empty(kvc.kvc_paged_block_evict_workspace_bytes(gc), dtype=torch.uint8, device="cuda")
    us_be = timed(lambda i: kvc.kvc_paged_block_evict(gc, sc, 0.5, dv, dsc, freed, fcount, max_len_hint=hint,
                                                      workspace=ws_be), 1)
    res["paged_b32_block_evict"] = {"workload": "paged_b32", "us_per_launch": round(us_be, 2), "retention": 0.5,
                                    "blocks": int(sum(nblk)), "blocks_freed": int(fcount.sum().item()),
                                    "score_bytes_moved": int(2 * 4 * H * (int(lengths.sum()) // 2))}
    del sc, dv, dsc, freed, fcount, ws_be
    del gc, ws
    torch.cuda.empty_cache()

    # GQA steady state (8193 tokens, 28/4 heads) and the 70B INT4 layer, H2O on.
    for name, L, n_bufs in (("qwen_gqa_stream", 8193, 8), ("llama70b_int4", 131072, 1)):
        w = get(name)
        B, Hq, H, D = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
        caches, scores = [], []
        for i in range(n_bufs):
            c = kvc.KVCache(B, H, D, L, w.bits)
            kv = torch.randn((2, B, H, L, D), device="cuda").half()
            kvc.kvc_quant_append(c, kv[0], kv[1], max_len_hint=0)
            del kv
            caches.append(c)
            scores.append(c.score_buffer())
        q = torch.randn((B, Hq, D), device="cuda").half()
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(caches[0], Hq, L, True), dtype=torch.uint8,
                         device="cuda")
        us = timed(lambda i: kvc.kvc_decode_attn(caches[i], q, out, h2o_score=scores[i], max_len_hint=L,
                                                 workspace=ws), n_bufs)
        report(name, w, B * H * L * 2 * (D * w.bits // 8 + 4) + q.numel() * 2, us,
               {"tokens": B * L, "h2o": True, "bits": w.bits, "q_heads": Hq, "kv_heads": H})
        del caches, scores, ws
        torch.cuda.empty_cache()

    # The LLaMA-7B layer with fp16 tiers, next to the same layer without: the
    # report's fp16 sinks on an INT8 cache (4 sinks), and the tutorial's hybrid
    # (INT4 codes, 4 fp16 sinks and the newest int(0.3 L) tokens at fp16). One
    # whole attention call (split, tier and merge kernels) with H2O, over 32
    # rotated layer buffers. Bytes: codes + scales of the coded slots, fp16
    # rows of the tier slots, and q.
    w = get("llama7b_8k")
    B, Hq, H, D, L = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.context
    n_bufs = 32
    for name, bits, s16, r16 in (("llama7b_8k_no_tiers", 8, 0, 0), ("llama7b_8k_fp16_sinks", 8, 4, 0),
                                 ("llama7b_8k_int4_hybrid", 4, 4, int(0.3 * L))):
        caches, scores = [], []
        for i in range(n_bufs):
            c = kvc.KVCache(B, H, D, L, bits, fp16_sinks=s16, fp16_recent=r16)
            kv = torch.randn((2, B, H, L, D), device="cuda").half()
            kvc.kvc_quant_append(c, kv[0], kv[1], max_len_hint=0)
            del kv
            caches.append(c)
            scores.append(c.score_buffer())
        q = torch.randn((B, Hq, D), device="cuda").half()
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(caches[0], Hq, L, True), dtype=torch.uint8,
                         device="cuda")
        us = timed(lambda i: kvc.kvc_decode_attn(caches[i], q, out, h2o_score=scores[i], max_len_hint=L,
                                                 workspace=ws), n_bufs, 64)
        tier = min(s16 + r16, L)
        kv_bytes = B * H * 2 * ((L - tier) * (D * bits // 8 + 4) + tier * D * 2) + q.numel() * 2
        report(name, w, kv_bytes, us, {"tokens": B * L, "h2o": True, "bits": bits, "fp16_sinks": s16,
                                       "fp16_recent": r16, "calls": "kvc_decode_attn (split, tiers, merge)"})
        del caches, scores, ws
        torch.cuda.empty_cache()

    # K/V-separated attention on the same layer: top_k = the 2457-token keep
    # budget per KV head, cold V rows read by the device from pinned host
    # memory; with no tiers every kept row is cold, with 4 fp16 sinks and a
    # 1024-token fp16 window those rows are hot (on the GPU). Timed eagerly:
    # each call is hundreds of microseconds of host-link reads.
    top_k = w.budget
    for name, s16, r16 in (("llama7b_8k_kvsep_all_cold", 0, 0), ("llama7b_8k_kvsep_hot_window", 4, 1024)):
        c = kvc.KVCache(B, H, D, L, 8, fp16_sinks=s16, fp16_recent=r16)
        kv = torch.randn((2, B, H, L, D), device="cuda").half()
        kvc.kvc_quant_append(c, kv[0], kv[1], max_len_hint=0)
        v_host = kv[1].cpu().pin_memory()
        del kv
        q = torch.randn((B, Hq, D), device="cuda").half()
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(kvc.kvc_decode_attn_kvsep_workspace_bytes(c, Hq, top_k, L), dtype=torch.uint8,
                         device="cuda")
        for _ in range(2):
            kvc.kvc_decode_attn_kvsep(c, q, top_k, v_host, out, max_len_hint=L, workspace=ws)
        torch.cuda.synchronize()
        n = 8
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            kvc.kvc_decode_attn_kvsep(c, q, top_k, v_host, out, max_len_hint=L, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        # at least top_k - (sinks + window) kept rows per KV head come from the host
        cold_rows = B * H * max(0, top_k - (s16 + r16))
        res[name] = {"workload": name, "us_per_launch": round(us, 2), "top_k": top_k, "fp16_sinks": s16,
                     "fp16_recent": r16, "kv_bytes_scored": int(B * H * L * (D + 4)),
                     "host_v_bytes_at_least": int(cold_rows * D * 2),
                     "calls": "kvc_decode_attn_kvsep (clear, split, merge, select, gather)"}
        del c, v_host, ws
        torch.cuda.empty_cache()

    # The GQA stream's whole decode step in steady state (c4 after its first
    # step): 8 sequences of 8192 kept tokens, append the new one, attend with
    # H2O over 8193, evict back to 8192 (4 sinks + 2048 recent + 6140 heavy),
    # one kvc_decode_step per step. In place (the cache as its destination):
    # the split kernel, then one launch that merges, selects and moves only
    # the tokens past the evicted one; out of place (into one other cache):
    # split, merge and the one-launch eviction copying every kept token.
    # 8 rotated caches share one lengths array, so a fill rewinds all of them
    # once per 8 steps; the fill is inside the timed graph.
    w = get("qwen_gqa_stream")
    B, Hq, H, D = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    Lk, n_bufs = w.budget, 8
    lengths_q = torch.zeros((n_bufs, B), dtype=torch.int32, device="cuda")
    seen_q = torch.zeros((n_bufs, B), dtype=torch.int32, device="cuda")
    caches, scores = [], []
    for i in range(n_bufs):
        c = kvc.KVCache(B, H, D, Lk + 1, w.bits)
        c.lengths, c.num_seen = lengths_q[i], seen_q[i]
        c.desc = c._make_desc()
        kv = torch.randn((2, B, H, Lk, D), device="cuda").half()
        kvc.kvc_quant_append(c, kv[0], kv[1], max_len_hint=0)
        del kv
        caches.append(c)
        scores.append(c.score_buffer())
    dstq = kvc.KVCache(B, H, D, Lk + 1, w.bits)
    dsc = dstq.score_buffer()
    kidx = torch.empty((B, H, Lk), dtype=torch.int32, device="cuda")
    knew = torch.randn((B, H, 1, D), device="cuda").half()
    vnew = torch.randn((B, H, 1, D), device="cuda").half()
    q = torch.randn((B, Hq, D), device="cuda").half()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(caches[0], Hq, Lk + 1, True), dtype=torch.uint8,
                     device="cuda")

    def step(i, in_place):
        if i % n_bufs == 0:
            lengths_q.fill_(Lk)
            seen_q.fill_(Lk)
        c, sc = caches[i % n_bufs], scores[i % n_bufs]
        dst, dst_sc = (c, sc) if in_place else (dstq, dsc)
        kvc.kvc_decode_step(c, knew, vnew, q, out, sc, Lk, w.n_sink, w.n_recent, kidx, dst, dst_sc, max_len_hint=Lk,
                            workspace=ws)

    # launch(i) gets the running index
    lengths_q.fill_(Lk)
    seen_q.fill_(Lk)
    us = timed(lambda i: step(i, True), 1 << 30, 64)
    lengths_q.fill_(Lk)
    seen_q.fill_(Lk)
    us_oop = timed(lambda i: step(i, False), 1 << 30, 64)
    res["qwen_gqa_stream_step"] = {"workload": "qwen_gqa_stream", "us_per_step": round(us, 2),
                                   "tokens_per_s_per_layer": round(B / (us * 1e-6), 1),
                                   "kv_bytes_attended": int(B * H * (Lk + 1) * 2 * (D + 4)),
                                   "calls": "kvc_decode_step in place (append, attention + H2O, evict 8193 -> 8192; "
                                            "only tokens past the first evicted slot move)",
                                   "us_per_step_out_of_place": round(us_oop, 2)}
    del caches, scores, dstq, dsc, ws
    torch.cuda.empty_cache()
    return res


def kernel_case(kvc, torch, name, reps=16):
    """16 eager launches of one case of the GQA stream's steady state (8
    sequences, 28 query / 4 KV heads, 8193 tokens, H2O on) over 8 rotated
    caches, for a profiler's kernel trace and counters: `qwen_attention` is
    kvc_decode_attn (split, merge); `qwen_step_in_place` is kvc_decode_step
    with the cache as its own destination (split, in-place eviction)."""
    from workloads import get
    w = get("qwen_gqa_stream")
    B, Hq, H, D, Lk, n_bufs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.budget, 8
    L = Lk + 1
    lengths = torch.zeros((n_bufs, B), dtype=torch.int32, device="cuda")
    seen = torch.zeros((n_bufs, B), dtype=torch.int32, device="cuda")
    caches, scores = [], []
    for i in range(n_bufs):
        c = kvc.KVCache(B, H, D, L, w.bits)
        c.lengths, c.num_seen = lengths[i], seen[i]
        c.desc = c._make_desc()
        n = L if name == "qwen_attention" else Lk
        kv = torch.randn((2, B, H, n, D), device="cuda").half()
        kvc.kvc_quant_append(c, kv[0], kv[1], max_len_hint=0)
        del kv
        caches.append(c)
        scores.append(c.score_buffer())
    q = torch.randn((B, Hq, D), device="cuda").half()
    knew, vnew = torch.randn((B, H, 1, D), device="cuda").half(), torch.randn((B, H, 1, D), device="cuda").half()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    kidx = torch.empty((B, H, Lk), dtype=torch.int32, device="cuda")
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(caches[0], Hq, L, True), dtype=torch.uint8, device="cuda")

    def launch(i):
        c, sc = caches[i % n_bufs], scores[i % n_bufs]
        if name == "qwen_attention":
            kvc.kvc_decode_attn(c, q, out, h2o_score=sc, max_len_hint=L, workspace=ws)
        else:
            if i % n_bufs == 0:
                lengths.fill_(Lk)
                seen.fill_(Lk)
            kvc.kvc_decode_step(c, knew, vnew, q, out, sc, Lk, w.n_sink, w.n_recent, kidx, c, sc, max_len_hint=Lk,
                                workspace=ws)

    for i in range(n_bufs):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    return {"kernel_case": name, "launches": reps, "us_per_call": round(e0.elapsed_time(e1) * 1e3 / reps, 2)}


def _graph_time(torch, fn, stream, reps, before=None):
    """Capture fn() once, then time `reps` replays with events on `stream`
    (before() runs eagerly, untimed, ahead of each replay); returns the mean
    and the best replay in microseconds."""
    with torch.cuda.stream(stream):
        if before:
            before()
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    times = []
    for _ in range(reps):
        if before:
            with torch.cuda.stream(stream):
                before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del g
    return sum(times) / len(times), min(times)


def config_legs(kvc, torch):
    """The configured workloads' other legs, each as configured, at full size:
    the prefill append of the LLaMA-7B layer (8191 tokens); the Qwen GQA
    stream's whole 64-step loop from 32767 prefilled tokens (step 0 evicts
    32768 -> 8192, steps 1-63 evict one token per row); the 70B INT4 layer's
    whole step (append, attention with H2O, the two-launch selection of 24162
    of 129020 candidates per row, compaction). Cache contents are random
    device data quantized by the library (timing does not depend on the
    values); each timed region is a replayed graph, with caches restored
    before it, untimed."""
    from workloads import get
    res = {}
    stream = torch.cuda.Stream()

    # ---- a1: the prefill append of the LLaMA-7B layer ----
    w = get("llama7b_8k")
    B, H, D, L = w.batch, w.num_kv_heads, w.head_dim, w.context
    c = kvc.KVCache(B, H, D, L, 8)
    sc = c.score_buffer()
    kv = torch.randn((2, B, H, L - 1, D), device="cuda").half()
    mean_us, best_us = _graph_time(torch, lambda: kvc.kvc_quant_append(c, kv[0], kv[1], h2o_score=sc,
                                                                       max_len_hint=0),
                                   stream, 8, before=lambda: (c.lengths.zero_(), c.num_seen.zero_()))
    n = B * H * (L - 1)
    nbytes = n * 2 * D * 2 + n * 2 * (D + 4) + n * 8  # fp16 in; codes + scales, position + score out
    res["llama7b_8k_prefill_append"] = {
        "calls": "kvc_quant_append of 8191 tokens x 32 KV heads", "us": round(mean_us, 2),
        "bytes": nbytes, "gbps": round(nbytes / (mean_us * 1e-6) / 1e9, 1),
        "frac": round(nbytes / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    del c, sc, kv
    torch.cuda.empty_cache()

    # ---- c4: the Qwen GQA stream, 64 steps from 32767 prefilled tokens ----
    w = get("qwen_gqa_stream")
    B, Hq, H, D, L, steps = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.context, w.steps
    budget, S, R = w.budget, w.n_sink, w.n_recent
    ca, cb = kvc.KVCache(B, H, D, L, 8), kvc.KVCache(B, H, D, L, 8)
    sa, sb = ca.score_buffer(), cb.score_buffer()
    kv = torch.randn((2, B, H, L - 1, D), device="cuda").half()
    kvc.kvc_quant_append(ca, kv[0], kv[1], max_len_hint=0)
    del kv
    pristine = {f: getattr(ca, f).clone() for f in ("k_codes", "v_codes", "k_scale", "v_scale", "positions",
                                                     "lengths", "num_seen")}
    qs = torch.randn((steps, B, Hq, D), device="cuda").half()
    ks = torch.randn((steps, B, H, 1, D), device="cuda").half()
    vs = torch.randn((steps, B, H, 1, D), device="cuda").half()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    kidx = torch.empty((B, H, budget), dtype=torch.int32, device="cuda")
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(ca, Hq, L, True), dtype=torch.uint8, device="cuda")

    def restore():
        for f, t in pristine.items():
            getattr(ca, f).copy_(t)
        sa.zero_()

    def step(i, in_place):
        if in_place:  # the cache is its own destination: only tokens past the first evicted slot move
            src, ssrc, dst, sdst = ca, sa, ca, sa
        else:
            src, ssrc, dst, sdst = (ca, sa, cb, sb) if i % 2 == 0 else (cb, sb, ca, sa)
        hint = L - 1 if i == 0 else budget
        kvc.kvc_decode_step(src, ks[i], vs[i], qs[i], out, ssrc, budget, S, R, kidx, dst, sdst, max_len_hint=hint,
                            workspace=ws)

    for in_place, key in ((True, "qwen_gqa_stream_loop"), (False, "qwen_gqa_stream_loop_out_of_place")):
        def loop():
            for i in range(steps):
                step(i, in_place)

        loop_us, loop_best = _graph_time(torch, loop, stream, 3, before=restore)
        step0_us, _ = _graph_time(torch, lambda: step(0, in_place), stream, 3, before=restore)
        res[key] = {
            "calls": "64 x kvc_decode_step (append, attention + H2O over 32768 then 8193 tokens, evict to 8192), "
                     + ("in place (dst = the cache)" if in_place else "into the other of two caches"),
            "loop_us": round(loop_us, 1), "step0_us": round(step0_us, 1),
            "steady_step_us": round((loop_us - step0_us) / (steps - 1), 2),
            "tokens_per_s": round(B * steps / (loop_us * 1e-6), 1)}
    del ca, cb, sa, sb, pristine, ws
    torch.cuda.empty_cache()

    # ---- c5: the 70B INT4 layer's whole step ----
    w = get("llama70b_int4")
    B, Hq, H, D, L = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.context
    budget, S, R = w.budget, w.n_sink, w.n_recent
    src, dst = kvc.KVCache(B, H, D, L, 4), kvc.KVCache(B, H, D, L, 4)
    ssrc, sdst = src.score_buffer(), dst.score_buffer()
    for b in range(B):  # one sequence at a time keeps the fp16 staging at 1 GB
        one = kvc.KvcCacheDesc.from_buffer_copy(src.desc)
        one.batch = 1
        for f in ("k_codes", "v_codes", "k_scale", "v_scale", "positions", "lengths", "num_seen"):
            t = getattr(src, f)
            setattr(one, f, t[b:b + 1].data_ptr())
        kv = torch.randn((2, 1, H, L - 1, D), device="cuda").half()
        kvc.kvc_quant_append(one, kv[0], kv[1], max_len_hint=0)
        del kv
    q = torch.randn((B, Hq, D), device="cuda").half()
    kn, vn = torch.randn((B, H, 1, D), device="cuda").half(), torch.randn((B, H, 1, D), device="cuda").half()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    kidx = torch.empty((B, H, budget), dtype=torch.int32, device="cuda")
    ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(src, Hq, L, True), dtype=torch.uint8, device="cuda")

    def rewind():
        src.lengths.fill_(L - 1)
        src.num_seen.fill_(L - 1)

    def c5_step():
        rewind()
        kvc.kvc_decode_step(src, kn, vn, q, out, ssrc, budget, S, R, kidx, dst, sdst, max_len_hint=L - 1,
                            workspace=ws)

    def c5_evict():
        kvc.kvc_h2o_evict(src, ssrc, budget, S, R, kidx, dst, sdst, max_len_hint=L)

    step_us, _ = _graph_time(torch, c5_step, stream, 5)
    evict_us, _ = _graph_time(torch, c5_evict, stream, 5)
    kv_bytes = B * H * L * 2 * (D // 2 + 4) + q.numel() * 2 + out.numel() * 4
    res["llama70b_int4_step"] = {
        "calls": "kvc_decode_step (split, merge, selection, gather: 131072 -> 26214 per row)",
        "us": round(step_us, 1), "evict_us": round(evict_us, 1),
        "kv_bytes": int(kv_bytes), "tokens_per_s_per_layer": round(B / (step_us * 1e-6), 1)}
    del src, dst, ssrc, sdst, ws
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024, help="timed steps")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the attention-only measurements of the paged, GQA and INT4 workloads")
    ap.add_argument("--legs-only", action="store_true",
                    help="instead of the benchmark, run only the configured workloads' other legs (prefill append, "
                         "GQA stream loop, 70B INT4 step) and print them as one JSON line")
    ap.add_argument("--kernel-case", choices=("qwen_attention", "qwen_step_in_place"), default=None,
                    help="instead of the benchmark, run 16 launches of one GQA-stream case (8 rotated caches of "
                         "8193 tokens) for a profiler, and print their mean time")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the benchmark, run 8 plain device-to-device copies of this many MiB "
                         "(the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence and KV head with no communication between GPUs).",
              file=sys.stderr)
        return 2

    import torch
    if args.copy_mib:
        return copy_calibration(torch, args.copy_mib)
    import compressed_kv_cache_kvc_amd as kvc
    from workloads import draw, get

    torch.cuda.set_device(0)
    if args.kernel_case:
        print(json.dumps(kernel_case(kvc, torch, args.kernel_case)))
        return 0
    if args.legs_only:
        print(json.dumps({"config_legs": config_legs(kvc, torch)}))
        return 0
    w = get("llama7b_8k")
    d = draw(w)
    B, Hq, H, D, L, bits = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.context, w.bits
    budget, S, R = w.budget, w.n_sink, w.n_recent
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    # ---- device state: 32 layer caches, shared lengths so one fill rewinds all ----
    lengths_all = torch.zeros((LAYERS, B), dtype=torch.int32, device="cuda")
    seen_all = torch.zeros((LAYERS, B), dtype=torch.int32, device="cuda")
    caches, scores, masks, keep_lists = [], [], [], []
    k_pre, v_pre = dev(d["k"][:, :, :L - 1]), dev(d["v"][:, :, :L - 1])
    for i in range(LAYERS):
        c = kvc.KVCache(B, H, D, L, bits)
        c.lengths, c.num_seen = lengths_all[i], seen_all[i]
        c.desc = c._make_desc()
        kvc.kvc_quant_append(c, k_pre, v_pre, max_len_hint=0)
        caches.append(c)
        scores.append(c.score_buffer())
        masks.append(torch.zeros((B, H, L), dtype=torch.uint8, device="cuda"))
        keep_lists.append(torch.zeros((B, H, budget), dtype=torch.int32, device="cuda"))
    del k_pre, v_pre
    dst = kvc.KVCache(B, H, D, L, bits)
    dst_score = dst.score_buffer()
    k_new, v_new, q = dev(d["k"][:, :, L - 1:]), dev(d["v"][:, :, L - 1:]), dev(d["q"])
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws_attn = torch.zeros(kvc.kvc_decode_attn_workspace_bytes(caches[0], Hq, L, True), dtype=torch.uint8,
                          device="cuda")
    torch.cuda.synchronize()

    # Phase by phase, the attention runs as its two calls, split (with the
    # append) then merge; each layer buffer has its own workspace, since all
    # the splits of a block run before the first merge.
    ws_layers = [torch.zeros_like(ws_attn) for _ in range(LAYERS)]

    def phase_split(n):
        lengths_all.fill_(L - 1)
        for i in range(n):
            kvc.kvc_decode_attn_split(caches[i], q, ws_layers[i], k_new=k_new, v_new=v_new, h2o_score=scores[i],
                                      max_len_hint=L - 1)

    def phase_merge(n):
        for i in range(n):
            kvc.kvc_decode_attn_merge(caches[i], Hq, out, ws_layers[i], appended=True, h2o_score=scores[i],
                                      max_len_hint=L - 1)

    def phase_evict(n):
        for i in range(n):
            kvc.kvc_h2o_evict(caches[i], scores[i], budget, S, R, keep_lists[i], dst, dst_score, keep_mask=masks[i],
                              max_len_hint=L)

    def whole_block(n):
        # Decode order: each layer's step (append, attention, H2O, eviction;
        # two launches) in turn.
        lengths_all.fill_(L - 1)
        for i in range(n):
            kvc.kvc_decode_step(caches[i], k_new, v_new, q, out, scores[i], budget, S, R, keep_lists[i], dst,
                                dst_score, keep_mask=masks[i], max_len_hint=L - 1, workspace=ws_attn)

    # ---- eager pass, then capture blocks of layer-steps as graphs ----
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        whole_block(LAYERS)
    torch.cuda.synchronize()
    eager_out = out.clone()
    eager_len = dst.lengths.clone()
    eager_keep = torch.stack(keep_lists)

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn(n)
        return g

    graphs = {}

    def block_graphs(n):
        """Graphs of n layer-steps (layers 0..n-1): the one-call step, and the
        three phases of the separate calls."""
        if n not in graphs:
            graphs[n] = (capture(whole_block, n), [capture(fn, n) for fn in (phase_split, phase_merge, phase_evict)])
        return graphs[n]

    def blocks_of(k):
        return [LAYERS] * (k // LAYERS) + ([k % LAYERS] if k % LAYERS else [])

    g_whole, g_phases = block_graphs(LAYERS)
    torch.cuda.synchronize()
    # Set-up check (not counted as warm-up): one 32-layer block replayed in
    # each order reproduces the eager result.
    for order in ([g_whole], g_phases):
        with torch.cuda.stream(stream):
            for g in order:
                g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out), "graph replay differs from the eager attention output"
        assert torch.equal(dst.lengths, eager_len)
        assert torch.equal(torch.stack(keep_lists), eager_keep), "graph replay differs from the eager keep lists"

    warm, timed = blocks_of(args.warmup), blocks_of(args.steps)
    for n in set(warm + timed):
        block_graphs(n)
    torch.cuda.synchronize()

    # ---- warm-up, then the timed steps as the one-call step ----
    with torch.cuda.stream(stream):
        for n in warm:
            block_graphs(n)[0].replay()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        t_start.record(stream)
        wall0 = time.perf_counter()
        for n in timed:
            block_graphs(n)[0].replay()
        t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    # ---- the same warm-up and timed steps as separate calls, events between phases ----
    # ev[bi][p] ends phase p of block bi; phase p starts where the previous
    # event (or p_start) ends.
    with torch.cuda.stream(stream):
        for n in warm:
            for g in block_graphs(n)[1]:
                g.replay()
    n_ph = 3
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ph)] for _ in timed]
    p_start, p_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        p_start.record(stream)
        for bi, n in enumerate(timed):
            for p, g in enumerate(block_graphs(n)[1]):
                g.replay()
                ev[bi][p].record(stream)
        p_end.record(stream)
    torch.cuda.synchronize()
    phase_ms = [0.0] * n_ph
    prev = p_start
    for bi in range(len(timed)):
        for p in range(n_ph):
            phase_ms[p] += prev.elapsed_time(ev[bi][p])
            prev = ev[bi][p]
    by_phase_ms = p_start.elapsed_time(p_end)
    steps = args.steps

    parts, split_alg, attn_alg = step_bytes(B, Hq, H, D, bits, L, budget)
    step_alg = sum(parts.values())
    ms_per_step = total_ms / steps
    split_us = phase_ms[0] * 1e3 / steps
    attn_us = (phase_ms[0] + phase_ms[1]) * 1e3 / steps
    split_gbps = split_alg / (split_us * 1e-6) / 1e9
    value = attn_alg / (attn_us * 1e-6) / 1e9

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 codes, fp32 math",
        "data": "synthetic (seeded N(0,1) fp16 K/V with 4 outlier channels per head x10)",
        "config": {"workload": "llama7b_8k", "batch": B, "q_heads": Hq, "kv_heads": H, "head_dim": D,
                   "context": L, "bits": bits, "budget": budget, "n_sink": S, "n_recent": R,
                   "layer_buffers_rotated": LAYERS},
        "value_definition": "decode attention's algorithmic bytes (KV codes + fp32 scales + q + out = "
                            f"{attn_alg} B) / the split + merge time per step (kvc_decode_attn_split with the "
                            "append, then kvc_decode_attn_merge with H2O), over the timed steps run as "
                            "separate calls",
        "attention_us": round(attn_us, 3),
        "attention_frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "attention_tokens_per_s": round(B / (attn_us * 1e-6), 1),
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "tokens_per_s_32_layers": round(B / (ms_per_step * 1e-3 * LAYERS), 1),
        "step": {"calls": "kvc_decode_step (two launches)", "us": round(ms_per_step * 1e3, 3),
                 "bytes": step_alg, "gbps": round(step_alg / (ms_per_step * 1e-3) / 1e9, 1),
                 "frac": round(step_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "wall_s": round(wall, 3),
        "phases": phase_table(phase_ms, steps, parts, split_alg),
        "ms_per_step_phase_by_phase": round(by_phase_ms / steps, 5),
        "roofline": {
            "bound": "hbm",
            "kernel": "attn_split_kernel<8, 8, 128, 1, false>: the KV stream (with the new token's append), timed "
                      "through kvc_decode_attn_split",
            "achieved": round(split_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(split_gbps / HBM_PEAK_GBPS, 4),
            "traffic": attention_traffic(),
            "bytes_per_launch": split_alg,
            "us_per_launch": round(split_us, 3),
            "frac_with_merge": round(value / HBM_PEAK_GBPS, 4),
        },
    }
    if not args.no_secondary:
        rec_sched = layer_schedules(kvc, torch, caches, scores, lengths_all, k_new, v_new, q, out, dst, dst_score,
                                    ws_attn, L, S, R, stream, max(1, len(timed)))
    probe = read_probe(kvc, torch, split_alg)
    probe["split_frac_of_probe"] = round(split_gbps / probe["gbps"], 4)
    rec["hbm_read_probe"] = probe
    if not args.no_secondary:
        rec["layer_schedules"] = rec_sched
        rec["secondary_attention"] = secondary_attention(kvc, torch)
        rec["config_legs"] = config_legs(kvc, torch)
    if not args.no_cpu_baseline:
        t_cpu, n_cpu, t_att, n_att, cores = cpu_baseline(w, d, args.cpu_seconds)
        rec["cpu_baseline"] = {
            "value": round(attn_alg / t_att / 1e9, 4),
            "unit": "GB/s",
            "cores": cores,
            "kind": "oracle",
            "sample": f"the fp64 oracle on the same 8192-token layer: attention + H2O alone best of {n_att} "
                      f"runs, {t_att * 1e3:.1f} ms ({attn_alg} B of decode-attention bytes); full step (append, "
                      f"attention + H2O, select, compact) best of {n_cpu}, {t_cpu * 1e3:.1f} ms, "
                      f"{B / t_cpu:.2f} tokens/s",
            "step_ms": round(t_cpu * 1e3, 2),
            "attention_ms": round(t_att * 1e3, 2),
            "step_gbps": round(step_alg / t_cpu / 1e9, 4),
        }
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
