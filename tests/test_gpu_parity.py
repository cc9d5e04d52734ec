"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Inputs are the seeded workload arrays; both sides get the same fp16 bits.
Sizes span several 256-token splits with a ragged tail; the LLaMA-7B-shaped
8192-token layer runs at full size in the launch configuration the benchmark
times.
"""
import numpy as np
import pytest

import oracle
from workloads import draw, get

from kvc_testlib import (assert_codes_equal, assert_keep_equivalent, assert_out_close, assert_scores_close, dev,
                         host, make_gpu_cache, oracle_code_bytes, prefill_both)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
kvc = pytest.importorskip("compressed_kv_cache_kvc_amd")


def _attend_both(gc, ref, q16, score):
    out = torch.empty((q16.shape[0], q16.shape[1], gc.head_dim), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn(gc, dev(q16), out, h2o_score=score)
    ro, _ = ref.attend(q16, h2o=score is not None)
    torch.cuda.synchronize()
    return host(out), ro


# ---------------------------------------------------------------- quantize ---

@pytest.mark.parametrize("name,bits,L", [
    ("tiny_mha", 8, 512), ("tiny_mha", 4, 512), ("tiny_mha", 8, 1), ("tiny_mha", 8, 300),
    ("llama7b_8k", 8, 8192), ("llama70b_int4", 4, 1100), ("qwen_gqa_stream", 8, 777),
])
def test_quant_append_bit_exact(name, bits, L):
    w = get(name).scaled(context=L, batch=min(get(name).batch, 2))
    print(f"[quant] {name} bits={bits} L={L}", flush=True)
    d = draw(w)
    gc, ref, _ = prefill_both(w, d, bits=bits)
    torch.cuda.synchronize()
    assert_codes_equal(gc, ref)
    assert host(gc.num_seen).tolist() == [L] * w.batch


@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("bits,v_bits,D", [(8, 8, 128), (4, 4, 128), (8, 4, 64), (4, 8, 128)])
def test_quant_append_bulk_edges(aligned, bits, v_bits, D):
    """Prefill-sized appends: 3 KV heads x 47 tokens per sequence (141 K rows,
    so a wave instruction straddles the last K and first V rows), appended
    after a short first append at different lengths and counts per sequence
    (13 and 6 tokens, seen 13 and 9); inputs offset by one fp16 element take
    the per-row kernel. Codes, scales, positions, lengths and counts
    bit-exact against the oracle."""
    print(f"[quant bulk] aligned={aligned} bits={bits} v_bits={v_bits} D={D}", flush=True)
    w = get("tiny_mha").scaled(context=60, batch=2, num_q_heads=3, num_kv_heads=3, head_dim=D, bits=bits)
    d = draw(w)
    gc = make_gpu_cache(w, 64, bits, v_bits=v_bits)
    ref = oracle.RefCache(2, 3, D, 64, bits, v_bits=v_bits)
    k0, v0 = d["k"][:, :, :13], d["v"][:, :, :13]
    kvc.kvc_quant_append(gc, dev(k0), dev(v0))
    ref.append(k0, v0)
    # Sequence 1 continues from 6 tokens (its later slots are overwritten).
    gc.lengths.copy_(dev(np.array([13, 6], np.int32)))
    gc.num_seen.copy_(dev(np.array([13, 9], np.int32)))
    ref.lengths[:] = [13, 6]
    ref.num_seen[:] = [13, 9]
    k1, v1 = d["k"][:, :, 13:60], d["v"][:, :, 13:60]
    if aligned:
        kd, vd = dev(k1), dev(v1)
    else:
        flat_k = torch.zeros(k1.size + 1, dtype=torch.float16, device="cuda")
        flat_v = torch.zeros(v1.size + 1, dtype=torch.float16, device="cuda")
        flat_k[1:] = dev(k1).reshape(-1)
        flat_v[1:] = dev(v1).reshape(-1)
        kd, vd = flat_k[1:].view(k1.shape), flat_v[1:].view(v1.shape)
        assert kd.data_ptr() % 16 != 0
    kvc.kvc_quant_append(gc, kd, vd)
    ref.append(k1, v1)
    torch.cuda.synchronize()
    assert_codes_equal(gc, ref)
    assert host(gc.lengths).tolist() == [60, 53]
    assert host(gc.num_seen).tolist() == [60, 56]


def test_quant_zero_rows_and_halfway_cases():
    """All-zero rows give scale 0 and code 0; amax = 127 rows hit exact halves."""
    w = get("tiny_mha").scaled(context=4)
    k = np.zeros((1, 4, 4, 64), np.float16)
    k[0, 1, :, 0] = 127.0
    k[0, 1, :, 1:12] = np.array([2.5, 3.5, -2.5, -3.5, 126.5, 0.5, -0.5, 1.5, 6.5, -6.5, 100.5], np.float16)
    v = -k
    d = {"k": k, "v": v}
    for bits in (8, 4):
        gc, ref, _ = prefill_both(w, d, capacity=8, bits=bits)
        torch.cuda.synchronize()
        assert_codes_equal(gc, ref)


def test_quant_bulk_halfway_cases():
    """The same exact-half quotients through the prefill-sized bulk kernel
    (4 heads x 64 tokens: 512 rows per sequence), for INT8 (max-abs 127:
    x / scale lands on .5) and INT4 (max-abs 7), between rows of random
    values, zero rows and rows whose max-abs is an fp16 subnormal."""
    w = get("tiny_mha").scaled(context=64)
    rng = np.random.default_rng(77)
    k = rng.standard_normal((1, 4, 64, 64)).astype(np.float16)
    halves = np.array([2.5, 3.5, -2.5, -3.5, 126.5, 0.5, -0.5, 1.5, 6.5, -6.5, 100.5], np.float16)
    for t in range(0, 64, 4):
        k[0, t % 4, t, :] = 0
        k[0, t % 4, t, 0] = 127.0
        k[0, t % 4, t, 1:12] = halves
        k[0, (t + 1) % 4, t + 1, :] = 0
        k[0, (t + 1) % 4, t + 1, 0] = 7.0
        k[0, (t + 1) % 4, t + 1, 1:7] = np.array([2.5, -2.5, 0.5, 3.5, -6.5, 1.5], np.float16)
        k[0, (t + 2) % 4, t + 2, :] = 0
        k[0, (t + 3) % 4, t + 3, :] = (np.arange(64) - 32).astype(np.float16) * np.float16(2.0 ** -24)
    v = -k[:, :, ::-1].copy()
    d = {"k": k, "v": v}
    for bits in (8, 4):
        print(f"[quant bulk halves] bits={bits}", flush=True)
        gc, ref, _ = prefill_both(w, d, capacity=64, bits=bits)
        torch.cuda.synchronize()
        assert_codes_equal(gc, ref)


# ---------------------------------------------------------------- attention --

@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("L", [1, 255, 256, 257, 512, 1000])
def test_decode_attn_tiny(bits, L):
    w = get("tiny_mha").scaled(context=L)
    print(f"[attn] tiny bits={bits} L={L}", flush=True)
    d = draw(w)
    gc, ref, score = prefill_both(w, d, bits=bits)
    out, ro = _attend_both(gc, ref, d["q"], score)
    assert_out_close(out, ro)
    assert_scores_close(host(score), ref.score, ref.lengths)


@pytest.mark.parametrize("hq,hkv,bits,D", [(8, 2, 8, 128), (28, 4, 8, 128), (16, 2, 4, 128), (12, 4, 8, 64),
                                           (6, 3, 4, 64), (64, 8, 4, 128)])
def test_decode_attn_gqa(hq, hkv, bits, D):
    w = get("qwen_gqa_stream").scaled(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, bits=bits, batch=2,
                                      context=1333)
    print(f"[attn] gqa hq={hq} hkv={hkv} bits={bits} D={D}", flush=True)
    d = draw(w)
    gc, ref, score = prefill_both(w, d)
    out, ro = _attend_both(gc, ref, d["q"], score)
    assert_out_close(out, ro)
    assert_scores_close(host(score), ref.score, ref.lengths)


@pytest.mark.parametrize("hq,hkv,bits", [(8, 8, 8), (16, 8, 8), (8, 8, 4)])
def test_decode_attn_multi_tile_splits(hq, hkv, bits):
    """Long rows: each split walks several 256-token tiles with an online
    softmax (70001 tokens x 8 KV heads gives 2 tiles per split)."""
    w = get("tiny_mha").scaled(num_q_heads=hq, num_kv_heads=hkv, head_dim=128, bits=bits, context=70001)
    print(f"[attn] multi-tile hq={hq} hkv={hkv} bits={bits}", flush=True)
    d = draw(w)
    gc, ref, score = prefill_both(w, d)
    out, ro = _attend_both(gc, ref, d["q"], score)
    assert_out_close(out, ro)
    assert_scores_close(host(score), ref.score, ref.lengths)


def test_decode_attn_is_deterministic():
    w = get("tiny_mha").scaled(context=700, num_q_heads=8, num_kv_heads=2)
    d = draw(w)
    gc, _, _ = prefill_both(w, d)
    outs = []
    for _ in range(2):
        o = torch.empty((1, 8, 64), dtype=torch.float32, device="cuda")
        s = gc.score_buffer()
        kvc.kvc_decode_attn(gc, dev(d["q"]), o, h2o_score=s)
        outs.append((host(o), host(s)))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


def test_workspace_reused_across_calls():
    """One workspace serves consecutive calls of different shapes (head
    counts, lengths and split counts); nothing from one call leaks into the
    next."""
    ws = None
    for hq, hkv, L in [(4, 4, 700), (4, 4, 3000), (8, 2, 1500), (2, 2, 9000), (8, 4, 700), (4, 4, 700)]:
        w = get("tiny_mha").scaled(num_q_heads=hq, num_kv_heads=hkv, context=L, batch=2)
        print(f"[attn] workspace reuse hq={hq} hkv={hkv} L={L}", flush=True)
        d = draw(w)
        gc, ref, score = prefill_both(w, d)
        if ws is None:
            ws = torch.full((1 << 22,), 0xA5, dtype=torch.uint8, device="cuda")
        assert kvc.kvc_decode_attn_workspace_bytes(gc, hq, L, True) <= ws.numel()
        out = torch.empty((2, hq, 64), dtype=torch.float32, device="cuda")
        kvc.kvc_decode_attn(gc, dev(d["q"]), out, h2o_score=score, workspace=ws)
        ro, _ = ref.attend(d["q"], h2o=True)
        torch.cuda.synchronize()
        assert_out_close(host(out), ro)
        assert_scores_close(host(score), ref.score, ref.lengths)


def test_empty_sequence_gives_zero_output():
    gc = kvc.KVCache(2, 2, 64, 64, 8)
    w = get("tiny_mha").scaled(context=5, num_q_heads=2, num_kv_heads=2, batch=1)
    d = draw(w)
    # Sequence 0 gets 5 tokens, sequence 1 stays empty (length 0).
    k = np.concatenate([d["k"], np.zeros_like(d["k"])])
    kvc.kvc_quant_append(gc, dev(k), dev(k))
    gc.lengths[1] = 0
    out = torch.full((2, 2, 64), 7.0, dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn(gc, dev(np.concatenate([d["q"], d["q"]])), out, max_len_hint=5)
    o = host(out)
    assert np.all(o[1] == 0) and np.all(np.isfinite(o[0]))


# --------------------------------------------------- read-bandwidth probe --

def test_bw_probe_reads_every_word():
    """The probe's per-workgroup XOR words fold to the XOR of the whole buffer
    (so every 16-byte word was read), on a size with a ragged tail."""
    rng = np.random.default_rng(11)
    words = rng.integers(0, 2**32, size=(4 << 20) // 4 + 20, dtype=np.uint32)
    src = dev(words.view(np.uint8))
    sink = torch.zeros(kvc.kvc_bw_probe_sink_bytes(), dtype=torch.uint8, device="cuda")
    kvc.kvc_bw_probe(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


# ------------------------------------------------- append + attention, fused --

def _append_attn_pair(gcA, gcB, sA, sB, knew, vnew, q, hint, hq):
    """The two-call step on cache A, the one-call step on cache B."""
    B, D = gcA.batch, gcA.head_dim
    outA = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    outB = torch.empty_like(outA)
    kvc.kvc_quant_append(gcA, knew, vnew, h2o_score=sA, max_len_hint=hint)
    kvc.kvc_decode_attn(gcA, q, outA, h2o_score=sA, max_len_hint=hint + 1)
    kvc.kvc_append_decode_attn(gcB, knew, vnew, q, outB, h2o_score=sB, max_len_hint=hint)
    torch.cuda.synchronize()
    return outA, outB


@pytest.mark.parametrize("hq,hkv,bits,D,lens,h2o,cap_extra", [
    (4, 4, 8, 128, [299, 100, 0], True, 5),      # MHA; one sequence starts empty
    (16, 4, 8, 128, [1000, 513, 64], True, 40),  # GQA 4
    (16, 2, 4, 128, [700, 255, 256], True, 0),   # INT4, GQA 8; new slot = last slot of sequence 0
    (8, 4, 8, 64, [300, 301, 302], True, 3),     # D = 64
    (32, 2, 8, 128, [600, 10, 599], True, 7),    # GQA 16: two passes of 8 heads
    (8, 4, 8, 128, [2100, 1500, 2048], False, 9),  # no H2O; several tiles per split
    # 64 rows just past 8 tiles: the last split takes the 9th tile (one
    # dispatch round of workgroups), and the new slot 2048 lies in it
    (16, 8, 8, 128, [2048, 2048, 1900, 2047, 1024, 2048, 5, 2000], True, 3),
    (8, 8, 4, 64, [2048, 1, 2048, 2040, 2048, 1500, 2048, 2047], True, 0),
])
def test_append_decode_attn_bit_exact(hq, hkv, bits, D, lens, h2o, cap_extra):
    """kvc_append_decode_attn equals kvc_quant_append + kvc_decode_attn on
    every cache buffer, the scores and the output, bit for bit, and the oracle's
    append and attention."""
    print(f"[append+attn] hq={hq} hkv={hkv} bits={bits} D={D} lens={lens} h2o={h2o}", flush=True)
    B, Lmax = len(lens), max(lens)
    w = get("tiny_mha").scaled(context=Lmax + 1, batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, bits=bits)
    d = draw(w)
    cap = Lmax + 1 + cap_extra
    rng = np.random.default_rng(Lmax + hq)
    sc = (rng.random((B, hkv, cap)) * 0.1).astype(np.float32)
    caches = []
    for _ in range(2):
        gc = make_gpu_cache(w, cap, bits)
        if Lmax:
            kvc.kvc_quant_append(gc, dev(d["k"][:, :, :Lmax]), dev(d["v"][:, :, :Lmax]))
        gc.lengths.copy_(dev(np.array(lens, np.int32)))
        gc.num_seen.copy_(dev(np.array(lens, np.int32) + 3))
        gc.max_len = Lmax
        caches.append((gc, dev(sc) if h2o else None))
    (gcA, sA), (gcB, sB) = caches
    ref = oracle.RefCache(B, hkv, D, cap, bits)
    if Lmax:
        ref.append(d["k"][:, :, :Lmax], d["v"][:, :, :Lmax])
    ref.lengths[:] = lens
    ref.num_seen[:] = np.array(lens) + 3
    ref.score[:] = sc
    knew, vnew = d["k"][:, :, Lmax:Lmax + 1], d["v"][:, :, Lmax:Lmax + 1]
    outA, outB = _append_attn_pair(gcA, gcB, sA, sB, dev(knew), dev(vnew), dev(d["q"]), Lmax, hq)
    _assert_same_cache(gcA, gcB, sA, sB)
    assert torch.equal(outA, outB)
    ref.append(knew, vnew)
    ro, _ = ref.attend(d["q"], h2o=h2o)
    assert_out_close(host(outB), ro)
    assert_codes_equal(gcB, ref)
    if h2o:
        assert_scores_close(host(sB), ref.score, ref.lengths)


@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("B,H,Hq,L", [
    (2, 4, 8, 1500),   # GQA 2
    (2, 4, 4, 1500),   # one query head per KV head
    (1, 1, 1, 70001),  # one row of 274 splits (more than 4 x 64 split states per head)
    (3, 2, 2, 5),      # one split per row
])
def test_split_then_merge_equals_one_call(append, B, H, Hq, L):
    """kvc_decode_attn_split + kvc_decode_attn_merge equal kvc_decode_attn
    (or, with the new token, kvc_append_decode_attn) bit for bit: output,
    scores and every cache buffer."""
    D = 128
    print(f"[attn] split + merge vs one call B={B} H={H} Hq={Hq} L={L} append={append}", flush=True)
    w = get("tiny_mha").scaled(context=L + 1, batch=B, num_q_heads=Hq, num_kv_heads=H, head_dim=D, bits=8)
    d = draw(w)
    runs = []
    for two_phase in (False, True):
        gc = make_gpu_cache(w, L + 1)
        sc = gc.score_buffer()
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :L]), dev(d["v"][:, :, :L]), h2o_score=sc)
        sc.copy_(torch.rand_like(sc, generator=torch.Generator(device="cuda").manual_seed(5)))
        q = dev(d["q"])
        kn, vn = (dev(d["k"][:, :, L:]), dev(d["v"][:, :, L:])) if append else (None, None)
        ws = torch.empty(kvc.kvc_decode_attn_workspace_bytes(gc, Hq, L + 1, True), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        if not two_phase:
            if append:
                kvc.kvc_append_decode_attn(gc, kn, vn, q, out, h2o_score=sc, max_len_hint=L, workspace=ws)
            else:
                kvc.kvc_decode_attn(gc, q, out, h2o_score=sc, max_len_hint=L, workspace=ws)
        else:
            kvc.kvc_decode_attn_split(gc, q, ws, k_new=kn, v_new=vn, h2o_score=sc, max_len_hint=L)
            kvc.kvc_decode_attn_merge(gc, Hq, out, ws, appended=append, h2o_score=sc, max_len_hint=L)
        torch.cuda.synchronize()
        runs.append((gc, sc, out))
    (ga, sa, oa), (gb, sb, ob) = runs
    assert torch.equal(oa, ob)
    _assert_same_cache(ga, gb, sa, sb)
    assert host(gb.lengths).tolist() == [L + int(append)] * B


def test_attention_consecutive_steps_on_one_workspace():
    """Several decode steps (with and without a new token) of the one-call
    attention on one workspace that starts as arbitrary bytes: each step's
    output, scores and cache (lengths and counts included) equal the split
    and merge calls' bit for bit, and the last step matches the oracle."""
    B, H, D, lens = 3, 4, 128, [700, 1, 0]
    print(f"[attn] consecutive steps on one workspace B={B} H={H} lens={lens}", flush=True)
    steps = 4
    Lmax = max(lens)
    w = get("tiny_mha").scaled(context=Lmax + steps, batch=B, num_q_heads=H, num_kv_heads=H, head_dim=D, bits=8)
    d = draw(w)
    cap = Lmax + steps + 3
    rng = np.random.default_rng(3)
    sc = (rng.random((B, H, cap)) * 0.1).astype(np.float32)
    pair = []
    for _ in range(2):
        gc = make_gpu_cache(w, cap, 8)
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :Lmax]), dev(d["v"][:, :, :Lmax]))
        gc.lengths.copy_(dev(np.array(lens, np.int32)))
        gc.num_seen.copy_(dev(np.array(lens, np.int32) + 5))
        pair.append((gc, dev(sc)))
    (gA, sA), (gB, sB) = pair
    ref = oracle.RefCache(B, H, D, cap, 8)
    ref.append(d["k"][:, :, :Lmax], d["v"][:, :, :Lmax])
    ref.lengths[:] = lens
    ref.num_seen[:] = np.array(lens) + 5
    ref.score[:] = sc
    nbytes = kvc.kvc_decode_attn_workspace_bytes(gB, H, cap, True)
    wsA = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    wsB = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    q = dev(d["q"])
    for i in range(steps):
        hint = Lmax + i
        kn, vn = dev(d["k"][:, :, Lmax + i:Lmax + i + 1]), dev(d["v"][:, :, Lmax + i:Lmax + i + 1])
        outA = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        outB = torch.empty_like(outA)
        append = i != 2  # step 2 attends without a new token
        kvc.kvc_decode_attn_split(gA, q, wsA, k_new=kn if append else None, v_new=vn if append else None,
                                  h2o_score=sA, max_len_hint=hint)
        kvc.kvc_decode_attn_merge(gA, H, outA, wsA, appended=append, h2o_score=sA, max_len_hint=hint)
        if append:
            kvc.kvc_append_decode_attn(gB, kn, vn, q, outB, h2o_score=sB, max_len_hint=hint, workspace=wsB)
            ref.append(d["k"][:, :, Lmax + i:Lmax + i + 1], d["v"][:, :, Lmax + i:Lmax + i + 1])
        else:
            kvc.kvc_decode_attn(gB, q, outB, h2o_score=sB, max_len_hint=hint, workspace=wsB)
        ro, _ = ref.attend(d["q"], h2o=True)
        torch.cuda.synchronize()
        assert torch.equal(outA, outB), f"step {i}"
        _assert_same_cache(gA, gB, sA, sB)
    assert host(gB.lengths).tolist() == [n + steps - 1 for n in lens]
    assert_out_close(host(outB), ro)
    assert_codes_equal(gB, ref)
    assert_scores_close(host(sB), ref.score, ref.lengths)


def test_append_decode_attn_paged():
    """Paged cache (16-token blocks, seeded block placement): the one-call
    step equals the two calls bit for bit."""
    B, H, hq, D, bs, L = 3, 4, 8, 128, 16, 333
    w = get("tiny_mha").scaled(context=L + 1, batch=B, num_q_heads=hq, num_kv_heads=H, head_dim=D, bits=8)
    d = draw(w)
    per = (L + 1 + bs - 1) // bs + 1
    perm = np.random.default_rng(5).permutation(B * per).astype(np.int32).reshape(B, per)
    caches = []
    for _ in range(2):
        gc = kvc.KVCache(B, H, D, 0, 8, block_size=bs, num_blocks=B * per, max_blocks_per_seq=per)
        gc.block_table.copy_(dev(perm))
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :L]), dev(d["v"][:, :, :L]), max_len_hint=0)
        gc.lengths.copy_(dev(np.array([L, L - 17, 5], np.int32)))
        caches.append((gc, gc.score_buffer()))
    (gcA, sA), (gcB, sB) = caches
    knew, vnew = dev(d["k"][:, :, L:L + 1]), dev(d["v"][:, :, L:L + 1])
    outA, outB = _append_attn_pair(gcA, gcB, sA, sB, knew, vnew, dev(d["q"]), L, hq)
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "lengths", "num_seen"):
        assert torch.equal(getattr(gcA, name), getattr(gcB, name)), name
    assert torch.equal(sA, sB) and torch.equal(outA, outB)


def test_append_decode_attn_llama7b_full_size():
    """The benchmarked step at full size (8191 cached tokens + the new one,
    32 heads): the one-call step equals the two calls bit for bit."""
    w = get("llama7b_8k")
    print("[append+attn] llama7b_8k full size", flush=True)
    d = draw(w)
    L = w.context - 1
    caches = []
    for _ in range(2):
        gc = make_gpu_cache(w)
        s = gc.score_buffer()
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :L]), dev(d["v"][:, :, :L]), h2o_score=s)
        caches.append((gc, s))
    (gcA, sA), (gcB, sB) = caches
    knew, vnew = dev(d["k"][:, :, L:]), dev(d["v"][:, :, L:])
    outA, outB = _append_attn_pair(gcA, gcB, sA, sB, knew, vnew, dev(d["q"]), L, w.num_q_heads)
    _assert_same_cache(gcA, gcB, sA, sB)
    assert torch.equal(outA, outB)


def _step_scores(w, lens, cap, seed):
    return (np.random.default_rng(seed).random((len(lens), w.num_kv_heads, cap)) * 0.1).astype(np.float32)


def _step_caches(w, lens, cap, seed, v_bits=0):
    """Two identical GPU caches with Lmax = max(lens) prefilled tokens, then
    per-sequence lengths `lens`, and the same random scores."""
    d = draw(w)
    Lmax = max(lens)
    sc = _step_scores(w, lens, cap, seed)
    out = []
    for _ in range(2):
        gc = make_gpu_cache(w, cap, v_bits=v_bits)
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :Lmax]), dev(d["v"][:, :, :Lmax]))
        gc.lengths.copy_(dev(np.array(lens, np.int32)))
        gc.num_seen.copy_(dev(np.array(lens, np.int32) + 2))
        gc.max_len = Lmax
        out.append((gc, dev(sc)))
    return d, out


def _oracle_step_check(w, d, lens, cap, seed, budget, S, R, out, dst, dst_score, kidx, mask, v_bits=0):
    """The oracle runs the same decode step from the state _step_caches built
    (the same prefill, lengths, token counts and scores): append, attention
    with H2O, selection and compaction. The GPU step's output, keep set (from
    its mask, else its keep list), compacted cache and kept scores are checked
    against it under the acceptance rules."""
    B, H, Lmax = len(lens), w.num_kv_heads, max(lens)
    ref = oracle.RefCache(B, H, w.head_dim, cap, w.bits, v_bits=v_bits or None)
    ref.append(d["k"][:, :, :Lmax], d["v"][:, :, :Lmax])
    ref.lengths[:] = lens
    ref.num_seen[:] = np.array(lens) + 2
    ref.score[:] = _step_scores(w, lens, cap, seed)
    ref.append(d["k"][:, :, Lmax:Lmax + 1], d["v"][:, :, Lmax:Lmax + 1])
    ro, _ = ref.attend(d["q"], h2o=True)
    assert_out_close(host(out), ro)
    L_new = ref.lengths.copy()
    keep = np.zeros((B, H, cap), bool)
    ki = host(kidx)
    m = host(mask) if mask is not None else None
    for b in range(B):
        L = int(L_new[b])
        n_keep = min(L, budget)
        for g in range(H):
            if m is not None:
                assert np.all(np.isin(m[b, g, :L], (0, 1))), (b, g)
                keep[b, g, :L] = m[b, g, :L] == 1
                assert np.array_equal(np.nonzero(keep[b, g])[0], ki[b, g, :n_keep]), (b, g)
            else:
                row = ki[b, g, :n_keep]
                assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < L, (b, g)
                keep[b, g, row] = True
    ambiguous = assert_keep_equivalent(keep, ref.score, L_new, budget, S, R)
    if ref.lengths.max() > budget:
        ref.compact(keep)
    else:
        assert keep[:, :, :Lmax + 1].sum() == int(L_new.sum()) * H
    assert_codes_equal(dst, ref)
    assert_scores_close(host(dst_score), ref.score, ref.lengths)
    assert host(dst.num_seen).tolist() == [n + 3 for n in lens]
    return ambiguous


def _step_pair(w, d, caches, lens, budget, S, R, with_mask):
    """kvc_append_decode_attn + kvc_h2o_evict on the first cache, kvc_decode_step
    on the second; returns both sides' outputs."""
    B, H, Hq, D, Lmax = len(lens), w.num_kv_heads, w.num_q_heads, w.head_dim, max(lens)
    knew, vnew = dev(d["k"][:, :, Lmax:Lmax + 1]), dev(d["v"][:, :, Lmax:Lmax + 1])
    q = dev(d["q"])
    res = []
    for i, (gc, sc) in enumerate(caches):
        dst = make_gpu_cache(w, gc.capacity, v_bits=gc.v_bits)
        dst.k_codes.fill_(0x33)
        dsc = dst.score_buffer()
        dsc.fill_(-2.0)
        kidx = torch.full((B, H, budget), -5, dtype=torch.int32, device="cuda")
        mask = torch.full((B, H, gc.capacity), 7, dtype=torch.uint8, device="cuda") if with_mask else None
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        if i == 0:
            kvc.kvc_append_decode_attn(gc, knew, vnew, q, out, h2o_score=sc, max_len_hint=Lmax)
            kvc.kvc_h2o_evict(gc, sc, budget, S, R, kidx, dst, dsc, keep_mask=mask, max_len_hint=Lmax + 1)
        else:
            kvc.kvc_decode_step(gc, knew, vnew, q, out, sc, budget, S, R, kidx, dst, dsc, keep_mask=mask,
                                max_len_hint=Lmax)
        res.append((gc, out, dst, dsc, kidx, mask))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("hq,hkv,bits,D,lens,budget,S,R,with_mask", [
    (4, 4, 8, 128, [2999, 1000, 500], 1000, 4, 100, True),     # MHA, two launches; one row within budget
    (8, 2, 8, 128, [3000, 2500, 2900], 1000, 4, 100, False),   # GQA 4, two launches, no mask
    (4, 2, 4, 128, [2000, 1999, 100], 700, 4, 64, True),       # INT4, GQA 2
    (8, 4, 8, 64, [1500, 1400, 1300], 500, 0, 64, True),       # D = 64, no sinks
    (4, 4, 8, 128, [1200, 1100, 1000], 1028, 4, 1024, True),   # no heavy hitters
    (16, 2, 8, 128, [2000, 1500, 1000], 600, 4, 64, True),     # GQA 8: the separate launches
    (4, 4, 8, 64, [20000, 19000, 100], 5000, 4, 256, True),    # long rows: selection + gather
    # 72 rows at GQA 4 (2 workgroups per row, so each merges two query heads)
    # and 136 rows at GQA 2 (1 workgroup per row), rows within and past the budget.
    (32, 8, 8, 128, [1200, 300, 1100, 499, 800, 1000, 200, 1300, 650], 500, 4, 64, True),
    (32, 8, 8, 128, [1200, 300, 1100, 499, 800, 1000, 200, 1300, 650], 500, 4, 64, False),
    (16, 8, 8, 128, [700, 150, 600, 299] * 4 + [640], 300, 4, 32, True),
])
def test_decode_step_bit_exact(hq, hkv, bits, D, lens, budget, S, R, with_mask):
    """kvc_decode_step equals kvc_append_decode_attn + kvc_h2o_evict: output,
    keep list, mask, the source cache and every buffer of dst (with the kept
    tokens' accumulated scores), bit for bit; and both equal the oracle's
    decode step (output, keep set, compacted cache, kept scores)."""
    print(f"[step] hq={hq} hkv={hkv} bits={bits} D={D} lens={lens} budget={budget}", flush=True)
    w = get("tiny_mha").scaled(context=max(lens) + 1, batch=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                               head_dim=D, bits=bits)
    cap, seed = max(lens) + 1 + 11, budget + hq
    d, caches = _step_caches(w, lens, cap, seed=seed)
    (gA, oA, dA, sA, kA, mA), (gB, oB, dB, sB, kB, mB) = _step_pair(w, d, caches, lens, budget, S, R, with_mask)
    assert torch.equal(oA, oB)
    assert torch.equal(kA, kB)
    if with_mask:
        assert torch.equal(mA, mB)
    _assert_same_cache(dA, dB, sA, sB)
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "positions", "lengths", "num_seen"):
        assert torch.equal(getattr(gA, name), getattr(gB, name)), name
    assert host(dB.lengths).tolist() == [min(n + 1, budget) for n in lens]
    _oracle_step_check(w, d, lens, cap, seed, budget, S, R, oB, dB, sB, kB, mB if with_mask else None)


@pytest.mark.parametrize("hq,hkv,bits,D,lens,budget,S,R,with_mask", [
    (28, 4, 8, 128, [1000, 1000, 990], 1000, 4, 256, True),      # GQA 7: one token evicted, one row within budget
    (28, 4, 8, 128, [1002, 1040, 999], 1000, 4, 256, True),      # 3 evicted (repeated minimum), 41 (radix), none
    (4, 2, 4, 128, [701, 700, 650], 700, 4, 64, False),          # INT4, GQA 2: 2 and 1 evicted
    (8, 1, 8, 128, [5000, 5000], 5000, 4, 2048, True),           # GQA 8, ten chunks of 512 rows per row
    (4, 4, 8, 128, [2999, 1000, 500], 1000, 4, 100, True),       # MHA, most tokens evicted
    (4, 2, 4, 128, [2000, 1999, 100], 700, 4, 64, False),        # INT4, GQA 2, no mask
    (8, 4, 8, 64, [1500, 1400, 1300], 500, 0, 64, True),         # D = 64, no sinks
    (4, 4, 8, 128, [1200, 1100, 1000], 1028, 4, 1024, True),     # no heavy hitters
    (4, 4, 8, 128, [800, 700, 600], 600, 4, 0, True),            # no recent window
    (32, 2, 8, 128, [2000, 1500, 1000], 600, 4, 64, True),       # GQA 16: merge kernel, then the in-place launch
    (4, 4, 8, 64, [20000, 19000, 100], 5000, 4, 256, True),      # long rows: selection kernel, then the moves
    # 72 rows of 4 workgroups each: more workgroups than CUs
    (32, 8, 8, 128, [1200, 300, 1100, 499, 800, 1000, 200, 1300, 650], 1100, 4, 64, True),
])
def test_decode_step_in_place(hq, hkv, bits, D, lens, budget, S, R, with_mask):
    """kvc_decode_step with the cache as its own destination: the kept tokens
    move down in place. Output, keep list, mask, codes, scales, positions,
    lengths, token counts and kept scores equal those of the out-of-place step
    bit for bit, and the oracle's decode step."""
    print(f"[step in place] hq={hq} hkv={hkv} bits={bits} D={D} lens={lens} budget={budget} R={R}", flush=True)
    w = get("tiny_mha").scaled(context=max(lens) + 1, batch=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                               head_dim=D, bits=bits)
    cap, seed = max(lens) + 1 + 11, budget + hq + 1
    d, ((gA, sA), (gB, sB)) = _step_caches(w, lens, cap, seed=seed)
    B, H, Lmax = len(lens), hkv, max(lens)
    knew, vnew, q = dev(d["k"][:, :, Lmax:Lmax + 1]), dev(d["v"][:, :, Lmax:Lmax + 1]), dev(d["q"])
    res = []
    for gc, sc, in_place in ((gA, sA, False), (gB, sB, True)):
        dst, dsc = (gc, sc) if in_place else (make_gpu_cache(w, cap), None)
        if dsc is None:
            dsc = dst.score_buffer()
        kidx = torch.full((B, H, budget), -5, dtype=torch.int32, device="cuda")
        mask = torch.full((B, H, cap), 7, dtype=torch.uint8, device="cuda") if with_mask else None
        out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
        kvc.kvc_decode_step(gc, knew, vnew, q, out, sc, budget, S, R, kidx, dst, dsc, keep_mask=mask,
                            max_len_hint=Lmax)
        res.append((out, dst, dsc, kidx, mask))
    torch.cuda.synchronize()
    (oA, dA, dsA, kA, mA), (oB, dB, dsB, kB, mB) = res
    assert torch.equal(oA, oB)
    assert torch.equal(kA, kB)
    if with_mask:
        assert torch.equal(mA, mB)
    new_len = host(dA.lengths)
    assert host(dB.lengths).tolist() == new_len.tolist() == [min(n + 1, budget) for n in lens]
    assert torch.equal(dA.num_seen, dB.num_seen)
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "positions"):
        a, b = host(getattr(dA, name)), host(getattr(dB, name))
        for i in range(B):
            assert np.array_equal(a[i, :, :new_len[i]], b[i, :, :new_len[i]]), (name, i)
    a, b = host(dsA), host(dsB)
    for i in range(B):
        assert np.array_equal(a[i, :, :new_len[i]].view(np.uint32), b[i, :, :new_len[i]].view(np.uint32)), i
    _oracle_step_check(w, d, lens, cap, seed, budget, S, R, oB, dB, dsB, kB, mB if with_mask else None)


def test_decode_step_llama7b_full_size():
    """The benchmarked step at full size (8191 cached tokens + the new one,
    32 heads, keep 2457): kvc_decode_step equals the two calls bit for bit."""
    w = get("llama7b_8k")
    print("[step] llama7b_8k full size", flush=True)
    L = w.context - 1
    d, caches = _step_caches(w, [L], w.context, seed=3)
    (gA, oA, dA, sA, kA, mA), (gB, oB, dB, sB, kB, mB) = _step_pair(w, d, caches, [L], w.budget, w.n_sink,
                                                                     w.n_recent, True)
    assert torch.equal(oA, oB) and torch.equal(kA, kB) and torch.equal(mA, mB)
    _assert_same_cache(dA, dB, sA, sB)
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "positions", "lengths", "num_seen"):
        assert torch.equal(getattr(gA, name), getattr(gB, name)), name


# ---------------------------------------------------------- select/compact --

@pytest.mark.parametrize("L,budget,S,R", [(512, 128, 4, 64), (3000, 1000, 4, 100), (9000, 2457, 4, 1024),
                                          (100, 100, 4, 10), (99, 100, 4, 10), (300, 20, 10, 10),
                                          (5000, 5000 - 1, 4, 2048), (20000, 5000, 4, 256),
                                          (30000, 23000, 4, 256), (40000, 12000, 4, 1024)])
def test_select_bit_exact_on_shared_scores(L, budget, S, R):
    """Same fp32 scores on both sides: the keep masks must be identical,
    including ties (broken toward the lower slot). Rows of more than 8192
    candidates take the memory path (keys re-read on every digit pass);
    30000 / 23000 puts the k-th key of row 0 in the 0.5 tie class."""
    rng = np.random.default_rng(L + budget)
    B, H = 2, 3
    sc = rng.random((B, H, L)).astype(np.float32) * 3
    sc[:, :, ::7] = np.float32(0.5)          # large tie classes
    sc[:, 1, :] = np.float32(1.0)            # one row of all-equal scores
    sc[:, 2, ::3] = 0.0
    cap = max(L, budget)
    gc = kvc.KVCache(B, H, 64, cap, 8)
    gc.lengths.fill_(L)
    score = dev(np.pad(sc, ((0, 0), (0, 0), (0, cap - L))))
    mask = torch.full((B, H, cap), 9, dtype=torch.uint8, device="cuda")
    kidx = torch.full((B, H, budget), -7, dtype=torch.int32, device="cuda")
    kvc.kvc_h2o_select(gc, score, budget, S, R, mask, keep_index=kidx, max_len_hint=L)
    m = host(mask)
    assert np.all(m[:, :, L:] == 9)          # slots past the length are untouched
    m = m[:, :, :L].astype(bool)
    ki = host(kidx)
    n_keep = min(L, budget)
    assert np.all(ki[:, :, n_keep:] == -7)
    for b in range(B):
        for g in range(H):
            ref = oracle.select_keep(sc[b, g].astype(np.float64), L, budget, S, R)
            assert np.array_equal(m[b, g], ref), (b, g)
            assert np.array_equal(ki[b, g, :n_keep], np.nonzero(ref)[0]), (b, g)


@pytest.mark.parametrize("bits,D,L,keep_n", [(8, 128, 2500, 900), (4, 128, 2500, 900), (8, 64, 2500, 900),
                                             (4, 64, 2500, 900), (8, 128, 40000, 12000)])
def test_compact_bit_exact(bits, D, L, keep_n):
    """Short rows take the one-launch path; 40000 slots (40 chunks) take the
    count-then-move path."""
    rng = np.random.default_rng(7 + bits + D)
    B, H, cap = 2, 3, L + 100
    w = get("tiny_mha").scaled(context=L, batch=B, num_q_heads=H, num_kv_heads=H, head_dim=D, bits=bits)
    d = draw(w)
    gc, ref, score = prefill_both(w, d, capacity=cap)
    sc = rng.random((B, H, cap)).astype(np.float32)
    score.copy_(dev(sc))
    mask = np.zeros((B, H, cap), np.uint8)
    for b in range(B):
        for g in range(H):
            mask[b, g, rng.choice(L, keep_n, replace=False)] = 1
    dst = make_gpu_cache(w, cap, bits)
    dst_score = dst.score_buffer()
    kvc.kvc_compact(gc, score, dev(mask), dst, dst_score)
    # The same compaction from the ascending keep list.
    kidx = np.stack([np.stack([np.nonzero(mask[b, g])[0] for g in range(H)]) for b in range(B)]).astype(np.int32)
    dst2 = make_gpu_cache(w, cap, bits)
    dst2_score = dst2.score_buffer()
    kvc.kvc_compact_gather(gc, score, dev(kidx), keep_n, dst2, dst2_score)
    torch.cuda.synchronize()
    ref.score[:] = sc
    ref.compact(mask.astype(bool))
    for out, out_score in ((dst, dst_score), (dst2, dst2_score)):
        assert_codes_equal(out, ref)
        assert np.array_equal(host(out_score)[:, :, :keep_n], sc[np.nonzero(mask)].reshape(B, H, keep_n))
        assert host(out.num_seen).tolist() == [L] * B


def _assert_same_cache(a, b, a_score=None, b_score=None):
    """Every buffer of two caches (and score arrays) equal bit for bit."""
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "positions", "lengths", "num_seen"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    if a_score is not None:
        assert torch.equal(a_score, b_score), "scores"


@pytest.mark.parametrize("bits,D,B,H,L,budget,S,R", [
    (8, 128, 2, 3, 9000, 2457, 4, 1024),   # one launch, 8 workgroups per row, 7972 candidates
    (4, 128, 2, 3, 3000, 1000, 4, 100),    # INT4 rows of 64 bytes
    (8, 64, 2, 3, 3000, 1000, 0, 100),     # no sinks
    (4, 64, 2, 3, 3000, 1000, 4, 100),     # rows of 32 bytes
    (8, 128, 2, 3, 99, 100, 4, 10),        # L <= budget: every slot kept
    (8, 128, 2, 3, 2000, 1028, 4, 1024),   # no heavy hitters
    (8, 64, 5, 32, 1500, 500, 4, 64),      # 160 rows: one workgroup per row
    (8, 64, 2, 3, 20000, 5000, 4, 256),    # 19740 candidates: the two-launch path
])
@pytest.mark.parametrize("with_mask", [True, False])
def test_evict_bit_exact(bits, D, B, H, L, budget, S, R, with_mask):
    """kvc_h2o_evict equals kvc_h2o_select followed by kvc_compact_gather on
    every buffer, and the oracle's selection and compaction on the kept slots;
    tie classes, an all-equal row and zero scores included."""
    print(f"[evict] bits={bits} D={D} B={B} H={H} L={L} budget={budget} S={S} R={R} mask={with_mask}", flush=True)
    rng = np.random.default_rng(L + budget + bits + D)
    w = get("tiny_mha").scaled(context=L, batch=B, num_q_heads=H, num_kv_heads=H, head_dim=D, bits=bits)
    d = draw(w)
    cap = max(L, budget) + 37
    gc, ref, score = prefill_both(w, d, capacity=cap)
    sc = rng.random((B, H, cap)).astype(np.float32) * 3
    sc[:, :, ::7] = np.float32(0.5)
    sc[:, min(1, H - 1), :] = np.float32(1.0)
    sc[:, :, ::3] = 0.0
    score.copy_(dev(sc))
    outs = []
    for fused in (True, False):
        dst = make_gpu_cache(w, cap)
        dst.k_codes.fill_(0x5A)
        dst_score = dst.score_buffer()
        dst_score.fill_(-1.0)
        kidx = torch.full((B, H, budget), -7, dtype=torch.int32, device="cuda")
        mask = torch.full((B, H, cap), 9, dtype=torch.uint8, device="cuda")
        if fused:
            kvc.kvc_h2o_evict(gc, score, budget, S, R, kidx, dst, dst_score, keep_mask=mask if with_mask else None,
                              max_len_hint=L)
        else:
            kvc.kvc_h2o_select(gc, score, budget, S, R, mask, keep_index=kidx, max_len_hint=L)
            kvc.kvc_compact_gather(gc, score, kidx, budget, dst, dst_score)
        outs.append((dst, dst_score, kidx, mask))
    torch.cuda.synchronize()
    (dst, dst_score, kidx, mask), (dst2, dst2_score, kidx2, mask2) = outs
    _assert_same_cache(dst, dst2, dst_score, dst2_score)
    assert torch.equal(kidx, kidx2)
    if with_mask:
        assert torch.equal(mask, mask2)
    else:
        assert torch.all(mask == 9)
    n_keep = min(L, budget)
    keep = np.stack([np.stack([oracle.select_keep(sc[b, g, :L].astype(np.float64), L, budget, S, R)
                               for g in range(H)]) for b in range(B)])
    ki = host(kidx)
    assert np.all(ki[:, :, n_keep:] == -7)
    for b in range(B):
        for g in range(H):
            assert np.array_equal(ki[b, g, :n_keep], np.nonzero(keep[b, g])[0]), (b, g)
    full = np.zeros((B, H, cap), bool)
    full[:, :, :L] = keep
    ref.score[:] = sc
    ref.compact(full)
    assert_codes_equal(dst, ref)
    ds = host(dst_score)
    assert np.array_equal(ds[:, :, :n_keep], sc[full].reshape(B, H, n_keep))
    assert np.all(ds[:, :, n_keep:] == -1.0)   # slots past the new length untouched
    assert np.all(host(dst.k_codes)[:, :, n_keep:] == 0x5A)
    assert host(dst.num_seen).tolist() == [L] * B


@pytest.mark.parametrize("sched,r", [(0, 0.0), (1, 0.2)])
def test_layer_budget_schedule(sched, r):
    """A 4-layer eviction loop with the pyramid schedule's budgets
    (kvc_layer_budgets): each layer's keep list and compacted cache equal the
    oracle's selection and compaction at that layer's budget."""
    B, H, D, L, S, R = 2, 4, 64, 3000, 4, 64
    budgets = kvc.kvc_layer_budgets(sched, 4, L, r, S + R)
    assert budgets == oracle.layer_budgets(sched, 4, L, r, S + R)
    print(f"[schedule] {sched} budgets {budgets}", flush=True)
    w = get("tiny_mha").scaled(context=L, batch=B, num_q_heads=H, num_kv_heads=H, head_dim=D, bits=8)
    d = draw(w)
    gc, ref, score = prefill_both(w, d, capacity=L)
    rng = np.random.default_rng(17 + sched)
    for layer, budget in enumerate(budgets):
        sc = rng.random((B, H, L)).astype(np.float32)
        score.copy_(dev(sc))
        dst = make_gpu_cache(w, L)
        dsc = dst.score_buffer()
        kidx = torch.full((B, H, budget), -1, dtype=torch.int32, device="cuda")
        kvc.kvc_h2o_evict(gc, score, budget, S, R, kidx, dst, dsc, max_len_hint=L)
        torch.cuda.synchronize()
        keep = np.stack([np.stack([oracle.select_keep(sc[b, g].astype(np.float64), L, budget, S, R)
                                   for g in range(H)]) for b in range(B)])
        ki = host(kidx)
        for b in range(B):
            for g in range(H):
                assert np.array_equal(ki[b, g, :min(L, budget)], np.nonzero(keep[b, g])[0]), (layer, b, g)
        r2 = oracle.RefCache(B, H, D, L, 8)
        r2.k_codes[:], r2.v_codes[:], r2.k_scale[:], r2.v_scale[:] = ref.k_codes, ref.v_codes, ref.k_scale, ref.v_scale
        r2.positions[:], r2.lengths[:], r2.num_seen[:] = ref.positions, ref.lengths, ref.num_seen
        r2.score[:] = sc
        r2.compact(keep)
        assert_codes_equal(dst, r2)
        assert host(dst.lengths).tolist() == [min(L, budget)] * B


# ------------------------------------------------------- whole decode step --

def _full_step(w, d, prior=()):
    gc, ref, score = prefill_both(w, d)
    for pq in prior:
        _attend_both(gc, ref, pq, score)
    out, ro = _attend_both(gc, ref, d["q"], score)
    err = assert_out_close(out, ro)
    rel = assert_scores_close(host(score), ref.score, ref.lengths)
    mask = torch.zeros((w.batch, w.num_kv_heads, gc.capacity), dtype=torch.uint8, device="cuda")
    kidx = torch.zeros((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device="cuda")
    kvc.kvc_h2o_select(gc, score, w.budget, w.n_sink, w.n_recent, mask, keep_index=kidx)
    torch.cuda.synchronize()
    amb = assert_keep_equivalent(host(mask), ref.score, ref.lengths, w.budget, w.n_sink, w.n_recent)
    m, ki = host(mask), host(kidx)
    for b in range(w.batch):   # the keep list is the mask's kept slots, ascending
        L = int(ref.lengths[b])
        for g in range(w.num_kv_heads):
            assert np.array_equal(ki[b, g, :min(L, w.budget)], np.nonzero(m[b, g, :L])[0])
    # Compact on the GPU with the oracle's keep list so that both caches keep
    # the same tokens, then compare the compacted caches bit for bit.
    keep_ref = ref.select(w.budget, w.n_sink, w.n_recent)
    ref_list = np.zeros((w.batch, w.num_kv_heads, w.budget), np.int32)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            idx = np.nonzero(keep_ref[b, g])[0]
            ref_list[b, g, :len(idx)] = idx
    dst = make_gpu_cache(w, gc.capacity)
    dst_score = dst.score_buffer()
    kvc.kvc_compact_gather(gc, score, dev(ref_list), w.budget, dst, dst_score)
    # The one-call eviction (the benchmark's launch configuration) equals the
    # GPU's own selection followed by the gather, on every buffer.
    dst_s, dst_e = make_gpu_cache(w, gc.capacity), make_gpu_cache(w, gc.capacity)
    dst_s_score, dst_e_score = dst_s.score_buffer(), dst_e.score_buffer()
    kidx_e, mask_e = torch.zeros_like(kidx), torch.zeros_like(mask)
    kvc.kvc_compact_gather(gc, score, kidx, w.budget, dst_s, dst_s_score)
    kvc.kvc_h2o_evict(gc, score, w.budget, w.n_sink, w.n_recent, kidx_e, dst_e, dst_e_score, keep_mask=mask_e)
    torch.cuda.synchronize()
    _assert_same_cache(dst_e, dst_s, dst_e_score, dst_s_score)
    assert torch.equal(kidx_e, kidx) and torch.equal(mask_e, mask)
    ref.compact(keep_ref)
    assert_codes_equal(dst, ref)
    print(f"max-abs out err {err:.2e}, worst score rel err {rel:.2e}, ambiguous {amb}", flush=True)
    return dst, ref


def test_tiny_mha_full_schedule():
    w = get("tiny_mha")
    d = draw(w)
    _full_step(w, d, prior=list(d["prior_q"]))


def test_llama7b_8k_full_size():
    """The benchmarked workload at full size: 32 heads, D=128, 8192 tokens,
    outlier channels, keep 2457 = 4 + 1024 + 1429."""
    w = get("llama7b_8k")
    print("[step] llama7b_8k full size", flush=True)
    d = draw(w)
    _full_step(w, d)


def test_int4_70b_shape_reduced():
    w = get("llama70b_int4").scaled(context=6000, batch=1, budget=1200, n_recent=256)
    print("[step] 70B-shaped INT4, L=6000", flush=True)
    d = draw(w)
    _full_step(w, d)


# ------------------------------------------------------------------ paged ---

@pytest.mark.parametrize("bits", [8, 4])
def test_paged_decode_reduced(bits):
    w = get("paged_b32").scaled(batch=4, num_q_heads=8, num_kv_heads=4, bits=bits, len_lo=100, len_hi=700)
    print(f"[paged] bits={bits}", flush=True)
    d = draw(w)
    B, H, D, bs = w.batch, w.num_kv_heads, w.head_dim, w.paged_block
    table = d["block_table"]
    nb = int(d["num_blocks"])
    lengths = d["lengths"]
    gc = kvc.KVCache(B, H, D, 0, bits, block_size=bs, num_blocks=nb, max_blocks_per_seq=table.shape[1])
    gc.block_table.copy_(dev(table))
    # Append each sequence's tokens in two pieces of a common count, padding the
    # short sequences' second piece is not possible with one call, so append
    # per sequence with a one-sequence view of the same pool.
    rb = D * bits // 8
    kp = np.zeros((nb, H, bs, D), np.int8)
    vp = np.zeros((nb, H, bs, D), np.int8)
    ksp = np.zeros((nb, H, bs), np.float32)
    vsp = np.zeros((nb, H, bs), np.float32)
    for b in range(B):
        one = kvc.KvcCacheDesc.from_buffer_copy(gc.desc)
        one.batch = 1
        one.block_table = gc.block_table[b].data_ptr()
        one.lengths = gc.lengths[b:b + 1].data_ptr()
        one.num_seen = gc.num_seen[b:b + 1].data_ptr()
        L = int(lengths[b])
        kvc.kvc_quant_append(one, dev(d["k_seq"][b][None]), dev(d["v_seq"][b][None]), max_len_hint=0)
        lens = np.zeros(1, np.int64)
        oracle.paged_append(kp, ksp, vp, vsp, table[b:b + 1], lens, d["k_seq"][b][None], d["v_seq"][b][None],
                            bits, bs)
    torch.cuda.synchronize()
    assert host(gc.lengths).tolist() == lengths.tolist()
    used = table[table >= 0]
    kc = host(gc.k_codes)[used]
    want = kp[used].view(np.uint8) if bits == 8 else oracle.pack_int4(kp[used])
    # Slots past a sequence's length inside its last block hold zeros on both sides.
    assert np.array_equal(kc, want)
    assert np.array_equal(host(gc.k_scale)[used].view(np.uint32), ksp[used].view(np.uint32))
    out = torch.empty((B, w.num_q_heads, D), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn(gc, dev(d["q"]), out, max_len_hint=int(lengths.max()))
    ro = oracle.paged_decode_attention(d["q"], kp, ksp, vp, vsp, table, lengths, bs)
    torch.cuda.synchronize()
    assert_out_close(host(out), ro)
    assert rb == kc.shape[-1]


def test_paged_block_evict():
    """Block-granular eviction: the rewritten table, lengths, freed blocks and
    moved scores equal the oracle's (exact ties included), attention through
    the new table equals the oracle's over the kept tokens, and the freed
    blocks go back to the pool."""
    B, H, Hq, D, bs = 3, 4, 8, 128, 16
    lens = np.array([333, 160, 17])
    mb = 24
    pool = kvc.BlockPool(80, bs, shuffle_seed=99)
    for b in range(B):
        pool.reserve(b, int(lens[b]))
    table = pool.block_table(list(range(B)), mb)
    gc = kvc.KVCache(B, H, D, 0, 8, block_size=bs, num_blocks=80, max_blocks_per_seq=mb)
    gc.block_table.copy_(dev(table))
    rng = np.random.default_rng(23)
    kp, vp = np.zeros((80, H, bs, D), np.int8), np.zeros((80, H, bs, D), np.int8)
    ksp, vsp = np.zeros((80, H, bs), np.float32), np.zeros((80, H, bs), np.float32)
    for b in range(B):
        k16 = rng.standard_normal((1, H, int(lens[b]), D)).astype(np.float16)
        v16 = rng.standard_normal((1, H, int(lens[b]), D)).astype(np.float16)
        one = kvc.KvcCacheDesc.from_buffer_copy(gc.desc)
        one.batch = 1
        one.block_table = gc.block_table[b].data_ptr()
        one.lengths = gc.lengths[b:b + 1].data_ptr()
        one.num_seen = gc.num_seen[b:b + 1].data_ptr()
        kvc.kvc_quant_append(one, dev(k16), dev(v16), max_len_hint=0)
        oracle.paged_append(kp, ksp, vp, vsp, table[b:b + 1], np.zeros(1, np.int64), k16, v16, 8, bs)
    cap = gc.capacity
    sc = rng.random((B, H, cap)).astype(np.float32)
    sc[0, :, 5 * bs:6 * bs] = sc[0, :, 2 * bs:3 * bs]      # exact tie between blocks 2 and 5
    sc[1, :, 0:bs] = sc[1, :, 7 * bs:8 * bs]               # and between blocks 0 and 7
    score = dev(sc)
    dst = gc.table_view()
    dst_score = torch.full((B, H, cap), -3.0, dtype=torch.float32, device="cuda")
    freed = torch.full((B, mb), -9, dtype=torch.int32, device="cuda")
    fcount = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    retention = 0.6
    kvc.kvc_paged_block_evict(gc, score, retention, dst, dst_score, freed, fcount, max_len_hint=int(lens.max()))
    torch.cuda.synchronize()
    new_table, new_lens = host(dst.block_table), host(dst.lengths)
    fr, fc, ds = host(freed), host(fcount), host(dst_score)
    want_table = np.zeros_like(table)
    for b in range(B):
        row, nl, fb, kept = oracle.block_evict(list(table[b]), int(lens[b]), sc[b].astype(np.float64), retention)
        want_table[b] = row
        assert new_table[b].tolist() == row, b
        assert int(new_lens[b]) == nl and int(fc[b]) == len(fb), b
        assert fr[b, :len(fb)].tolist() == fb and np.all(fr[b, len(fb):] == -9), b
        moved = oracle.move_block_scores(sc[b], kept, int(lens[b]))
        assert np.array_equal(ds[b, :, :nl], moved[:, :nl]), b
        assert np.all(ds[b, :, nl:] == -3.0), b
        pool.release(b, fb)
    assert host(dst.num_seen).tolist() == lens.tolist()
    assert pool.num_free == 80 - sum(int(x) for x in ((new_lens + bs - 1) // bs))
    assert pool.block_table(list(range(B)), mb).tolist() == want_table.tolist()
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn(dst, dev(q), out, max_len_hint=int(new_lens.max()))
    ro = oracle.paged_decode_attention(q, kp, ksp, vp, vsp, want_table, new_lens.astype(np.int64), bs)
    torch.cuda.synchronize()
    assert_out_close(host(out), ro)


# ------------------------------------------------ full-size configurations --
# The larger workloads run at full size on the GPU, in the launch configuration
# the library picks for them; the oracle checks sampled sequences or rows
# (it computes each sampled row from the fp16 inputs on its own).

def _row_check(gpu_codes, gpu_scale, codes_ref, scale_ref, bits):
    want = codes_ref.view(np.uint8) if bits == 8 else oracle.pack_int4(codes_ref)
    assert np.array_equal(gpu_codes, want)
    assert np.array_equal(gpu_scale.view(np.uint32), scale_ref.astype(np.float32).view(np.uint32))


def test_paged_b32_full_size():
    """32 sequences of 1024..4096 tokens in 16-token INT8 blocks placed by a
    seeded permutation; all 32 appended and attended on the GPU, 4 sampled
    sequences checked in full (codes, scales, every query head's output)."""
    w = get("paged_b32")
    print("[paged] full size B=32", flush=True)
    d = draw(w)
    B, Hq, H, D, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.paged_block
    table, nb, lengths = d["block_table"], int(d["num_blocks"]), d["lengths"]
    gc = kvc.KVCache(B, H, D, 0, 8, block_size=bs, num_blocks=nb, max_blocks_per_seq=table.shape[1])
    gc.block_table.copy_(dev(table))
    for b in range(B):
        one = kvc.KvcCacheDesc.from_buffer_copy(gc.desc)
        one.batch = 1
        one.block_table = gc.block_table[b].data_ptr()
        one.lengths = gc.lengths[b:b + 1].data_ptr()
        one.num_seen = gc.num_seen[b:b + 1].data_ptr()
        kvc.kvc_quant_append(one, dev(d["k_seq"][b][None]), dev(d["v_seq"][b][None]), max_len_hint=0)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn(gc, dev(d["q"]), out, max_len_hint=int(lengths.max()))
    torch.cuda.synchronize()
    assert host(gc.lengths).tolist() == lengths.tolist()
    kc_all, ks_all, o = host(gc.k_codes), host(gc.k_scale), host(out)
    for b in np.random.default_rng(33).choice(B, 4, replace=False):
        L, nbk = int(lengths[b]), (int(lengths[b]) + bs - 1) // bs
        blocks = table[b, :nbk]
        local = np.arange(nbk, dtype=np.int32)[None]          # the sequence's blocks, renumbered
        kp = np.zeros((nbk, H, bs, D), np.int8); vp = np.zeros_like(kp)
        ksp = np.zeros((nbk, H, bs), np.float32); vsp = np.zeros_like(ksp)
        oracle.paged_append(kp, ksp, vp, vsp, local, np.zeros(1, np.int64), d["k_seq"][b][None],
                            d["v_seq"][b][None], 8, bs)
        assert np.array_equal(kc_all[blocks], kp.view(np.uint8)), b
        assert np.array_equal(ks_all[blocks].view(np.uint32), ksp.view(np.uint32)), b
        ro = oracle.paged_decode_attention(d["q"][b:b + 1], kp, ksp, vp, vsp, local, lengths[b:b + 1], bs)
        assert_out_close(o[b:b + 1], ro)


def test_qwen_gqa_stream_full_size():
    """8 sequences x 32768 tokens, 28 query / 4 KV heads: 64 decode steps of
    append, attention with H2O, keep-set selection (checked against the
    oracle's) and compaction back to 8192, all at full size. Both sides
    compact with the oracle's keep list so that they stay on the same tokens."""
    w = get("qwen_gqa_stream")
    print("[stream] full size, 64 steps", flush=True)
    d = draw(w)
    B, Hq, H, D, L = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.context
    gc, ref, score = prefill_both(w, d)
    other = make_gpu_cache(w, L)
    other_score = other.score_buffer()
    worst_err, ambiguous = 0.0, 0
    for s in range(w.steps):
        if s > 0:
            kvc.kvc_quant_append(gc, dev(d["step_k"][s]), dev(d["step_v"][s]), h2o_score=score)
            ref.append(d["step_k"][s], d["step_v"][s])
        out, ro = _attend_both(gc, ref, d["step_q"][s], score)
        worst_err = max(worst_err, assert_out_close(out, ro))
        assert_scores_close(host(score), ref.score, ref.lengths)
        if int(ref.lengths.max()) <= w.budget:
            continue
        mask = torch.zeros((B, H, gc.capacity), dtype=torch.uint8, device="cuda")
        kidx = torch.zeros((B, H, w.budget), dtype=torch.int32, device="cuda")
        kvc.kvc_h2o_select(gc, score, w.budget, w.n_sink, w.n_recent, mask, keep_index=kidx)
        torch.cuda.synchronize()
        ambiguous += assert_keep_equivalent(host(mask), ref.score, ref.lengths, w.budget, w.n_sink, w.n_recent)
        keep_ref = ref.select(w.budget, w.n_sink, w.n_recent)
        ref_list = np.stack([np.stack([np.nonzero(keep_ref[b, g])[0] for g in range(H)])
                             for b in range(B)]).astype(np.int32)
        kvc.kvc_compact_gather(gc, score, dev(ref_list), w.budget, other, other_score)
        ref.compact(keep_ref)
        gc, other, score, other_score = other, gc, other_score, score
    torch.cuda.synchronize()
    assert_codes_equal(gc, ref)
    assert host(gc.lengths).tolist() == [w.budget] * B
    print(f"64 steps: worst max-abs out err {worst_err:.2e}, ambiguous keep slots {ambiguous}", flush=True)


def test_llama70b_int4_full_size():
    """4 sequences x 131072 tokens, INT4, 64 query / 8 KV heads, 1% outlier
    tokens x8: prefill, append, attention with H2O, selection and compaction
    at full size on the GPU; two sampled (sequence, KV head) rows checked end
    to end (codes, scales, the 8 query heads' outputs, H2O scores, keep-set,
    compacted row)."""
    w = get("llama70b_int4")
    print("[70b] full size INT4", flush=True)
    d = draw(w)
    B, Hq, H, D, L, G = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.context, w.group
    gc = make_gpu_cache(w, L)
    score = gc.score_buffer()
    k16, v16 = dev(d["k"]), dev(d["v"])
    kvc.kvc_quant_append(gc, k16[:, :, :L - 1].contiguous(), v16[:, :, :L - 1].contiguous(), h2o_score=score)
    kvc.kvc_quant_append(gc, k16[:, :, L - 1:].contiguous(), v16[:, :, L - 1:].contiguous(), h2o_score=score)
    del k16, v16
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn(gc, dev(d["q"]), out, h2o_score=score)
    mask = torch.zeros((B, H, L), dtype=torch.uint8, device="cuda")
    kidx = torch.zeros((B, H, w.budget), dtype=torch.int32, device="cuda")
    kvc.kvc_h2o_select(gc, score, w.budget, w.n_sink, w.n_recent, mask, keep_index=kidx)
    torch.cuda.synchronize()
    samples = [(0, 3), (2, 6)]
    lists = host(kidx).copy()
    refs = {}
    for b, g in samples:
        kc, ks = oracle.quantize_rows(d["k"][b, g], 4)
        vc, vs = oracle.quantize_rows(d["v"][b, g], 4)
        _row_check(host(gc.k_codes[b, g]), host(gc.k_scale[b, g]), kc, ks, 4)
        _row_check(host(gc.v_codes[b, g]), host(gc.v_scale[b, g]), vc, vs, 4)
        ro, p = oracle.attend_head_group(d["q"][b, g * G:(g + 1) * G], kc, ks, vc, vs)
        assert_out_close(host(out[b, g * G:(g + 1) * G]), ro)
        sref = oracle.h2o_accumulate(np.zeros(L), p)
        assert_scores_close(host(score[b, g])[None, None], sref[None, None], np.array([L]))
        assert_keep_equivalent(host(mask[b, g])[None, None], sref[None, None], np.array([L]), w.budget,
                               w.n_sink, w.n_recent)
        keep = oracle.select_keep(sref, L, w.budget, w.n_sink, w.n_recent)
        lists[b, g] = np.nonzero(keep)[0]
        refs[(b, g)] = oracle.compact_row(keep, kc, vc, ks, vs, np.arange(L), sref)
    dst = make_gpu_cache(w, L)
    dst_score = dst.score_buffer()
    kvc.kvc_compact_gather(gc, score, dev(lists), w.budget, dst, dst_score)
    torch.cuda.synchronize()
    assert host(dst.lengths).tolist() == [w.budget] * B
    for (b, g), (kc, vc, ks, vs, pos, sc) in refs.items():
        _row_check(host(dst.k_codes[b, g, :w.budget]), host(dst.k_scale[b, g, :w.budget]), kc, ks, 4)
        _row_check(host(dst.v_codes[b, g, :w.budget]), host(dst.v_scale[b, g, :w.budget]), vc, vs, 4)
        assert np.array_equal(host(dst.positions[b, g, :w.budget]), pos)
        gpu_sc = host(dst_score[b, g, :w.budget]).astype(np.float64)
        assert np.all(np.abs(gpu_sc - sc) <= 1e-5 * np.abs(sc) + 1e-30)


# ------------------------------------------- K and V at different widths --

MIXED = [(8, 4), (4, 8)]


@pytest.mark.parametrize("bits,v_bits", MIXED)
@pytest.mark.parametrize("D,L", [(128, 300), (64, 700)])
def test_mixed_quant_append_bit_exact(bits, v_bits, D, L):
    """K codes at `bits`, V codes at `v_bits`: both append kernels (the
    prefill-sized rows kernel, then the one-token sequence kernel)."""
    print(f"[mixed quant] bits={bits} v_bits={v_bits} D={D} L={L}", flush=True)
    w = get("tiny_mha").scaled(context=L, head_dim=D, batch=2)
    d = draw(w)
    gc, ref, _ = prefill_both(w, d, bits=bits, v_bits=v_bits)
    torch.cuda.synchronize()
    assert gc.v_codes.shape[-1] == D * v_bits // 8
    assert_codes_equal(gc, ref)


@pytest.mark.parametrize("bits,v_bits", MIXED)
@pytest.mark.parametrize("hq,hkv,D", [(4, 4, 128), (8, 4, 128), (16, 4, 128), (16, 2, 128), (8, 8, 64)])
def test_mixed_decode_attn(bits, v_bits, hq, hkv, D):
    """Attention over mixed-width codes (every query-head grouping the kernel
    has: 1, 2, 4 and 8 per pass) against the oracle, with the H2O scores."""
    print(f"[mixed attn] bits={bits} v_bits={v_bits} hq={hq} hkv={hkv} D={D}", flush=True)
    w = get("tiny_mha").scaled(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, batch=2, context=1333)
    d = draw(w)
    gc, ref, score = prefill_both(w, d, bits=bits, v_bits=v_bits)
    out, ro = _attend_both(gc, ref, d["q"], score)
    assert_out_close(out, ro)
    assert_scores_close(host(score), ref.score, ref.lengths)


@pytest.mark.parametrize("bits,v_bits", MIXED)
def test_mixed_append_decode_attn(bits, v_bits):
    """The one-call append + attention equals the two calls bit for bit, and
    the oracle's append and attention, on ragged lengths."""
    lens, hq, hkv, D = [700, 255, 64], 8, 2, 128
    print(f"[mixed append+attn] bits={bits} v_bits={v_bits}", flush=True)
    B, Lmax = len(lens), max(lens)
    w = get("tiny_mha").scaled(context=Lmax + 1, batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=D)
    d = draw(w)
    cap = Lmax + 6
    sc = (np.random.default_rng(9).random((B, hkv, cap)) * 0.1).astype(np.float32)
    caches = []
    for _ in range(2):
        gc = make_gpu_cache(w, cap, bits, v_bits=v_bits)
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :Lmax]), dev(d["v"][:, :, :Lmax]))
        gc.lengths.copy_(dev(np.array(lens, np.int32)))
        gc.num_seen.copy_(dev(np.array(lens, np.int32)))
        gc.max_len = Lmax
        caches.append((gc, dev(sc)))
    (gcA, sA), (gcB, sB) = caches
    ref = oracle.RefCache(B, hkv, D, cap, bits, v_bits=v_bits)
    ref.append(d["k"][:, :, :Lmax], d["v"][:, :, :Lmax])
    ref.lengths[:] = lens
    ref.num_seen[:] = lens
    ref.score[:] = sc
    knew, vnew = d["k"][:, :, Lmax:Lmax + 1], d["v"][:, :, Lmax:Lmax + 1]
    outA, outB = _append_attn_pair(gcA, gcB, sA, sB, dev(knew), dev(vnew), dev(d["q"]), Lmax, hq)
    _assert_same_cache(gcA, gcB, sA, sB)
    assert torch.equal(outA, outB)
    ref.append(knew, vnew)
    ro, _ = ref.attend(d["q"], h2o=True)
    assert_out_close(host(outB), ro)
    assert_codes_equal(gcB, ref)
    assert_scores_close(host(sB), ref.score, ref.lengths)


@pytest.mark.parametrize("bits,v_bits", MIXED)
def test_mixed_paged_decode_attn(bits, v_bits):
    """Paged mixed-width cache (16-token blocks in seeded places): the codes
    gathered through the table equal the oracle's, and the attention equals
    the oracle's over the same tokens."""
    B, H, hq, D, bs, L = 3, 4, 8, 128, 16, 333
    lens = [L, L - 17, 5]
    print(f"[mixed paged] bits={bits} v_bits={v_bits}", flush=True)
    w = get("tiny_mha").scaled(context=L, batch=B, num_q_heads=hq, num_kv_heads=H, head_dim=D)
    d = draw(w)
    per = (L + bs - 1) // bs + 1
    perm = np.random.default_rng(6).permutation(B * per).astype(np.int32).reshape(B, per)
    gc = kvc.KVCache(B, H, D, 0, bits, block_size=bs, num_blocks=B * per, max_blocks_per_seq=per, v_bits=v_bits)
    gc.block_table.copy_(dev(perm))
    kvc.kvc_quant_append(gc, dev(d["k"]), dev(d["v"]), max_len_hint=0)
    gc.lengths.copy_(dev(np.array(lens, np.int32)))
    ref = oracle.RefCache(B, H, D, L, bits, v_bits=v_bits)
    ref.append(d["k"], d["v"])
    ref.lengths[:] = lens
    out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attn(gc, dev(d["q"]), out, max_len_hint=L)
    ro, _ = ref.attend(d["q"], h2o=False)
    torch.cuda.synchronize()
    assert_out_close(host(out), ro)
    kc, vc = host(gc.k_codes), host(gc.v_codes)
    for b in range(B):
        n = lens[b]
        blocks = perm[b, :(n + bs - 1) // bs]
        # pool [block, head, slot, bytes] -> [head, token, bytes]
        kg = kc[blocks].transpose(1, 0, 2, 3).reshape(H, -1, kc.shape[-1])[:, :n]
        vg = vc[blocks].transpose(1, 0, 2, 3).reshape(H, -1, vc.shape[-1])[:, :n]
        for g in range(H):
            assert np.array_equal(kg[g], oracle_code_bytes(ref.k_codes[b, g, :n], bits)), (b, g)
            assert np.array_equal(vg[g], oracle_code_bytes(ref.v_codes[b, g, :n], v_bits)), (b, g)


@pytest.mark.parametrize("bits,v_bits", MIXED)
@pytest.mark.parametrize("D,L,budget", [(128, 3000, 1000), (64, 20000, 5000)])
def test_mixed_evict_and_compact(bits, v_bits, D, L, budget):
    """Eviction (one launch, and selection + gather for the long rows) and the
    mask compaction on mixed-width rows: equal to each other and to the
    oracle's selection and compaction."""
    print(f"[mixed evict] bits={bits} v_bits={v_bits} D={D} L={L}", flush=True)
    B, H, S, R = 2, 3, 4, 100
    rng = np.random.default_rng(L + bits)
    w = get("tiny_mha").scaled(context=L, batch=B, num_q_heads=H, num_kv_heads=H, head_dim=D)
    d = draw(w)
    cap = L + 37
    gc, ref, score = prefill_both(w, d, capacity=cap, bits=bits, v_bits=v_bits)
    sc = rng.random((B, H, cap)).astype(np.float32) * 3
    sc[:, :, ::7] = np.float32(0.5)
    score.copy_(dev(sc))
    dsts = []
    for _ in range(3):
        dst = make_gpu_cache(w, cap, bits, v_bits=v_bits)
        dst_score = dst.score_buffer()
        dsts.append((dst, dst_score))
    kidx = torch.full((B, H, budget), -7, dtype=torch.int32, device="cuda")
    mask = torch.zeros((B, H, cap), dtype=torch.uint8, device="cuda")
    kvc.kvc_h2o_evict(gc, score, budget, S, R, kidx, dsts[0][0], dsts[0][1], keep_mask=mask, max_len_hint=L)
    kvc.kvc_compact_gather(gc, score, kidx, budget, dsts[1][0], dsts[1][1])
    kvc.kvc_compact(gc, score, mask, dsts[2][0], dsts[2][1])
    torch.cuda.synchronize()
    keep = np.stack([np.stack([oracle.select_keep(sc[b, g, :L].astype(np.float64), L, budget, S, R)
                               for g in range(H)]) for b in range(B)])
    assert np.array_equal(host(mask)[:, :, :L].astype(bool), keep)
    full = np.zeros((B, H, cap), bool)
    full[:, :, :L] = keep
    ref.score[:] = sc
    ref.compact(full)
    for dst, dst_score in dsts:
        assert_codes_equal(dst, ref)
        assert np.array_equal(host(dst_score)[:, :, :budget], sc[full].reshape(B, H, budget))
    _assert_same_cache(dsts[0][0], dsts[1][0], dsts[0][1], dsts[1][1])


@pytest.mark.parametrize("bits,v_bits", MIXED)
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_mixed_decode_step(bits, v_bits, hq, hkv):
    """The one-call decode step (merged attention statistics, H2O update and
    eviction) on a mixed-width cache equals the separate calls bit for bit,
    and its output equals the oracle's attention."""
    lens, budget, S, R = [2999, 1000, 500], 1000, 4, 100
    print(f"[mixed step] bits={bits} v_bits={v_bits} hq={hq} hkv={hkv}", flush=True)
    w = get("tiny_mha").scaled(context=max(lens) + 1, batch=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                               head_dim=128, bits=bits)
    d, caches = _step_caches(w, lens, max(lens) + 12, seed=hq, v_bits=v_bits)
    ref = oracle.RefCache(len(lens), hkv, 128, max(lens) + 12, bits, v_bits=v_bits)
    ref.append(d["k"][:, :, :max(lens)], d["v"][:, :, :max(lens)])
    ref.lengths[:] = lens
    ref.append(d["k"][:, :, max(lens):max(lens) + 1], d["v"][:, :, max(lens):max(lens) + 1])
    ro, _ = ref.attend(d["q"], h2o=False)
    (gA, oA, dA, sA, kA, mA), (gB, oB, dB, sB, kB, mB) = _step_pair(w, d, caches, lens, budget, S, R, True)
    assert torch.equal(oA, oB) and torch.equal(kA, kB) and torch.equal(mA, mB)
    _assert_same_cache(dA, dB, sA, sB)
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "positions", "lengths", "num_seen"):
        assert torch.equal(getattr(gA, name), getattr(gB, name)), name
    assert_out_close(host(oB), ro)
    assert host(dB.lengths).tolist() == [min(n + 1, budget) for n in lens]
