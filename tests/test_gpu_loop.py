"""A decode loop of the benchmarked call at full size, against the oracle.

Four ``kvc_decode_step`` calls (append, attention with H2O, eviction) on the
LLaMA-7B layer: the first evicts the 8192-token row to its 2457-token budget
(4 sinks, 1024 recent, 1429 heavy hitters), the next three run in the steady
state (2458 -> 2457), the destination of one step being the source of the
next. Each step's output and kept scores are checked against
``oracle.RefCache``, and its keep mask against the oracle's selection (equal
except on scores within the tolerance band of the threshold). The oracle
then compacts with the GPU's mask, a valid keep-set, so that both caches hold
the same tokens, and the compacted caches must agree bit for bit.
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


def test_decode_step_loop_llama7b_full_size():
    steps = 4
    w = get("llama7b_8k").scaled(steps=steps)
    d = draw(w)
    B, Hq, H, D, L, bits = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.context, w.bits
    budget, S, R = w.budget, w.n_sink, w.n_recent
    print(f"[loop] LLaMA-7B layer, {steps} decode steps, budget {budget}", flush=True)
    caches = [kvc.KVCache(B, H, D, L, bits) for _ in range(2)]
    scores = [c.score_buffer() for c in caches]
    ref = oracle.RefCache(B, H, D, L, bits)
    kvc.kvc_quant_append(caches[0], dev(d["k"][:, :, :L - 1]), dev(d["v"][:, :, :L - 1]), h2o_score=scores[0])
    ref.append(d["k"][:, :, :L - 1], d["v"][:, :, :L - 1])
    kidx = torch.zeros((B, H, budget), dtype=torch.int32, device="cuda")
    mask = torch.zeros((B, H, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ambiguous = candidates = 0
    for i in range(steps):
        src, dst = caches[i % 2], caches[(i + 1) % 2]
        ssc, dsc = scores[i % 2], scores[(i + 1) % 2]
        mask.zero_()
        kvc.kvc_decode_step(src, dev(d["step_k"][i]), dev(d["step_v"][i]), dev(d["step_q"][i]), out, ssc, budget, S,
                            R, kidx, dst, dsc, keep_mask=mask, max_len_hint=int(ref.lengths.max()))
        ref.append(d["step_k"][i], d["step_v"][i])
        ro, _ = ref.attend(d["step_q"][i])
        candidates += B * H * (int(ref.lengths.max()) - S - R)
        torch.cuda.synchronize()
        err = assert_out_close(host(out), ro)
        m = host(mask)
        ambiguous += assert_keep_equivalent(m, ref.score, ref.lengths, budget, S, R)
        ref.compact(m[:, :, :L].astype(bool))
        assert_codes_equal(dst, ref)
        rel = assert_scores_close(host(dsc), ref.score, ref.lengths)
        print(f"step {i}: length {int(ref.lengths[0])}, max-abs out err {err:.2e}, score rel err {rel:.2e}",
              flush=True)
    # Candidates inside the threshold's tolerance band (where either choice is
    # a correct keep-set) must stay rare.
    print(f"{ambiguous} of {candidates} candidates within the threshold band", flush=True)
    assert ambiguous <= candidates // 100, (ambiguous, candidates)


def test_decode_step_in_place_loop_qwen_full_size():
    """The GQA stream's decode loop in place at full size: 8 sequences, 28
    query / 4 KV heads, 32767 prefilled tokens; each kvc_decode_step names the
    cache as its own destination. Step 0 evicts 32768 -> 8192 (the selection
    kernel, then the in-place moves); the next steps run the steady state
    (8193 -> 8192, one launch that merges, selects and moves). Each step is
    checked against the oracle as above."""
    steps = 4
    w = get("qwen_gqa_stream").scaled(steps=steps)
    d = draw(w)
    B, Hq, H, D, L, bits = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.context, w.bits
    budget, S, R = w.budget, w.n_sink, w.n_recent
    print(f"[loop in place] Qwen GQA stream, {steps} decode steps, budget {budget}", flush=True)
    gc = kvc.KVCache(B, H, D, L, bits)
    score = gc.score_buffer()
    ref = oracle.RefCache(B, H, D, L, bits)
    kvc.kvc_quant_append(gc, dev(d["k"][:, :, :L - 1]), dev(d["v"][:, :, :L - 1]), h2o_score=score)
    ref.append(d["k"][:, :, :L - 1], d["v"][:, :, :L - 1])
    kidx = torch.zeros((B, H, budget), dtype=torch.int32, device="cuda")
    mask = torch.zeros((B, H, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ambiguous = candidates = 0
    for i in range(steps):
        mask.zero_()
        kvc.kvc_decode_step(gc, dev(d["step_k"][i]), dev(d["step_v"][i]), dev(d["step_q"][i]), out, score, budget,
                            S, R, kidx, gc, score, keep_mask=mask, max_len_hint=int(ref.lengths.max()))
        ref.append(d["step_k"][i], d["step_v"][i])
        ro, _ = ref.attend(d["step_q"][i])
        candidates += B * H * (int(ref.lengths.max()) - S - R)
        torch.cuda.synchronize()
        err = assert_out_close(host(out), ro)
        m = host(mask)
        ambiguous += assert_keep_equivalent(m, ref.score, ref.lengths, budget, S, R)
        ref.compact(m[:, :, :L].astype(bool))
        assert_codes_equal(gc, ref)
        rel = assert_scores_close(host(score), ref.score, ref.lengths)
        print(f"step {i}: length {int(ref.lengths[0])}, max-abs out err {err:.2e}, score rel err {rel:.2e}",
              flush=True)
    print(f"{ambiguous} of {candidates} candidates within the threshold band", flush=True)
    assert ambiguous <= candidates // 100, (ambiguous, candidates)
