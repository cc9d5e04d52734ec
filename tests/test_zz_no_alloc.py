"""The allocation-free decode step (kvc_decode_step_noalloc) against the
ordinary one (kvc_decode_step with a caller workspace), through the C ABI.

Both run the same kernels, so every output must match bit for bit: the
attention output, the keep list and mask, the source cache's codes, scales,
positions and lengths, and every buffer of the destination with the kept
scores. Two calls in a row share the library's static workspace; the second
is smaller than the first, so it runs over what the first left there.
"""
import numpy as np
import pytest

from workloads import draw, get

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
kvc = pytest.importorskip("compressed_kv_cache_kvc_amd")

from kvc_testlib import dev, make_gpu_cache  # noqa: E402

CACHE_FIELDS = ("k_codes", "v_codes", "k_scale", "v_scale", "positions", "lengths", "num_seen")


def _pair(w, lens, cap, seed):
    """Two identical caches holding max(lens) prefilled tokens, per-sequence
    lengths `lens`, and the same random scores."""
    d = draw(w)
    Lmax = max(lens)
    sc = (np.random.default_rng(seed).random((len(lens), w.num_kv_heads, cap)) * 0.1).astype(np.float32)
    caches = []
    for _ in range(2):
        gc = make_gpu_cache(w, cap)
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :Lmax]), dev(d["v"][:, :, :Lmax]))
        gc.lengths.copy_(dev(np.array(lens, np.int32)))
        gc.num_seen.copy_(dev(np.array(lens, np.int32) + 5))
        caches.append((gc, dev(sc)))
    return d, caches


def _run(w, d, caches, lens, budget, S, R):
    B, H, Hq, D, Lmax = len(lens), w.num_kv_heads, w.num_q_heads, w.head_dim, max(lens)
    knew, vnew = dev(d["k"][:, :, Lmax:Lmax + 1]), dev(d["v"][:, :, Lmax:Lmax + 1])
    q = dev(d["q"])
    res = []
    for noalloc, (gc, sc) in zip((False, True), caches):
        dst = make_gpu_cache(w, gc.capacity)
        dst.k_codes.fill_(0x44)
        dsc = dst.score_buffer()
        dsc.fill_(-3.0)
        kidx = torch.full((B, H, budget), -9, dtype=torch.int32, device="cuda")
        mask = torch.full((B, H, gc.capacity), 5, dtype=torch.uint8, device="cuda")
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        args = (gc, knew, vnew, q, out, sc, budget, S, R, kidx, dst, dsc)
        if noalloc:
            kvc.kvc_decode_step_noalloc(*args, keep_mask=mask, max_len_hint=Lmax)
        else:
            kvc.kvc_decode_step(*args, keep_mask=mask, max_len_hint=Lmax)
        res.append((gc, out, dst, dsc, kidx, mask))
    torch.cuda.synchronize()
    return res


def test_noalloc_step_equals_workspace_step_twice():
    """A 3-sequence GQA-4 step (the eviction kernel merges the splits), then a
    smaller 2-sequence MHA step over the same static workspace."""
    for hq, hkv, D, lens, budget, S, R in ((8, 2, 128, [2999, 1000, 500], 1000, 4, 100),
                                           (4, 4, 64, [700, 300], 256, 4, 32)):
        print(f"[noalloc] hq={hq} hkv={hkv} D={D} lens={lens} budget={budget}", flush=True)
        w = get("tiny_mha").scaled(context=max(lens) + 1, batch=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                                   head_dim=D, bits=8)
        d, caches = _pair(w, lens, max(lens) + 9, seed=budget)
        (gA, oA, dA, sA, kA, mA), (gB, oB, dB, sB, kB, mB) = _run(w, d, caches, lens, budget, S, R)
        assert torch.isfinite(oA).all()
        assert torch.equal(oA, oB), "attention output"
        assert torch.equal(kA, kB), "keep list"
        assert torch.equal(mA, mB), "keep mask"
        assert torch.equal(sA, sB), "kept scores"
        for name in CACHE_FIELDS:
            assert torch.equal(getattr(gA, name), getattr(gB, name)), f"source {name}"
            assert torch.equal(getattr(dA, name), getattr(dB, name)), f"destination {name}"
        assert dB.lengths.cpu().tolist() == [min(n + 1, budget) for n in lens]
