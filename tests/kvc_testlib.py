"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
read GPU state back, and compare it with the oracle under the acceptance rules:

* INT8/INT4 codes and fp32 scales: bit-exact;
* attention outputs: max-abs error <= 2e-3;
* H2O scores: |gpu - ref| <= 1e-5 * |ref| + 1e-30;
* keep sets: same size per row, and identical except for candidates whose
  oracle score lies within 1e-5 (relative) of the oracle's k-th threshold.
"""
from __future__ import annotations

import numpy as np

import oracle

OUT_ATOL = 2e-3
SCORE_RTOL = 1e-5
SCORE_FLOOR = 1e-30


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def oracle_code_bytes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Oracle codes as the bytes the cache stores."""
    if bits == 8:
        return np.ascontiguousarray(codes).view(np.uint8)
    return oracle.pack_int4(codes)


def assert_codes_equal(gpu_cache, ref: "oracle.RefCache", rows=None):
    """Bit-exact codes, scales and positions on every slot below the length."""
    k = host(gpu_cache.k_codes)
    v = host(gpu_cache.v_codes)
    ks = host(gpu_cache.k_scale)
    vs = host(gpu_cache.v_scale)
    pos = host(gpu_cache.positions) if gpu_cache.positions is not None else None
    lens = host(gpu_cache.lengths)
    assert np.array_equal(lens, ref.lengths.astype(np.int32)), (lens, ref.lengths)
    B, H = ref.k_scale.shape[:2]
    for b in range(B):
        L = int(ref.lengths[b])
        for g in range(H):
            if rows is not None and (b, g) not in rows:
                continue
            assert np.array_equal(k[b, g, :L], oracle_code_bytes(ref.k_codes[b, g, :L], ref.bits)), (b, g)
            assert np.array_equal(v[b, g, :L], oracle_code_bytes(ref.v_codes[b, g, :L], ref.v_bits)), (b, g)
            assert np.array_equal(ks[b, g, :L].view(np.uint32), ref.k_scale[b, g, :L].view(np.uint32)), (b, g)
            assert np.array_equal(vs[b, g, :L].view(np.uint32), ref.v_scale[b, g, :L].view(np.uint32)), (b, g)
            if pos is not None:
                assert np.array_equal(pos[b, g, :L], ref.positions[b, g, :L]), (b, g)


def assert_out_close(out_gpu: np.ndarray, out_ref: np.ndarray, atol=OUT_ATOL):
    err = np.abs(out_gpu.astype(np.float64) - out_ref)
    assert np.all(np.isfinite(out_gpu))
    assert err.max() <= atol, f"max-abs error {err.max():.3e} > {atol}"
    return float(err.max())


def assert_scores_close(score_gpu: np.ndarray, score_ref: np.ndarray, lengths):
    worst = 0.0
    for b, L in enumerate(lengths):
        L = int(L)
        g = score_gpu[b, :, :L].astype(np.float64)
        r = score_ref[b, :, :L]
        tol = SCORE_RTOL * np.abs(r) + SCORE_FLOOR
        bad = np.abs(g - r) > tol
        assert not bad.any(), f"seq {b}: {bad.sum()} scores off, worst rel {np.max(np.abs(g - r) / (np.abs(r) + 1e-300)):.3e}"
        worst = max(worst, float(np.max(np.abs(g - r) / (np.abs(r) + 1e-30))))
    return worst


def assert_keep_equivalent(mask_gpu: np.ndarray, score_ref: np.ndarray, lengths, budget, n_sink, n_recent):
    """Keep sets agree except on candidates within the tolerance band of the threshold."""
    ambiguous_total = 0
    B, H = score_ref.shape[:2]
    for b in range(B):
        L = int(lengths[b])
        for g in range(H):
            ref = oracle.select_keep(score_ref[b, g, :L], L, budget, n_sink, n_recent)
            got = mask_gpu[b, g, :L].astype(bool)
            assert got.sum() == ref.sum(), (b, g, got.sum(), ref.sum())
            T = oracle.kth_threshold(score_ref[b, g, :L], L, budget, n_sink, n_recent)
            if T is None:
                assert np.array_equal(got, ref), (b, g)
                continue
            sc = score_ref[b, g, :L]
            amb = np.zeros(L, bool)
            amb[n_sink:L - n_recent] = np.abs(sc[n_sink:L - n_recent] - T) <= SCORE_RTOL * T + SCORE_FLOOR
            ambiguous_total += int(amb.sum())
            assert np.array_equal(got[~amb], ref[~amb]), (b, g, np.nonzero(got[~amb] != ref[~amb])[0][:10])
    return ambiguous_total


def make_gpu_cache(w, capacity=None, bits=None, positions=True, v_bits=0):
    import compressed_kv_cache_kvc_amd as kvc
    return kvc.KVCache(w.batch, w.num_kv_heads, w.head_dim, capacity or w.context, bits or w.bits,
                       positions=positions, v_bits=v_bits)


def prefill_both(w, d, capacity=None, bits=None, with_score=True, v_bits=0):
    """Prefill L-1 tokens and append the L-th with both the GPU and the oracle
    (V at ``v_bits`` when set, else at the K width)."""
    import compressed_kv_cache_kvc_amd as kvc
    bits = bits or w.bits
    cap = capacity or w.context
    L = d["k"].shape[2]
    gc = make_gpu_cache(w, cap, bits, v_bits=v_bits)
    score = gc.score_buffer() if with_score else None
    ref = oracle.RefCache(w.batch, w.num_kv_heads, w.head_dim, cap, bits, v_bits=v_bits or None)
    if L > 1:
        kvc.kvc_quant_append(gc, dev(d["k"][:, :, :L - 1]), dev(d["v"][:, :, :L - 1]), h2o_score=score)
        ref.append(d["k"][:, :, :L - 1], d["v"][:, :, :L - 1])
    kvc.kvc_quant_append(gc, dev(d["k"][:, :, L - 1:]), dev(d["v"][:, :, L - 1:]), h2o_score=score)
    ref.append(d["k"][:, :, L - 1:], d["v"][:, :, L - 1:])
    return gc, ref, score
