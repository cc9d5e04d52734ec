"""Compressed-KV decode attention for AMD MI355X: Python binding of libkvc.

Argument marshalling only. Every step of the path runs in the HIP kernels of
``libkvc.so``; this module turns torch tensors into device pointers, calls the
C ABI declared in ``include/kvc.h`` through ctypes, and raises
:class:`KvcError` on a non-OK status. There is no CPU fallback: importing the
package fails loudly when the library has not been built.

Function names match the C entry points (``kvc_quant_append``,
``kvc_decode_attn`` and its fused and split forms, ``kvc_h2o_select``,
``kvc_compact``, ``kvc_h2o_evict``, ``kvc_decode_step``, the paged block
eviction, K/V-separated attention, ``kvc_layer_budgets`` and the
``kvc_pool_*`` calls). :class:`KVCache` owns the device buffers one cache
descriptor points to; :class:`BlockPool` wraps the host block pool.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "KvcError", "KVCache", "BlockPool", "lib", "LIB_PATH",
    "kvc_abi_version", "kvc_status_str", "kvc_last_error",
    "kvc_quant_append", "kvc_decode_attn", "kvc_decode_attn_workspace_bytes",
    "kvc_append_decode_attn", "kvc_decode_attn_split", "kvc_decode_attn_merge",
    "kvc_h2o_select", "kvc_compact", "kvc_compact_workspace_bytes", "kvc_compact_gather",
    "kvc_h2o_evict", "kvc_decode_step", "kvc_decode_step_noalloc", "kvc_decode_step_noalloc_max_bytes",
    "kvc_layer_budgets",
    "kvc_paged_block_evict", "kvc_paged_block_evict_workspace_bytes",
    "kvc_decode_attn_kvsep", "kvc_decode_attn_kvsep_workspace_bytes",
    "kvc_bw_probe", "kvc_bw_probe_sink_bytes",
    "row_bytes",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvc.so")

KVC_OK, KVC_ERR_INVALID_ARG, KVC_ERR_CAPACITY, KVC_ERR_UNSUPPORTED, KVC_ERR_DEVICE = range(5)


class KvcCacheDesc(ctypes.Structure):
    """ctypes mirror of ``kvc_cache_t``."""
    _fields_ = [
        ("bits", ctypes.c_int32), ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("lengths", ctypes.c_void_p), ("num_seen", ctypes.c_void_p),
        ("positions", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("v_bits", ctypes.c_int32),
        ("fp16_sinks", ctypes.c_int32), ("fp16_recent", ctypes.c_int32),
        ("k_sink16", ctypes.c_void_p), ("v_sink16", ctypes.c_void_p),
        ("k_recent16", ctypes.c_void_p), ("v_recent16", ctypes.c_void_p),
    ]


def _load():
    # torch brings its own HIP runtime (libamdhip64.so, soname libamdhip64.so.7).
    # Loading torch first lets libkvc.so bind to that same runtime by soname;
    # otherwise the process would hold two HIP runtimes and the second finds no device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python compressed_kv_cache_kvc_amd/build.py` "
            "(or __graft_entry__.build()). There is no fallback implementation.")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_uint64
    D = ctypes.POINTER(KvcCacheDesc)
    sig = {
        "kvc_abi_version": (I32, []),
        "kvc_status_str": (ctypes.c_char_p, [I32]),
        "kvc_last_error": (ctypes.c_char_p, []),
        "kvc_quant_append": (I32, [D, P, P, I32, P, I32, P]),
        "kvc_decode_attn_workspace_bytes": (SZ, [D, I32, I32, I32]),
        "kvc_decode_attn": (I32, [D, P, I32, P, P, I32, P, SZ, P]),
        "kvc_append_decode_attn": (I32, [D, P, P, P, I32, P, P, I32, P, SZ, P]),
        "kvc_decode_attn_split": (I32, [D, P, P, P, I32, P, I32, P, SZ, P]),
        "kvc_decode_attn_merge": (I32, [D, I32, I32, P, P, I32, P, SZ, P]),
        "kvc_h2o_select": (I32, [D, P, I32, I32, I32, P, P, I32, P]),
        "kvc_compact_workspace_bytes": (SZ, [D, I32]),
        "kvc_compact": (I32, [D, P, P, D, P, I32, P, SZ, P]),
        "kvc_compact_gather": (I32, [D, P, P, I32, D, P, P]),
        "kvc_h2o_evict": (I32, [D, P, I32, I32, I32, P, P, D, P, I32, P]),
        "kvc_decode_step": (I32, [D, P, P, P, I32, P, P, I32, I32, I32, P, P, D, P, I32, P, SZ, P]),
        "kvc_decode_step_noalloc_max_bytes": (SZ, []),
        "kvc_decode_step_noalloc": (I32, [D, P, P, P, I32, P, P, I32, I32, I32, P, P, D, P, I32, P]),
        "kvc_decode_attn_kvsep_workspace_bytes": (SZ, [D, I32, I32, I32]),
        "kvc_decode_attn_kvsep": (I32, [D, P, I32, I32, P, P, I32, P, SZ, P]),
        "kvc_bw_probe_sink_bytes": (SZ, []),
        "kvc_bw_probe": (I32, [P, SZ, P, SZ, P]),
        "kvc_layer_budgets": (I32, [I32, I32, I32, ctypes.c_double, I32, P]),
        "kvc_paged_block_evict_workspace_bytes": (SZ, [D]),
        "kvc_paged_block_evict": (I32, [D, P, ctypes.c_double, D, P, P, P, I32, P, SZ, P]),
        "kvc_pool_create": (P, [I32, I32, U64]),
        "kvc_pool_destroy": (None, [P]),
        "kvc_pool_reserve": (I32, [P, I32, I32]),
        "kvc_pool_free": (I32, [P, I32]),
        "kvc_pool_release": (I32, [P, I32, P, I32]),
        "kvc_pool_num_free": (I32, [P]),
        "kvc_pool_num_blocks": (I32, [P, I32]),
        "kvc_pool_block_table": (I32, [P, P, I32, I32, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.kvc_last_error().decode()
        super().__init__(f"{where}: {lib.kvc_status_str(status).decode()}: {msg}")


def _check(status: int, where: str) -> None:
    if status != KVC_OK:
        raise KvcError(status, where)


def kvc_abi_version() -> int:
    return lib.kvc_abi_version()


def kvc_status_str(status: int) -> str:
    return lib.kvc_status_str(status).decode()


def kvc_last_error() -> str:
    return lib.kvc_last_error().decode()


def row_bytes(head_dim: int, bits: int) -> int:
    """Bytes of one token row of one KV head (codes only)."""
    return head_dim * bits // 8


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(t, dtype, name, numel=None):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")


class KVCache:
    """Device buffers of one compressed cache (one layer) and its descriptor.

    Contiguous layout (``block_size=0``): codes ``[B][Hkv][capacity][RB]`` uint8
    (RB = head_dim * bits / 8 for K, with ``v_bits`` (if set) for V),
    scales ``[B][Hkv][capacity]`` fp32, positions int32 of the same shape.
    Paged layout (``block_size=16``): codes ``[num_blocks][Hkv][16][RB]``,
    scales ``[num_blocks][Hkv][16]``, a ``[B][max_blocks]`` int32 block table,
    and no positions. ``lengths`` and ``num_seen`` are ``[B]`` int32.

    fp16 tiers (``fp16_sinks``, ``fp16_recent`` > 0): fp16 rows
    ``[B][Hkv][fp16_sinks][head_dim]`` of the first slots and a ring
    ``[B][Hkv][fp16_recent][head_dim]`` of the newest positions, attended at
    fp16. A compaction destination passes ``share_tiers_with=src`` so that both
    descriptors name the same tier buffers.
    """

    def __init__(self, batch: int, num_kv_heads: int, head_dim: int, capacity: int, bits: int = 8,
                 device="cuda", block_size: int = 0, num_blocks: int = 0, max_blocks_per_seq: int = 0,
                 positions: bool = True, v_bits: int = 0, fp16_sinks: int = 0, fp16_recent: int = 0,
                 share_tiers_with: "Optional[KVCache]" = None):
        import torch
        self.batch, self.num_kv_heads, self.head_dim, self.bits = batch, num_kv_heads, head_dim, bits
        self.v_bits = v_bits            # 0: V at the K width
        self.block_size = block_size
        rb = row_bytes(head_dim, bits)
        rbv = row_bytes(head_dim, v_bits or bits)
        if block_size:
            self.capacity = max_blocks_per_seq * block_size
            rows = (num_blocks, num_kv_heads, block_size)
            self.block_table = torch.full((batch, max_blocks_per_seq), -1, dtype=torch.int32, device=device)
            self.positions = None
        else:
            self.capacity = capacity
            rows = (batch, num_kv_heads, capacity)
            self.block_table = None
            self.positions = torch.zeros(rows, dtype=torch.int32, device=device) if positions else None
        self.num_blocks, self.max_blocks_per_seq = num_blocks, max_blocks_per_seq
        self.k_codes = torch.zeros(rows + (rb,), dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros(rows + (rbv,), dtype=torch.uint8, device=device)
        self.k_scale = torch.zeros(rows, dtype=torch.float32, device=device)
        self.v_scale = torch.zeros(rows, dtype=torch.float32, device=device)
        self.lengths = torch.zeros(batch, dtype=torch.int32, device=device)
        self.num_seen = torch.zeros(batch, dtype=torch.int32, device=device)
        if share_tiers_with is not None:
            o = share_tiers_with
            fp16_sinks, fp16_recent = o.fp16_sinks, o.fp16_recent
            self.k_sink16, self.v_sink16 = o.k_sink16, o.v_sink16
            self.k_recent16, self.v_recent16 = o.k_recent16, o.v_recent16
        else:
            def tier(n):
                return torch.zeros((batch, num_kv_heads, n, head_dim), dtype=torch.float16,
                                   device=device) if n else None
            self.k_sink16, self.v_sink16 = tier(fp16_sinks), tier(fp16_sinks)
            self.k_recent16, self.v_recent16 = tier(fp16_recent), tier(fp16_recent)
        self.fp16_sinks, self.fp16_recent = fp16_sinks, fp16_recent
        self.max_len = 0   # host-side upper bound of the device lengths
        self.desc = self._make_desc()

    def _make_desc(self) -> KvcCacheDesc:
        d = KvcCacheDesc()
        d.bits, d.batch, d.num_kv_heads, d.head_dim = self.bits, self.batch, self.num_kv_heads, self.head_dim
        d.v_bits = self.v_bits
        d.capacity, d.block_size = self.capacity, self.block_size
        d.max_blocks_per_seq, d.num_blocks = self.max_blocks_per_seq, self.num_blocks
        d.k_codes, d.v_codes = _ptr(self.k_codes), _ptr(self.v_codes)
        d.k_scale, d.v_scale = _ptr(self.k_scale), _ptr(self.v_scale)
        d.lengths, d.num_seen = _ptr(self.lengths), _ptr(self.num_seen)
        d.positions = _ptr(self.positions)
        d.block_table = _ptr(self.block_table)
        d.fp16_sinks, d.fp16_recent = self.fp16_sinks, self.fp16_recent
        d.k_sink16, d.v_sink16 = _ptr(self.k_sink16), _ptr(self.v_sink16)
        d.k_recent16, d.v_recent16 = _ptr(self.k_recent16), _ptr(self.v_recent16)
        return d

    def table_view(self):
        """A paged cache over the same pools with its own block table, lengths
        and num_seen: the destination of ``kvc_paged_block_evict``."""
        import copy
        import torch
        if not self.block_size:
            raise ValueError("table_view needs a paged cache")
        v = copy.copy(self)
        v.block_table = torch.full_like(self.block_table, -1)
        v.lengths = torch.zeros_like(self.lengths)
        v.num_seen = torch.zeros_like(self.num_seen)
        v.desc = v._make_desc()
        return v

    def score_buffer(self):
        """A zeroed fp32 H2O score array ``[B][Hkv][capacity]``."""
        import torch
        return torch.zeros((self.batch, self.num_kv_heads, self.capacity), dtype=torch.float32,
                           device=self.k_codes.device)


def _desc(cache) -> KvcCacheDesc:
    return cache.desc if isinstance(cache, KVCache) else cache


def kvc_quant_append(cache, k_new, v_new, h2o_score=None, max_len_hint: Optional[int] = None, stream=None):
    """Quantize ``k_new``/``v_new`` fp16 ``[B][Hkv][n][D]`` into the cache (see kvc.h)."""
    import torch
    d = _desc(cache)
    n_new = k_new.shape[2]
    _need(k_new, torch.float16, "k_new", d.batch * d.num_kv_heads * n_new * d.head_dim)
    _need(v_new, torch.float16, "v_new", d.batch * d.num_kv_heads * n_new * d.head_dim)
    _need(h2o_score, torch.float32, "h2o_score", d.batch * d.num_kv_heads * d.capacity)
    if max_len_hint is None:
        max_len_hint = cache.max_len
    _check(lib.kvc_quant_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new), n_new, _ptr(h2o_score),
                                max_len_hint, _stream(stream)), "kvc_quant_append")
    if isinstance(cache, KVCache):
        cache.max_len = max_len_hint + n_new


def kvc_decode_attn_workspace_bytes(cache, num_q_heads: int, max_len_hint: int, with_h2o: bool) -> int:
    return lib.kvc_decode_attn_workspace_bytes(ctypes.byref(_desc(cache)), num_q_heads, max_len_hint,
                                               int(bool(with_h2o)))


def kvc_decode_attn(cache, q, out, h2o_score=None, max_len_hint: Optional[int] = None, workspace=None,
                    stream=None):
    """Decode attention; ``q`` fp16 ``[B][Hq][D]``, ``out`` fp32 ``[B][Hq][D]`` (see kvc.h)."""
    import torch
    d = _desc(cache)
    Hq = q.shape[1]
    _need(q, torch.float16, "q", d.batch * Hq * d.head_dim)
    _need(out, torch.float32, "out", d.batch * Hq * d.head_dim)
    _need(h2o_score, torch.float32, "h2o_score", d.batch * d.num_kv_heads * d.capacity)
    if max_len_hint is None:
        max_len_hint = cache.max_len
    if workspace is None:
        n = kvc_decode_attn_workspace_bytes(d, Hq, max_len_hint, h2o_score is not None)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check(lib.kvc_decode_attn(ctypes.byref(d), _ptr(q), Hq, _ptr(out), _ptr(h2o_score), max_len_hint,
                               _ptr(workspace), workspace.numel(), _stream(stream)), "kvc_decode_attn")


def kvc_append_decode_attn(cache, k_new, v_new, q, out, h2o_score=None, max_len_hint: Optional[int] = None,
                           workspace=None, stream=None):
    """Append one token per sequence (``k_new``/``v_new`` fp16 ``[B][Hkv][1][D]``
    or ``[B][Hkv][D]``) and attend over the cache that includes it, in one call
    (see kvc.h). ``max_len_hint`` bounds the lengths before the append."""
    import torch
    d = _desc(cache)
    Hq = q.shape[1]
    _need(k_new, torch.float16, "k_new", d.batch * d.num_kv_heads * d.head_dim)
    _need(v_new, torch.float16, "v_new", d.batch * d.num_kv_heads * d.head_dim)
    _need(q, torch.float16, "q", d.batch * Hq * d.head_dim)
    _need(out, torch.float32, "out", d.batch * Hq * d.head_dim)
    _need(h2o_score, torch.float32, "h2o_score", d.batch * d.num_kv_heads * d.capacity)
    if max_len_hint is None:
        max_len_hint = cache.max_len
    if workspace is None:
        n = kvc_decode_attn_workspace_bytes(d, Hq, max_len_hint + 1, h2o_score is not None)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check(lib.kvc_append_decode_attn(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), Hq, _ptr(out),
                                      _ptr(h2o_score), max_len_hint, _ptr(workspace), workspace.numel(),
                                      _stream(stream)), "kvc_append_decode_attn")
    if isinstance(cache, KVCache):
        cache.max_len = max_len_hint + 1


def kvc_decode_attn_split(cache, q, workspace, k_new=None, v_new=None, h2o_score=None,
                          max_len_hint: Optional[int] = None, stream=None):
    """The split phase of the attention (with the new token's append when
    ``k_new``/``v_new`` are given); finish with ``kvc_decode_attn_merge``."""
    import torch
    d = _desc(cache)
    Hq = q.shape[1]
    _need(q, torch.float16, "q", d.batch * Hq * d.head_dim)
    _need(k_new, torch.float16, "k_new", d.batch * d.num_kv_heads * d.head_dim)
    _need(v_new, torch.float16, "v_new", d.batch * d.num_kv_heads * d.head_dim)
    _need(h2o_score, torch.float32, "h2o_score", d.batch * d.num_kv_heads * d.capacity)
    if max_len_hint is None:
        max_len_hint = cache.max_len
    _check(lib.kvc_decode_attn_split(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), Hq, _ptr(h2o_score),
                                     max_len_hint, _ptr(workspace), workspace.numel(), _stream(stream)),
           "kvc_decode_attn_split")


def kvc_decode_attn_merge(cache, num_q_heads: int, out, workspace, appended: bool = False, h2o_score=None,
                          max_len_hint: Optional[int] = None, stream=None):
    """The merge phase after ``kvc_decode_attn_split`` (see kvc.h)."""
    import torch
    d = _desc(cache)
    _need(out, torch.float32, "out", d.batch * num_q_heads * d.head_dim)
    _need(h2o_score, torch.float32, "h2o_score", d.batch * d.num_kv_heads * d.capacity)
    if max_len_hint is None:
        max_len_hint = cache.max_len
    _check(lib.kvc_decode_attn_merge(ctypes.byref(d), int(bool(appended)), num_q_heads, _ptr(out), _ptr(h2o_score),
                                     max_len_hint, _ptr(workspace), workspace.numel(), _stream(stream)),
           "kvc_decode_attn_merge")
    if appended and isinstance(cache, KVCache):
        cache.max_len = max_len_hint + 1


def kvc_h2o_select(cache, h2o_score, budget: int, n_sink: int, n_recent: int, keep_mask, keep_index=None,
                   max_len_hint: Optional[int] = None, stream=None):
    """Keep mask uint8 ``[B][Hkv][capacity]`` (and optionally the ascending keep
    list int32 ``[B][Hkv][budget]``): sinks + recent + top-k by score (see kvc.h)."""
    import torch
    d = _desc(cache)
    _need(h2o_score, torch.float32, "h2o_score", d.batch * d.num_kv_heads * d.capacity)
    _need(keep_mask, torch.uint8, "keep_mask", d.batch * d.num_kv_heads * d.capacity)
    _need(keep_index, torch.int32, "keep_index", d.batch * d.num_kv_heads * budget)
    if max_len_hint is None:
        max_len_hint = cache.max_len
    _check(lib.kvc_h2o_select(ctypes.byref(d), _ptr(h2o_score), budget, n_sink, n_recent, _ptr(keep_mask),
                              _ptr(keep_index), max_len_hint, _stream(stream)), "kvc_h2o_select")


def kvc_compact_workspace_bytes(cache, max_len_hint: int) -> int:
    return lib.kvc_compact_workspace_bytes(ctypes.byref(_desc(cache)), max_len_hint)


def kvc_compact(src, src_score, keep_mask, dst, dst_score=None, max_len_hint: Optional[int] = None,
                workspace=None, stream=None):
    """Stable out-of-place compaction of the kept slots from ``src`` to ``dst`` (see kvc.h)."""
    import torch
    ds, dd = _desc(src), _desc(dst)
    _need(src_score, torch.float32, "src_score", ds.batch * ds.num_kv_heads * ds.capacity)
    _need(dst_score, torch.float32, "dst_score", dd.batch * dd.num_kv_heads * dd.capacity)
    _need(keep_mask, torch.uint8, "keep_mask", ds.batch * ds.num_kv_heads * ds.capacity)
    if max_len_hint is None:
        max_len_hint = src.max_len
    if workspace is None:
        n = kvc_compact_workspace_bytes(ds, max_len_hint)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=keep_mask.device)
    _check(lib.kvc_compact(ctypes.byref(ds), _ptr(src_score), _ptr(keep_mask), ctypes.byref(dd), _ptr(dst_score),
                           max_len_hint, _ptr(workspace), workspace.numel(), _stream(stream)), "kvc_compact")
    if isinstance(dst, KVCache) and isinstance(src, KVCache):
        dst.max_len = src.max_len


def kvc_compact_gather(src, src_score, keep_index, n_keep: int, dst, dst_score=None, stream=None):
    """Compaction from the ascending keep list ``[B][Hkv][n_keep]`` (see kvc.h)."""
    import torch
    ds, dd = _desc(src), _desc(dst)
    _need(src_score, torch.float32, "src_score", ds.batch * ds.num_kv_heads * ds.capacity)
    _need(dst_score, torch.float32, "dst_score", dd.batch * dd.num_kv_heads * dd.capacity)
    _need(keep_index, torch.int32, "keep_index", ds.batch * ds.num_kv_heads * n_keep)
    _check(lib.kvc_compact_gather(ctypes.byref(ds), _ptr(src_score), _ptr(keep_index), n_keep, ctypes.byref(dd),
                                  _ptr(dst_score), _stream(stream)), "kvc_compact_gather")
    if isinstance(dst, KVCache) and isinstance(src, KVCache):
        dst.max_len = min(src.max_len, n_keep)


def kvc_h2o_evict(src, h2o_score, budget: int, n_sink: int, n_recent: int, keep_index, dst, dst_score=None,
                  keep_mask=None, max_len_hint: Optional[int] = None, stream=None):
    """Selection and compaction in one call: the keep set of ``kvc_h2o_select``
    copied into ``dst`` as ``kvc_compact_gather`` copies it (see kvc.h)."""
    import torch
    ds, dd = _desc(src), _desc(dst)
    _need(h2o_score, torch.float32, "h2o_score", ds.batch * ds.num_kv_heads * ds.capacity)
    _need(dst_score, torch.float32, "dst_score", dd.batch * dd.num_kv_heads * dd.capacity)
    _need(keep_index, torch.int32, "keep_index", ds.batch * ds.num_kv_heads * budget)
    _need(keep_mask, torch.uint8, "keep_mask", ds.batch * ds.num_kv_heads * ds.capacity)
    if max_len_hint is None:
        max_len_hint = src.max_len
    _check(lib.kvc_h2o_evict(ctypes.byref(ds), _ptr(h2o_score), budget, n_sink, n_recent, _ptr(keep_mask),
                             _ptr(keep_index), ctypes.byref(dd), _ptr(dst_score), max_len_hint, _stream(stream)),
           "kvc_h2o_evict")
    if isinstance(dst, KVCache) and isinstance(src, KVCache):
        dst.max_len = min(src.max_len, budget)


def kvc_decode_step(cache, k_new, v_new, q, out, h2o_score, budget: int, n_sink: int, n_recent: int, keep_index,
                    dst, dst_score, keep_mask=None, max_len_hint: Optional[int] = None, workspace=None, stream=None):
    """A whole decode step in one call (see kvc.h): append the new token,
    attend with H2O, evict from ``cache`` into ``dst`` (``dst_score`` receives
    the kept tokens' accumulated scores)."""
    import torch
    d, dd = _desc(cache), _desc(dst)
    Hq = q.shape[1]
    _need(k_new, torch.float16, "k_new", d.batch * d.num_kv_heads * d.head_dim)
    _need(v_new, torch.float16, "v_new", d.batch * d.num_kv_heads * d.head_dim)
    _need(q, torch.float16, "q", d.batch * Hq * d.head_dim)
    _need(out, torch.float32, "out", d.batch * Hq * d.head_dim)
    _need(h2o_score, torch.float32, "h2o_score", d.batch * d.num_kv_heads * d.capacity)
    _need(dst_score, torch.float32, "dst_score", dd.batch * dd.num_kv_heads * dd.capacity)
    _need(keep_index, torch.int32, "keep_index", d.batch * d.num_kv_heads * budget)
    _need(keep_mask, torch.uint8, "keep_mask", d.batch * d.num_kv_heads * d.capacity)
    if max_len_hint is None:
        max_len_hint = cache.max_len
    if workspace is None:
        n = kvc_decode_attn_workspace_bytes(d, Hq, max_len_hint + 1, True)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check(lib.kvc_decode_step(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), Hq, _ptr(out), _ptr(h2o_score),
                               budget, n_sink, n_recent, _ptr(keep_mask), _ptr(keep_index), ctypes.byref(dd),
                               _ptr(dst_score), max_len_hint, _ptr(workspace), workspace.numel(), _stream(stream)),
           "kvc_decode_step")
    if isinstance(cache, KVCache):
        cache.max_len = max_len_hint + 1
    if isinstance(dst, KVCache):
        dst.max_len = min(max_len_hint + 1, budget)


def kvc_decode_step_noalloc_max_bytes() -> int:
    return lib.kvc_decode_step_noalloc_max_bytes()


def kvc_decode_step_noalloc(cache, k_new, v_new, q, out, h2o_score, budget: int, n_sink: int, n_recent: int,
                            keep_index, dst, dst_score, keep_mask=None, max_len_hint: Optional[int] = None,
                            stream=None):
    """``kvc_decode_step`` with the library's static device scratch as its
    workspace: allocates nothing (see kvc.h)."""
    import torch
    d, dd = _desc(cache), _desc(dst)
    Hq = q.shape[1]
    _need(k_new, torch.float16, "k_new", d.batch * d.num_kv_heads * d.head_dim)
    _need(v_new, torch.float16, "v_new", d.batch * d.num_kv_heads * d.head_dim)
    _need(q, torch.float16, "q", d.batch * Hq * d.head_dim)
    _need(out, torch.float32, "out", d.batch * Hq * d.head_dim)
    _need(h2o_score, torch.float32, "h2o_score", d.batch * d.num_kv_heads * d.capacity)
    _need(dst_score, torch.float32, "dst_score", dd.batch * dd.num_kv_heads * dd.capacity)
    _need(keep_index, torch.int32, "keep_index", d.batch * d.num_kv_heads * budget)
    _need(keep_mask, torch.uint8, "keep_mask", d.batch * d.num_kv_heads * d.capacity)
    if max_len_hint is None:
        max_len_hint = cache.max_len
    _check(lib.kvc_decode_step_noalloc(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), Hq, _ptr(out),
                                       _ptr(h2o_score), budget, n_sink, n_recent, _ptr(keep_mask), _ptr(keep_index),
                                       ctypes.byref(dd), _ptr(dst_score), max_len_hint, _stream(stream)),
           "kvc_decode_step_noalloc")
    if isinstance(cache, KVCache):
        cache.max_len = max_len_hint + 1
    if isinstance(dst, KVCache):
        dst.max_len = min(max_len_hint + 1, budget)


def kvc_paged_block_evict_workspace_bytes(src) -> int:
    return lib.kvc_paged_block_evict_workspace_bytes(ctypes.byref(_desc(src)))


def kvc_paged_block_evict(src, h2o_score, retention: float, dst, dst_score, freed, freed_count,
                          max_len_hint: Optional[int] = None, workspace=None, stream=None):
    """Block-granular H2O eviction on a paged cache (see kvc.h): ``dst`` shares
    ``src``'s pools (``src.table_view()``); ``freed`` int32 ``[B][max_blocks]``
    and ``freed_count`` int32 ``[B]`` receive the released physical blocks."""
    import torch
    ds, dd = _desc(src), _desc(dst)
    if workspace is None:
        n = kvc_paged_block_evict_workspace_bytes(ds)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=h2o_score.device)
    _need(h2o_score, torch.float32, "h2o_score", ds.batch * ds.num_kv_heads * ds.capacity)
    _need(dst_score, torch.float32, "dst_score", dd.batch * dd.num_kv_heads * dd.capacity)
    _need(freed, torch.int32, "freed", ds.batch * ds.max_blocks_per_seq)
    _need(freed_count, torch.int32, "freed_count", ds.batch)
    if max_len_hint is None:
        max_len_hint = src.max_len
    _check(lib.kvc_paged_block_evict(ctypes.byref(ds), _ptr(h2o_score), float(retention), ctypes.byref(dd),
                                     _ptr(dst_score), _ptr(freed), _ptr(freed_count), max_len_hint,
                                     _ptr(workspace), workspace.numel(), _stream(stream)), "kvc_paged_block_evict")
    if isinstance(dst, KVCache) and isinstance(src, KVCache):
        dst.max_len = src.max_len


KVC_SCHEDULE_LINEAR, KVC_SCHEDULE_QUADRATIC = 0, 1


def kvc_layer_budgets(schedule: int, num_layers: int, base: int, base_ratio: float = 0.0,
                      min_budget: int = 0) -> list:
    """Per-layer keep budgets of a pyramid schedule (see kvc.h), as a list."""
    out = (ctypes.c_int32 * max(num_layers, 1))()
    _check(lib.kvc_layer_budgets(schedule, num_layers, base, float(base_ratio), min_budget, out),
           "kvc_layer_budgets")
    return list(out)[:num_layers]


def kvc_decode_attn_kvsep_workspace_bytes(cache, num_q_heads: int, top_k: int, max_len_hint: int) -> int:
    return lib.kvc_decode_attn_kvsep_workspace_bytes(ctypes.byref(_desc(cache)), num_q_heads, top_k, max_len_hint)


def kvc_decode_attn_kvsep(cache, q, top_k: int, v_host, out, max_len_hint: Optional[int] = None, workspace=None,
                          stream=None):
    """K/V-separated attention (see kvc.h): scores on the cache's quantized K,
    the output from the top_k tokens' fp16 V rows per KV head, hot rows from
    the cache's fp16 tiers and cold rows from ``v_host``, a pinned CPU fp16
    tensor ``[B][Hkv][capacity][D]`` indexed by slot."""
    import torch
    d = _desc(cache)
    Hq = q.shape[1]
    _need(q, torch.float16, "q", d.batch * Hq * d.head_dim)
    _need(out, torch.float32, "out", d.batch * Hq * d.head_dim)
    if v_host.device.type != "cpu" or not v_host.is_pinned() or v_host.dtype != torch.float16 \
            or not v_host.is_contiguous() or v_host.numel() != d.batch * d.num_kv_heads * d.capacity * d.head_dim:
        raise ValueError("v_host must be a contiguous pinned CPU fp16 tensor [B][Hkv][capacity][D]")
    if max_len_hint is None:
        max_len_hint = cache.max_len
    if workspace is None:
        n = kvc_decode_attn_kvsep_workspace_bytes(d, Hq, top_k, max_len_hint)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check(lib.kvc_decode_attn_kvsep(ctypes.byref(d), _ptr(q), Hq, top_k, v_host.data_ptr(), _ptr(out),
                                     max_len_hint, _ptr(workspace), workspace.numel(), _stream(stream)),
           "kvc_decode_attn_kvsep")


def kvc_bw_probe_sink_bytes() -> int:
    return lib.kvc_bw_probe_sink_bytes()


def kvc_bw_probe(src, sink, stream=None):
    """One streaming read of the device tensor ``src`` (see kvc.h); ``sink`` is
    a device uint8 tensor of ``kvc_bw_probe_sink_bytes()`` bytes."""
    _check(lib.kvc_bw_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                            sink.numel() * sink.element_size(), _stream(stream)), "kvc_bw_probe")


class BlockPool:
    """Host block pool (``kvc_pool_*``): seeded block placement and block tables."""

    def __init__(self, num_blocks: int, block_size: int = 16, shuffle_seed: int = 0):
        self._p = lib.kvc_pool_create(num_blocks, block_size, shuffle_seed)
        if not self._p:
            raise KvcError(KVC_ERR_INVALID_ARG, "kvc_pool_create")
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self):
        if self._p:
            lib.kvc_pool_destroy(self._p)
            self._p = None

    __del__ = close

    def reserve(self, seq_id: int, num_tokens: int) -> None:
        _check(lib.kvc_pool_reserve(self._p, seq_id, num_tokens), "kvc_pool_reserve")

    def free(self, seq_id: int) -> None:
        _check(lib.kvc_pool_free(self._p, seq_id), "kvc_pool_free")

    def release(self, seq_id: int, blocks) -> None:
        """Give back the listed blocks of a sequence (refcounted, all or nothing)."""
        arr = (ctypes.c_int32 * max(len(blocks), 1))(*[int(x) for x in blocks])
        _check(lib.kvc_pool_release(self._p, seq_id, arr, len(blocks)), "kvc_pool_release")

    @property
    def num_free(self) -> int:
        return lib.kvc_pool_num_free(self._p)

    def num_blocks_of(self, seq_id: int) -> int:
        return lib.kvc_pool_num_blocks(self._p, seq_id)

    def block_table(self, seq_ids: Sequence[int], max_blocks: int):
        """``[len(seq_ids)][max_blocks]`` int32 host table (a numpy array)."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))
        table = np.empty((len(ids), max_blocks), dtype=np.int32)
        _check(lib.kvc_pool_block_table(self._p, ids.ctypes.data, len(ids), max_blocks, table.ctypes.data),
               "kvc_pool_block_table")
        return table
