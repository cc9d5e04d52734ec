// libkvc entry points: host-side validation, workspace sizing and launches.
//
// Every entry point checks its arguments before touching the GPU, so each
// error status is returned with nothing enqueued. No entry point allocates
// device memory or synchronizes.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "kvc_internal.h"

namespace kvc {

namespace {
thread_local std::string g_last_error;
}

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int device_cus() {
  constexpr int kMaxDev = 64, kDefault = 256;
  static std::mutex m;
  static int cus[kMaxDev];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return kDefault;
  }
  std::lock_guard<std::mutex> lock(m);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      n = kDefault;
    }
    cus[dev] = n;
  }
  return cus[dev];
}

namespace {

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int32_t device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVC_OK;
  return fail(KVC_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Shape and pointer checks shared by every device call.
int32_t check_cache(const kvc_cache_t* c, const char* name) {
  if (!c) return fail(KVC_ERR_INVALID_ARG, "%s is NULL", name);
  if (c->bits != 8 && c->bits != 4) return fail(KVC_ERR_INVALID_ARG, "%s: bits must be 8 or 4 (got %d)", name, c->bits);
  if (c->v_bits != 0 && c->v_bits != 8 && c->v_bits != 4)
    return fail(KVC_ERR_INVALID_ARG, "%s: v_bits must be 0, 8 or 4 (got %d)", name, c->v_bits);
  if (c->batch < 1 || c->num_kv_heads < 1)
    return fail(KVC_ERR_INVALID_ARG, "%s: batch and num_kv_heads must be >= 1", name);
  if (c->head_dim != 64 && c->head_dim != 128) {
    if (c->head_dim > 0 && c->head_dim % 16 == 0 && c->head_dim <= 256)
      return fail(KVC_ERR_UNSUPPORTED, "%s: head_dim %d is not built (64 and 128 are)", name, c->head_dim);
    return fail(KVC_ERR_INVALID_ARG, "%s: head_dim must be a multiple of 16 in [16, 256]", name);
  }
  if (c->capacity < 1) return fail(KVC_ERR_INVALID_ARG, "%s: capacity must be >= 1", name);
  if (!c->k_codes || !c->v_codes || !c->k_scale || !c->v_scale || !c->lengths || !c->num_seen)
    return fail(KVC_ERR_INVALID_ARG, "%s: NULL buffer in the descriptor", name);
  if (c->block_size == 0) {
    if (c->block_table) return fail(KVC_ERR_INVALID_ARG, "%s: contiguous cache with a block table", name);
    if ((long long)c->batch * c->num_kv_heads * c->capacity > (1LL << 40))
      return fail(KVC_ERR_INVALID_ARG, "%s: cache too large", name);
  } else if (c->block_size == 16) {
    if (!c->block_table || c->max_blocks_per_seq < 1 || c->num_blocks < 1)
      return fail(KVC_ERR_INVALID_ARG, "%s: paged cache needs a block table, max_blocks_per_seq and num_blocks", name);
    if ((long long)c->max_blocks_per_seq * c->block_size != c->capacity)
      return fail(KVC_ERR_INVALID_ARG, "%s: paged capacity must equal max_blocks_per_seq * block_size", name);
    if (c->positions) return fail(KVC_ERR_INVALID_ARG, "%s: paged caches keep no positions", name);
  } else {
    return fail(KVC_ERR_UNSUPPORTED, "%s: block_size must be 0 (contiguous) or 16 (got %d)", name, c->block_size);
  }
  if (c->fp16_sinks < 0 || c->fp16_recent < 0)
    return fail(KVC_ERR_INVALID_ARG, "%s: fp16_sinks and fp16_recent must be >= 0", name);
  if ((c->fp16_sinks && (!c->k_sink16 || !c->v_sink16)) || (c->fp16_recent && (!c->k_recent16 || !c->v_recent16)))
    return fail(KVC_ERR_INVALID_ARG, "%s: NULL fp16 tier buffer", name);
  if (((uintptr_t)c->k_sink16 | (uintptr_t)c->v_sink16 | (uintptr_t)c->k_recent16 | (uintptr_t)c->v_recent16) % 16)
    return fail(KVC_ERR_INVALID_ARG, "%s: fp16 tier buffers must be 16-byte aligned", name);
  return KVC_OK;
}

bool tiered(const kvc_cache_t* c) { return c->fp16_sinks > 0 || c->fp16_recent > 0; }

// The tier kernels copy new rows 16 bytes at a time.
int32_t check_tier_inputs(const kvc_cache_t* c, const void* k_new, const void* v_new) {
  if (tiered(c) && (((uintptr_t)k_new | (uintptr_t)v_new) % 16))
    return fail(KVC_ERR_INVALID_ARG, "with fp16 tiers, k_new and v_new must be 16-byte aligned");
  return KVC_OK;
}

// Eviction keeps the fp16 tiers whole only if the sink and recent counts cover
// them (the tiers are the first and the newest slots of a row).
int32_t check_tiers_kept(const kvc_cache_t* c, int32_t n_sink, int32_t n_recent) {
  if (n_sink < c->fp16_sinks || n_recent < c->fp16_recent)
    return fail(KVC_ERR_INVALID_ARG, "eviction must keep the fp16 tiers (n_sink %d >= fp16_sinks %d, n_recent %d >= "
                "fp16_recent %d)", n_sink, c->fp16_sinks, n_recent, c->fp16_recent);
  return KVC_OK;
}

// A compaction's destination uses the source's fp16 tier buffers.
int32_t check_same_tiers(const kvc_cache_t* src, const kvc_cache_t* dst) {
  if (src->fp16_sinks != dst->fp16_sinks || src->fp16_recent != dst->fp16_recent ||
      (src->fp16_sinks && (src->k_sink16 != dst->k_sink16 || src->v_sink16 != dst->v_sink16)) ||
      (src->fp16_recent && (src->k_recent16 != dst->k_recent16 || src->v_recent16 != dst->v_recent16)))
    return fail(KVC_ERR_INVALID_ARG, "src and dst must name the same fp16 tiers");
  return KVC_OK;
}

struct AttnGeom {
  int splits, tiles, last_tiles, tier_parts;
  size_t off_ml, off_logits, off_stash, off_ip, total;
};

// Launch geometry of the decode-attention kernels. A split covers `tiles`
// 256-token tiles (one 64-token block per wave per tile); tiles are grouped so
// that the grid has about two workgroups per CU (512 on MI355X's 256 CUs, all
// resident); longer contexts loop over tiles.
int32_t attn_geometry(const kvc_cache_t* c, int32_t Hq, int32_t hint, int32_t with_h2o, AttnGeom* g) {
  int32_t st = check_cache(c, "cache");
  if (st) return st;
  if (Hq < 1 || Hq % c->num_kv_heads) return fail(KVC_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  const int G = Hq / c->num_kv_heads;
  if (G > 16) return fail(KVC_ERR_INVALID_ARG, "more than 16 query heads per KV head");
  if (hint < 1) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 1");
  if (hint > c->capacity) return fail(KVC_ERR_CAPACITY, "max_len_hint %d exceeds capacity %d", hint, c->capacity);
  const long long rb = std::max(k_row_bytes(*c), v_row_bytes(*c));
  if ((long long)c->capacity * rb >= (1LL << 32) - 4096)
    return fail(KVC_ERR_UNSUPPORTED, "one (sequence, KV head) row must stay below 4 GiB");
  if (c->block_size && (long long)c->num_blocks * c->num_kv_heads * c->block_size * rb >= (1LL << 32))
    return fail(KVC_ERR_UNSUPPORTED, "paged pools must stay below 4 GiB of codes");
  const long long tiles_total = (hint + kSplitTokens - 1) / kSplitTokens;
  const long long rows = (long long)c->batch * c->num_kv_heads;
  const long long target = 2LL * device_cus();
  const long long nt = std::max(1LL, tiles_total * rows / target);
  long long S = (tiles_total + nt - 1) / nt;
  // When the last splits of the rows would spill into a second round of
  // workgroups (a row just past a multiple of the split size, e.g. a budget
  // plus the appended token), the last split takes the remainder instead, up
  // to half a split more.
  const long long s_fit = std::max(1LL, target / rows);
  if (S > s_fit && tiles_total - (s_fit - 1) * nt <= nt + (nt + 1) / 2) S = s_fit;
  const long long last = tiles_total - (S - 1) * nt;
  // fp16 tiers: one extra partial state per 64 tier tokens, after the splits.
  const long long tier_tok = std::min<long long>((long long)c->fp16_sinks + c->fp16_recent, hint);
  const long long TP = (tier_tok + kTierTokens - 1) / kTierTokens;
  const long long P = S + TP;
  if (P * (G + 2) > 16384) return fail(KVC_ERR_UNSUPPORTED, "too many splits for one KV head (%lld x %d)", P, G);
  const size_t BH = (size_t)c->batch * Hq;
  const size_t part_o = align256(BH * P * c->head_dim * sizeof(float));
  const size_t part_ml = align256(BH * P * 2 * sizeof(float));
  const size_t logits = with_h2o ? align256(BH * ((S - 1) * nt + last) * kSplitTokens * sizeof(float)) : 0;
  g->splits = (int)S;
  g->tiles = (int)nt;
  g->last_tiles = (int)last;
  g->tier_parts = (int)TP;
  g->off_ml = part_o;
  g->off_logits = part_o + part_ml;
  g->off_stash = part_o + part_ml + logits;
  g->off_ip = g->off_stash + align256(2 * (size_t)c->batch * sizeof(int32_t));
  // With H2O (a decode step may follow), room for the control words of an
  // in-place eviction to any budget up to the capacity.
  const size_t ip_words = with_h2o && !c->block_size ? evict_inplace_words_bound(*c, c->capacity) : 0;
  g->total = g->off_ip + align256(ip_words * sizeof(int32_t));
  return KVC_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Compaction is out of place: no destination buffer (nor the workspace) may
// overlap any source buffer, the keep mask or list, or the source scores.
int32_t check_out_of_place(const kvc_cache_t* src, const float* src_score, const void* keep, size_t keep_bytes,
                           const kvc_cache_t* dst, const float* dst_score, const void* workspace, size_t ws_bytes) {
  const size_t rows = (size_t)src->batch * src->num_kv_heads * src->capacity;
  const size_t RBK = k_row_bytes(*src), RBV = v_row_bytes(*src);
  const void* s_bufs[] = {src->k_codes, src->v_codes, src->k_scale, src->v_scale, src->positions, src_score,
                          keep, src->lengths, src->num_seen};
  const size_t s_len[] = {rows * RBK, rows * RBV, rows * 4, rows * 4, rows * 4, rows * 4, keep_bytes,
                          (size_t)src->batch * 4, (size_t)src->batch * 4};
  const void* d_bufs[] = {dst->k_codes, dst->v_codes, dst->k_scale, dst->v_scale, dst->positions, dst_score,
                          dst->lengths, dst->num_seen, workspace};
  const size_t d_len[] = {rows * RBK, rows * RBV, rows * 4, rows * 4, rows * 4, rows * 4, (size_t)src->batch * 4,
                          (size_t)src->batch * 4, ws_bytes};
  for (int i = 0; i < 9; ++i)
    for (int j = 0; j < 9; ++j)
      if (overlap(s_bufs[i], s_len[i], d_bufs[j], d_len[j]))
        return fail(KVC_ERR_INVALID_ARG, "dst buffer %d overlaps src buffer %d (compaction is out of place)", j, i);
  return KVC_OK;
}

// Shared checks of both compaction entry points.
int32_t check_compact_pair(const kvc_cache_t* src, const kvc_cache_t* dst, const float* src_score,
                           const float* dst_score) {
  int32_t st = check_cache(src, "src");
  if (st) return st;
  if ((st = check_cache(dst, "dst"))) return st;
  if (src->block_size || dst->block_size) return fail(KVC_ERR_UNSUPPORTED, "compaction of paged caches is not built");
  if (src->bits != dst->bits || vbits_of(*src) != vbits_of(*dst) || src->batch != dst->batch ||
      src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim || src->capacity != dst->capacity)
    return fail(KVC_ERR_INVALID_ARG, "src and dst geometries differ");
  if ((st = check_same_tiers(src, dst))) return st;
  if ((src_score == nullptr) != (dst_score == nullptr))
    return fail(KVC_ERR_INVALID_ARG, "pass both src_score and dst_score, or neither");
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" {

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_status_str(int32_t s) {
  switch (s) {
    case KVC_OK: return "KVC_OK";
    case KVC_ERR_INVALID_ARG: return "KVC_ERR_INVALID_ARG";
    case KVC_ERR_CAPACITY: return "KVC_ERR_CAPACITY";
    case KVC_ERR_UNSUPPORTED: return "KVC_ERR_UNSUPPORTED";
    case KVC_ERR_DEVICE: return "KVC_ERR_DEVICE";
    default: return "KVC_UNKNOWN";
  }
}

const char* kvc_last_error(void) { return g_last_error.c_str(); }

int32_t kvc_quant_append(const kvc_cache_t* cache, const void* k_new, const void* v_new, int32_t n_new,
                         float* h2o_score, int32_t max_len_hint, void* stream) {
  clear_error();
  int32_t st = check_cache(cache, "cache");
  if (st) return st;
  if (!k_new || !v_new) return fail(KVC_ERR_INVALID_ARG, "k_new and v_new must not be NULL");
  if (n_new < 1) return fail(KVC_ERR_INVALID_ARG, "n_new must be >= 1");
  if (max_len_hint < 0) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 0");
  if ((long long)max_len_hint + n_new > cache->capacity)
    return fail(KVC_ERR_CAPACITY, "max_len_hint %d + n_new %d exceeds capacity %d", max_len_hint, n_new,
                cache->capacity);
  if ((st = check_tier_inputs(cache, k_new, v_new))) return st;
  return device_status(launch_quant_append(*cache, static_cast<const __half*>(k_new),
                                           static_cast<const __half*>(v_new), n_new, h2o_score,
                                           static_cast<hipStream_t>(stream)),
                       "kvc_quant_append launch");
}

size_t kvc_decode_attn_workspace_bytes(const kvc_cache_t* cache, int32_t num_q_heads, int32_t max_len_hint,
                                       int32_t with_h2o) {
  AttnGeom g;
  if (attn_geometry(cache, num_q_heads, max_len_hint, with_h2o, &g)) return 0;
  return g.total;
}

}  // extern "C"

namespace kvc {
namespace {

// Validation and launch arguments shared by the attention entry points;
// `span_hint` is the largest length the attention sees (after the append, if
// any).
int32_t prepare_attn(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                     int32_t num_q_heads, float* out, float* h2o_score, int32_t span_hint, void* workspace,
                     size_t workspace_bytes, AttnLaunch* a) {
  AttnGeom g;
  int32_t st = attn_geometry(cache, num_q_heads, span_hint, h2o_score != nullptr, &g);
  if (st) return st;
  if (!q || !out) return fail(KVC_ERR_INVALID_ARG, "q and out must not be NULL");
  if (!workspace || workspace_bytes < g.total)
    return fail(KVC_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", g.total, workspace ? workspace_bytes : 0);
  if ((uintptr_t)workspace % 256) return fail(KVC_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if ((st = check_tier_inputs(cache, k_new, v_new))) return st;
  a->c = *cache;
  a->q = static_cast<const __half*>(q);
  a->out = out;
  a->score = h2o_score;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a->part_o = reinterpret_cast<float*>(ws);
  a->part_ml = reinterpret_cast<float*>(ws + g.off_ml);
  a->logits = h2o_score ? reinterpret_cast<float*>(ws + g.off_logits) : nullptr;
  a->k_new = static_cast<const __half*>(k_new);
  a->v_new = static_cast<const __half*>(v_new);
  a->stash = reinterpret_cast<int32_t*>(ws + g.off_stash);
  a->append = k_new != nullptr;
  a->num_q_heads = num_q_heads;
  a->splits = g.splits;
  a->tiles = g.tiles;
  a->last_tiles = g.last_tiles;
  a->tier_parts = g.tier_parts;
  a->parts = g.splits + g.tier_parts;
  a->qk_log2 = (float)(1.4426950408889634 / sqrt((double)cache->head_dim));
  a->zero_words = nullptr;
  a->zero_count = 0;
  // One tier part, one query head per KV head and a contiguous cache (the
  // split kernel variant that holds the tier code): the split kernel computes it.
  a->fold_tier = g.tier_parts == 1 && num_q_heads == cache->num_kv_heads && cache->block_size == 0;
  return KVC_OK;
}

int32_t decode_attn_call(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                         int32_t num_q_heads, float* out, float* h2o_score, int32_t span_hint, void* workspace,
                         size_t workspace_bytes, void* stream) {
  AttnLaunch a;
  const int32_t st = prepare_attn(cache, k_new, v_new, q, num_q_heads, out, h2o_score, span_hint, workspace,
                                  workspace_bytes, &a);
  if (st) return st;
  return device_status(launch_decode_attn(a, static_cast<hipStream_t>(stream)), "decode attention launch");
}

// The step's workspace (written by the split kernel, read by the eviction
// kernel) may overlap no buffer of either cache, their scores, nor the keep
// list or mask.
int32_t check_workspace_disjoint(const void* ws, size_t ws_bytes, const kvc_cache_t* c, const float* c_score,
                                 const kvc_cache_t* d, const float* d_score, const void* keep_index,
                                 size_t keep_bytes, const void* keep_mask, size_t mask_bytes) {
  const size_t rows = (size_t)c->batch * c->num_kv_heads * c->capacity;
  const size_t RBK = k_row_bytes(*c), RBV = v_row_bytes(*c);
  const void* bufs[] = {c->k_codes, c->v_codes, c->k_scale, c->v_scale, c->positions, c_score, c->lengths,
                        c->num_seen, d->k_codes, d->v_codes, d->k_scale, d->v_scale, d->positions, d_score,
                        d->lengths, d->num_seen, keep_index, keep_mask};
  const size_t lens[] = {rows * RBK, rows * RBV, rows * 4, rows * 4, rows * 4, rows * 4, (size_t)c->batch * 4,
                         (size_t)c->batch * 4, rows * RBK, rows * RBV, rows * 4, rows * 4, rows * 4, rows * 4,
                         (size_t)c->batch * 4, (size_t)c->batch * 4, keep_bytes, mask_bytes};
  for (int i = 0; i < 18; ++i)
    if (overlap(ws, ws_bytes, bufs[i], lens[i]))
      return fail(KVC_ERR_INVALID_ARG, "the workspace overlaps buffer %d of the caches, scores or keep outputs", i);
  return KVC_OK;
}

// Checks of the eviction arguments shared by kvc_h2o_evict and kvc_decode_step
// (`max_len` is the largest length the eviction sees).
int32_t check_evict(const kvc_cache_t* src, const float* h2o_score, int32_t budget, int32_t n_sink, int32_t n_recent,
                    const uint8_t* keep_mask, const int32_t* keep_index, const kvc_cache_t* dst,
                    const float* dst_score, int32_t max_len, const void* workspace, size_t ws_bytes,
                    bool in_place = false) {
  int32_t st = check_compact_pair(src, dst, nullptr, nullptr);
  if (st) return st;
  if (!h2o_score || !keep_index) return fail(KVC_ERR_INVALID_ARG, "h2o_score and keep_index must not be NULL");
  if (budget < 1) return fail(KVC_ERR_INVALID_ARG, "budget must be >= 1");
  if (n_sink < 0 || n_recent < 0) return fail(KVC_ERR_INVALID_ARG, "n_sink and n_recent must be >= 0");
  if ((long long)n_sink + n_recent > budget) return fail(KVC_ERR_INVALID_ARG, "n_sink + n_recent exceeds budget");
  if ((st = check_tiers_kept(src, n_sink, n_recent))) return st;
  if (budget > src->capacity) return fail(KVC_ERR_CAPACITY, "budget exceeds capacity");
  if (max_len < 0) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 0");
  if (max_len > src->capacity) return fail(KVC_ERR_CAPACITY, "max_len_hint exceeds capacity");
  const size_t rows = (size_t)src->batch * src->num_kv_heads;
  if (in_place) {
    // The cache is its own destination: every dst buffer is the cache's; the
    // keep outputs (written during the step) overlap none of them.
    const bool same = dst->k_codes == src->k_codes && dst->v_codes == src->v_codes && dst->k_scale == src->k_scale &&
                      dst->v_scale == src->v_scale && dst->positions == src->positions &&
                      dst->lengths == src->lengths && dst->num_seen == src->num_seen && dst_score == h2o_score;
    if (!same)
      return fail(KVC_ERR_INVALID_ARG, "in place, every dst buffer must be the cache's own and dst_score h2o_score");
    const size_t slots = rows * src->capacity;
    const void* bufs[] = {src->k_codes, src->v_codes, src->k_scale, src->v_scale, src->positions, h2o_score,
                          src->lengths, src->num_seen, keep_mask};
    const size_t lens[] = {slots * k_row_bytes(*src), slots * v_row_bytes(*src), slots * 4, slots * 4, slots * 4,
                           slots * 4, (size_t)src->batch * 4, (size_t)src->batch * 4, keep_mask ? slots : 0};
    for (int i = 0; i < 9; ++i) {
      if (overlap(keep_index, rows * budget * sizeof(int32_t), bufs[i], lens[i]) ||
          (i < 8 && overlap(keep_mask, keep_mask ? slots : 0, bufs[i], lens[i])))
        return fail(KVC_ERR_INVALID_ARG, "keep_index or keep_mask overlaps a cache buffer, the scores or each other");
    }
    return KVC_OK;
  }
  if ((st = check_out_of_place(src, h2o_score, keep_index, rows * budget * sizeof(int32_t), dst, dst_score, workspace,
                               ws_bytes)))
    return st;
  if (keep_mask && (st = check_out_of_place(src, h2o_score, keep_mask, rows * src->capacity, dst, dst_score,
                                            workspace, ws_bytes)))
    return st;
  return KVC_OK;
}

// Eviction launches: one kernel for rows of up to 8192 candidates, else the
// selection kernel writes the keep list and the gather copies it.
int32_t evict_launch(const EvictArgs& e, hipStream_t s, const char* what) {
  if (evict_fits_one_launch(e.max_len, e.n_sink, e.n_recent)) return device_status(launch_evict(e, s), what);
  int32_t st = device_status(launch_select(e.c, e.score, e.budget, e.n_sink, e.n_recent, e.mask, e.keep_index,
                                           e.max_len, s),
                             what);
  if (st) return st;
  return device_status(launch_compact_gather(e.c, e.dst_score ? e.score : nullptr, e.keep_index, e.budget, e.dst,
                                             e.dst_score, s),
                       what);
}

EvictArgs evict_args(const kvc_cache_t* src, const float* h2o_score, int32_t budget, int32_t n_sink,
                     int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index, const kvc_cache_t* dst,
                     float* dst_score, int32_t max_len) {
  EvictArgs e{};
  e.c = *src;
  e.score = h2o_score;
  e.budget = budget;
  e.n_sink = n_sink;
  e.n_recent = n_recent;
  e.mask = keep_mask;
  e.keep_index = keep_index;
  e.dst = *dst;
  e.dst_score = dst_score;
  e.max_len = max_len;
  return e;
}

}  // namespace
}  // namespace kvc

extern "C" {

int32_t kvc_decode_attn(const kvc_cache_t* cache, const void* q, int32_t num_q_heads, float* out, float* h2o_score,
                        int32_t max_len_hint, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return decode_attn_call(cache, nullptr, nullptr, q, num_q_heads, out, h2o_score, max_len_hint, workspace,
                          workspace_bytes, stream);
}

int32_t kvc_decode_attn_split(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                              int32_t num_q_heads, float* h2o_score, int32_t max_len_hint, void* workspace,
                              size_t workspace_bytes, void* stream) {
  clear_error();
  int32_t st = check_cache(cache, "cache");
  if (st) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(KVC_ERR_INVALID_ARG, "pass both k_new and v_new, or neither");
  const int app = k_new != nullptr;
  if (max_len_hint < 0 || (!app && max_len_hint < 1)) return fail(KVC_ERR_INVALID_ARG, "bad max_len_hint");
  if ((long long)max_len_hint + app > cache->capacity) return fail(KVC_ERR_CAPACITY, "max_len_hint exceeds capacity");
  float dummy_out;
  AttnLaunch a;
  if ((st = prepare_attn(cache, k_new, v_new, q, num_q_heads, &dummy_out, h2o_score, max_len_hint + app, workspace,
                         workspace_bytes, &a)))
    return st;
  a.out = nullptr;
  return device_status(launch_attn_split(a, static_cast<hipStream_t>(stream)), "kvc_decode_attn_split launch");
}

int32_t kvc_decode_attn_merge(const kvc_cache_t* cache, int32_t appended, int32_t num_q_heads, float* out,
                              float* h2o_score, int32_t max_len_hint, void* workspace, size_t workspace_bytes,
                              void* stream) {
  clear_error();
  int32_t st = check_cache(cache, "cache");
  if (st) return st;
  const int app = appended != 0;
  if (max_len_hint < 0 || (!app && max_len_hint < 1)) return fail(KVC_ERR_INVALID_ARG, "bad max_len_hint");
  if ((long long)max_len_hint + app > cache->capacity) return fail(KVC_ERR_CAPACITY, "max_len_hint exceeds capacity");
  // The merge reads no q (the shared checks want one: the workspace stands
  // in) and no new token; `appended` says where the lengths come from.
  AttnLaunch a;
  if ((st = prepare_attn(cache, nullptr, nullptr, workspace, num_q_heads, out, h2o_score, max_len_hint + app,
                         workspace, workspace_bytes, &a)))
    return st;
  a.q = nullptr;
  a.append = app;
  return device_status(launch_attn_merge(a, static_cast<hipStream_t>(stream)), "kvc_decode_attn_merge launch");
}

int32_t kvc_append_decode_attn(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                               int32_t num_q_heads, float* out, float* h2o_score, int32_t max_len_hint,
                               void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int32_t st = check_cache(cache, "cache");
  if (st) return st;
  if (!k_new || !v_new) return fail(KVC_ERR_INVALID_ARG, "k_new and v_new must not be NULL");
  if (max_len_hint < 0) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 0");
  if ((long long)max_len_hint + 1 > cache->capacity)
    return fail(KVC_ERR_CAPACITY, "max_len_hint %d + 1 exceeds capacity %d", max_len_hint, cache->capacity);
  return decode_attn_call(cache, k_new, v_new, q, num_q_heads, out, h2o_score, max_len_hint + 1, workspace,
                          workspace_bytes, stream);
}

int32_t kvc_h2o_select(const kvc_cache_t* cache, const float* h2o_score, int32_t budget, int32_t n_sink,
                       int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index, int32_t max_len_hint,
                       void* stream) {
  clear_error();
  int32_t st = check_cache(cache, "cache");
  if (st) return st;
  if (!h2o_score || !keep_mask) return fail(KVC_ERR_INVALID_ARG, "h2o_score and keep_mask must not be NULL");
  if (budget < 1) return fail(KVC_ERR_INVALID_ARG, "budget must be >= 1");
  if (n_sink < 0 || n_recent < 0) return fail(KVC_ERR_INVALID_ARG, "n_sink and n_recent must be >= 0");
  if ((long long)n_sink + n_recent > budget) return fail(KVC_ERR_INVALID_ARG, "n_sink + n_recent exceeds budget");
  if ((st = check_tiers_kept(cache, n_sink, n_recent))) return st;
  if (budget > cache->capacity) return fail(KVC_ERR_CAPACITY, "budget exceeds capacity");
  if (max_len_hint < 0) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 0");
  if (max_len_hint > cache->capacity) return fail(KVC_ERR_CAPACITY, "max_len_hint exceeds capacity");
  // The kernel reads at most max_len_hint slots per row.
  return device_status(launch_select(*cache, h2o_score, budget, n_sink, n_recent, keep_mask, keep_index,
                                     max_len_hint, static_cast<hipStream_t>(stream)),
                       "kvc_h2o_select launch");
}

size_t kvc_compact_workspace_bytes(const kvc_cache_t* src, int32_t max_len_hint) {
  if (check_cache(src, "src") || max_len_hint < 0 || max_len_hint > src->capacity) return 0;
  const int chunks = max_len_hint > 0 ? (max_len_hint + kCompactChunk - 1) / kCompactChunk : 1;
  return align256((size_t)src->batch * src->num_kv_heads * chunks * sizeof(int32_t));
}

int32_t kvc_compact(const kvc_cache_t* src, const float* src_score, const uint8_t* keep_mask, const kvc_cache_t* dst,
                    float* dst_score, int32_t max_len_hint, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int32_t st = check_compact_pair(src, dst, src_score, dst_score);
  if (st) return st;
  if (!keep_mask) return fail(KVC_ERR_INVALID_ARG, "keep_mask must not be NULL");
  if (max_len_hint < 0) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 0");
  if (max_len_hint > src->capacity) return fail(KVC_ERR_CAPACITY, "max_len_hint exceeds capacity");
  const size_t need = kvc_compact_workspace_bytes(src, max_len_hint);
  if (!workspace || workspace_bytes < need)
    return fail(KVC_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need, workspace ? workspace_bytes : 0);
  if ((st = check_out_of_place(src, src_score, keep_mask, (size_t)src->batch * src->num_kv_heads * src->capacity,
                                dst, dst_score, workspace, need)))
    return st;
  // Kernels read at most `chunks` * kCompactChunk slots per row.
  const int chunks = max_len_hint > 0 ? (max_len_hint + kCompactChunk - 1) / kCompactChunk : 1;
  return device_status(launch_compact(*src, src_score, keep_mask, *dst, dst_score, static_cast<int32_t*>(workspace),
                                      chunks, static_cast<hipStream_t>(stream)),
                       "kvc_compact launch");
}

int32_t kvc_compact_gather(const kvc_cache_t* src, const float* src_score, const int32_t* keep_index,
                           int32_t n_keep, const kvc_cache_t* dst, float* dst_score, void* stream) {
  clear_error();
  int32_t st = check_compact_pair(src, dst, src_score, dst_score);
  if (st) return st;
  if (!keep_index) return fail(KVC_ERR_INVALID_ARG, "keep_index must not be NULL");
  if (n_keep < 1) return fail(KVC_ERR_INVALID_ARG, "n_keep must be >= 1");
  if (n_keep > src->capacity) return fail(KVC_ERR_CAPACITY, "n_keep exceeds capacity");
  if ((st = check_out_of_place(src, src_score, keep_index,
                               (size_t)src->batch * src->num_kv_heads * n_keep * sizeof(int32_t), dst, dst_score,
                               nullptr, 0)))
    return st;
  return device_status(launch_compact_gather(*src, src_score, keep_index, n_keep, *dst, dst_score,
                                             static_cast<hipStream_t>(stream)),
                       "kvc_compact_gather launch");
}

size_t kvc_paged_block_evict_workspace_bytes(const kvc_cache_t* src) {
  if (!src || src->batch < 1 || src->max_blocks_per_seq < 1) return 0;
  return align256((size_t)src->batch * src->max_blocks_per_seq * sizeof(float));
}

int32_t kvc_paged_block_evict(const kvc_cache_t* src, const float* h2o_score, double retention,
                              const kvc_cache_t* dst, float* dst_score, int32_t* freed, int32_t* freed_count,
                              int32_t max_len_hint, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int32_t st = check_cache(src, "src");
  if (st) return st;
  if ((st = check_cache(dst, "dst"))) return st;
  if (src->block_size == 0 || dst->block_size == 0)
    return fail(KVC_ERR_INVALID_ARG, "block eviction needs paged caches");
  if (tiered(src) || tiered(dst))
    return fail(KVC_ERR_UNSUPPORTED, "block eviction keeps no sinks or window, so it cannot keep fp16 tiers");
  if (src->bits != dst->bits || vbits_of(*src) != vbits_of(*dst) || src->batch != dst->batch ||
      src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim || src->capacity != dst->capacity ||
      src->max_blocks_per_seq != dst->max_blocks_per_seq || src->num_blocks != dst->num_blocks)
    return fail(KVC_ERR_INVALID_ARG, "src and dst geometries differ");
  if (src->k_codes != dst->k_codes || src->v_codes != dst->v_codes || src->k_scale != dst->k_scale ||
      src->v_scale != dst->v_scale)
    return fail(KVC_ERR_INVALID_ARG, "dst must share src's code and scale pools");
  if (!h2o_score || !dst_score || !freed || !freed_count)
    return fail(KVC_ERR_INVALID_ARG, "h2o_score, dst_score, freed and freed_count must not be NULL");
  if (!(retention >= 0.0 && retention <= 1.0)) return fail(KVC_ERR_INVALID_ARG, "retention must lie in [0, 1]");
  if (max_len_hint < 0) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 0");
  if (max_len_hint > src->capacity) return fail(KVC_ERR_CAPACITY, "max_len_hint exceeds capacity");
  if (src->max_blocks_per_seq > kBlockEvictMaxBlocks)
    return fail(KVC_ERR_UNSUPPORTED, "block eviction supports up to %d blocks per sequence", kBlockEvictMaxBlocks);
  const size_t B = (size_t)src->batch, MB = (size_t)src->max_blocks_per_seq;
  const size_t score_bytes = B * src->num_kv_heads * (size_t)src->capacity * sizeof(float);
  // Outputs (dst table, lengths, num_seen, scores, freed lists) overlap no input
  // (src table, lengths, num_seen, scores) and no other output.
  const void* in[] = {src->block_table, src->lengths, src->num_seen, h2o_score};
  const size_t in_len[] = {B * MB * 4, B * 4, B * 4, score_bytes};
  const size_t ws_need = kvc_paged_block_evict_workspace_bytes(src);
  if (!workspace || workspace_bytes < ws_need)
    return fail(KVC_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", ws_need, workspace ? workspace_bytes : 0);
  if ((uintptr_t)workspace % 256) return fail(KVC_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const void* out[] = {dst->block_table, dst->lengths, dst->num_seen, dst_score, freed, freed_count, workspace};
  const size_t out_len[] = {B * MB * 4, B * 4, B * 4, score_bytes, B * MB * 4, B * 4, ws_need};
  for (int i = 0; i < 7; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlap(out[i], out_len[i], in[j], in_len[j]))
        return fail(KVC_ERR_INVALID_ARG, "output %d overlaps input %d (eviction is out of place)", i, j);
    for (int j = 0; j < i; ++j)
      if (overlap(out[i], out_len[i], out[j], out_len[j]))
        return fail(KVC_ERR_INVALID_ARG, "outputs %d and %d overlap", j, i);
  }
  return device_status(launch_block_evict(*src, h2o_score, retention, *dst, dst_score, freed, freed_count,
                                          static_cast<float*>(workspace), max_len_hint,
                                          static_cast<hipStream_t>(stream)),
                       "kvc_paged_block_evict launch");
}

size_t kvc_decode_attn_kvsep_workspace_bytes(const kvc_cache_t* cache, int32_t num_q_heads, int32_t top_k,
                                             int32_t max_len_hint) {
  AttnGeom g;
  if (!cache || top_k < 1 || top_k > cache->capacity || attn_geometry(cache, num_q_heads, max_len_hint, 1, &g))
    return 0;
  const size_t rows = (size_t)cache->batch * cache->num_kv_heads;
  return g.total + align256(rows * cache->capacity * sizeof(float)) + align256(rows * top_k * sizeof(int32_t)) +
         align256((size_t)cache->batch * num_q_heads * kKvsepMaxParts * cache->head_dim * sizeof(float));
}

int32_t kvc_decode_attn_kvsep(const kvc_cache_t* cache, const void* q, int32_t num_q_heads, int32_t top_k,
                              const void* v_host, float* out, int32_t max_len_hint, void* workspace,
                              size_t workspace_bytes, void* stream) {
  clear_error();
  int32_t st = check_cache(cache, "cache");
  if (st) return st;
  if (top_k < 1) return fail(KVC_ERR_INVALID_ARG, "top_k must be >= 1");
  if (top_k > cache->capacity) return fail(KVC_ERR_CAPACITY, "top_k %d exceeds capacity %d", top_k, cache->capacity);
  if (!v_host || (uintptr_t)v_host % 16) return fail(KVC_ERR_INVALID_ARG, "v_host must be a 16-byte aligned host array");
  AttnGeom g;
  if ((st = attn_geometry(cache, num_q_heads, max_len_hint, 1, &g))) return st;
  const size_t rows = (size_t)cache->batch * cache->num_kv_heads;
  const size_t off_score = g.total, off_keep = off_score + align256(rows * cache->capacity * sizeof(float));
  const size_t off_part = off_keep + align256(rows * top_k * sizeof(int32_t));
  const size_t need =
      off_part + align256((size_t)cache->batch * num_q_heads * kKvsepMaxParts * cache->head_dim * sizeof(float));
  if (!workspace || workspace_bytes < need)
    return fail(KVC_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need, workspace ? workspace_bytes : 0);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* tscore = reinterpret_cast<float*>(ws + off_score);
  int32_t* keep = reinterpret_cast<int32_t*>(ws + off_keep);
  AttnLaunch a;
  if ((st = prepare_attn(cache, nullptr, nullptr, q, num_q_heads, out, tscore, max_len_hint, workspace,
                         workspace_bytes, &a)))
    return st;
  // The cold V rows are read by the device straight from pinned host memory.
  void* v_dev = nullptr;
  if (hipHostGetDevicePointer(&v_dev, const_cast<void*>(v_host), 0) != hipSuccess || !v_dev) {
    (void)hipGetLastError();  // do not leave the failed query's error for the next call
    return fail(KVC_ERR_INVALID_ARG, "v_host must be pinned host memory the device can read (hipHostMalloc)");
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = device_status(launch_fill_zero(tscore, (long long)(rows * cache->capacity), s), "kvsep score clear")))
    return st;
  if ((st = device_status(launch_decode_attn(a, s), "kvsep attention launch"))) return st;
  if ((st = device_status(launch_select(*cache, tscore, top_k, 0, 0, nullptr, keep, max_len_hint, s),
                          "kvsep selection launch")))
    return st;
  KvsepArgs k{};
  k.c = *cache;
  k.logits = a.logits;
  k.span = attn_span(a);
  k.keep = keep;
  k.top_k = top_k;
  k.max_len = max_len_hint;
  k.v_host = static_cast<const __half*>(v_dev);
  k.out = out;
  k.part_o = reinterpret_cast<float*>(ws + off_part);
  // Workgroups per row: about 512 in all (the host link needs many reads in
  // flight), at most one per 64 kept tokens.
  k.parts = (int)std::max<long long>(1, std::min<long long>({(long long)kKvsepMaxParts,
                                                             512 / (long long)rows, ((long long)top_k + 63) / 64}));
  k.num_q_heads = num_q_heads;
  return device_status(launch_kvsep_gather(k, s), "kvsep gather launch");
}

size_t kvc_bw_probe_sink_bytes(void) { return (size_t)bw_probe_workgroups() * sizeof(uint32_t); }

int32_t kvc_bw_probe(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
  clear_error();
  if (!src || !sink) return fail(KVC_ERR_INVALID_ARG, "src and sink must not be NULL");
  if (bytes == 0 || bytes % 16) return fail(KVC_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if ((uintptr_t)src % 16) return fail(KVC_ERR_INVALID_ARG, "src must be 16-byte aligned");
  if (sink_bytes < kvc_bw_probe_sink_bytes())
    return fail(KVC_ERR_INVALID_ARG, "sink needs %zu bytes", kvc_bw_probe_sink_bytes());
  if (overlap(src, bytes, sink, sink_bytes)) return fail(KVC_ERR_INVALID_ARG, "sink overlaps src");
  return device_status(launch_bw_probe(src, bytes, static_cast<unsigned*>(sink), static_cast<hipStream_t>(stream)),
                       "kvc_bw_probe launch");
}

int32_t kvc_h2o_evict(const kvc_cache_t* src, const float* h2o_score, int32_t budget, int32_t n_sink,
                      int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index, const kvc_cache_t* dst,
                      float* dst_score, int32_t max_len_hint, void* stream) {
  clear_error();
  const int32_t st = check_evict(src, h2o_score, budget, n_sink, n_recent, keep_mask, keep_index, dst, dst_score,
                                 max_len_hint, nullptr, 0);
  if (st) return st;
  return evict_launch(evict_args(src, h2o_score, budget, n_sink, n_recent, keep_mask, keep_index, dst, dst_score,
                                 max_len_hint),
                      static_cast<hipStream_t>(stream), "kvc_h2o_evict launch");
}

}  // extern "C"

namespace kvc {
namespace {

int32_t decode_step_call(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                         int32_t num_q_heads, float* out, float* h2o_score, int32_t budget, int32_t n_sink,
                         int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index, const kvc_cache_t* dst,
                         float* dst_score, int32_t max_len_hint, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int32_t st = check_cache(cache, "cache");
  if (st) return st;
  if (!k_new || !v_new) return fail(KVC_ERR_INVALID_ARG, "k_new and v_new must not be NULL");
  if (!h2o_score || !dst_score) return fail(KVC_ERR_INVALID_ARG, "h2o_score and dst_score must not be NULL");
  if (max_len_hint < 0) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 0");
  if ((long long)max_len_hint + 1 > cache->capacity)
    return fail(KVC_ERR_CAPACITY, "max_len_hint %d + 1 exceeds capacity %d", max_len_hint, cache->capacity);
  AttnLaunch a;
  if ((st = prepare_attn(cache, k_new, v_new, q, num_q_heads, out, h2o_score, max_len_hint + 1, workspace,
                         workspace_bytes, &a)))
    return st;
  const bool in_place = dst && dst->k_codes == cache->k_codes;
  if ((st = check_evict(cache, h2o_score, budget, n_sink, n_recent, keep_mask, keep_index, dst, dst_score,
                        max_len_hint + 1, workspace, workspace_bytes, in_place)))
    return st;
  const size_t rows = (size_t)cache->batch * cache->num_kv_heads;
  if ((st = check_workspace_disjoint(workspace, workspace_bytes, cache, h2o_score, dst, dst_score, keep_index,
                                     rows * budget * sizeof(int32_t), keep_mask, rows * cache->capacity)))
    return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  EvictArgs e = evict_args(cache, h2o_score, budget, n_sink, n_recent, keep_mask, keep_index, dst, dst_score,
                           max_len_hint + 1);
  if (in_place) {
    // The split kernel clears the control words; then one eviction launch
    // selects and moves in place (merging the splits when it can, else after
    // the merge kernel). Rows past one launch's selection are selected by the
    // selection kernel first and only moved by the in-place launch.
    AttnGeom g;
    if ((st = attn_geometry(cache, num_q_heads, max_len_hint + 1, 1, &g))) return st;
    // Moving workgroups: about one CU each with the selectors (so that every
    // workgroup of the launch is resident at once), each moving
    // kInplaceMinPasses to kInplaceMaxPasses passes of rows.
    // Movers cover the larger of the budget (destinations) and the longest
    // row (sources).
    const long long rows_ip = (long long)cache->batch * cache->num_kv_heads;
    const long long rpp = evict_inplace_rows_per_pass(*cache);
    const long long cover = std::max<long long>(budget, e.max_len);
    const long long movers = std::max(1LL, device_cus() / rows_ip - 1);
    const int passes = (int)std::min<long long>(kInplaceMaxPasses(std::max(k_row_bytes(*cache), v_row_bytes(*cache))),
                                                std::max<long long>(kInplaceMinPasses, (cover + movers * rpp - 1) /
                                                                                           (movers * rpp)));
    const int chunks = (int)((cover + passes * rpp - 1) / (passes * rpp));
    int32_t* ip = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + g.off_ip);
    a.zero_words = ip;
    a.zero_count = (int)(1 + rows_ip + rows_ip * chunks + rows_ip * kInplaceMaxEvicted);
    e.ip = ip;
    e.ip_chunks = chunks;
    e.ip_passes = passes;
    e.stash = a.stash;
    if (evict_fits_one_launch(e.max_len, n_sink, n_recent) &&
        evict_inplace_can_merge(num_q_heads, cache->num_kv_heads, a.parts)) {
      if ((st = device_status(launch_attn_split(a, s), "kvc_decode_step split launch"))) return st;
      e.part_o = a.part_o;
      e.part_ml = a.part_ml;
      e.logits = a.logits;
      e.out = out;
      e.num_q_heads = num_q_heads;
      e.splits = a.parts;
      e.span = attn_span(a);
      return device_status(launch_evict_inplace(e, s), "kvc_decode_step in-place eviction launch");
    }
    if ((st = device_status(launch_decode_attn(a, s), "kvc_decode_step attention launch"))) return st;
    if (!evict_fits_one_launch(e.max_len, n_sink, n_recent)) {
      if ((st = device_status(launch_select(e.c, e.score, budget, n_sink, n_recent, e.mask, e.keep_index, e.max_len,
                                            s),
                              "kvc_decode_step selection launch")))
        return st;
      e.ip_preselected = 1;
    }
    return device_status(launch_evict_inplace(e, s), "kvc_decode_step in-place eviction launch");
  }
  if (evict_fits_one_launch(e.max_len, n_sink, n_recent) &&
      evict_can_merge(num_q_heads, cache->num_kv_heads, a.parts)) {
    // Two launches: the split kernel (with the append), then the eviction
    // kernel that also merges the splits.
    if ((st = device_status(launch_attn_split(a, s), "kvc_decode_step split launch"))) return st;
    e.part_o = a.part_o;
    e.part_ml = a.part_ml;
    e.logits = a.logits;
    e.stash = a.stash;
    e.out = out;
    e.num_q_heads = num_q_heads;
    e.splits = a.parts;  // partial states per head: the splits and the fp16-tier parts
    e.span = attn_span(a);
    return device_status(launch_evict(e, s), "kvc_decode_step eviction launch");
  }
  if ((st = device_status(launch_decode_attn(a, s), "kvc_decode_step attention launch"))) return st;
  return evict_launch(e, s, "kvc_decode_step eviction launch");
}

// The workspace of kvc_decode_step_noalloc: a static device array, one copy
// per GPU, held until the process ends. Host code uses its device address
// from hipGetSymbolAddress (taken once per device, with that device current),
// never the array's name.
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

int32_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVC_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVC_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

extern "C" {

int32_t kvc_decode_step(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                        int32_t num_q_heads, float* out, float* h2o_score, int32_t budget, int32_t n_sink,
                        int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index, const kvc_cache_t* dst,
                        float* dst_score, int32_t max_len_hint, void* workspace, size_t workspace_bytes,
                        void* stream) {
  clear_error();
  return decode_step_call(cache, k_new, v_new, q, num_q_heads, out, h2o_score, budget, n_sink, n_recent, keep_mask,
                          keep_index, dst, dst_score, max_len_hint, workspace, workspace_bytes, stream);
}

size_t kvc_decode_step_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

int32_t kvc_decode_step_noalloc(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                                int32_t num_q_heads, float* out, float* h2o_score, int32_t budget, int32_t n_sink,
                                int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index, const kvc_cache_t* dst,
                                float* dst_score, int32_t max_len_hint, void* stream) {
  clear_error();
  int32_t st = check_cache(cache, "cache");
  if (st) return st;
  if (max_len_hint < 0) return fail(KVC_ERR_INVALID_ARG, "max_len_hint must be >= 0");
  if ((long long)max_len_hint + 1 > cache->capacity)
    return fail(KVC_ERR_CAPACITY, "max_len_hint %d + 1 exceeds capacity %d", max_len_hint, cache->capacity);
  AttnGeom g;
  if ((st = attn_geometry(cache, num_q_heads, max_len_hint + 1, 1, &g))) return st;
  if (g.total > kNoallocScratchBytes)
    return fail(KVC_ERR_CAPACITY, "the step needs %zu bytes of workspace; the static scratch holds %zu", g.total,
                kNoallocScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return decode_step_call(cache, k_new, v_new, q, num_q_heads, out, h2o_score, budget, n_sink, n_recent, keep_mask,
                          keep_index, dst, dst_score, max_len_hint, ws, kNoallocScratchBytes, stream);
}

}  // extern "C"
