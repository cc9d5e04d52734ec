// Internal declarations shared by libkvc's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <algorithm>
#include <string>
#include <type_traits>

#include "kvc.h"

namespace kvc {

// Code widths of K and V, and their bytes per token row.
__host__ __device__ inline int kbits_of(const kvc_cache_t& c) { return c.bits; }
__host__ __device__ inline int vbits_of(const kvc_cache_t& c) { return c.v_bits ? c.v_bits : c.bits; }
__host__ __device__ inline int k_row_bytes(const kvc_cache_t& c) { return c.head_dim * kbits_of(c) / 8; }
__host__ __device__ inline int v_row_bytes(const kvc_cache_t& c) { return c.head_dim * vbits_of(c) / 8; }

// Calls f(RBK, RBV) with the cache's K and V row bytes as compile-time
// constants (std::integral_constant): 32, 64 or 128 each (head_dim 64 or 128
// at 4 or 8 bits), equal or one twice the other. Other sizes: invalid value.
template <typename F>
hipError_t with_row_bytes(const kvc_cache_t& c, F&& f) {
  using I32 = std::integral_constant<int, 32>;
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  const int rbk = k_row_bytes(c), rbv = v_row_bytes(c);
  if (rbk == 32 && rbv == 32) return f(I32{}, I32{});
  if (rbk == 64 && rbv == 64) return f(I64{}, I64{});
  if (rbk == 128 && rbv == 128) return f(I128{}, I128{});
  if (rbk == 64 && rbv == 32) return f(I64{}, I32{});
  if (rbk == 32 && rbv == 64) return f(I32{}, I64{});
  if (rbk == 128 && rbv == 64) return f(I128{}, I64{});
  if (rbk == 64 && rbv == 128) return f(I64{}, I128{});
  return hipErrorInvalidValue;
}

// ---- host-side error reporting (thread-local message of the last failure) ----
void set_error(const char* fmt, ...);
void clear_error();
int32_t fail(int32_t status, const char* fmt, ...);

// Compute units of the current device (host; 256, MI355X's count, when no
// device answers). Launch geometries aim at a multiple of it.
int device_cus();

// Tokens per split of the decode-attention kernel (one workgroup per split).
constexpr int kSplitTokens = 256;
// fp16-tier tokens per workgroup (one wave) of the tier attention kernel.
constexpr int kTierTokens = 64;
// Slots per chunk of the compaction kernels.
constexpr int kCompactChunk = 256;
// Rows of at most this many chunks are compacted in one launch (each
// workgroup recounts the kept slots before its chunk from the mask).
constexpr int kCompactRecountChunks = 64;

// ---- launchers (defined in the .hip files; return the first HIP error) ----
hipError_t launch_quant_append(const kvc_cache_t& c, const __half* k_new, const __half* v_new,
                               int n_new, float* score, hipStream_t st);

struct AttnLaunch {
  kvc_cache_t c;
  const __half* q;
  float* out;
  float* score;      // NULL = no H2O
  float* part_o;     // [B][Hq][parts][D]
  float* part_ml;    // [B][Hq][parts][2]  (max in log2 units, sum)
  float* logits;     // [B][Hq][S * tiles * kSplitTokens], log2 units (only with H2O)
  // With k_new and v_new ([B][Hkv][D] fp16): append one token per sequence
  // first (slot lengths[b]); NULL: attention only.
  const __half* k_new;
  const __half* v_new;
  int32_t* stash;    // [2][B]: lengths and num_seen before the append
  int append;        // the split appended (the merge takes the lengths from stash)
  int num_q_heads;
  int splits;        // S: workgroups per (sequence, KV head)
  int tiles;         // 256-token tiles per split, except the last
  int last_tiles;    // tiles of the last split (it may take a small remainder past `tiles`)
  int tier_parts;    // TP: fp16-tier partial states per (sequence, query head), after the S splits
  int parts;         // S + TP: partial states per query head in part_o / part_ml
  float qk_log2;     // log2(e) / sqrt(head_dim)
  // Words the split kernel sets to zero (NULL: none): the control words of an
  // in-place eviction later in the same decode step.
  int32_t* zero_words;
  int zero_count;
  // Set when the tiers make one part (at most kTierTokens tier tokens, e.g.
  // the sinks alone), each KV head serves one query head and the cache is
  // contiguous: the first split's workgroups compute it at their end, and no
  // tier launch follows.
  int fold_tier;
};
// Logit slots per query head: the tiles of all splits.
__host__ __device__ inline long long attn_span(const AttnLaunch& a) {
  return ((long long)(a.splits - 1) * a.tiles + a.last_tiles) * kSplitTokens;
}
hipError_t launch_decode_attn(const AttnLaunch& a, hipStream_t st);  // split, then merge
// The code splits, then (on a tiered cache) the fp16-tier parts S .. S + TP - 1
// in a second kernel (with an append, it also stores the new token's tier
// rows).
hipError_t launch_attn_split(const AttnLaunch& a, hipStream_t st);
// Stores the fp16 rows of n_new appended tokens in the cache's tiers (before
// the append advances the lengths).
hipError_t launch_tier_append(const kvc_cache_t& c, const __half* k_new, const __half* v_new, int n_new,
                              hipStream_t st);
hipError_t launch_attn_merge(const AttnLaunch& a, hipStream_t st);

hipError_t launch_select(const kvc_cache_t& c, const float* score, int budget, int n_sink,
                         int n_recent, uint8_t* mask, int32_t* keep_index, int max_len, hipStream_t st);

// Selection and compaction in one launch; only for rows of at most 8192
// candidates (evict_fits_one_launch). With part_ml set, the launch also merges
// the attention splits of the same step (evict_can_merge).
struct EvictArgs {
  kvc_cache_t c;
  const float* score;
  int budget, n_sink, n_recent;
  uint8_t* mask;        // may be NULL
  int32_t* keep_index;  // may be NULL
  kvc_cache_t dst;
  float* dst_score;     // may be NULL
  int max_len;
  int log2_parts;       // set by the launcher
  int xcd_rows;         // set by the launcher: the workgroups of a row share an XCD
  // Merging (part_ml NULL: none): the split kernel's outputs of the step.
  const float* part_o;
  const float* part_ml;
  const float* logits;
  const int32_t* stash;
  float* out;
  int num_q_heads, splits;
  long long span;
  // In-place eviction (dst is the source cache; NULL: out of place): control
  // words, zero on entry (ticket, per-row and per-chunk flags, then per-row
  // first moved slot), and whether a selection kernel already wrote the keep
  // list (the workgroups then only move rows).
  int32_t* ip;
  int ip_chunks;      // moving workgroups per row
  int ip_passes;      // passes per moving workgroup
  int ip_preselected;
};
constexpr int kEvictMaxMergeHeads = 4;  // query heads per KV head
constexpr int kEvictMaxSplits = 1024;
bool evict_fits_one_launch(int max_len, int n_sink, int n_recent);
bool evict_can_merge(int num_q_heads, int num_kv_heads, int splits);
hipError_t launch_evict(const EvictArgs& a, hipStream_t st);
// In-place eviction. A moving workgroup (kEvictThreads threads, one 16-byte
// access each per pass and row part) takes the kept entries of `passes`
// times evict_inplace_rows_per_pass consecutive destination slots.
// Control words: a ticket, a flag per row, a flag per (row, chunk), the
// row's first kInplaceMaxEvicted evicted slots, then its first moved slot;
// all but the last `rows` words must be zero when it starts.
constexpr int kEvictThreads = 1024;
constexpr int kInplaceMinPasses = 4;
// Passes of codes held in registers: 10 for 128-byte rows; fewer for shorter
// rows, whose passes cover more entries and so more scales, positions,
// scores and logits per thread.
__host__ __device__ constexpr int kInplaceMaxPasses(int row_bytes) {
  return row_bytes >= 128 ? 10 : row_bytes >= 64 ? 8 : 4;
}
// Rows with at most this many evicted slots are moved by workgroups that load
// their rows before the selection is known.
constexpr int kInplaceMaxEvicted = 64;
inline int evict_inplace_rows_per_pass(const kvc_cache_t& c) {
  const int rb = k_row_bytes(c) > v_row_bytes(c) ? k_row_bytes(c) : v_row_bytes(c);
  return kEvictThreads * 16 / rb;
}
// Control words for any pass count and any budget up to `budget`.
inline size_t evict_inplace_words_bound(const kvc_cache_t& c, int budget) {
  const size_t rows = (size_t)c.batch * c.num_kv_heads;
  const size_t chunk = (size_t)kInplaceMinPasses * evict_inplace_rows_per_pass(c);
  return 1 + rows + rows * (((size_t)budget + chunk - 1) / chunk) + rows * kInplaceMaxEvicted + rows;
}
// The in-place launch merges the attention splits for up to 8 query heads per
// KV head.
inline bool evict_inplace_can_merge(int num_q_heads, int num_kv_heads, int splits) {
  return num_q_heads / num_kv_heads <= 8 && (long long)splits <= kEvictMaxSplits;
}
hipError_t launch_evict_inplace(const EvictArgs& a, hipStream_t st);

hipError_t launch_compact(const kvc_cache_t& src, const float* src_score, const uint8_t* mask,
                          const kvc_cache_t& dst, float* dst_score, int32_t* counts, int chunks,
                          hipStream_t st);
hipError_t launch_compact_gather(const kvc_cache_t& src, const float* src_score, const int32_t* keep_index,
                                 int n_keep, const kvc_cache_t& dst, float* dst_score, hipStream_t st);

// Block-granular eviction on a paged cache: the block means (to `means`,
// [batch][max_blocks_per_seq] fp32), then selection, table rewrite and score
// move with block_evict_lds_bytes of dynamic LDS per workgroup.
size_t block_evict_lds_bytes(int max_blocks_per_seq);
constexpr int kBlockEvictMaxBlocks = 8192;
hipError_t launch_block_evict(const kvc_cache_t& src, const float* score, double retention, const kvc_cache_t& dst,
                              float* dst_score, int32_t* freed, int32_t* freed_count, float* means, int max_len,
                              hipStream_t st);

// K/V-separated attention's last step (kvsep.hip): per (sequence, KV head),
// the output of each query head from the kept tokens' fp16 V rows.
struct KvsepArgs {
  kvc_cache_t c;
  const float* logits;   // [B][Hq][span] from the attention kernels, log2 units
  long long span;
  const int32_t* keep;   // [B][Hkv][top_k] kept slots, ascending
  int top_k;
  int max_len;           // the length bound the selection used
  const __half* v_host;  // device-visible pointer to [B][Hkv][capacity][D] fp16
  float* out;            // [B][Hq][D]
  float* part_o;         // [B][Hq][parts][D] workspace: each part's sums
  int parts;             // workgroups per (sequence, KV head), 1..kKvsepMaxParts
  int num_q_heads;
};
constexpr int kKvsepMaxParts = 16;
hipError_t launch_fill_zero(float* p, long long n, hipStream_t st);
hipError_t launch_kvsep_gather(const KvsepArgs& a, hipStream_t st);

// Read-bandwidth probe: reads bytes (a multiple of 16) from src once; writes
// bw_probe_workgroups() words to sink.
int bw_probe_workgroups();
hipError_t launch_bw_probe(const void* src, size_t bytes, unsigned* sink, hipStream_t st);

// ---- device helpers ----
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                                               false));
}

// Max over the wave, returned in every lane: DPP inside each 16-lane row
// (xor 1, xor 2, half-row and row mirrors), row broadcasts across rows, then
// a read of lane 63. No LDS traffic.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v, v));
  v = fmaxf(v, dpp_f<0x4E>(v, v));
  v = fmaxf(v, dpp_f<0x141>(v, v));
  v = fmaxf(v, dpp_f<0x140>(v, v));
  v = fmaxf(v, dpp_f<0x142, 0xA>(v, v));
  v = fmaxf(v, dpp_f<0x143, 0xC>(v, v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, BOUND_ZERO);
}

// Inclusive prefix sum over the 64 lanes of a wave, all in DPP (no LDS):
// three row shifts build 4-lane sums inside each 16-lane row, shifts by 4 and
// 8 on the upper banks complete the row, and two row broadcasts carry row
// totals forward. Lanes whose DPP source is masked off receive 0.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int v0 = v;
  v += dpp_i<0x111, 0xF, 0xF, true>(v0);  // row_shr:1
  v += dpp_i<0x112, 0xF, 0xF, true>(v0);  // row_shr:2
  v += dpp_i<0x113, 0xF, 0xF, true>(v0);  // row_shr:3
  v += dpp_i<0x114, 0xF, 0xE>(v);         // row_shr:4 into lanes 4..15 of each row
  v += dpp_i<0x118, 0xF, 0xC>(v);         // row_shr:8 into lanes 8..15
  v += dpp_i<0x142, 0xA>(v);              // row_bcast:15 into rows 1 and 3
  v += dpp_i<0x143, 0xC>(v);              // row_bcast:31 into rows 2 and 3
  return v;
}

// Sum over the wave, returned in every lane (DPP, then a read of lane 63).
__device__ __forceinline__ int wave_sum_i(int v) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan(v), 63);
}

// Unsigned min / max over the wave, returned in every lane.
template <bool MAX>
__device__ __forceinline__ unsigned wave_minmax_u(unsigned v) {
  auto op = [](unsigned x, unsigned y) { return MAX ? (x > y ? x : y) : (x < y ? x : y); };
  // Masked-off lanes of the broadcasts read 0, a no-op only for max; the
  // row-broadcast steps therefore pass the value itself as the fallback.
  v = op(v, (unsigned)dpp_i<0xB1>((int)v));
  v = op(v, (unsigned)dpp_i<0x4E>((int)v));
  v = op(v, (unsigned)dpp_i<0x141>((int)v));
  v = op(v, (unsigned)dpp_i<0x140>((int)v));
  v = op(v, (unsigned)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = op(v, (unsigned)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over a workgroup of NT threads. `tmp` is NT/64 ints of
// LDS; two barriers.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_inclusive_scan(v);
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) add += (w < wave) ? tmp[w] : 0;
  __syncthreads();
  return v + add;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Row index (token of one KV head) of cache slot `slot` of sequence b, KV head h;
// -1 when the slot has no storage. Codes of the row start at row * RB bytes,
// its scale at element `row` of the scale array.
__device__ __forceinline__ long long cache_row(const kvc_cache_t& c, int b, int h, int slot) {
  if ((unsigned)slot >= (unsigned)c.capacity) return -1;
  if (c.block_size == 0) return ((long long)b * c.num_kv_heads + h) * c.capacity + slot;
  const int bi = slot / c.block_size;
  const int blk = c.block_table[(long long)b * c.max_blocks_per_seq + bi];
  if ((unsigned)blk >= (unsigned)c.num_blocks) return -1;
  return ((long long)blk * c.num_kv_heads + h) * c.block_size + (slot - bi * c.block_size);
}

}  // namespace kvc
