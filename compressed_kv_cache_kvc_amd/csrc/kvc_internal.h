// Internal declarations shared by libkvc's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <algorithm>
#include <string>

#include "kvc.h"

namespace kvc {

// ---- host-side error reporting (thread-local message of the last failure) ----
void set_error(const char* fmt, ...);
void clear_error();
int32_t fail(int32_t status, const char* fmt, ...);

// Tokens per split of the decode-attention kernel (one workgroup per split).
constexpr int kSplitTokens = 256;
// Slots per chunk of the compaction kernels.
constexpr int kCompactChunk = 256;
// Rows of at most this many chunks are compacted in one launch (each
// workgroup recounts the kept slots before its chunk from the mask).
constexpr int kCompactRecountChunks = 64;
// Candidate keys the selection kernel stages in LDS (48 KiB).
constexpr int kSelectResidentKeys = 12288;

// ---- launchers (defined in the .hip files; return the first HIP error) ----
hipError_t launch_quant_append(const kvc_cache_t& c, const __half* k_new, const __half* v_new,
                               int n_new, float* score, hipStream_t st);

struct AttnLaunch {
  kvc_cache_t c;
  const __half* q;
  float* out;
  float* score;      // NULL = no H2O
  float* part_o;     // [B][Hq][S][D]
  float* part_ml;    // [B][Hq][S][2]  (max in log2 units, sum)
  float* logits;     // [B][Hq][S * tiles * kSplitTokens], log2 units (only with H2O)
  int num_q_heads;
  int splits;        // S: workgroups per (sequence, KV head)
  int tiles;         // 256-token tiles per split
  float qk_log2;     // log2(e) / sqrt(head_dim)
};
hipError_t launch_decode_attn(const AttnLaunch& a, hipStream_t st);
// Query heads one split-kernel pass serves; with more heads per KV head than
// this, a split holds a single tile.
int attn_heads_per_pass(int G);

hipError_t launch_select(const kvc_cache_t& c, const float* score, int budget, int n_sink,
                         int n_recent, uint8_t* mask, int max_len, hipStream_t st);

hipError_t launch_compact(const kvc_cache_t& src, const float* src_score, const uint8_t* mask,
                          const kvc_cache_t& dst, float* dst_score, int32_t* counts, int chunks,
                          hipStream_t st);

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
