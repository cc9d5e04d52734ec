// Internal declarations shared by libkvc's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

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
constexpr int kCompactChunk = 1024;

// ---- launchers (defined in the .hip files; return the first HIP error) ----
hipError_t launch_quant_append(const kvc_cache_t& c, const __half* k_new, const __half* v_new,
                               int n_new, float* score, hipStream_t st);

struct AttnLaunch {
  kvc_cache_t c;
  const __half* q;
  float* out;
  float* score;      // NULL = no H2O
  float* part_o;     // [B][Hq][S][D]
  float* part_ml;    // [B][Hq][S][2]  (running max in log2 units, sum)
  float* pexp;       // [B][Hq][S * kSplitTokens]  (only with H2O)
  int num_q_heads;
  int splits;
  float qk_log2;     // log2(e) / sqrt(head_dim)
};
hipError_t launch_decode_attn(const AttnLaunch& a, hipStream_t st);

hipError_t launch_select(const kvc_cache_t& c, const float* score, int budget, int n_sink,
                         int n_recent, uint8_t* mask, int max_len, hipStream_t st);

hipError_t launch_compact(const kvc_cache_t& src, const float* src_score, const uint8_t* mask,
                          const kvc_cache_t& dst, float* dst_score, int32_t* counts, int chunks,
                          hipStream_t st);

// ---- device helpers ----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
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
