// Block-granular H2O eviction on a paged cache: whole 16-token blocks leave,
// and compaction is a rewrite of the block table.
//
// The eviction-and-reuse survey (section 4) evicts KV blocks by attention
// score: the blocks are sorted by their mean score (a stable sort, lowest
// first) and the first int(n * (1 - retention)) of them are evicted, their
// references released so the pool can reuse them ("KV Cache optimization
// techniques" tutorial, section 3.2: a block returns to the free set when its
// reference count drops to zero). Here a block's score is the mean H2O score
// over its filled slots and every KV head of the sequence (a physical block
// holds all heads), and n is the number of blocks the sequence's length
// covers. The kept blocks keep their order, so the tokens keep theirs: the
// destination's table lists them first, its length counts their tokens (only
// the last block can be partial), and the scores move with their blocks. The
// codes and scales stay where they are: source and destination share the
// pools.
//
// Two launches. block_mean_kernel: one wave per block, lanes over (head,
// quarter row) pairs, 16-byte loads, a fixed-order sum of the filled slots
// (blocks holding equal scores get equal means), the means to a workspace.
// block_select_kernel: several workgroups per sequence, each with the means
// in LDS as 64-bit keys (the mean's order-preserving bits, then the block
// index, so that one unsigned compare gives the stable order): every block's
// rank by counting (n^2 compares, made for decode-sized tables), a block scan for the kept and
// freed positions (workgroup 0 writes the table, the freed list and the
// lengths), and a share of the score rows moved in 16-byte pieces, eight
// loads in flight per thread. One workgroup per sequence doing all of it took
// about 43 us on the 32-sequence paged batch (5114 blocks), bound by one CU's
// latency per sequence.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kBT = 256;

// Mean H2O score of each block over its filled slots and all heads.
__global__ __launch_bounds__(kBT) void block_mean_kernel(kvc_cache_t src, const float* __restrict__ score,
                                                         float* __restrict__ means, int max_len) {
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  const int j = blockIdx.x * (kBT / 64) + (threadIdx.x >> 6);  // this wave's block
  const int H = src.num_kv_heads, BS = src.block_size, MB = src.max_blocks_per_seq;
  const long long cap = src.capacity;
  const int L = __builtin_amdgcn_readfirstlane(min(min(src.lengths[b], src.capacity), max_len));
  const int nb = (L + BS - 1) / BS;
  if (j >= nb) return;  // uniform per wave
  const int fill = min(BS, L - BS * j);
  // Lane r of each pass takes head r / 4, quarter r % 4 of the 16-slot row (in
  // bounds: the capacity is a whole number of blocks).
  float acc = 0.f;
  for (int r = lane; r < 4 * H; r += 64) {
    const int h = r >> 2, q = r & 3;
    const float4 w = reinterpret_cast<const float4*>(score + ((long long)b * H + h) * cap + (long long)BS * j)[q];
    const float x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (4 * q + c < fill) acc += x[c];
  }
  acc = wave_sum(acc);
  if (lane == 0) means[(long long)b * MB + j] = acc / (float)(fill * H);
}

// Workgroup (part, b): ranks, keep flags and kept positions of sequence b
// (every part the same), the table rewrite (part 0) and a 1/parts share of
// the score move.
__global__ __launch_bounds__(kBT) void block_select_kernel(kvc_cache_t src, const float* __restrict__ score,
                                                           const float* __restrict__ means, double retention,
                                                           kvc_cache_t dst, float* __restrict__ dst_score,
                                                           int32_t* __restrict__ freed,
                                                           int32_t* __restrict__ freed_count, int max_len) {
  extern __shared__ __align__(16) unsigned long long lds_keys[];
  const int part = blockIdx.x, parts = gridDim.x, b = blockIdx.y, tid = threadIdx.x;
  const int H = src.num_kv_heads, BS = src.block_size, MB = src.max_blocks_per_seq;
  const long long cap = src.capacity;
  unsigned long long* key = lds_keys;                   // [MB]: (order key of the mean) << 32 | block index
  int* keep = reinterpret_cast<int*>(lds_keys + MB);    // [MB]: 1 kept, 0 evicted
  int* src_of = reinterpret_cast<int*>(lds_keys);       // [MB]: kept block at each new position (after the ranks)
  __shared__ int scan_tmp[kBT / 64];
  const int L = __builtin_amdgcn_readfirstlane(min(min(src.lengths[b], src.capacity), max_len));
  const int nb = (L + BS - 1) / BS;
  const int32_t* srow = src.block_table + (long long)b * MB;
  for (int j = tid; j < nb; j += kBT) {
    // + 0: -0 becomes +0, which the float order holds equal to it
    unsigned u = __float_as_uint(means[(long long)b * MB + j] + 0.f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    key[j] = ((unsigned long long)u << 32) | (unsigned)j;
  }
  __syncthreads();
  // Stable ascending order by mean: block j's rank counts the blocks with a
  // lower mean, or an equal mean and a lower index (a smaller key); ranks
  // below n_evict go.
  const int n_evict = (int)((double)nb * (1.0 - retention));
  for (int j = tid; j < nb; j += kBT) {
    const unsigned long long kj = key[j];
    int rank = 0;
    for (int i = 0; i < nb; ++i) rank += key[i] < kj;
    keep[j] = rank >= n_evict;
  }
  __syncthreads();  // the keys are read no more: src_of takes their place
  // Kept and freed positions: thread t owns blocks [t*per, t*per + per).
  const int per = (nb + kBT - 1) / kBT;
  const int j0 = min(tid * per, nb), j1 = min(j0 + per, nb);
  int kc = 0;
  for (int j = j0; j < j1; ++j) kc += keep[j];
  int kpos = block_inclusive_scan<kBT>(kc, scan_tmp) - kc;  // kept blocks before j0
  int fpos = j0 - kpos;                                       // evicted blocks before j0
  const int n_kept = nb - n_evict;
  int32_t* drow = const_cast<int32_t*>(dst.block_table) + (long long)b * MB;
  int32_t* frow = freed + (long long)b * MB;
  for (int j = j0; j < j1; ++j) {
    if (keep[j]) {
      src_of[kpos] = j;
      if (part == 0) drow[kpos] = srow[j];
      ++kpos;
    } else {
      if (part == 0) frow[fpos] = srow[j];
      ++fpos;
    }
  }
  if (part == 0)
    for (int i = n_kept + tid; i < MB; i += kBT) drow[i] = -1;
  __syncthreads();
  // Scores move with their blocks: new block i takes old block src_of[i], in
  // 16-byte pieces (4 per block row); this part moves pieces [w_lo, w_hi),
  // kMB per thread loaded before any is stored; slots past a partial block's
  // fill are not written.
  constexpr int kMB = 8;
  const long long pieces = (long long)n_kept * H * 4;
  const long long w_lo = pieces * part / parts, w_hi = pieces * (part + 1) / parts;
  for (long long w0 = w_lo + tid; w0 < w_hi; w0 += (long long)kBT * kMB) {
    float4 v[kMB];
#pragma unroll
    for (int u = 0; u < kMB; ++u) {
      const long long w = min(w0 + (long long)u * kBT, w_hi - 1);
      const int q = (int)(w & 3);
      const long long r = w >> 2;
      const int h = (int)(r % H), i = (int)(r / H);
      v[u] = reinterpret_cast<const float4*>(score + ((long long)b * H + h) * cap + (long long)BS * src_of[i])[q];
    }
#pragma unroll
    for (int u = 0; u < kMB; ++u) {
      const long long w = w0 + (long long)u * kBT;
      if (w < w_hi) {
        const int q = (int)(w & 3);
        const long long r = w >> 2;
        const int h = (int)(r % H), i = (int)(r / H);
        const int fill = min(BS, L - BS * src_of[i]);
        float* d = dst_score + ((long long)b * H + h) * cap + (long long)BS * i + 4 * q;
        if (4 * q + 4 <= fill) {
          *reinterpret_cast<float4*>(d) = v[u];
        } else {
          const float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
          for (int c = 0; c < 4; ++c)
            if (4 * q + c < fill) d[c] = x[c];
        }
      }
    }
  }
  if (part == 0 && tid == 0) {
    // Only the last block can be partial; it stays last when kept.
    const int last_fill = nb > 0 ? L - BS * (nb - 1) : 0;
    const int new_len = n_kept == 0 ? 0 : (nb > 0 && keep[nb - 1] ? BS * (n_kept - 1) + last_fill : BS * n_kept);
    dst.lengths[b] = new_len;
    dst.num_seen[b] = src.num_seen[b];
    freed_count[b] = n_evict;
  }
}

}  // namespace

size_t block_evict_lds_bytes(int max_blocks_per_seq) {
  return (size_t)max_blocks_per_seq * (sizeof(unsigned long long) + sizeof(int));
}

hipError_t launch_block_evict(const kvc_cache_t& src, const float* score, double retention, const kvc_cache_t& dst,
                              float* dst_score, int32_t* freed, int32_t* freed_count, float* means, int max_len,
                              hipStream_t st) {
  const int MB = src.max_blocks_per_seq;
  hipLaunchKernelGGL(block_mean_kernel, dim3((MB + kBT / 64 - 1) / (kBT / 64), src.batch), dim3(kBT), 0, st, src,
                     score, means, max_len);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Workgroups per sequence: about 256 in all, at most 8.
  const int parts = std::max(1, std::min(8, 256 / std::max(1, src.batch)));
  hipLaunchKernelGGL(block_select_kernel, dim3(parts, src.batch), dim3(kBT), block_evict_lds_bytes(MB), st, src,
                     score, means, retention, dst, dst_score, freed, freed_count, max_len);
  return hipGetLastError();
}

}  // namespace kvc
