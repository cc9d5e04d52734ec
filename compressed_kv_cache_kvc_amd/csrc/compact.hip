// Stable out-of-place compaction of the kept cache slots.
//
// The kept slots keep their relative (ascending) order and carry their scores
// with them ("KV Cache optimization techniques" tutorial, section 2.2; "KV
// Cache Compression Report", section 3.4). The destination slot of a kept
// slot is the number of kept slots before it: an exclusive prefix sum of the
// mask. Two launches: per-chunk counts, then each chunk adds the counts of
// the chunks before it, scans its own 1024 slots and moves the kept rows.
// Reading src and writing dst, which may not overlap, removes every race.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int CH = kCompactChunk;
constexpr int NT = 256;
constexpr int PER = CH / NT;

__device__ __forceinline__ int block_sum(int v, int* tmp) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  const int r = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(NT) void compact_count_kernel(kvc_cache_t src, const uint8_t* __restrict__ mask,
                                                           int32_t* __restrict__ counts, int chunks) {
  const int ch = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = min(min(src.lengths[b], src.capacity), chunks * CH);
  const uint8_t* m = mask + ((long long)b * src.num_kv_heads + g) * src.capacity;
  int n = 0;
  for (int q = 0; q < PER; ++q) {
    const int i = ch * CH + q * NT + threadIdx.x;
    if (i < L) n += m[i] != 0;
  }
  __shared__ int tmp[4];
  n = block_sum(n, tmp);
  if (threadIdx.x == 0) counts[((long long)b * src.num_kv_heads + g) * chunks + ch] = n;
}

template <int RB>
__device__ __forceinline__ void copy_row(const uint8_t* __restrict__ s, uint8_t* __restrict__ d) {
  if (RB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < RB / 16; ++i) reinterpret_cast<uint4*>(d)[i] = reinterpret_cast<const uint4*>(s)[i];
  } else {
#pragma unroll
    for (int i = 0; i < RB / 8; ++i) reinterpret_cast<uint2*>(d)[i] = reinterpret_cast<const uint2*>(s)[i];
  }
}

template <int RB>
__global__ __launch_bounds__(NT) void compact_move_kernel(kvc_cache_t src, const float* __restrict__ src_score,
                                                          const uint8_t* __restrict__ mask, kvc_cache_t dst,
                                                          float* __restrict__ dst_score,
                                                          const int32_t* __restrict__ counts, int chunks) {
  const int ch = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int H = src.num_kv_heads;
  const int L = min(min(src.lengths[b], src.capacity), chunks * CH);
  const long long rowoff = ((long long)b * H + g) * src.capacity;
  __shared__ int tmp[16];
  // Offset of this chunk: kept slots in the chunks before it.
  int off = 0;
  const int32_t* cr = counts + ((long long)b * H + g) * chunks;
  for (int q = tid; q < ch; q += NT) off += cr[q];
  off = block_sum(off, tmp);
  if (ch * CH >= L) {
    if (ch == 0 && g == 0 && tid == 0) {
      dst.lengths[b] = 0;
      dst.num_seen[b] = src.num_seen[b];
    }
    return;
  }
  // Each thread scans PER consecutive slots.
  const int i0 = ch * CH + tid * PER;
  int flags = 0, n = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = i0 + q;
    const int f = (i < L) && mask[rowoff + i] != 0;
    flags |= f << q;
    n += f;
  }
  // Inclusive scan of n over the workgroup.
  const int lane = tid & 63, wave = tid >> 6;
  int incl = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) tmp[8 + wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += tmp[8 + w];
  int d = off + incl - n;
  const uint8_t* sk = static_cast<const uint8_t*>(src.k_codes);
  const uint8_t* sv = static_cast<const uint8_t*>(src.v_codes);
  uint8_t* dk = static_cast<uint8_t*>(dst.k_codes);
  uint8_t* dv = static_cast<uint8_t*>(dst.v_codes);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (flags & (1 << q)) {
      const long long si = rowoff + i0 + q, di = rowoff + d;
      copy_row<RB>(sk + si * RB, dk + di * RB);
      copy_row<RB>(sv + si * RB, dv + di * RB);
      dst.k_scale[di] = src.k_scale[si];
      dst.v_scale[di] = src.v_scale[si];
      if (src.positions && dst.positions) dst.positions[di] = src.positions[si];
      if (src_score && dst_score) dst_score[di] = src_score[si];
      ++d;
    }
  }
  // The chunk holding the row's last slot knows the row's total.
  if (g == 0 && ch == (L - 1) / CH && tid == NT - 1) {
    dst.lengths[b] = d;
    dst.num_seen[b] = src.num_seen[b];
  }
}

template <int RB>
hipError_t launch_move(const kvc_cache_t& src, const float* ss, const uint8_t* mask, const kvc_cache_t& dst,
                       float* ds, const int32_t* counts, int chunks, hipStream_t st) {
  hipLaunchKernelGGL(compact_move_kernel<RB>, dim3(chunks, src.num_kv_heads, src.batch), dim3(NT), 0, st, src, ss,
                     mask, dst, ds, counts, chunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compact(const kvc_cache_t& src, const float* src_score, const uint8_t* mask,
                          const kvc_cache_t& dst, float* dst_score, int32_t* counts, int chunks, hipStream_t st) {
  hipLaunchKernelGGL(compact_count_kernel, dim3(chunks, src.num_kv_heads, src.batch), dim3(NT), 0, st, src, mask,
                     counts, chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int RB = src.head_dim * src.bits / 8;
  switch (RB) {
    case 32: return launch_move<32>(src, src_score, mask, dst, dst_score, counts, chunks, st);
    case 64: return launch_move<64>(src, src_score, mask, dst, dst_score, counts, chunks, st);
    case 128: return launch_move<128>(src, src_score, mask, dst, dst_score, counts, chunks, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvc
