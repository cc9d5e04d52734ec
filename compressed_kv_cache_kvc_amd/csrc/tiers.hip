// Storing the fp16 rows of appended tokens in the fp16 tiers of a cache.
//
// "KV Cache Compression Report", section 3.2 keeps the attention sinks' K and
// V in fp16; the "KV Cache optimization techniques" tutorial, section 1.3
// keeps recent tokens at fp16 (its "int4_hybrid" mode). The sink rows are
// indexed by slot (slot j < fp16_sinks is always the j-th token: eviction
// keeps the sinks and compaction is stable); the recent rows form a ring
// indexed by position % fp16_recent. The appends still quantize every token;
// the attention over the tiers is in tiers.h.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Store the fp16 rows of appended tokens in the tiers. Thread i of the grid
// copies 16 bytes: token t = i / (D / 8), chunk i % (D / 8). Slot
// lengths[b] + t < fp16_sinks goes to the sink rows; the newest fp16_recent
// of the n_new tokens go to the ring (older ones would be overwritten).
template <int D>
__global__ __launch_bounds__(256) void tier_append_kernel(kvc_cache_t c, const __half* __restrict__ kn,
                                                          const __half* __restrict__ vn, int n_new) {
  constexpr int NCH = D / 8;
  const int g = blockIdx.y, b = blockIdx.z, H = c.num_kv_heads;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int t = i / NCH, ch = i % NCH;
  if (t >= n_new) return;
  const int L0 = c.lengths[b], ns0 = c.num_seen[b];
  const long long row = (long long)b * H + g;
  const long long src = (row * n_new + t) * D + ch * 8;
  const u32x4 kx = *reinterpret_cast<const u32x4*>(kn + src);
  const u32x4 vx = *reinterpret_cast<const u32x4*>(vn + src);
  const long long slot = (long long)L0 + t;
  if (slot >= 0 && slot < c.fp16_sinks) {
    const long long dst = (row * c.fp16_sinks + slot) * D + ch * 8;
    *reinterpret_cast<u32x4*>(static_cast<__half*>(c.k_sink16) + dst) = kx;
    *reinterpret_cast<u32x4*>(static_cast<__half*>(c.v_sink16) + dst) = vx;
  }
  if (c.fp16_recent > 0 && t >= n_new - c.fp16_recent) {
    const unsigned p = (unsigned)(ns0 + t) % (unsigned)c.fp16_recent;
    const long long dst = (row * c.fp16_recent + p) * D + ch * 8;
    *reinterpret_cast<u32x4*>(static_cast<__half*>(c.k_recent16) + dst) = kx;
    *reinterpret_cast<u32x4*>(static_cast<__half*>(c.v_recent16) + dst) = vx;
  }
}

}  // namespace

hipError_t launch_tier_append(const kvc_cache_t& c, const __half* kn, const __half* vn, int n_new,
                              hipStream_t st) {
  if (c.fp16_sinks <= 0 && c.fp16_recent <= 0) return hipSuccess;
  const long long threads = (long long)n_new * (c.head_dim / 8);
  const dim3 grid((unsigned)((threads + 255) / 256), c.num_kv_heads, c.batch);
  if (c.head_dim == 64) hipLaunchKernelGGL((tier_append_kernel<64>), grid, dim3(256), 0, st, c, kn, vn, n_new);
  else hipLaunchKernelGGL((tier_append_kernel<128>), grid, dim3(256), 0, st, c, kn, vn, n_new);
  return hipGetLastError();
}

}  // namespace kvc
