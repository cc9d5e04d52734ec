// Read-bandwidth probe: one streaming read of a device buffer, for measuring
// the HBM read ceiling a single launch reaches on this GPU (the context for
// the decode-attention roofline, whose KV stream is a read of the same size).
//
// Every lane reads 16-byte words with the attention kernel's load width, a
// grid-stride loop over 4096 workgroups of 256 threads (16 per CU, eight
// words in flight per lane per iteration: the fastest of the shapes measured,
// about 5.2 TB/s on 66 MiB, with 8192 x 4 equal); each workgroup folds what it
// read into one word (XOR) and writes it, so no load can be dropped.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void bw_probe_kernel(const u32x4* __restrict__ src, long long words,
                                                                 unsigned* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * kProbeThreads;
  long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < words; i += kProbeUnroll * stride) {
    u32x4 w[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) w[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= w[u];
  }
  for (; i < words; i += stride) acc ^= src[i];
  unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ unsigned red[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

int bw_probe_workgroups() { return 4096; }

hipError_t launch_bw_probe(const void* src, size_t bytes, unsigned* sink, hipStream_t st) {
  hipLaunchKernelGGL(bw_probe_kernel, dim3(bw_probe_workgroups()), dim3(kProbeThreads), 0, st,
                     static_cast<const u32x4*>(src), (long long)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace kvc
