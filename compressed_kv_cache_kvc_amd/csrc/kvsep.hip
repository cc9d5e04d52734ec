// K/V-separated attention: the output from the top-k tokens' fp16 V rows.
//
// "KV Cache Compression Report", section 3.5: the quantized K of every token
// stays on the GPU and scores the query; full-precision V is split into hot
// rows on the GPU and cold rows in host memory, fetched on demand for the
// top-scored tokens. Here the scores, the softmax statistics and the H2O mass
// come from the ordinary attention kernels, the selection from the keep-set
// kernel (top_k per KV head by the step's group mass, no sinks or window),
// and kvsep_gather_kernel (several workgroups per row, each over a share of
// the kept tokens, their sums added in order) forms, per query head,
//   out = sum over kept i of exp2(s_i - m) / l * v_i,
// with m and l taken over the kept tokens only and v_i the token's fp16 row:
// from the cache's fp16 tiers when slot i is on one (hot), else from the
// caller's pinned host array (cold; the kernel reads host memory directly).
#include "kvc_internal.h"

namespace kvc {
namespace {

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* tmp) {
  v = MAX ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // tmp is free
  if (lane == 0) tmp[wave] = v;
  __syncthreads();
  return MAX ? fmaxf(fmaxf(tmp[0], tmp[1]), fmaxf(tmp[2], tmp[3])) : (tmp[0] + tmp[1]) + (tmp[2] + tmp[3]);
}

// Workgroup (g, b, part): KV head g of sequence b, kept tokens
// [part * chunk, (part + 1) * chunk) of the row's list; GM >= G query heads.
// Each part writes its sum for every head to a.part_o; kvsep_reduce_kernel
// adds the parts in order.
template <int D, int GM>
__global__ __launch_bounds__(256) void kvsep_gather_kernel(KvsepArgs a) {
  constexpr int CPL = D / 64;  // channels per lane
  constexpr int UN = 32;       // kept tokens per wave per round (their V loads go out together)
  const kvc_cache_t& c = a.c;
  const int g = blockIdx.x, b = blockIdx.y, part = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H;
  // The selection saw at most max_len slots; kept slots are below L.
  const int L = __builtin_amdgcn_readfirstlane(
      max(0, min(min(min(c.lengths[b], c.capacity), (int)a.span), a.max_len)));
  const int seen = __builtin_amdgcn_readfirstlane(c.num_seen[b]);
  const int n = min(L, a.top_k);
  const int chunk = (n + a.parts - 1) / a.parts;
  const int i_lo = min(n, part * chunk), i_hi = min(n, i_lo + chunk);
  const long long row = (long long)b * H + g;
  const int32_t* keep = a.keep + row * a.top_k;
  const float* lg = a.logits + ((long long)b * Hq + g * G) * a.span;
  const int ns = min(c.fp16_sinks, L), nr = min(c.fp16_recent, L - ns);
  const __half* sink = static_cast<const __half*>(c.v_sink16) + row * c.fp16_sinks * D;
  const __half* ring = static_cast<const __half*>(c.v_recent16) + row * c.fp16_recent * D;
  const __half* host = a.v_host + row * (long long)c.capacity * D;

  __shared__ float tmp[4];
  __shared__ float m_s[GM], inv_s[GM];
  __shared__ float red_o[4][GM * D];

  // ---- per head: max and sum of exp2 over the kept tokens' logits ----
  for (int h = 0; h < G; ++h) {
    float mx = -INFINITY;
    for (int i = tid; i < n; i += 256) {
      const int s = keep[i];
      if ((unsigned)s < (unsigned)L) mx = fmaxf(mx, lg[h * a.span + s]);
    }
    mx = block_reduce<true>(mx, tmp);
    float sm = 0.f;
    for (int i = tid; i < n; i += 256) {
      const int s = keep[i];
      if ((unsigned)s < (unsigned)L) sm += __builtin_amdgcn_exp2f(lg[h * a.span + s] - mx);
    }
    sm = block_reduce<false>(sm, tmp);
    if (tid == 0) {
      m_s[h] = mx;
      inv_s[h] = sm > 0.f ? 1.f / sm : 0.f;
    }
  }
  __syncthreads();

  // ---- o = sum p v: wave w takes kept tokens w, w + 4, ...; lanes over channels ----
  float o[GM][CPL];
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < CPL; ++e) o[h][e] = 0.f;
  for (int i0 = i_lo + wave; i0 < i_hi; i0 += 4 * UN) {
    float v[UN][CPL];
    int sl[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int i = i0 + 4 * u;
      sl[u] = i < i_hi ? keep[i] : -1;
      if ((unsigned)sl[u] >= (unsigned)L) sl[u] = -1;
      const int s = sl[u];
      const __half* src = s < 0 ? nullptr
                          : s < ns ? sink + (long long)s * D
                          : s >= L - nr ? ring + (long long)((unsigned)(seen - L + s) % (unsigned)c.fp16_recent) * D
                                        : host + (long long)s * D;
#pragma unroll
      for (int e = 0; e < CPL; ++e) v[u][e] = src ? __half2float(src[lane * CPL + e]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (sl[u] < 0) continue;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h >= G) break;
        const float p = __builtin_amdgcn_exp2f(lg[h * a.span + sl[u]] - m_s[h]) * inv_s[h];
#pragma unroll
        for (int e = 0; e < CPL; ++e) o[h][e] = fmaf(p, v[u][e], o[h][e]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < CPL; ++e) red_o[wave][h * D + lane * CPL + e] = o[h][e];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const float r = (red_o[0][idx] + red_o[1][idx]) + (red_o[2][idx] + red_o[3][idx]);
    const int h = idx / D, d = idx - h * D;
    a.part_o[(((long long)b * Hq + g * G + h) * a.parts + part) * D + d] = r;
  }
}

// out[b][h][:] = the parts' sums, added in part order (deterministic).
__global__ __launch_bounds__(128) void kvsep_reduce_kernel(const float* __restrict__ part_o, float* __restrict__ out,
                                                           int parts, int D) {
  const long long bh = blockIdx.x;
  for (int d = threadIdx.x; d < D; d += 128) {
    float r = 0.f;
    for (int p = 0; p < parts; ++p) r += part_o[(bh * parts + p) * D + d];
    out[bh * D + d] = r;
  }
}

template <int D>
hipError_t launch_d(const KvsepArgs& a, hipStream_t st) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const dim3 grid(a.c.num_kv_heads, a.c.batch, a.parts);
  if (G == 1) hipLaunchKernelGGL((kvsep_gather_kernel<D, 1>), grid, dim3(256), 0, st, a);
  else if (G == 2) hipLaunchKernelGGL((kvsep_gather_kernel<D, 2>), grid, dim3(256), 0, st, a);
  else if (G <= 4) hipLaunchKernelGGL((kvsep_gather_kernel<D, 4>), grid, dim3(256), 0, st, a);
  else if (G <= 8) hipLaunchKernelGGL((kvsep_gather_kernel<D, 8>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((kvsep_gather_kernel<D, 16>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_zero(float* p, long long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_kvsep_gather(const KvsepArgs& a, hipStream_t st) {
  const hipError_t e = a.c.head_dim == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kvsep_reduce_kernel, dim3((unsigned)((long long)a.c.batch * a.num_q_heads)), dim3(128), 0, st,
                     a.part_o, a.out, a.parts, a.c.head_dim);
  return hipGetLastError();
}

}  // namespace kvc
