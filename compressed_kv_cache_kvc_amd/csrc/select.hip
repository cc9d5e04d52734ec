// Keep-set selection: attention sinks + recent window + top-k heavy hitters.
//
// Sinks are the first tokens of the sequence and the window its most recent
// tokens ("KV Cache Compression Report", section 3.3); the rest of the budget
// goes to the tokens with the largest accumulated attention (section 3.4 of the
// report; "KV Cache optimization techniques" tutorial, section 2.2). Equal
// scores go to the lower slot, so the result is unique.
//
// One 1024-thread workgroup per (sequence, KV head) row. The k-th largest score
// among the candidates is found by an MSB-first radix select over the fp32 bit
// patterns (mapped to an unsigned order-preserving key), four passes of 8-bit
// digits with an LDS histogram; the digit search is a wave-wide suffix scan.
// Candidates strictly above the threshold are kept; of those equal to it, the
// first `need` in slot order are kept, ranked by a block-wide prefix count.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int NT = 1024;

__device__ __forceinline__ unsigned order_key(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the workgroup; `tmp` holds 16 ints of LDS.
__device__ __forceinline__ int block_inclusive_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += tmp[w];
  __syncthreads();
  return v + add;
}

__global__ __launch_bounds__(NT) void select_kernel(kvc_cache_t c, const float* __restrict__ score, int budget,
                                                    int n_sink, int n_recent, uint8_t* __restrict__ mask,
                                                    int max_len) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = min(min(c.lengths[b], c.capacity), max_len);
  const long long rowoff = ((long long)b * c.num_kv_heads + g) * c.capacity;
  const float* row = score + rowoff;
  uint8_t* m = mask + rowoff;
  if (L <= budget) {
    for (int i = tid; i < L; i += NT) m[i] = 1;
    return;
  }
  const int lo = n_sink, hi = L - n_recent;
  int k = budget - n_sink - n_recent;

  __shared__ int hist[256];
  __shared__ int sel_digit, sel_k;
  __shared__ int scan_tmp[16];

  unsigned prefix = 0, pmask = 0;
  if (k > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += NT) hist[i] = 0;
      __syncthreads();
      for (int i = lo + tid; i < hi; i += NT) {
        const unsigned u = order_key(row[i]);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns digits 255-4l .. 252-4l (descending order)
        int cnt[4], tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          cnt[q] = hist[255 - 4 * tid - q];
          tot += cnt[q];
        }
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int n = __shfl_up(incl, o);
          if (tid >= o) incl += n;
        }
        int before = incl - tot;  // count of keys with a larger digit than this lane's first
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (before < k && k <= before + cnt[q]) {
            sel_digit = 255 - 4 * tid - q;
            sel_k = k - before;
          }
          before += cnt[q];
        }
      }
      __syncthreads();
      prefix |= (unsigned)sel_digit << shift;
      pmask |= 255u << shift;
      k = sel_k;
      __syncthreads();
    }
  }
  // `prefix` is the threshold key (valid when the heavy-hitter count > 0) and
  // `k` the number of threshold-equal candidates to keep.
  const bool any_heavy = budget - n_sink - n_recent > 0;
  const int per = (L + NT - 1) / NT;
  const int i0 = tid * per, i1 = min(i0 + per, L);
  int ties = 0;
  if (any_heavy) {
    for (int i = max(i0, lo); i < min(i1, hi); ++i) ties += order_key(row[i]) == prefix;
  }
  const int incl = block_inclusive_scan(ties, scan_tmp);
  int rank = incl - ties;
  for (int i = i0; i < i1; ++i) {
    uint8_t keep;
    if (i < lo || i >= hi) {
      keep = 1;
    } else if (!any_heavy) {
      keep = 0;
    } else {
      const unsigned u = order_key(row[i]);
      if (u > prefix) {
        keep = 1;
      } else if (u == prefix) {
        keep = rank < k;
        ++rank;
      } else {
        keep = 0;
      }
    }
    m[i] = keep;
  }
}

}  // namespace

hipError_t launch_select(const kvc_cache_t& c, const float* score, int budget, int n_sink, int n_recent,
                         uint8_t* mask, int max_len, hipStream_t st) {
  hipLaunchKernelGGL(select_kernel, dim3(c.num_kv_heads, c.batch), dim3(NT), 0, st, c, score, budget, n_sink,
                     n_recent, mask, max_len);
  return hipGetLastError();
}

}  // namespace kvc
