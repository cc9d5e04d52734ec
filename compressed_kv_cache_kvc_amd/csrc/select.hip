// Keep-set selection: attention sinks + recent window + top-k heavy hitters.
//
// Sinks are the first tokens of the sequence and the window its most recent
// tokens ("KV Cache Compression Report", section 3.3); the rest of the budget
// goes to the tokens with the largest accumulated attention (section 3.4 of the
// report; "KV Cache optimization techniques" tutorial, section 2.2). Equal
// scores go to the lower slot, so the result is unique.
//
// One workgroup per (sequence, KV head) row; scores become order-preserving
// unsigned keys and the threshold T is the k-th largest key, found by an
// MSB-first radix select:
//  * the bits shared by the row's smallest and largest key are known at once
//    (one block reduction), so digits start at the first bit that varies;
//  * digits are up to 11 bits wide (2048-bin LDS histogram, at most three
//    passes). Wide digits that start where keys differ spread each wave's
//    histogram increments over many bins (LDS atomics that collide on one
//    address within a wave instruction serialize; scores are probability mass
//    and mostly share a few binary exponents);
//  * the bin holding the k-th key comes from a block-wide suffix scan; once
//    that bin holds at most 64 keys, they are gathered into LDS and one wave
//    ranks them directly (each lane counts the keys above and equal to its
//    own), which ends the search without further passes.
// Rows of up to 8192 candidates use 1024 threads holding up to 8 keys each in
// registers, with no per-key branches (unused slots hold key 0); with a single
// workgroup per row the kernel is latency-bound, and 16 waves per CU hide each
// other's latency. Longer rows use 1024 threads that re-read their keys from
// memory on every pass. Keys above T are kept; of the
// keys equal to T, the first (k - count above T) in slot order are kept,
// ranked by a block-wide prefix count over thread-contiguous slot ranges.
//
// Besides the mask, the kernel can emit the sorted list of kept slots (the
// gather list of the compaction that follows).
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

__device__ __forceinline__ unsigned order_key(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide min and max of unsigned keys (every thread gets both): DPP wave
// reductions, then the wave results through LDS.
template <int NT>
__device__ __forceinline__ void block_minmax(unsigned& lo, unsigned& hi, unsigned* tmp) {
  lo = wave_minmax_u<false>(lo);
  hi = wave_minmax_u<true>(hi);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    tmp[wave] = lo;
    tmp[16 + wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    lo = min(lo, tmp[w]);
    hi = max(hi, tmp[16 + w]);
  }
  __syncthreads();
}

// Radix select over the candidates. `for_keys(f)` calls f(key) for each of the
// calling thread's candidate keys. On return, T is the k-th largest key and
// `k` the number of keys equal to T that are kept.
template <int NT, typename ForKeys>
__device__ __forceinline__ unsigned radix_threshold(ForKeys for_keys, int& k, int* hist, int* scan_tmp,
                                                    unsigned* mm_tmp, int* sel, unsigned* small) {
  constexpr int BPT = kBins / NT;  // bins per thread in the digit search
  const int tid = threadIdx.x;
  unsigned kmin = 0xFFFFFFFFu, kmax = 0u;
  for_keys([&](unsigned u) {  // key 0 marks an unused register slot
    kmin = min(kmin, u == 0u ? 0xFFFFFFFFu : u);
    kmax = max(kmax, u);
  });
  block_minmax<NT>(kmin, kmax, mm_tmp);
  const unsigned diff = kmin ^ kmax;
  if (diff == 0) return kmin;  // every candidate equal: keep the lowest k slots
  int remaining = 32 - __clz(diff);  // low bits still undecided
  const unsigned low = (remaining == 32) ? 0xFFFFFFFFu : ((1u << remaining) - 1u);
  unsigned T = kmin & ~low, pmask = ~low;
  for (int i = tid; i < kBins; i += NT) hist[i] = 0;
  if (tid == 0) sel[3] = 0;  // keys gathered into `small`
  __syncthreads();
  bool first = true;
  while (remaining > 0) {
    const int width = min(kDigitBits, remaining);
    const int shift = remaining - width;
    const unsigned dmask = (1u << width) - 1u;
    if (first) {
      // Every real key shares the prefix T of the first pass: add the match
      // flag instead of branching per key.
      for_keys([&](unsigned u) { atomicAdd(&hist[(u >> shift) & dmask], (int)((u & pmask) == T)); });
    } else {
      for_keys([&](unsigned u) {
        if ((u & pmask) == T) atomicAdd(&hist[(u >> shift) & dmask], 1);
      });
    }
    first = false;
    __syncthreads();
    // Thread t owns the BPT bins just below kBins - BPT*t, so the inclusive
    // scan over threads counts keys from the largest digit down; each bin is
    // cleared once read.
    const int top = kBins - BPT * tid - 1;
    int c[BPT], tot = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = hist[top - j];
      hist[top - j] = 0;
      tot += c[j];
    }
    const int incl = block_inclusive_scan<NT>(tot, scan_tmp);
    int before = incl - tot;  // keys with a digit above this thread's bins
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (before < k && k <= before + c[j]) {
        sel[0] = top - j;
        sel[1] = k - before;
        sel[2] = c[j];
      }
      before += c[j];
    }
    __syncthreads();
    T |= (unsigned)sel[0] << shift;
    pmask |= dmask << shift;
    k = sel[1];
    remaining = shift;
    if (remaining > 0 && sel[2] <= 64) {
      // Few keys share the prefix found so far: gather them and rank them in
      // one wave. The k-th largest key u has g keys above it and e equal,
      // with g < k <= g + e.
      for_keys([&](unsigned u) {
        if ((u & pmask) == T) small[atomicAdd(&sel[3], 1)] = u;
      });
      __syncthreads();
      const int n_small = sel[2];
      if (tid < 64) {
        const unsigned u = small[min(tid, n_small - 1)];
        int gt = 0, eq = 0;
        for (int j = 0; j < n_small; ++j) {
          const unsigned w = small[j];
          gt += w > u;
          eq += w == u;
        }
        if (tid < n_small && gt < k && k <= gt + eq) {
          sel[0] = (int)u;
          sel[1] = k - gt;
        }
      }
      __syncthreads();
      k = sel[1];
      return (unsigned)sel[0];
    }
  }
  return T;
}

// NT threads; REG: each thread holds KPT consecutive candidates in registers.
template <int NT, int KPT, bool REG>
__global__ __launch_bounds__(NT) void select_kernel(kvc_cache_t c, const float* __restrict__ score, int budget,
                                                    int n_sink, int n_recent, uint8_t* __restrict__ mask,
                                                    int32_t* __restrict__ keep_index, int max_len) {
  __shared__ int hist[kBins];
  __shared__ int scan_tmp[16];
  __shared__ unsigned mm_tmp[32];
  __shared__ int sel[4];
  __shared__ unsigned small[64];
  __shared__ __align__(16) unsigned stage_lds[REG ? NT * KPT : 1];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const long long rowoff = ((long long)b * c.num_kv_heads + g) * c.capacity;
  const float* row = score + rowoff;
  // The register path's coalesced loads cover slots n_sink .. n_sink + NT*KPT
  // - 1 (clamped to the row) and do not wait for the sequence length.
  unsigned v[REG ? KPT : 1];
  if (REG) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) v[j] = order_key(row[min(n_sink + tid + j * NT, c.capacity - 1)]);
  }
  const int L = __builtin_amdgcn_readfirstlane(min(min(c.lengths[b], c.capacity), max_len));
  uint8_t* m = mask + rowoff;
  int32_t* kidx = keep_index ? keep_index + ((long long)b * c.num_kv_heads + g) * budget : nullptr;
  if (L <= budget) {
    for (int i = tid; i < L; i += NT) {
      m[i] = 1;
      if (kidx) kidx[i] = i;
    }
    return;
  }
  const int lo = n_sink, hi = L - n_recent, n = hi - lo;
  int k = budget - n_sink - n_recent;
  // Thread t holds candidates [lo + t*per, lo + t*per + per); per is a
  // multiple of 4, so that its range starts on a 16-byte boundary of the
  // staging buffer.
  const int per = ((n + NT - 1) / NT + 3) & ~3;
  const int i0 = lo + min(tid * per, n), cnt = min(tid * per + per, n) - min(tid * per, n);
  unsigned key[REG ? KPT : 1];
  if (REG) {
    // The coalesced loads (slot lo + tid + j*NT) go to LDS, then each thread
    // reads its contiguous range back with 16-byte LDS reads (its range starts
    // at a multiple of 4 words); staged slots past the candidates are unused.
    unsigned* stage = reinterpret_cast<unsigned*>(stage_lds);
#pragma unroll
    for (int j = 0; j < KPT; ++j) stage[tid + j * NT] = v[j];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KPT; q += 4) {
      const uint4 w = *reinterpret_cast<const uint4*>(stage + min(tid * per + q, NT * KPT - 4));
      key[q] = w.x;
      key[q + 1] = w.y;
      key[q + 2] = w.z;
      key[q + 3] = w.w;
    }
    // Slots past the thread's candidates hold key 0, below every real key
    // (scores are non-negative, so real keys have the top bit set): loops over
    // the keys then need no per-key branch.
#pragma unroll
    for (int q = 0; q < KPT; ++q) key[q] = q < cnt ? key[q] : 0u;
  }
  // Every candidate once, in any order (the histogram passes). Register path:
  // the thread's own keys. Memory path: slots strided over the workgroup
  // (coalesced), KPT unconditional loads from clamped slots in flight at a time.
  auto for_keys = [&](auto f) {
    if (REG) {
#pragma unroll
      for (int q = 0; q < KPT; ++q) f(key[q]);  // key 0 in unused slots
    } else {
      for (int base = lo + tid; base < hi; base += KPT * NT) {
        unsigned kk[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) kk[j] = order_key(row[min(base + j * NT, hi - 1)]);
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          if (base + j * NT < hi) f(kk[j]);
      }
    }
  };
  // The thread's contiguous candidates in slot order: f(slot, key).
  auto for_own = [&](auto f) {
    if (REG) {
#pragma unroll
      for (int q = 0; q < KPT; ++q)
        if (q < cnt) f(i0 + q, key[q]);
    } else {
      for (int q0 = 0; q0 < cnt; q0 += KPT) {
        unsigned kk[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) kk[j] = order_key(row[i0 + min(q0 + j, cnt - 1)]);
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          if (q0 + j < cnt) f(i0 + q0 + j, kk[j]);
      }
    }
  };
  const bool any_heavy = k > 0;
  unsigned T = 0;
  if (any_heavy) T = radix_threshold<NT>(for_keys, k, hist, scan_tmp, mm_tmp, sel, small);

  // Sinks and the recent window are always kept.
  const int n_heavy = budget - n_sink - n_recent;
  for (int i = tid; i < lo; i += NT) {
    m[i] = 1;
    if (kidx) kidx[i] = i;
  }
  for (int i = hi + tid; i < L; i += NT) {
    m[i] = 1;
    if (kidx) kidx[lo + n_heavy + (i - hi)] = i;
  }
  // Candidates: rank the threshold ties in slot order; with a gather list,
  // also count the candidates above T before this thread.
  int ties = 0, above = 0;
  if (REG) {
    // Unused slots hold key 0, never equal to or above T.
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      ties += any_heavy & (key[q] == T);
      above += any_heavy & (key[q] > T);
    }
  } else {
    for_own([&](int, unsigned u) {
      ties += any_heavy & (u == T);
      above += any_heavy & (u > T);
    });
  }
  // Both prefix counts at once when every count fits 16 bits (ties in the
  // low half); longer rows scan them separately.
  int tie_rank, above_before;
  if (n < 65536) {
    const int packed = ties | (above << 16);
    const int before = block_inclusive_scan<NT>(packed, scan_tmp) - packed;
    tie_rank = before & 0xFFFF;
    above_before = before >> 16;
  } else {
    tie_rank = block_inclusive_scan<NT>(ties, scan_tmp) - ties;
    above_before = block_inclusive_scan<NT>(above, scan_tmp) - above;
  }
  // Kept before this thread = candidates above T before it + ties kept before it.
  int out = above_before + min(tie_rank, k);
  for_own([&](int i, unsigned u) {
    uint8_t keepb = 0;
    if (any_heavy) {
      if (u > T) {
        keepb = 1;
      } else if (u == T) {
        keepb = tie_rank < k;
        ++tie_rank;
      }
    }
    m[i] = keepb;
    if (kidx && keepb) kidx[lo + out++] = i;
  });
}

}  // namespace

hipError_t launch_select(const kvc_cache_t& c, const float* score, int budget, int n_sink, int n_recent,
                         uint8_t* mask, int32_t* keep_index, int max_len, hipStream_t st) {
  const long long cand = (long long)max_len - n_sink - n_recent;
  const dim3 grid(c.num_kv_heads, c.batch);
  if (cand <= 1024 * 8)
    hipLaunchKernelGGL((select_kernel<1024, 8, true>), grid, dim3(1024), 0, st, c, score, budget, n_sink, n_recent,
                       mask, keep_index, max_len);
  else
    hipLaunchKernelGGL((select_kernel<1024, 8, false>), grid, dim3(1024), 0, st, c, score, budget, n_sink,
                       n_recent, mask, keep_index, max_len);
  return hipGetLastError();
}

}  // namespace kvc
