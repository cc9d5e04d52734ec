// Radix selection of the k-th largest H2O score of a row, shared by the
// selection kernel and the fused selection-and-compaction kernel.
//
// Scores become order-preserving unsigned keys and the threshold T is the k-th
// largest key, found by an MSB-first radix select ("KV Cache Compression
// Report", section 3.4: keep the top-scoring tokens; "KV Cache optimization
// techniques" tutorial, section 2.2):
//  * the bits shared by the row's smallest and largest key are known at once
//    (one block reduction), so digits start at the first bit that varies;
//  * digits are up to 11 bits wide (2048-bin LDS histogram, at most three
//    passes). Wide digits that start where keys differ spread each wave's
//    histogram increments over many bins (LDS atomics that collide on one
//    address within a wave instruction serialize; scores are probability mass
//    and mostly share a few binary exponents);
//  * the histogram can be replicated (COPIES copies, a lane adding into copy
//    lane % COPIES, the copies of a bin adjacent): lanes of one wave whose
//    keys fall in the same bin then collide in groups of at most 64 / COPIES
//    instead of 64;
//  * the bin holding the k-th key comes from a block-wide suffix scan; once
//    that bin holds at most 64 keys, they are gathered into LDS and ranked
//    directly (every key's count of keys above and equal to it, spread over
//    the whole workgroup), which ends the search without further passes.
#pragma once

#include "kvc_internal.h"

namespace kvc {
namespace radix {

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

// Inclusive prefix sum over a workgroup of NT threads with a single barrier:
// `tmp` (NT/64 ints of LDS) must not be written again before another barrier.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan_1b(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_inclusive_scan(v);
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) add += (w < wave) ? tmp[w] : 0;
  return v + add;
}

// Clears the histogram (kBins * COPIES ints) and the gather counter; a
// barrier must follow before radix_threshold_range runs.
template <int NT, int COPIES = 1>
__device__ __forceinline__ void radix_clear(int* hist, int* sel) {
  for (int i = threadIdx.x; i < kBins * COPIES; i += NT) hist[i] = 0;
  if (threadIdx.x == 0) sel[3] = 0;
}

// Radix select over the candidates, whose smallest and largest keys are kmin
// and kmax. `for_keys(f)` calls f(key) for each of the calling thread's
// candidate keys (key 0 may stand for an unused slot: it is never counted).
// On entry `hist` is zero and sel[3] == 0 (radix_clear, then a barrier). On
// return, T is the k-th largest key and `k` the number of keys equal to T that
// are kept.
template <int NT, int COPIES = 1, typename ForKeys>
__device__ __forceinline__ unsigned radix_threshold_range(ForKeys for_keys, int& k, unsigned kmin, unsigned kmax,
                                                          int* hist, int* scan_tmp, int* sel, unsigned* small) {
  constexpr int BPT = kBins / NT;  // bins per thread in the digit search
  static_assert(COPIES == 1 || COPIES == 4 || COPIES == 8, "COPIES");
  const int tid = threadIdx.x;
  const int cp = COPIES > 1 ? (tid & (COPIES - 1)) : 0;
  const unsigned diff = kmin ^ kmax;
  if (diff == 0) return kmin;  // every candidate equal: keep the lowest k slots
  int remaining = 32 - __clz(diff);  // low bits still undecided
  const unsigned low = (remaining == 32) ? 0xFFFFFFFFu : ((1u << remaining) - 1u);
  unsigned T = kmin & ~low, pmask = ~low;
  bool first = true;
  while (remaining > 0) {
    const int width = min(kDigitBits, remaining);
    const int shift = remaining - width;
    const unsigned dmask = (1u << width) - 1u;
    if (first) {
      // Every real key shares the prefix T of the first pass: add the match
      // flag instead of branching per key.
      for_keys([&](unsigned u) {
        atomicAdd(&hist[((u >> shift) & dmask) * COPIES + cp], (int)((u & pmask) == T));
      });
    } else {
      for_keys([&](unsigned u) {
        if ((u & pmask) == T) atomicAdd(&hist[((u >> shift) & dmask) * COPIES + cp], 1);
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
      if constexpr (COPIES == 1) {
        c[j] = hist[top - j];
        hist[top - j] = 0;
      } else {
        int4* h4 = reinterpret_cast<int4*>(hist + (top - j) * COPIES);
        c[j] = 0;
#pragma unroll
        for (int q = 0; q < COPIES / 4; ++q) {
          const int4 x = h4[q];
          c[j] += x.x + x.y + x.z + x.w;
          h4[q] = make_int4(0, 0, 0, 0);
        }
      }
      tot += c[j];
    }
    // scan_tmp is next written after the barrier below and the histogram's.
    const int incl = block_inclusive_scan_1b<NT>(tot, scan_tmp);
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
      // Every wave ranks: NT / 64 adjacent threads per gathered key, each
      // comparing it with 64 / (NT / 64) of the others, then a sum over the
      // key's threads. Equal keys write the same result.
      constexpr int TPK = NT / 64, JPT = 64 / TPK;
      static_assert(TPK >= 1 && TPK <= 64 && TPK * JPT == 64, "NT");
      const int n_small = sel[2];
      const int ki = tid / TPK, part = tid % TPK;
      const unsigned u = small[min(ki, n_small - 1)];
      int gt = 0, eq = 0;
#pragma unroll
      for (int q = 0; q < JPT; ++q) {
        const int j = part * JPT + q;
        const unsigned w = small[min(j, n_small - 1)];
        gt += (j < n_small) & (w > u);
        eq += (j < n_small) & (w == u);
      }
#pragma unroll
      for (int o = 1; o < TPK; o <<= 1) {
        gt += __shfl_xor(gt, o);
        eq += __shfl_xor(eq, o);
      }
      if (part == 0 && ki < n_small && gt < k && k <= gt + eq) {
        sel[0] = (int)u;
        sel[1] = k - gt;
      }
      __syncthreads();
      k = sel[1];
      return (unsigned)sel[0];
    }
  }
  return T;
}

// The same with the key range found here: one block reduction, the clear and
// a barrier come first.
template <int NT, int COPIES = 1, typename ForKeys>
__device__ __forceinline__ unsigned radix_threshold(ForKeys for_keys, int& k, int* hist, int* scan_tmp,
                                                    unsigned* mm_tmp, int* sel, unsigned* small) {
  unsigned kmin = 0xFFFFFFFFu, kmax = 0u;
  for_keys([&](unsigned u) {  // key 0 marks an unused register slot
    kmin = min(kmin, u == 0u ? 0xFFFFFFFFu : u);
    kmax = max(kmax, u);
  });
  block_minmax<NT>(kmin, kmax, mm_tmp);
  radix_clear<NT, COPIES>(hist, sel);
  __syncthreads();
  return radix_threshold_range<NT, COPIES>(for_keys, k, kmin, kmax, hist, scan_tmp, sel, small);
}

}  // namespace radix
}  // namespace kvc
