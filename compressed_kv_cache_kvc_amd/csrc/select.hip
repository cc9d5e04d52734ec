// Keep-set selection: attention sinks + recent window + top-k heavy hitters.
//
// Sinks are the first tokens of the sequence and the window its most recent
// tokens ("KV Cache Compression Report", section 3.3); the rest of the budget
// goes to the tokens with the largest accumulated attention (section 3.4 of the
// report; "KV Cache optimization techniques" tutorial, section 2.2). Equal
// scores go to the lower slot, so the result is unique.
//
// One 1024-thread workgroup per (sequence, KV head) row; scores become
// order-preserving unsigned keys. The threshold T is the k-th largest key:
//  * T is found by an MSB-first radix select: four passes of 8-bit digits,
//    each a histogram of the keys that still match the digits chosen so far,
//    then a wave-wide suffix scan that picks the digit holding the k-th key;
//  * rows of up to 16 candidates per thread keep their keys in registers and
//    give every wave its own LDS histogram (two barriers per pass);
//  * longer rows read their keys from memory on every pass and share eight
//    sub-histograms.
// Keys above T are kept; of the keys equal to T, the first (k - count above T)
// in slot order are kept, ranked by a block-wide prefix count over
// thread-contiguous slot ranges.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int NT = 1024;
constexpr int NSUB = 8;
constexpr int kRegKeys = 16;  // keys per thread in the register path

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

// Write the mask of one row given the threshold key T and the number of
// T-equal candidates to keep. `key_at(i)` returns the key of candidate slot i.
template <typename KeyAt>
__device__ __forceinline__ void write_mask(uint8_t* m, int L, int lo, int hi, bool any_heavy, unsigned T,
                                           int need, KeyAt key_at, int* scan_tmp) {
  const int tid = threadIdx.x;
  for (int i = tid; i < lo; i += NT) m[i] = 1;
  for (int i = hi + tid; i < L; i += NT) m[i] = 1;
  const int n = hi - lo;
  const int per = (n + NT - 1) / NT;
  const int i0 = lo + min(tid * per, n), i1 = lo + min(tid * per + per, n);
  int ties = 0;
  if (any_heavy)
    for (int i = i0; i < i1; ++i) ties += key_at(i) == T;
  int rank = block_inclusive_scan(ties, scan_tmp) - ties;
  for (int i = i0; i < i1; ++i) {
    uint8_t keep = 0;
    if (any_heavy) {
      const unsigned u = key_at(i);
      if (u > T) {
        keep = 1;
      } else if (u == T) {
        keep = rank < need;
        ++rank;
      }
    }
    m[i] = keep;
  }
}

__global__ __launch_bounds__(NT) void select_reg_kernel(kvc_cache_t c, const float* __restrict__ score, int budget,
                                                        int n_sink, int n_recent, uint8_t* __restrict__ mask,
                                                        int max_len) {
  constexpr int NWAVE = NT / 64;
  __shared__ int hist[NWAVE][256];  // one histogram per wave: no cross-wave contention
  __shared__ int sel_digit, sel_k;
  __shared__ int scan_tmp[16];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = __builtin_amdgcn_readfirstlane(min(min(c.lengths[b], c.capacity), max_len));
  const long long rowoff = ((long long)b * c.num_kv_heads + g) * c.capacity;
  const float* row = score + rowoff;
  uint8_t* m = mask + rowoff;
  if (L <= budget) {
    for (int i = tid; i < L; i += NT) m[i] = 1;
    return;
  }
  const int lo = n_sink, hi = L - n_recent, n = hi - lo;
  int k = budget - n_sink - n_recent;
  // Thread t holds candidates [lo + t*per, lo + t*per + per) (per <= kRegKeys;
  // the host routes longer rows to the radix kernel). Unconditional loads from
  // clamped slots keep all of them in flight at once.
  const int per = (n + NT - 1) / NT;
  const int i0 = lo + min(tid * per, n), cnt = min(tid * per + per, n) - min(tid * per, n);
  unsigned key[kRegKeys];
#pragma unroll
  for (int q = 0; q < kRegKeys; ++q) key[q] = order_key(row[lo + min(i0 - lo + q, n - 1)]);

  unsigned T = 0, pmask = 0;
  const bool any_heavy = k > 0;
  if (any_heavy) {
    for (int i = tid; i < NWAVE * 256; i += NT) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
#pragma unroll
      for (int q = 0; q < kRegKeys; ++q)
        if (q < cnt && (key[q] & pmask) == T) atomicAdd(&hist[wave][(key[q] >> shift) & 255u], 1);
      __syncthreads();
      if (wave == 0) {
        // Lane l owns digits 4l .. 4l+3: sum them over the per-wave
        // histograms (and clear those for the next pass), then a suffix scan
        // from the largest digit finds the one holding the k-th largest key.
        int cnt4[4] = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
          int4* hp = reinterpret_cast<int4*>(&hist[w][4 * lane]);
          const int4 h4 = *hp;
          cnt4[0] += h4.x;
          cnt4[1] += h4.y;
          cnt4[2] += h4.z;
          cnt4[3] += h4.w;
          *hp = make_int4(0, 0, 0, 0);
        }
        const int tot = cnt4[0] + cnt4[1] + cnt4[2] + cnt4[3];
        // Inclusive scan from the top: lanes 63 .. lane.
        int suf = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int nb = __shfl_down(suf, o);
          if (lane + o < 64) suf += nb;
        }
        int above = suf - tot;  // keys whose digit is larger than this lane's four
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (above < k && k <= above + cnt4[q]) {
            sel_digit = 4 * lane + q;
            sel_k = k - above;
          }
          above += cnt4[q];
        }
      }
      __syncthreads();
      T |= (unsigned)sel_digit << shift;
      pmask |= 255u << shift;
      k = sel_k;
    }
  }
  // T is the threshold key and k the number of T-equal candidates to keep,
  // lowest slots first.
  for (int i = tid; i < lo; i += NT) m[i] = 1;
  for (int i = hi + tid; i < L; i += NT) m[i] = 1;
  int ties = 0;
#pragma unroll
  for (int q = 0; q < kRegKeys; ++q) ties += any_heavy & (q < cnt) & (key[q] == T);
  int rank = block_inclusive_scan(ties, scan_tmp) - ties;
#pragma unroll
  for (int q = 0; q < kRegKeys; ++q) {
    if (q < cnt) {
      uint8_t keep = 0;
      if (any_heavy) {
        if (key[q] > T) {
          keep = 1;
        } else if (key[q] == T) {
          keep = rank < k;
          ++rank;
        }
      }
      m[i0 + q] = keep;
    }
  }
}

__global__ __launch_bounds__(NT) void select_radix_kernel(kvc_cache_t c, const float* __restrict__ score,
                                                          int budget, int n_sink, int n_recent,
                                                          uint8_t* __restrict__ mask, int max_len) {
  __shared__ int hist[NSUB][256];
  __shared__ int sel_digit, sel_k;
  __shared__ int scan_tmp[16];

  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = __builtin_amdgcn_readfirstlane(min(min(c.lengths[b], c.capacity), max_len));
  const long long rowoff = ((long long)b * c.num_kv_heads + g) * c.capacity;
  const float* row = score + rowoff;
  uint8_t* m = mask + rowoff;
  if (L <= budget) {
    for (int i = tid; i < L; i += NT) m[i] = 1;
    return;
  }
  const int lo = n_sink, hi = L - n_recent;
  const int k_heavy = budget - n_sink - n_recent;
  auto key_at = [&](int i) -> unsigned { return order_key(row[i]); };

  unsigned prefix = 0, pmask = 0;
  int k = k_heavy;
  if (k > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < NSUB * 256; i += NT) (&hist[0][0])[i] = 0;
      __syncthreads();
      int* h = hist[(tid >> 6) & (NSUB - 1)];
      for (int i = lo + tid; i < hi; i += NT) {
        const unsigned u = key_at(i);
        if ((u & pmask) == prefix) atomicAdd(&h[(u >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns digits 255-4l .. 252-4l (descending order)
        int cnt[4], tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int s = 0;
#pragma unroll
          for (int sub = 0; sub < NSUB; ++sub) s += hist[sub][255 - 4 * tid - q];
          cnt[q] = s;
          tot += s;
        }
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int n = __shfl_up(incl, o);
          if (tid >= o) incl += n;
        }
        int before = incl - tot;  // keys with a larger digit than this lane's first
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
    }
  }
  write_mask(m, L, lo, hi, k_heavy > 0, prefix, k, key_at, scan_tmp);
}

}  // namespace

hipError_t launch_select(const kvc_cache_t& c, const float* score, int budget, int n_sink, int n_recent,
                         uint8_t* mask, int max_len, hipStream_t st) {
  const long long cand = (long long)max_len - n_sink - n_recent;
  if (cand <= (long long)NT * kRegKeys)
    hipLaunchKernelGGL(select_reg_kernel, dim3(c.num_kv_heads, c.batch), dim3(NT), 0, st, c, score, budget, n_sink,
                       n_recent, mask, max_len);
  else
    hipLaunchKernelGGL(select_radix_kernel, dim3(c.num_kv_heads, c.batch), dim3(NT), 0, st, c, score, budget,
                       n_sink, n_recent, mask, max_len);
  return hipGetLastError();
}

}  // namespace kvc
