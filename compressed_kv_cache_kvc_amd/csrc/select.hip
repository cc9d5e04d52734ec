// Keep-set selection: attention sinks + recent window + top-k heavy hitters.
//
// Sinks are the first tokens of the sequence and the window its most recent
// tokens ("KV Cache Compression Report", section 3.3); the rest of the budget
// goes to the tokens with the largest accumulated attention (section 3.4 of the
// report; "KV Cache optimization techniques" tutorial, section 2.2). Equal
// scores go to the lower slot, so the result is unique.
//
// One workgroup per (sequence, KV head) row finds the threshold T (the k-th
// largest key) with the radix select of radix_select.h. Rows of up to 8192
// candidates use 1024 threads holding up to 8 keys each in registers, with no
// per-key branches (unused slots hold key 0); with a single workgroup per row
// the kernel is latency-bound, and 16 waves per CU hide each other's latency.
// Longer rows use 1024 threads that re-read their keys from memory on every
// pass. Keys above T are kept; of the keys equal to T, the first
// (k - count above T) in slot order are kept, ranked by a block-wide prefix
// count over thread-contiguous slot ranges.
//
// Besides the mask, the kernel can emit the sorted list of kept slots (the
// gather list of the compaction that follows).
#include "radix_select.h"

namespace kvc {
namespace {

using radix::kBins;
using radix::order_key;
using radix::radix_threshold;

// NT threads; REG: each thread holds KPT consecutive candidates in registers;
// else the keys are re-read, KMEM loads in flight per thread.
// The histogram has 8 copies (radix_select.h).
constexpr int kHistCopies = 8;
constexpr int KMEM = 32;
template <int NT, int KPT, bool REG>
__global__ __launch_bounds__(NT) void select_kernel(kvc_cache_t c, const float* __restrict__ score, int budget,
                                                    int n_sink, int n_recent, uint8_t* __restrict__ mask,
                                                    int32_t* __restrict__ keep_index, int max_len) {
  __shared__ __align__(16) int hist[kBins * kHistCopies];
  __shared__ int scan_tmp[16];
  __shared__ unsigned mm_tmp[32];
  __shared__ int sel[4];
  __shared__ unsigned small[64];
  // Register path: the staged keys. Memory path: one tile of the output pass.
  __shared__ __align__(16) unsigned stage_lds[NT * KPT];
  __shared__ int tile_tot[2];
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
  uint8_t* m = mask ? mask + rowoff : nullptr;  // NULL: keep list only
  int32_t* kidx = keep_index ? keep_index + ((long long)b * c.num_kv_heads + g) * budget : nullptr;
  if (L <= budget) {
    for (int i = tid; i < L; i += NT) {
      if (m) m[i] = 1;
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
  unsigned kmin = 0xFFFFFFFFu, kmax = 0u;
  if (REG) {
    // The candidates' key range (wave reductions now, the workgroup's after
    // the staging barrier) and the histogram's clear share that barrier.
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool cand = n_sink + tid + j * NT < hi;
      kmin = min(kmin, cand ? v[j] : 0xFFFFFFFFu);
      kmax = max(kmax, cand ? v[j] : 0u);
    }
    kmin = wave_minmax_u<false>(kmin);
    kmax = wave_minmax_u<true>(kmax);
    if ((tid & 63) == 0) {
      mm_tmp[tid >> 6] = kmin;
      mm_tmp[16 + (tid >> 6)] = kmax;
    }
    radix::radix_clear<NT, kHistCopies>(hist, sel);
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
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      kmin = min(kmin, mm_tmp[w]);
      kmax = max(kmax, mm_tmp[16 + w]);
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
      for (int base = lo + tid; base < hi; base += KMEM * NT) {
        unsigned kk[KMEM];
#pragma unroll
        for (int j = 0; j < KMEM; ++j) kk[j] = order_key(row[min(base + j * NT, hi - 1)]);
#pragma unroll
        for (int j = 0; j < KMEM; ++j)
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
      for (int q0 = 0; q0 < cnt; q0 += KMEM) {
        unsigned kk[KMEM];
#pragma unroll
        for (int j = 0; j < KMEM; ++j) kk[j] = order_key(row[i0 + min(q0 + j, cnt - 1)]);
#pragma unroll
        for (int j = 0; j < KMEM; ++j)
          if (q0 + j < cnt) f(i0 + q0 + j, kk[j]);
      }
    }
  };
  const bool any_heavy = k > 0;
  unsigned T = 0;
  if (any_heavy)
    T = REG ? radix::radix_threshold_range<NT, kHistCopies>(for_keys, k, kmin, kmax, hist, scan_tmp, sel, small)
            : radix_threshold<NT, kHistCopies>(for_keys, k, hist, scan_tmp, mm_tmp, sel, small);

  // Sinks and the recent window are always kept.
  const int n_heavy = budget - n_sink - n_recent;
  for (int i = tid; i < lo; i += NT) {
    if (m) m[i] = 1;
    if (kidx) kidx[i] = i;
  }
  for (int i = hi + tid; i < L; i += NT) {
    if (m) m[i] = 1;
    if (kidx) kidx[lo + n_heavy + (i - hi)] = i;
  }
  // Candidates: rank the threshold ties in slot order; with a gather list,
  // also count the candidates above T before this thread.
  auto decide = [&](int i, unsigned u, int& tie_rank, int& out) {
    uint8_t keepb = 0;
    if (any_heavy) {
      if (u > T) {
        keepb = 1;
      } else if (u == T) {
        keepb = tie_rank < k;
        ++tie_rank;
      }
    }
    if (m) m[i] = keepb;
    if (kidx && keepb) kidx[lo + out++] = i;
  };
  if (REG) {
    // Unused slots hold key 0, never equal to or above T; every count fits
    // 16 bits, so one packed scan gives both prefix counts.
    int ties = 0, above = 0;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      ties += any_heavy & (key[q] == T);
      above += any_heavy & (key[q] > T);
    }
    const int packed = ties | (above << 16);
    const int before = block_inclusive_scan<NT>(packed, scan_tmp) - packed;
    int tie_rank = before & 0xFFFF;
    // Kept before this thread = candidates above T before it + ties kept before it.
    int out = (before >> 16) + min(tie_rank, k);
    for_own([&](int i, unsigned u) { decide(i, u, tie_rank, out); });
  } else {
    // Memory path: the candidates in tiles of NT * KPT slots, in order. Each
    // tile is loaded coalesced into LDS, then every thread takes KPT
    // consecutive slots of it (so that slot order is tile, thread, key) and
    // the tile's prefix counts come from one packed block scan, on top of
    // the counts of the tiles before it. (Reading a thread's own range
    // straight from memory would touch 64 cache lines per load.)
    constexpr int TILE = NT * KPT;
    int run_ties = 0, run_above = 0;  // uniform: counts of the tiles before
    // The next tile's keys load while this one is processed.
    float nxt[KPT];
    auto load_tile = [&](int t0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) nxt[j] = row[lo + min(t0 + tid + j * NT, n - 1)];
    };
    load_tile(0);
    for (int t0 = 0; t0 < n; t0 += TILE) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) stage_lds[tid + j * NT] = t0 + tid + j * NT < n ? order_key(nxt[j]) : 0u;
      if (t0 + TILE < n) load_tile(t0 + TILE);
      __syncthreads();
      unsigned kk[KPT];
#pragma unroll
      for (int q = 0; q < KPT; q += 4) {
        const uint4 w = *reinterpret_cast<const uint4*>(stage_lds + tid * KPT + q);
        kk[q] = w.x;
        kk[q + 1] = w.y;
        kk[q + 2] = w.z;
        kk[q + 3] = w.w;
      }
      const int cnt_t = min(max(n - t0 - tid * KPT, 0), KPT);
      int ties = 0, above = 0;
#pragma unroll
      for (int q = 0; q < KPT; ++q) {
        ties += any_heavy & (q < cnt_t) & (kk[q] == T);
        above += any_heavy & (q < cnt_t) & (kk[q] > T);
      }
      const int packed = ties | (above << 16);  // a tile's counts fit 16 bits
      const int incl = block_inclusive_scan<NT>(packed, scan_tmp);
      if (tid == NT - 1) {
        tile_tot[0] = incl & 0xFFFF;
        tile_tot[1] = incl >> 16;
      }
      const int before = incl - packed;
      int tie_rank = run_ties + (before & 0xFFFF);
      int out = run_above + (before >> 16) + min(tie_rank, k);
#pragma unroll
      for (int q = 0; q < KPT; ++q)
        if (q < cnt_t) decide(lo + t0 + tid * KPT + q, kk[q], tie_rank, out);
      __syncthreads();  // the tile's totals are written; LDS is free for the next tile
      run_ties += tile_tot[0];
      run_above += tile_tot[1];
    }
  }
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
