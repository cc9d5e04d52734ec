// Selection and compaction in one launch (rows of up to 8192 candidates).
//
// The keep set is the one kvc_h2o_select chooses: the first n_sink tokens
// (attention sinks, "KV Cache Compression Report", section 3.3), the n_recent
// most recent ones and, from the rest, the tokens with the largest accumulated
// attention (report, section 3.4; "KV Cache optimization techniques" tutorial,
// section 2.2), equal scores going to the lower slot. The kept slots move to
// the destination cache in ascending order, with their scales, positions and
// scores, as kvc_compact_gather moves them (tutorial, section 2.2).
//
// A row's selection is latency-bound work for one workgroup; its compaction
// is bandwidth work that wants many CUs. So P workgroups take each
// (sequence, KV head) row. Each loads the row's scores (an L2 hit right after
// the attention launch that updated them), finds the same threshold and tie
// ranks (the selection is deterministic, so the P copies agree exactly), then
// writes its share: 1/P of the sinks and window entries and 1/P of the heavy
// hitters (keep-list entries, mask bytes and rows). The sinks and the window
// are known from the length alone, so the first pass of each workgroup's share
// of their rows loads while the threshold search runs; the heavy hitters
// follow it. One launch instead of two: no drain between selection
// and compaction, and the kept-slot list never travels through memory on its
// way to the copy.
#include "radix_select.h"

namespace kvc {
namespace {

constexpr int kLog2NT = 10;
constexpr int kNT = 1 << kLog2NT;  // threads per workgroup
constexpr int kKPT = 8;    // candidate keys per thread (in registers)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Row copies. An entry e of a row moves source slot slot_of(e) to destination
// slot dest_of(e): K and V codes (RB/16 lanes per row, 16-byte accesses),
// scales, position and score. A pass covers up to RPP = kNT * 16 / RB
// consecutive entries: lane group r0 = tid / (RB/16) holds the codes of entry
// e0 + r0, thread tid the other fields of entry e0 + tid.
template <int RB>
struct Pass {
  static constexpr int LPR = RB / 16;
  static constexpr int RPP = kNT / LPR;
  u32x4 k, v;
  float ks, vs, sc;
  int pos;
};

struct RowIO {
  const uint8_t* sk;
  const uint8_t* sv;
  uint8_t* dk;
  uint8_t* dv;
  const float* sks;
  const float* svs;
  float* dks;
  float* dvs;
  const int* spos;  // NULL unless both caches keep positions
  int* dpos;
  const float* ssc;  // NULL unless dst scores are written
  float* dsc;
};

template <int RB, typename SlotOf>
__device__ __forceinline__ void load_pass(Pass<RB>& P, const RowIO& io, int e0, int e1, SlotOf slot_of) {
  const int tid = threadIdx.x, part = tid % Pass<RB>::LPR, r0 = tid / Pass<RB>::LPR;
  if (e0 >= e1) return;  // uniform
  const long long s = slot_of(min(e0 + r0, e1 - 1));  // every lane loads; spare lanes repeat the last entry
  P.k = *reinterpret_cast<const u32x4*>(io.sk + s * RB + part * 16);
  P.v = *reinterpret_cast<const u32x4*>(io.sv + s * RB + part * 16);
  if (tid < e1 - e0) {
    const long long se = slot_of(e0 + tid);
    P.ks = io.sks[se];
    P.vs = io.svs[se];
    if (io.spos) P.pos = io.spos[se];
    if (io.ssc) P.sc = io.ssc[se];
  }
}

template <int RB, typename DestOf>
__device__ __forceinline__ void store_pass(const Pass<RB>& P, const RowIO& io, int e0, int e1, DestOf dest_of) {
  const int tid = threadIdx.x, part = tid % Pass<RB>::LPR, r0 = tid / Pass<RB>::LPR;
  if (e0 >= e1) return;
  if (e0 + r0 < e1) {
    const long long d = dest_of(e0 + r0);
    // Streaming stores: the compacted rows are not read again here.
    __builtin_nontemporal_store(P.k, reinterpret_cast<u32x4*>(io.dk + d * RB + part * 16));
    __builtin_nontemporal_store(P.v, reinterpret_cast<u32x4*>(io.dv + d * RB + part * 16));
  }
  if (tid < e1 - e0) {
    const long long de = dest_of(e0 + tid);
    io.dks[de] = P.ks;
    io.dvs[de] = P.vs;
    if (io.spos) io.dpos[de] = P.pos;
    if (io.ssc) io.dsc[de] = P.sc;
  }
}

// Entries [e0, e1), BATCH passes in flight at a time.
template <int RB, int BATCH, typename SlotOf, typename DestOf>
__device__ __forceinline__ void copy_entries(const RowIO& io, int e0, int e1, SlotOf slot_of, DestOf dest_of) {
  constexpr int RPP = Pass<RB>::RPP;
  for (int e = e0; e < e1; e += RPP * BATCH) {
    Pass<RB> ps[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) load_pass<RB>(ps[q], io, e + q * RPP, min(e1, e + (q + 1) * RPP), slot_of);
#pragma unroll
    for (int q = 0; q < BATCH; ++q) store_pass<RB>(ps[q], io, e + q * RPP, min(e1, e + (q + 1) * RPP), dest_of);
  }
}

// Grid (num_kv_heads << log2_parts, batch); 2^log2_parts workgroups per row,
// at most kNT.
//
// gfx9 counts stores in the same counter as loads, so a wait for a load also
// waits for every store issued before it: stores come after the loads whose
// data the workgroup waits for.
template <int RB>
__global__ __launch_bounds__(kNT) void evict_kernel(kvc_cache_t c, const float* __restrict__ score, int budget,
                                                    int n_sink, int n_recent, uint8_t* __restrict__ mask,
                                                    int32_t* __restrict__ keep_index, kvc_cache_t dst,
                                                    float* __restrict__ dst_score, int max_len, int log2_parts) {
  constexpr int NT = kNT, KPT = kKPT;
  __shared__ int hist[radix::kBins];
  __shared__ int scan_tmp[16];
  __shared__ unsigned mm_tmp[32];
  __shared__ int sel[4];
  __shared__ unsigned small[64];
  // Staged keys; after the threshold search, the kept candidates in order.
  __shared__ __align__(16) unsigned stage_lds[NT * KPT];
  const int parts = 1 << log2_parts;
  const int p = blockIdx.x & (parts - 1), g = blockIdx.x >> log2_parts, b = blockIdx.y, tid = threadIdx.x;
  const long long bg = (long long)b * c.num_kv_heads + g;
  const long long rowoff = bg * c.capacity;
  const float* row = score + rowoff;
  // Coalesced loads of slots n_sink .. n_sink + NT*KPT - 1 (clamped to the
  // row), issued before the sequence length is known.
  unsigned v[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) v[j] = radix::order_key(row[min(n_sink + tid + j * NT, c.capacity - 1)]);
  const int L = __builtin_amdgcn_readfirstlane(min(min(c.lengths[b], c.capacity), max_len));
  // The new length, written last (after every load this workgroup waits for).
  auto set_length = [&]() {
    if (p == 0 && g == 0 && tid == 0) {
      dst.lengths[b] = min(L, budget);
      dst.num_seen[b] = c.num_seen[b];
    }
  };
  uint8_t* m = mask ? mask + rowoff : nullptr;
  int32_t* kidx = keep_index ? keep_index + bg * budget : nullptr;
  const RowIO io{static_cast<const uint8_t*>(c.k_codes) + rowoff * RB,
                 static_cast<const uint8_t*>(c.v_codes) + rowoff * RB,
                 static_cast<uint8_t*>(dst.k_codes) + rowoff * RB,
                 static_cast<uint8_t*>(dst.v_codes) + rowoff * RB,
                 c.k_scale + rowoff, c.v_scale + rowoff, dst.k_scale + rowoff, dst.v_scale + rowoff,
                 (c.positions && dst.positions) ? c.positions + rowoff : nullptr,
                 (c.positions && dst.positions) ? dst.positions + rowoff : nullptr,
                 dst_score ? row : nullptr, dst_score ? dst_score + rowoff : nullptr};
  // Kept entries: "fixed" ones (sinks and the recent window; every slot when
  // L <= budget), known from L alone, and heavy hitters, known after the
  // threshold search. Each kind is split evenly over the row's workgroups:
  // this one takes fixed entries [f0, f1) and heavy ranks [h0, h1), writes
  // their keep-list entries (and mask bytes), and copies their rows.
  const bool all = L <= budget;
  const int lo = n_sink, hi = L - n_recent;
  const int n_heavy = all ? 0 : budget - n_sink - n_recent;
  const int n_self = all ? L : n_sink;  // fixed entries that stay in place
  const int n_fixed = all ? L : n_sink + n_recent;
  auto fixed_slot = [&](int f) { return f < n_self ? f : hi + (f - n_self); };
  auto fixed_dest = [&](int f) { return f < n_self ? f : lo + n_heavy + (f - n_self); };
  constexpr int RPP = Pass<RB>::RPP;
  const int f0 = (int)(((long long)n_fixed * p) >> log2_parts);
  const int f1 = (int)(((long long)n_fixed * (p + 1)) >> log2_parts);
  const int fa = min(f1, f0 + RPP);  // the first pass of fixed entries
  const int h0 = (int)(((long long)n_heavy * p) >> log2_parts);
  const int h1 = (int)(((long long)n_heavy * (p + 1)) >> log2_parts);
  auto fixed_entries = [&]() {
    for (int f = f0 + tid; f < f1; f += NT) {
      if (m) m[fixed_slot(f)] = 1;
      if (kidx) kidx[fixed_dest(f)] = fixed_slot(f);
    }
  };
  Pass<RB> pre;
  if (all) {
    load_pass<RB>(pre, io, f0, fa, fixed_slot);
    fixed_entries();
    store_pass<RB>(pre, io, f0, fa, fixed_dest);
    copy_entries<RB, 2>(io, fa, f1, fixed_slot, fixed_dest);
    set_length();
    return;
  }
  const int n = hi - lo;
  int k = n_heavy;
  // Thread t holds candidates [lo + t*per, lo + t*per + per) (per <= KPT, a
  // multiple of 4): staged through LDS, read back with 16-byte reads.
  const int per = ((n + NT - 1) / NT + 3) & ~3;
  const int i0 = lo + min(tid * per, n), cnt = min(tid * per + per, n) - min(tid * per, n);
  // The candidates' key range (wave reductions now, the workgroup's after the
  // staging barrier) and the histogram's clear share that one barrier.
  unsigned kmin = 0xFFFFFFFFu, kmax = 0u;
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
  radix::radix_clear<NT>(hist, sel);
  unsigned key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) stage_lds[tid + j * NT] = v[j];
  // The first pass of fixed rows loads during the search (barriers here wait
  // for LDS only), and is stored after it.
  load_pass<RB>(pre, io, f0, fa, fixed_slot);
  __syncthreads();
  fixed_entries();  // stores: after the wait for the scores
#pragma unroll
  for (int q = 0; q < KPT; q += 4) {
    const uint4 w = *reinterpret_cast<const uint4*>(stage_lds + min(tid * per + q, NT * KPT - 4));
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
  // Unused slots hold key 0, below every real key (scores are non-negative).
#pragma unroll
  for (int q = 0; q < KPT; ++q) key[q] = q < cnt ? key[q] : 0u;
  auto for_keys = [&](auto f) {
#pragma unroll
    for (int q = 0; q < KPT; ++q) f(key[q]);
  };
  const bool any_heavy = k > 0;
  unsigned T = 0;
  if (any_heavy) T = radix::radix_threshold_range<NT>(for_keys, k, kmin, kmax, hist, scan_tmp, sel, small);

  // Threshold ties ranked in slot order; candidates above T before this
  // thread (both counts fit 16 bits: n <= NT * KPT).
  int ties = 0, above = 0;
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    ties += any_heavy & (key[q] == T);
    above += any_heavy & (key[q] > T);
  }
  const int packed = ties | (above << 16);
  const int before = block_inclusive_scan<NT>(packed, scan_tmp) - packed;
  int tie_rank = before & 0xFFFF;
  int out = (before >> 16) + min(tie_rank, k);  // kept candidates before this thread
  // Kept candidates into LDS in rank order (the heavy list); mask bytes of
  // the threads [p*NT/parts, (p+1)*NT/parts).
  int* heavy = reinterpret_cast<int*>(stage_lds);
  const bool my_threads = m && (tid >> (kLog2NT - log2_parts)) == p;
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    if (q < cnt) {
      const unsigned u = key[q];
      int keepb = 0;
      if (any_heavy) {
        if (u > T) {
          keepb = 1;
        } else if (u == T) {
          keepb = tie_rank < k;
          ++tie_rank;
        }
      }
      if (my_threads) m[i0 + q] = (uint8_t)keepb;
      if (keepb) heavy[min(out++, NT * KPT - 1)] = i0 + q;
    }
  }
  __syncthreads();
  // The rest of this workgroup's share, as one list: its fixed entries past
  // the first pass, then its heavy hitters h (slot heavy[h] to slot lo + h).
  const int nfr = f1 - fa, total = nfr + (h1 - h0);
  auto rest_slot = [&](int e) { return e < nfr ? fixed_slot(fa + e) : heavy[h0 + e - nfr]; };
  auto rest_dest = [&](int e) { return e < nfr ? fixed_dest(fa + e) : lo + h0 + (e - nfr); };
  constexpr int HB = 2;
  Pass<RB> hp[HB];
#pragma unroll
  for (int q = 0; q < HB; ++q) load_pass<RB>(hp[q], io, q * RPP, min(total, (q + 1) * RPP), rest_slot);
  store_pass<RB>(pre, io, f0, fa, fixed_dest);
  if (kidx)
    for (int h = h0 + tid; h < h1; h += NT) kidx[lo + h] = heavy[h];
#pragma unroll
  for (int q = 0; q < HB; ++q) store_pass<RB>(hp[q], io, q * RPP, min(total, (q + 1) * RPP), rest_dest);
  copy_entries<RB, 2>(io, HB * RPP, total, rest_slot, rest_dest);
  set_length();
}

template <int RB>
hipError_t launch_rb(const kvc_cache_t& c, const float* score, int budget, int n_sink, int n_recent, uint8_t* mask,
                     int32_t* keep_index, const kvc_cache_t& dst, float* dst_score, int max_len, hipStream_t st) {
  // About 256 workgroups over the rows, at most 8 per row.
  const long long rows = (long long)c.batch * c.num_kv_heads;
  int lp = 0;
  while (lp < 3 && rows << (lp + 1) <= 256) ++lp;
  hipLaunchKernelGGL((evict_kernel<RB>), dim3(c.num_kv_heads << lp, c.batch), dim3(kNT), 0, st, c, score, budget,
                     n_sink, n_recent, mask, keep_index, dst, dst_score, max_len, lp);
  return hipGetLastError();
}

}  // namespace

bool evict_fits_one_launch(int max_len, int n_sink, int n_recent) {
  return (long long)max_len - n_sink - n_recent <= (long long)kNT * kKPT;
}

hipError_t launch_evict(const kvc_cache_t& c, const float* score, int budget, int n_sink, int n_recent,
                        uint8_t* mask, int32_t* keep_index, const kvc_cache_t& dst, float* dst_score, int max_len,
                        hipStream_t st) {
  switch (c.head_dim * c.bits / 8) {
    case 32: return launch_rb<32>(c, score, budget, n_sink, n_recent, mask, keep_index, dst, dst_score, max_len, st);
    case 64: return launch_rb<64>(c, score, budget, n_sink, n_recent, mask, keep_index, dst, dst_score, max_len, st);
    case 128:
      return launch_rb<128>(c, score, budget, n_sink, n_recent, mask, keep_index, dst, dst_score, max_len, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvc
