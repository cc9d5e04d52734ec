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
//
// In a one-call decode step (kvc_decode_step) the same kernel also takes over
// the attention's merge: it reads the split kernel's per-split statistics and
// spilled logits, applies the H2O update to the scores it loads (the merge
// kernel's arithmetic, merge.h), selects on the updated scores, copies the
// kept tokens with them, and merges the attention output of the row's query
// heads. The step then takes two launches: the split kernel, this one.
#include "merge.h"
#include "radix_select.h"

namespace kvc {
namespace {

constexpr int kLog2NT = 10;
constexpr int kNT = 1 << kLog2NT;  // threads per workgroup
constexpr int kKPT = 8;            // candidate keys per thread (in registers)
constexpr int kHistCopies = 4;     // histogram copies (radix_select.h)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Row copies. An entry e of a row moves source slot slot_of(e) to destination
// slot dest_of(e): K and V codes (RBK and RBV bytes per row; RB/16 lanes per
// row, RB the wider of the two, 16-byte accesses, lanes past the narrower
// row's end idle for it), scales, position and score. A pass covers up to
// RPP = kNT * 16 / RB consecutive entries: lane group r0 = tid / (RB/16) holds
// the codes of entry e0 + r0, thread tid the other fields of entry e0 + tid.
// GK > 0: the score is updated with the step's H2O mass (GK logits per entry)
// when stored.
template <int RBK, int RBV, int GK>
struct Pass {
  static constexpr int RB = RBK > RBV ? RBK : RBV;
  static constexpr int LPR = RB / 16;
  static constexpr int RPP = kNT / LPR;
  u32x4 k, v;
  float ks, vs, sc;
  int pos;
  float lg[GK > 0 ? GK : 1];
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
  // H2O update of the copied scores (merging kernels): the row's logits
  // (head h of slot t at lg[h * span + t]), the heads' (m, 1/l) and the
  // number of slots the update covers.
  const float* lg;
  long long span;
  const float* mstat;
  int G, L_h2o;
};

template <int GK>
__device__ __forceinline__ float updated_score(const RowIO& io, float sc, const float* lg, int slot) {
  if (GK == 0 || slot >= io.L_h2o) return sc;
  float add = 0.f;
#pragma unroll
  for (int h = 0; h < (GK > 0 ? GK : 1); ++h)
    if (h < io.G) add = merge::h2o_add(add, lg[h], io.mstat[2 * h], io.mstat[2 * h + 1]);
  return sc + add;
}

template <int RBK, int RBV, int GK, typename SlotOf>
__device__ __forceinline__ void load_pass(Pass<RBK, RBV, GK>& P, const RowIO& io, int e0, int e1, SlotOf slot_of) {
  using PS = Pass<RBK, RBV, GK>;
  const int tid = threadIdx.x, part = tid % PS::LPR, r0 = tid / PS::LPR;
  if (e0 >= e1) return;  // uniform
  const long long s = slot_of(min(e0 + r0, e1 - 1));  // every lane loads; spare lanes repeat the last entry
  if (RBK == PS::RB || part * 16 < RBK) P.k = *reinterpret_cast<const u32x4*>(io.sk + s * RBK + part * 16);
  if (RBV == PS::RB || part * 16 < RBV) P.v = *reinterpret_cast<const u32x4*>(io.sv + s * RBV + part * 16);
  if (tid < e1 - e0) {
    const int se = slot_of(e0 + tid);
    P.ks = io.sks[se];
    P.vs = io.svs[se];
    if (io.spos) P.pos = io.spos[se];
    if (io.ssc) {
      P.sc = io.ssc[se];
      if (GK > 0) {
#pragma unroll
        for (int h = 0; h < (GK > 0 ? GK : 1); ++h)
          P.lg[h] = io.lg[min(h, io.G - 1) * io.span + min((long long)se, io.span - 1)];
      }
    }
  }
}

template <int RBK, int RBV, int GK, typename SlotOf, typename DestOf>
__device__ __forceinline__ void store_pass(const Pass<RBK, RBV, GK>& P, const RowIO& io, int e0, int e1,
                                           SlotOf slot_of, DestOf dest_of) {
  using PS = Pass<RBK, RBV, GK>;
  const int tid = threadIdx.x, part = tid % PS::LPR, r0 = tid / PS::LPR;
  if (e0 >= e1) return;
  if (e0 + r0 < e1) {
    const long long d = dest_of(e0 + r0);
    // Streaming stores: the compacted rows are not read again here.
    if (RBK == PS::RB || part * 16 < RBK)
      __builtin_nontemporal_store(P.k, reinterpret_cast<u32x4*>(io.dk + d * RBK + part * 16));
    if (RBV == PS::RB || part * 16 < RBV)
      __builtin_nontemporal_store(P.v, reinterpret_cast<u32x4*>(io.dv + d * RBV + part * 16));
  }
  if (tid < e1 - e0) {
    const long long de = dest_of(e0 + tid);
    io.dks[de] = P.ks;
    io.dvs[de] = P.vs;
    if (io.spos) io.dpos[de] = P.pos;
    if (io.ssc) io.dsc[de] = updated_score<GK>(io, P.sc, P.lg, slot_of(e0 + tid));
  }
}

// Entries [e0, e1), BATCH passes in flight at a time.
template <int RBK, int RBV, int GK, int BATCH, typename SlotOf, typename DestOf>
__device__ __forceinline__ void copy_entries(const RowIO& io, int e0, int e1, SlotOf slot_of, DestOf dest_of) {
  constexpr int RPP = Pass<RBK, RBV, GK>::RPP;
  for (int e = e0; e < e1; e += RPP * BATCH) {
    Pass<RBK, RBV, GK> ps[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q)
      load_pass<RBK, RBV, GK>(ps[q], io, e + q * RPP, min(e1, e + (q + 1) * RPP), slot_of);
#pragma unroll
    for (int q = 0; q < BATCH; ++q)
      store_pass<RBK, RBV, GK>(ps[q], io, e + q * RPP, min(e1, e + (q + 1) * RPP), slot_of, dest_of);
  }
}

}  // namespace

// One-dimensional grid of rows << log2_parts workgroups (2^log2_parts per
// (sequence, KV head) row, at most kNT). Workgroups go to the 8 XCDs round
// robin by index; when the row count is a multiple of 8 (xcd_rows), the
// workgroups of a row get indices that are equal mod 8, so they share one
// XCD and its L2 serves the row's scores (and logits) to all of them after
// the first. GK > 0: merge the attention splits first (num_q_heads /
// num_kv_heads <= GK query heads per KV head).
//
// gfx9 counts stores in the same counter as loads, so a wait for a load also
// waits for every store issued before it: stores come after the loads whose
// data the workgroup waits for.
template <int RBK, int RBV, int GK>
__global__ __launch_bounds__(kNT) void evict_kernel(EvictArgs e) {
  constexpr int NT = kNT, KPT = kKPT;
  constexpr bool MERGE = GK > 0;
  constexpr int GL = MERGE ? GK : 1;
  __shared__ __align__(16) int hist[radix::kBins * kHistCopies];
  __shared__ int scan_tmp[16];
  __shared__ unsigned mm_tmp[32];
  __shared__ int sel[4];
  __shared__ unsigned small[64];
  // Staged keys; after the threshold search, the kept candidates in order.
  __shared__ __align__(16) unsigned stage_lds[NT * KPT];
  // Merging: the heads' (m, 1/l), their split weights, the output partials.
  __shared__ float mstat[2 * GL];
  __shared__ float facl[MERGE ? GL * kEvictMaxSplits : 1];
  __shared__ float opart[MERGE ? 256 : 1];
  const kvc_cache_t& c = e.c;
  const int budget = e.budget, n_sink = e.n_sink, n_recent = e.n_recent, log2_parts = e.log2_parts;
  const int parts = 1 << log2_parts;
  const unsigned wg = blockIdx.x;
  const unsigned rowi = e.xcd_rows ? (wg & 7u) + 8u * (wg >> (3 + log2_parts)) : wg >> log2_parts;
  const int p = e.xcd_rows ? (int)((wg >> 3) & (unsigned)(parts - 1)) : (int)(wg & (unsigned)(parts - 1));
  const int g = (int)(rowi % (unsigned)c.num_kv_heads), b = (int)(rowi / (unsigned)c.num_kv_heads);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const long long bg = (long long)b * c.num_kv_heads + g;
  const long long rowoff = bg * c.capacity;
  const float* row = e.score + rowoff;
  const int Hq = MERGE ? e.num_q_heads : 0, G = MERGE ? Hq / c.num_kv_heads : 0, S = e.splits;
  const float* lrow = MERGE ? e.logits + ((long long)b * Hq + g * G) * e.span : nullptr;
  // Merging: wave h < G holds head h's split states (loaded first, so the
  // statistics wait for nothing else).
  const float* mlh = MERGE ? e.part_ml + ((long long)b * Hq + g * G + min(wave, G - 1)) * S * 2 : nullptr;
  merge::SplitML mlr;
  if (MERGE && wave < G) mlr = merge::load_split_ml(mlh, S);
  // Merging, output of the row's first query head merged here (h = p): the
  // split partials of thread (pi, d) = (tid / D, tid % D), tid < 256, load
  // before the scores; the sum is taken once the statistics are known.
  constexpr int kPre = 8;
  const int D = c.head_dim, PARTS = 256 / D;
  const bool merges = MERGE && p < G;
  float opre[MERGE ? kPre : 1];
  const float* po = MERGE ? e.part_o + ((long long)b * Hq + g * G + p) * S * D + tid % D : nullptr;
  if (merges && tid < 256) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) opre[k] = po[(long long)min(tid / D + k * PARTS, S - 1) * D];
  }
  // Coalesced loads of slots n_sink .. n_sink + NT*KPT - 1 (clamped to the
  // row), issued before the sequence length is known: scores, and when
  // merging the heads' logits of the same slots.
  float sv[KPT];
  float lgv[KPT][GL];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int slot = min(n_sink + tid + j * NT, c.capacity - 1);
    sv[j] = row[slot];
    if (MERGE) {
#pragma unroll
      for (int h = 0; h < GL; ++h) lgv[j][h] = lrow[min(h, G - 1) * e.span + min((long long)slot, e.span - 1)];
    }
  }
  // Merging: the lengths before this step's append come from the split
  // kernel (this kernel advances the cache's own); the H2O update covers the
  // slots the merge kernel would update.
  const int L_src = MERGE ? e.stash[b] + 1 : c.lengths[b];
  const int L = __builtin_amdgcn_readfirstlane(min(min(L_src, c.capacity), e.max_len));
  const int L_h2o = MERGE ? __builtin_amdgcn_readfirstlane(min(min(L_src, c.capacity), (int)min(e.span, (long long)c.capacity))) : 0;
  if (MERGE) {
    // Statistics: wave h takes head h (G <= GK <= 16 waves).
    if (wave < G) {
      float m, inv;
      merge::split_stats(mlr, mlh, S, facl + wave * S, m, inv);
      if ((tid & 63) == 0) {
        mstat[2 * wave] = m;
        mstat[2 * wave + 1] = inv;
      }
    }
    __syncthreads();
  }
  // The new lengths, written last (after every load this workgroup waits for).
  auto set_length = [&]() {
    if (p == 0 && g == 0 && tid == 0) {
      const int seen = MERGE ? e.stash[c.batch + b] + 1 : c.num_seen[b];
      if (MERGE) {
        c.lengths[b] = L_src;
        c.num_seen[b] = seen;
      }
      e.dst.lengths[b] = min(L, budget);
      e.dst.num_seen[b] = seen;
    }
  };
  // Merging: the attention output of the row's query heads h = p, p + parts,
  // ... in the merge kernel's order (PARTS threads per channel over every
  // PARTS-th split, then the PARTS sums). Head p: the partial sums right after
  // the statistics (merge_first), the total after a later barrier
  // (merge_first_out); further heads at the end (merge_rest).
  auto merge_first = [&]() {
    if (merges && tid < 256) {
      const int pi = tid / D;
      float o = 0.f;
#pragma unroll
      for (int k = 0; k < kPre; ++k)
        if (pi + k * PARTS < S) o = fmaf(opre[k], facl[p * S + pi + k * PARTS], o);
      for (int sp = pi + kPre * PARTS; sp < S; sp += PARTS) o = fmaf(po[(long long)sp * D], facl[p * S + sp], o);
      opart[tid] = o;  // = opart[pi * D + d]
    }
  };
  auto merge_first_out = [&]() {
    if (merges && tid < D) {
      float r = opart[tid];
      for (int q = 1; q < PARTS; ++q) r += opart[q * D + tid];
      e.out[((long long)b * Hq + g * G + p) * D + tid] = r;
    }
  };
  auto merge_rest = [&]() {
    if (!MERGE) return;
    for (int h = p + parts; h < G; h += parts) {
      // Every earlier reader of opart (merge_first_out, the previous head's
      // sum) is done before it is overwritten.
      __syncthreads();
      if (tid < 256) {
        const int d = tid % D, pi = tid / D;
        const float* po = e.part_o + ((long long)b * Hq + g * G + h) * S * D + d;
        float o = 0.f;
        for (int sp = pi; sp < S; sp += PARTS) o = fmaf(po[(long long)sp * D], facl[h * S + sp], o);
        opart[pi * D + d] = o;
      }
      __syncthreads();
      if (tid < D) {
        float r = opart[tid];
        for (int q = 1; q < PARTS; ++q) r += opart[q * D + tid];
        e.out[((long long)b * Hq + g * G + h) * D + tid] = r;
      }
    }
  };
  merge_first();
  uint8_t* m = e.mask ? e.mask + rowoff : nullptr;
  int32_t* kidx = e.keep_index ? e.keep_index + bg * budget : nullptr;
  const RowIO io{static_cast<const uint8_t*>(c.k_codes) + rowoff * RBK,
                 static_cast<const uint8_t*>(c.v_codes) + rowoff * RBV,
                 static_cast<uint8_t*>(e.dst.k_codes) + rowoff * RBK,
                 static_cast<uint8_t*>(e.dst.v_codes) + rowoff * RBV,
                 c.k_scale + rowoff, c.v_scale + rowoff, e.dst.k_scale + rowoff, e.dst.v_scale + rowoff,
                 (c.positions && e.dst.positions) ? c.positions + rowoff : nullptr,
                 (c.positions && e.dst.positions) ? e.dst.positions + rowoff : nullptr,
                 e.dst_score ? row : nullptr, e.dst_score ? e.dst_score + rowoff : nullptr,
                 lrow, e.span, mstat, G, L_h2o};
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
  constexpr int RPP = Pass<RBK, RBV, GK>::RPP;
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
  Pass<RBK, RBV, GK> pre;
  if (all) {
    load_pass<RBK, RBV, GK>(pre, io, f0, fa, fixed_slot);
    fixed_entries();
    store_pass<RBK, RBV, GK>(pre, io, f0, fa, fixed_slot, fixed_dest);
    copy_entries<RBK, RBV, GK, 2>(io, fa, f1, fixed_slot, fixed_dest);
    __syncthreads();
    merge_first_out();
    merge_rest();
    set_length();
    return;
  }
  // Keys of the coalesced slots: the scores, with this step's H2O mass when
  // merging (slots below L_h2o, as the merge kernel updates them).
  unsigned v[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    float s = sv[j];
    if (MERGE && n_sink + tid + j * NT < L_h2o) {
      float add = 0.f;
#pragma unroll
      for (int h = 0; h < GL; ++h)
        if (h < G) add = merge::h2o_add(add, lgv[j][h], mstat[2 * h], mstat[2 * h + 1]);
      s = s + add;
    }
    v[j] = radix::order_key(s);
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
  radix::radix_clear<NT, kHistCopies>(hist, sel);
  unsigned key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) stage_lds[tid + j * NT] = v[j];
  // The first pass of fixed rows loads during the search (barriers here wait
  // for LDS only), and is stored after it.
  load_pass<RBK, RBV, GK>(pre, io, f0, fa, fixed_slot);
  __syncthreads();
  merge_first_out();
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
  if (any_heavy) T = radix::radix_threshold_range<NT, kHistCopies>(for_keys, k, kmin, kmax, hist, scan_tmp, sel, small);

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
  Pass<RBK, RBV, GK> hp[HB];
#pragma unroll
  for (int q = 0; q < HB; ++q) load_pass<RBK, RBV, GK>(hp[q], io, q * RPP, min(total, (q + 1) * RPP), rest_slot);
  store_pass<RBK, RBV, GK>(pre, io, f0, fa, fixed_slot, fixed_dest);
  if (kidx)
    for (int h = h0 + tid; h < h1; h += NT) kidx[lo + h] = heavy[h];
#pragma unroll
  for (int q = 0; q < HB; ++q)
    store_pass<RBK, RBV, GK>(hp[q], io, q * RPP, min(total, (q + 1) * RPP), rest_slot, rest_dest);
  copy_entries<RBK, RBV, GK, 2>(io, HB * RPP, total, rest_slot, rest_dest);
  merge_rest();
  set_length();
}

namespace {

template <int RBK, int RBV, int GK>
hipError_t launch_rb(const EvictArgs& a, hipStream_t st) {
  // About one workgroup per CU over the rows, at most 8 per row.
  const long long rows = (long long)a.c.batch * a.c.num_kv_heads;
  const long long target = device_cus();
  int lp = 0;
  while (lp < 3 && rows << (lp + 1) <= target) ++lp;
  EvictArgs e = a;
  e.log2_parts = lp;
  e.xcd_rows = rows % 8 == 0;
  const long long wgs = rows << lp;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((evict_kernel<RBK, RBV, GK>), dim3((unsigned)wgs), dim3(kNT), 0, st, e);
  return hipGetLastError();
}

template <int GK>
hipError_t launch_gk(const EvictArgs& a, hipStream_t st) {
  return with_row_bytes(a.c, [&](auto rbk, auto rbv) { return launch_rb<decltype(rbk)::value, decltype(rbv)::value, GK>(a, st); });
}

}  // namespace

bool evict_fits_one_launch(int max_len, int n_sink, int n_recent) {
  return (long long)max_len - n_sink - n_recent <= (long long)kNT * kKPT;
}

bool evict_can_merge(int num_q_heads, int num_kv_heads, int splits) {
  const int G = num_q_heads / num_kv_heads;
  return G <= kEvictMaxMergeHeads && (long long)splits <= kEvictMaxSplits;
}

hipError_t launch_evict(const EvictArgs& a, hipStream_t st) {
  if (!a.part_ml) return launch_gk<0>(a, st);
  const int G = a.num_q_heads / a.c.num_kv_heads;
  if (G <= 1) return launch_gk<1>(a, st);
  if (G <= 2) return launch_gk<2>(a, st);
  return launch_gk<4>(a, st);
}

}  // namespace kvc
