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
static_assert(kNT == kEvictThreads, "eviction workgroup size");
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
  if (MERGE) mlr = merge::load_split_ml(mlh, S);  // every wave (clamped head): no branch to wait in
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
    if (MERGE) {
      // Computed for every slot (clamped loads, so the logits are some
      // row's), kept only below L_h2o: a select, not a branch per key.
      float add = 0.f;
#pragma unroll
      for (int h = 0; h < GL; ++h)
        if (h < G) add = merge::h2o_add(add, lgv[j][h], mstat[2 * h], mstat[2 * h + 1]);
      s = n_sink + tid + j * NT < L_h2o ? s + add : s;
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
  // The decisions take no branch per key (keys past cnt are 0, below T);
  // the mask bytes go out four to a store where the slots are 4-byte aligned.
  int* heavy = reinterpret_cast<int*>(stage_lds);
  const bool my_threads = m && (tid >> (kLog2NT - log2_parts)) == p;
  unsigned keep_bytes[KPT / 4];
#pragma unroll
  for (int w = 0; w < KPT / 4; ++w) keep_bytes[w] = 0u;
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const unsigned u = key[q];
    const bool tie = any_heavy && u == T;
    const bool keepb = (any_heavy && u > T) || (tie && tie_rank < k);
    tie_rank += tie;
    keep_bytes[q / 4] |= (unsigned)keepb << (8 * (q % 4));
    if (keepb) heavy[min(out, NT * KPT - 1)] = i0 + q;
    out += keepb;
  }
  if (my_threads) {
#pragma unroll
    for (int w = 0; w < KPT / 4; ++w) {
      if (4 * w + 4 <= cnt && ((uintptr_t)(m + i0 + 4 * w) & 3u) == 0u) {
        *reinterpret_cast<unsigned*>(m + i0 + 4 * w) = keep_bytes[w];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * w + e < cnt) m[i0 + 4 * w + e] = (uint8_t)(keep_bytes[w] >> (8 * e));
      }
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

// ---- In-place eviction ----
//
// A decode step may name the source cache as its destination. The kept
// tokens keep their order and move down to their rank, so only those past the
// first evicted slot move: with one token evicted per step the rows before it
// stay where they are. Each (sequence, KV head) row gets one selecting
// workgroup and ip_chunks moving ones; mover j moves the kept entries of the
// C destination slots starting C * j past the row's first moved slot.
//
// A slot may be overwritten only after every workgroup that reads it has read
// it, so the workgroups order themselves through flags in the workspace
// (agent-scope release and acquire):
//  * roles follow a ticket taken at start from a counter, so a workgroup only
//    waits for workgroups that started before it, which never wait for it;
//  * the selector reads the row's scores, chooses, writes the keep list, the
//    mask, the first moved slot and (when it merges the attention) the
//    updated scores, then sets its flag; the movers of the row wait for it;
//  * a mover loads its chunk's source rows, sets its flag, waits for the
//    flags of the row's lower chunks, then stores. An entry's source slot is
//    never below its destination, so every reader of a slot in this chunk's
//    destination range is this chunk or a lower one.
// Every wait is bounded (about half a second of polling): no wave waits
// forever, whatever the memory holds.
constexpr long long kIpSpin = 1LL << 23;  // polls of one wait before it gives up
constexpr int kIpFewEvicted = 4;  // at most this many evicted: selection by repeated minimum
// Buffer resource word 3 for gfx9-family raw buffers (32-bit dword format).
constexpr int kEvictBufferFlags = 0x00020000;

// Wave 0 polls flags f[0 .. n) until each is non-zero (or the bound is hit);
// with `acquire` it then invalidates this CU's and XCD's cached copies (one
// agent-scope acquire), so the workgroup reads what the flags' writers
// published. Waits that only order this workgroup's stores after other
// workgroups' loads need no acquire.
__device__ __forceinline__ void ip_wait(const int32_t* f, int n, bool acquire) {
  if (threadIdx.x < 64) {
    for (int i = threadIdx.x; i < n; i += 64) {
      for (long long k = 0; k < kIpSpin; ++k) {
        if (__hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (acquire) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Every wave's earlier loads have returned (their data is in registers) and
// its stores have reached the L2; with `release`, the L2 is also written back
// (one agent-scope release) so that other XCDs see those stores. Then flag f
// is set.
__device__ __forceinline__ void ip_post(int32_t* f, bool release) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    if (release) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(f, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroup minimum of 64-bit values (every thread gets it); tmp: NT / 64
// words of LDS, reusable after return.
template <int NT>
__device__ __forceinline__ unsigned long long block_min_u64(unsigned long long x, unsigned long long* tmp) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned long long y = __shfl_xor(x, o);
    x = y < x ? y : x;
  }
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = x;
  __syncthreads();
  x = tmp[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) x = tmp[w] < x ? tmp[w] : x;
  __syncthreads();
  return x;
}

// In-place destination of slot x when the E <= EMAX evicted slots ev[] (LDS,
// ascending) are the only ones removed: x moves down by the number of
// evicted slots below it; -1 if x stays where it is or is evicted (a
// fixed-step binary search).
template <int EMAX>
__device__ __forceinline__ int ip_dest_n(const int* ev, int E, int x) {
  int below = 0;
#pragma unroll
  for (int step = EMAX; step >= 1; step >>= 1)
    if (below + step <= E && ev[below + step - 1] < x) below += step;
  if (below == 0 || (below < E && ev[below] == x)) return -1;
  return x - below;
}
__device__ __forceinline__ int ip_dest(const int* ev, int E, int x) { return ip_dest_n<kInplaceMaxEvicted>(ev, E, x); }

template <int NT>
__device__ __forceinline__ int block_min_int(int x, unsigned* tmp) {
  unsigned lo = (unsigned)x, hi = 0u;
  radix::block_minmax<NT>(lo, hi, tmp);
  return (int)lo;
}

template <int RBK, int RBV, int GK>
__global__ __launch_bounds__(kNT) void evict_inplace_kernel(EvictArgs e) {
  constexpr int NT = kNT, KPT = kKPT;
  constexpr bool MERGE = GK > 0;
  constexpr int GL = MERGE ? GK : 1;
  constexpr int RB = RBK > RBV ? RBK : RBV, LPR = RB / 16, RPP = NT / LPR;
  constexpr int MAXP = kInplaceMaxPasses(RB);
  constexpr int FPT = (MAXP * RPP + NT - 1) / NT;  // entries per thread for scales, position and score
  constexpr int EMAX = kInplaceMaxEvicted;
  __shared__ __align__(16) int hist[radix::kBins * kHistCopies];
  __shared__ int scan_tmp[16];
  __shared__ unsigned mm_tmp[32];
  __shared__ int sel[4];
  __shared__ unsigned small[64];
  // Selector: staged keys, then the heavy list. Mover: its entries' sources.
  __shared__ __align__(16) unsigned stage_lds[NT * KPT];
  __shared__ float mstat[2 * GL];
  __shared__ float facl[MERGE ? GL * kEvictMaxSplits : 1];
  __shared__ float opart[MERGE ? 256 : 1];
  __shared__ int evl[EMAX];
  __shared__ unsigned long long wmin_tmp[NT / 64];
  __shared__ int ticket_lds;
  const kvc_cache_t& c = e.c;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int H = c.num_kv_heads, rows = c.batch * H;
  const int NCH = e.ip_chunks;
  int32_t* const sel_flag = e.ip + 1;  // the row's selection is published
  int32_t* const mv_flag = e.ip + 1 + rows;
  // [rows][EMAX]: a row's first evicted slots, ascending, each plus one (zero:
  // not written yet), then the rows' first moved slots.
  int32_t* const evicted = e.ip + 1 + rows + (long long)rows * NCH;
  int32_t* const first_moved = evicted + (long long)rows * EMAX;
  if (tid == 0) ticket_lds = atomicAdd(e.ip, 1);
  __syncthreads();
  const int t = ticket_lds;
  const bool selector = t < rows;
  const int r = selector ? t : (t - rows) % rows;
  const int chunk = selector ? 0 : (t - rows) / rows;
  const int g = r % H, b = r / H;
  const long long rowoff = (long long)r * c.capacity;
  const int budget = e.budget, n_sink = e.n_sink, n_recent = e.n_recent;
  const int Hq = MERGE ? e.num_q_heads : 0, G = MERGE ? Hq / H : 0, S = e.splits;
  // The lengths before this step's append come from the split kernel.
  const int L_src = e.stash[b] + 1;
  const int L = __builtin_amdgcn_readfirstlane(min(min(L_src, c.capacity), e.max_len));
  const int K = min(L, budget);  // kept entries
  const int E = L - K;           // evicted entries
  const int L_h2o =
      MERGE ? __builtin_amdgcn_readfirstlane(min(min(L_src, c.capacity), (int)min(e.span, (long long)c.capacity))) : 0;
  float* const srow = e.dst_score + rowoff;  // the step's scores (dst_score == h2o_score)
  const float* const lrow = MERGE ? e.logits + ((long long)b * Hq + g * G) * e.span : nullptr;
  int32_t* const kidx = e.keep_index + (long long)r * budget;
  uint8_t* const m = e.mask ? e.mask + rowoff : nullptr;
  // This step's H2O mass of a slot below L_h2o (lg_of(h): head h's logit).
  auto h2o_mass = [&](auto lg_of) {
    float add = 0.f;
#pragma unroll
    for (int h = 0; h < GL; ++h)
      if (h < G) add = merge::h2o_add(add, lg_of(h), mstat[2 * h], mstat[2 * h + 1]);
    return add;
  };

  if (!selector) {
    // ---- a mover ----
    // The selector writes the updated scores of the slots that stay; a mover
    // adds the step's H2O mass to the scores it moves (merging).
    const int np = e.ip_passes, CH = np * RPP;
    const int part = tid % LPR, r0 = tid / LPR;
    // The row's codes as raw buffers (32-bit offsets: one register per
    // access instead of a 64-bit address).
    const __amdgpu_buffer_rsrc_t kb = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t*>(c.k_codes) + rowoff * RBK, 0, c.capacity * RBK, kEvictBufferFlags);
    const __amdgpu_buffer_rsrc_t vb = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t*>(c.v_codes) + rowoff * RBV, 0, c.capacity * RBV, kEvictBufferFlags);
    // Per-slot fields of the row, and (merging) its logits, likewise.
    const unsigned slots_b = (unsigned)c.capacity * 4;
    const __amdgpu_buffer_rsrc_t ksb = __builtin_amdgcn_make_buffer_rsrc(c.k_scale + rowoff, 0, slots_b, kEvictBufferFlags);
    const __amdgpu_buffer_rsrc_t vsb = __builtin_amdgcn_make_buffer_rsrc(c.v_scale + rowoff, 0, slots_b, kEvictBufferFlags);
    const __amdgpu_buffer_rsrc_t scb = __builtin_amdgcn_make_buffer_rsrc(srow, 0, slots_b, kEvictBufferFlags);
    int32_t* const pos = c.positions ? c.positions + rowoff : nullptr;
    const __amdgpu_buffer_rsrc_t psb = __builtin_amdgcn_make_buffer_rsrc(pos, 0, pos ? slots_b : 0, kEvictBufferFlags);
    const __amdgpu_buffer_rsrc_t lb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(lrow), 0, MERGE ? (unsigned)(G * e.span * 4) : 0, kEvictBufferFlags);
    int32_t* const own = mv_flag + (long long)r * NCH;
    u32x4 kk[MAXP], vv[MAXP];
    float fks[FPT], fvs[FPT], fsc[FPT], flg[FPT][GL];
    int fpos[FPT];
    // Loads of the rows of source slot sl_of(x) for entries x of [x0, x1):
    // codes by pass (lane group r0 holds entry x0 + q RPP + r0; spare lanes
    // repeat the last entry), the other fields (and logits) of entries
    // x0 + tid + k NT.
    auto load_logits = [&](int x0, int x1, auto sl_of) {
      if (MERGE) {
#pragma unroll
        for (int k = 0; k < FPT; ++k) {
          const int x = x0 + tid + k * NT;
          if (x < x1) {
            const int sl = sl_of(x);
#pragma unroll
            for (int h = 0; h < GL; ++h)
              flg[k][h] = __builtin_bit_cast(
                  float, __builtin_amdgcn_raw_buffer_load_b32(
                             lb, (unsigned)(min(h, G - 1) * e.span + min((long long)sl, e.span - 1)) * 4, 0, 0));
          }
        }
      }
    };
    auto load_rows = [&](int x0, int x1, auto sl_of, bool with_logits) {
#pragma unroll
      for (int q = 0; q < MAXP; ++q) {
        if (q < np) {
          const unsigned sl = sl_of(min(x0 + q * RPP + r0, x1 - 1));
          if (RBK == RB || part * 16 < RBK)
            kk[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kb, sl * RBK + part * 16, 0, 0));
          if (RBV == RB || part * 16 < RBV)
            vv[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vb, sl * RBV + part * 16, 0, 0));
        }
      }
#pragma unroll
      for (int k = 0; k < FPT; ++k) {
        const int x = x0 + tid + k * NT;
        if (x < x1) {
          const unsigned o = (unsigned)sl_of(x) * 4;
          fks[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksb, o, 0, 0));
          fvs[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vsb, o, 0, 0));
          fsc[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(scb, o, 0, 0));
          if (pos) fpos[k] = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(psb, o, 0, 0));
        }
      }
      if (with_logits) load_logits(x0, x1, sl_of);
    };
    // Merging: the moved scores take this step's H2O mass once the
    // statistics are known (then the logits need no registers while the
    // mover waits).
    auto fold_mass = [&](int x0, int x1, auto sl_of) {
      if (MERGE) {
#pragma unroll
        for (int k = 0; k < FPT; ++k) {
          const int x = x0 + tid + k * NT;
          if (x < x1 && sl_of(x) < L_h2o) fsc[k] = fsc[k] + h2o_mass([&](int h) { return flg[k][h]; });
        }
      }
    };
    // Merging: the statistics of every head (and the split weights of this
    // mover's output heads `mine`, i = 0, 1, ...).
    auto head_stats = [&](auto mine_of) {
      if (MERGE) {
        if (wave < G) {
          const float* mlh = e.part_ml + ((long long)b * Hq + g * G + wave) * S * 2;
          const int i = mine_of(wave);
          float mm, inv;
          merge::split_stats(merge::load_split_ml(mlh, S), mlh, S, i >= 0 ? facl + i * kEvictMaxSplits : nullptr,
                             mm, inv);
          if ((tid & 63) == 0) {
            mstat[2 * wave] = mm;
            mstat[2 * wave + 1] = inv;
          }
        }
        __syncthreads();
      }
    };
    // Stores of entries [x0, x1) to destination dest_of(x) (< 0: none).
    auto store_rows = [&](int x0, int x1, auto dest_of) {
#pragma unroll
      for (int q = 0; q < MAXP; ++q) {
        const int x = x0 + q * RPP + r0;
        if (q < np && x < x1) {
          const int d = dest_of(x);
          if (d >= 0) {
            if (RBK == RB || part * 16 < RBK)
              __builtin_amdgcn_raw_buffer_store_b128(kk[q], kb, (unsigned)d * RBK + part * 16, 0, 0);
            if (RBV == RB || part * 16 < RBV)
              __builtin_amdgcn_raw_buffer_store_b128(vv[q], vb, (unsigned)d * RBV + part * 16, 0, 0);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < FPT; ++k) {
        const int x = x0 + tid + k * NT;
        if (x < x1) {
          const int d = dest_of(x);
          if (d >= 0) {
            const unsigned o = (unsigned)d * 4;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, fks[k]), ksb, o, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, fvs[k]), vsb, o, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, fsc[k]), scb, o, 0, 0);
            if (pos) __builtin_amdgcn_raw_buffer_store_b32((unsigned)fpos[k], psb, o, 0, 0);
          }
        }
      }
    };
    // Few evicted slots: this mover owns source slots [s0, s1) and loads them
    // (after its share of the output merge) before the selection is known; its rows move down by the number of
    // evicted slots below them, at most E <= CH, into slots owned by this
    // mover or the one below. Else it takes destination slots past the first
    // moved one, from the keep list, after the selection.
    const bool early = !e.ip_preselected && E > 0 && E <= EMAX;
    const int s0 = chunk * CH, s1 = min(s0 + CH, L);
    auto self = [](int x) { return x; };
    // A chunk that reaches into the recent window moves whenever anything is
    // evicted: with few evicted slots it loads at once, during the selection,
    // and merges no output (its own branch, so the merge code does not hold
    // registers while its rows are in flight).
    // Chunk 0 never takes this branch: it always merges output heads.
    if (early && chunk > 0 && s0 < s1 && s1 > L - n_recent) {
      // The statistics first (a short round trip), so that no register holds
      // a row while they are computed.
      head_stats([](int) { return -1; });
      load_rows(s0, s1, self, true);
      fold_mass(s0, s1, self);
      ip_post(own + chunk, false);  // this mover's sources are read
      ip_wait(evicted + (long long)r * EMAX, E, false);
      if (tid < E) evl[tid] = min(max(__hip_atomic_load(evicted + (long long)r * EMAX + tid, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT) - 1, 0), L);
      __syncthreads();
      auto dest_of = [&](int x) -> int { return ip_dest(evl, E, x); };
      ip_wait(own + chunk - 1, chunk > 0 ? 1 : 0, false);
      store_rows(s0, s1, dest_of);
      return;
    }
    if (MERGE) {
      // The attention output of query heads chunk, chunk + MC, ... (the merge
      // kernel's arithmetic and order), by the movers that wait for the
      // selection before they load: chunks [0, MC).
      const int MC = early ? max(1, min(NCH, (L - n_recent) / CH)) : NCH;
      head_stats([&](int w) { return chunk < MC && w >= chunk && (w - chunk) % MC == 0 ? (w - chunk) / MC : -1; });
      const int D = c.head_dim, PARTS = 256 / D;
      for (int h = chunk, i = 0; chunk < MC && h < G; h += MC, ++i) {
        if (tid < 256) {
          const int d = tid % D, pi = tid / D;
          const float* po = e.part_o + ((long long)b * Hq + g * G + h) * S * D + d;
          float o = 0.f;
          for (int sp = pi; sp < S; sp += PARTS) o = fmaf(po[(long long)sp * D], facl[i * kEvictMaxSplits + sp], o);
          opart[pi * D + d] = o;
        }
        __syncthreads();
        if (tid < D) {
          float rr = opart[tid];
          for (int q = 1; q < PARTS; ++q) rr += opart[q * D + tid];
          e.out[((long long)b * Hq + g * G + h) * D + tid] = rr;
        }
        __syncthreads();
      }
    }
    if (early) {
      // The others wait for the selection and load only their rows at or
      // past the first evicted slot.
      if (s0 >= s1) {
        ip_post(own + chunk, false);
        return;
      }
      // The selection reaches this mover through the evicted-slot list alone,
      // each entry its own flag (agent-scope atomics): no cache writeback or
      // invalidation is needed. The selector has read every score it needs
      // by then.
      ip_wait(evicted + (long long)r * EMAX, E, false);
      if (tid < E) evl[tid] = min(max(__hip_atomic_load(evicted + (long long)r * EMAX + tid, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT) - 1, 0), L);
      __syncthreads();
      // Slot x keeps its token iff it is not evicted; it moves down by the
      // number of evicted slots below it (a fixed-step binary search over the
      // E <= EMAX ascending slots).
      auto dest_of = [&](int x) -> int { return ip_dest(evl, E, x); };
      // Rows below the first evicted slot stay where they are; nobody writes
      // them, so only the rest is loaded before the flag.
      const int x0 = __builtin_amdgcn_readfirstlane(max(s0, min(evl[0], s1)));
      if (x0 < s1) {
        load_rows(x0, s1, self, true);
        fold_mass(x0, s1, self);
      }
      ip_post(own + chunk, false);
      if (x0 >= s1) return;
      ip_wait(own + chunk - 1, chunk > 0 ? 1 : 0, false);
      store_rows(x0, s1, dest_of);
      return;
    }
    ip_wait(sel_flag + r, 1, true);
    // Clamped, like the sources below, so that even a wait that gave up
    // cannot send an access out of the row.
    const int d0 = __builtin_amdgcn_readfirstlane(
        min(max(__hip_atomic_load(first_moved + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), 0), K));
    const int e0 = d0 + chunk * CH, e1 = min(e0 + CH, K);
    if (e0 >= e1) {
      ip_post(own + chunk, false);
      return;
    }
    int* src = reinterpret_cast<int*>(stage_lds);
    for (int i = tid; i < e1 - e0; i += NT) src[i] = min(max(kidx[e0 + i], 0), c.capacity - 1);
    __syncthreads();
    auto src_of = [&](int x) { return src[x - e0]; };
    load_rows(e0, e1, src_of, true);
    fold_mass(e0, e1, src_of);
    ip_post(own + chunk, false);  // this mover's sources are read
    // A slot is a source only for an entry whose destination is not above
    // it, so the readers of this mover's destinations are it and lower chunks.
    ip_wait(own, chunk, false);
    store_rows(e0, e1, self);
    return;
  }

  // ---- the row's selector ----
  auto set_length = [&]() {
    if (g == 0 && tid == 0) {
      c.lengths[b] = K;
      c.num_seen[b] = e.stash[c.batch + b] + 1;
    }
  };
  if (e.ip_preselected) {
    // A selection kernel wrote the keep list (on scores the merge kernel
    // updated): the first moved slot is the first entry whose source is not
    // its own slot.
    int first = K;
    for (int d = tid; d < K; d += NT)
      if (kidx[d] != d) {
        first = d;
        break;
      }
    first = block_min_int<NT>(first, mm_tmp);
    if (tid == 0) first_moved[r] = first;
    ip_post(sel_flag + r, true);
    set_length();
    return;
  }
  const float* mlh = MERGE ? e.part_ml + ((long long)b * Hq + g * G + min(wave, G - 1)) * S * 2 : nullptr;
  merge::SplitML mlr;
  if (MERGE) mlr = merge::load_split_ml(mlh, S);  // every wave (clamped head): no branch to wait in
  float sv[KPT];
  float lgv[KPT][GL];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int slot = min(n_sink + tid + j * NT, c.capacity - 1);
    sv[j] = srow[slot];
    if (MERGE) {
#pragma unroll
      for (int h = 0; h < GL; ++h) lgv[j][h] = lrow[min(h, G - 1) * e.span + min((long long)slot, e.span - 1)];
    }
  }
  // Merging: the sinks' scores and logits (the first NT sinks) load now too.
  float ssc = 0.f, slg[GL];
  const int sink_slot = min(tid, max(min(n_sink, L) - 1, 0));
  if (MERGE) {
    ssc = srow[sink_slot];
#pragma unroll
    for (int h = 0; h < GL; ++h) slg[h] = lrow[min(h, G - 1) * e.span + min((long long)sink_slot, e.span - 1)];
    if (wave < G) {
      float mm, inv;
      merge::split_stats(mlr, mlh, S, nullptr, mm, inv);
      if ((tid & 63) == 0) {
        mstat[2 * wave] = mm;
        mstat[2 * wave + 1] = inv;
      }
    }
    __syncthreads();
  }
  // Keys: the scores with this step's H2O mass when merging.
  float u[KPT];
  unsigned v[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int slot = n_sink + tid + j * NT;
    u[j] = sv[j];
    if (MERGE && slot < L_h2o) u[j] = u[j] + h2o_mass([&](int h) { return lgv[j][h]; });
    v[j] = radix::order_key(u[j]);
  }
  const bool all = L <= budget;
  const int lo = n_sink, hi = L - n_recent;
  const int n_heavy = all ? 0 : budget - n_sink - n_recent;
  int d0 = K;  // first moved slot
  if (all) {
    for (int d = tid; d < L; d += NT) {
      kidx[d] = d;
      if (m) m[d] = 1;
    }
  } else if (E <= kIpFewEvicted) {
    // Few evicted tokens (the steady state of a decode loop evicts one):
    // the evicted ones are the E smallest candidates by (score ascending,
    // slot descending), the complement of the keep rule; E rounds of a
    // block-wide minimum of (key, ~slot) find them without a radix pass.
    unsigned long long kv[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const unsigned slot = (unsigned)(n_sink + tid + j * NT);
      kv[j] = slot < (unsigned)hi ? ((unsigned long long)v[j] << 32) | (0xFFFFFFFFu - slot) : ~0ull;
    }
    int ev[kIpFewEvicted];
#pragma unroll
    for (int i = 0; i < kIpFewEvicted; ++i) {
      ev[i] = 0;
      if (i < E) {
        unsigned long long mn = kv[0];
#pragma unroll
        for (int j = 1; j < KPT; ++j) mn = kv[j] < mn ? kv[j] : mn;
        mn = block_min_u64<NT>(mn, wmin_tmp);
        ev[i] = (int)(0xFFFFFFFFu - (unsigned)mn);
#pragma unroll
        for (int j = 0; j < KPT; ++j) kv[j] = kv[j] == mn ? ~0ull : kv[j];
      }
    }
    // ascending (every thread sorts the same E <= kIpFewEvicted slots)
#pragma unroll
    for (int i = 1; i < kIpFewEvicted; ++i)
#pragma unroll
      for (int j = kIpFewEvicted - 1; j >= i; --j)
        if (j < E && ev[j - 1] > ev[j]) {
          const int x = ev[j - 1];
          ev[j - 1] = ev[j];
          ev[j] = x;
        }
    if (tid < E) {
      int x = ev[0];
#pragma unroll
      for (int i = 1; i < kIpFewEvicted; ++i) x = tid == i ? ev[i] : x;
      __hip_atomic_store(evicted + (long long)r * EMAX + tid, x + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Keep list: destination d takes source d plus the evicted slots at or
    // below the running source.
    for (int d = tid; d < K; d += NT) {
      int src = d;
#pragma unroll
      for (int i = 0; i < kIpFewEvicted; ++i)
        if (i < E && ev[i] <= src) ++src;
      kidx[d] = src;
    }
    if (m) {
      for (int sl = tid; sl < L; sl += NT) {
        bool keep = true;
#pragma unroll
        for (int i = 0; i < kIpFewEvicted; ++i) keep = keep && !(i < E && ev[i] == sl);
        m[sl] = (uint8_t)keep;
      }
    }
    d0 = ev[0];
  } else {
    const int n = hi - lo;
    int k = n_heavy;
    const int per = ((n + NT - 1) / NT + 3) & ~3;
    const int i0 = lo + min(tid * per, n), cnt = min(tid * per + per, n) - min(tid * per, n);
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
#pragma unroll
    for (int j = 0; j < KPT; ++j) stage_lds[tid + j * NT] = v[j];
    __syncthreads();
    unsigned key[KPT];
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
#pragma unroll
    for (int q = 0; q < KPT; ++q) key[q] = q < cnt ? key[q] : 0u;
    auto for_keys = [&](auto f) {
#pragma unroll
      for (int q = 0; q < KPT; ++q) f(key[q]);
    };
    const bool any_heavy = k > 0;
    unsigned T = 0;
    if (any_heavy) T = radix::radix_threshold_range<NT, kHistCopies>(for_keys, k, kmin, kmax, hist, scan_tmp, sel, small);
    int ties = 0, above = 0;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      ties += any_heavy & (key[q] == T);
      above += any_heavy & (key[q] > T);
    }
    const int packed = ties | (above << 16);
    const int before = block_inclusive_scan<NT>(packed, scan_tmp) - packed;
    int tie_rank = before & 0xFFFF;
    int out = (before >> 16) + min(tie_rank, k);
    int* heavy = reinterpret_cast<int*>(stage_lds);
    // The scan's barrier ordered every read of the staged keys before these
    // writes of the heavy list into the same LDS.
    int first = n_heavy;  // first heavy rank not in its own slot
    int32_t* const evrow = evicted + (long long)r * EMAX;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      if (q < cnt) {
        const unsigned uk = key[q];
        int keepb = 0;
        if (any_heavy) {
          if (uk > T) {
            keepb = 1;
          } else if (uk == T) {
            keepb = tie_rank < k;
            ++tie_rank;
          }
        }
        if (m) m[i0 + q] = (uint8_t)keepb;
        if (keepb) {
          if (i0 + q != lo + out) first = min(first, out);
          heavy[min(out, NT * KPT - 1)] = i0 + q;
          ++out;
        } else {
          const int ev = i0 + q - lo - out;  // evicted candidates below this one
          if (ev < EMAX) __hip_atomic_store(evrow + ev, i0 + q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    first = block_min_int<NT>(first, mm_tmp);  // its barriers also publish the heavy list
    for (int h = tid; h < n_heavy; h += NT) kidx[lo + h] = heavy[h];
    for (int d = tid; d < n_sink; d += NT) {
      kidx[d] = d;
      if (m) m[d] = 1;
    }
    for (int i = tid; i < L - hi; i += NT) {
      kidx[lo + n_heavy + i] = hi + i;
      if (m) m[hi + i] = 1;
    }
    d0 = first < n_heavy ? lo + first : (L > hi ? lo + n_heavy : K);
  }
  // Merging: the updated scores of the slots that stay (below d0); the
  // movers write those of the tokens they move.
  if (MERGE) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int slot = n_sink + tid + j * NT;
      if (slot < d0) srow[slot] = u[j];
    }
    if (tid < min(n_sink, d0)) srow[tid] = ssc + (tid < L_h2o ? h2o_mass([&](int h) { return slg[h]; }) : 0.f);
    auto update = [&](int slot) {
      float s = srow[slot];
      if (slot < L_h2o) s = s + h2o_mass([&](int h) { return lrow[h * e.span + slot]; });
      srow[slot] = s;
    };
    for (int slot = NT + tid; slot < min(n_sink, d0); slot += NT) update(slot);
    for (int slot = n_sink + NT * KPT + tid; slot < d0; slot += NT) update(slot);
  }
  if (tid == 0) first_moved[r] = d0;
  // Movers of the keep-list path read the keep list, the first moved slot and
  // the scores through the cache: the L2 is written back first. (Movers of
  // the early path wait for the evicted-slot list instead.)
  ip_post(sel_flag + r, true);
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

template <int RBK, int RBV, int GK>
hipError_t launch_ip_rb(const EvictArgs& a, hipStream_t st) {
  const long long rows = (long long)a.c.batch * a.c.num_kv_heads;
  const long long wgs = rows * (1 + (long long)a.ip_chunks);
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((evict_inplace_kernel<RBK, RBV, GK>), dim3((unsigned)wgs), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

template <int GK>
hipError_t launch_ip_gk(const EvictArgs& a, hipStream_t st) {
  return with_row_bytes(a.c, [&](auto rbk, auto rbv) {
    return launch_ip_rb<decltype(rbk)::value, decltype(rbv)::value, GK>(a, st);
  });
}

}  // namespace

hipError_t launch_evict_inplace(const EvictArgs& a, hipStream_t st) {
  if (!a.part_ml) return launch_ip_gk<0>(a, st);
  const int G = a.num_q_heads / a.c.num_kv_heads;
  if (G <= 1) return launch_ip_gk<1>(a, st);
  if (G <= 2) return launch_ip_gk<2>(a, st);
  if (G <= 4) return launch_ip_gk<4>(a, st);
  return launch_ip_gk<8>(a, st);
}

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
