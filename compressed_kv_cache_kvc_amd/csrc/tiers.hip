// fp16 precision tiers at both ends of a quantized cache.
//
// "KV Cache Compression Report", section 3.2 keeps the K and V of the
// attention-sink tokens in fp16; the "KV Cache optimization techniques"
// tutorial, section 1.3 keeps recent tokens at fp16 and older ones quantized
// (its "int4_hybrid" mode). In a row of L slots the sink tier is slots
// [0, ns), ns = min(fp16_sinks, L), and the recent tier the newest
// nr = min(fp16_recent, L - ns) slots. The codes of every token are still
// written (quantize on write); attention reads the tier slots' fp16 rows.
//
// Storage: the sink rows are indexed by slot (slot j < fp16_sinks is always
// the j-th token, since eviction keeps the sinks and compaction is stable);
// the recent rows form a ring indexed by position % fp16_recent (slot i of the
// recent tier holds position num_seen - L + i, since eviction keeps the
// newest slots). Neither moves under compaction.
//
// Attention: the split kernel masks the tier slots out of the code path, and
// attn_tier_kernel adds the tiers as extra partial softmax states (parts
// S .. S + TP - 1 of each query head, 64 tier tokens per part), which the
// merge folds in with the splits. Logits and values are fp32 from the fp16
// rows; the H2O logits of the tier slots are written at their slots.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Row of tier index j (the tier's j-th slot, sinks first) of one
// (sequence, KV head); `nw` is the appended token's row when slot L_old was
// appended in this call.
struct TierRows {
  const __half* sink;   // [fp16_sinks][D] of this row
  const __half* ring;   // [fp16_recent][D] of this row
  const __half* nw;     // [D] or NULL
  int ns, nr, L, L_old, seen, recent;
  __device__ const __half* row(int j, int D) const {
    const int slot = j < ns ? j : L - nr + (j - ns);
    if (nw && slot == L_old) return nw;
    if (j < ns) return sink + (long long)slot * D;
    const unsigned p = (unsigned)(seen - L + slot) % (unsigned)recent;
    return ring + (long long)p * D;
  }
};

// Store the fp16 rows of appended tokens in the tiers. Thread i of the grid
// copies 16 bytes: token t = i / (D / 8), chunk i % (D / 8). Slot
// lengths[b] + t < fp16_sinks goes to the sink rows; the newest fp16_recent
// of the n_new tokens go to the ring (older ones would be overwritten).
template <int D>
__global__ __launch_bounds__(256) void tier_append_kernel(kvc_cache_t c, const __half* __restrict__ kn,
                                                          const __half* __restrict__ vn, int n_new) {
  constexpr int NCH = D / 8;
  const int g = blockIdx.y, b = blockIdx.z, H = c.num_kv_heads;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int t = i / NCH, ch = i % NCH;
  if (t >= n_new) return;
  const int L0 = c.lengths[b], ns0 = c.num_seen[b];
  const long long row = (long long)b * H + g;
  const long long src = (row * n_new + t) * D + ch * 8;
  const u32x4 kx = *reinterpret_cast<const u32x4*>(kn + src);
  const u32x4 vx = *reinterpret_cast<const u32x4*>(vn + src);
  const long long slot = (long long)L0 + t;
  if (slot >= 0 && slot < c.fp16_sinks) {
    const long long dst = (row * c.fp16_sinks + slot) * D + ch * 8;
    *reinterpret_cast<u32x4*>(static_cast<__half*>(c.k_sink16) + dst) = kx;
    *reinterpret_cast<u32x4*>(static_cast<__half*>(c.v_sink16) + dst) = vx;
  }
  if (c.fp16_recent > 0 && t >= n_new - c.fp16_recent) {
    const unsigned p = (unsigned)(ns0 + t) % (unsigned)c.fp16_recent;
    const long long dst = (row * c.fp16_recent + p) * D + ch * 8;
    *reinterpret_cast<u32x4*>(static_cast<__half*>(c.k_recent16) + dst) = kx;
    *reinterpret_cast<u32x4*>(static_cast<__half*>(c.v_recent16) + dst) = vx;
  }
}

// One wave per part: tier tokens [64 x, 64 x + 64) of row (b, g), for the G
// query heads of g (GM >= G, padded). Lane t holds token 64 x + t for the
// logits; for P.V, lane l holds channels CPL l .. CPL l + CPL - 1.
template <int D, int GM>
__global__ __launch_bounds__(64) void attn_tier_kernel(AttnLaunch a) {
  constexpr int NCH = D / 8;   // 16-byte chunks per row
  constexpr int CPL = D / 64;  // channels per lane in P.V
  static_assert(CPL == 1 || CPL == 2, "head_dim 64 or 128");
  const kvc_cache_t& c = a.c;
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.splits, P = a.parts;
  const long long span = (long long)S * a.tiles * kSplitTokens;
  const bool app = a.k_new != nullptr;
  const int L_old = __builtin_amdgcn_readfirstlane(c.lengths[b]);
  const int L = max(0, __builtin_amdgcn_readfirstlane(min(min(L_old + (app ? 1 : 0), c.capacity), (int)span)));
  const int seen = __builtin_amdgcn_readfirstlane(c.num_seen[b]) + (app ? 1 : 0);
  const long long rowid = (long long)b * H + g;

  TierRows kr, vr;
  kr.ns = vr.ns = min(c.fp16_sinks, L);
  kr.nr = vr.nr = min(c.fp16_recent, L - kr.ns);
  kr.L = vr.L = L;
  kr.L_old = vr.L_old = L_old;
  kr.seen = vr.seen = seen;
  kr.recent = vr.recent = c.fp16_recent;
  kr.sink = static_cast<const __half*>(c.k_sink16) + rowid * c.fp16_sinks * D;
  vr.sink = static_cast<const __half*>(c.v_sink16) + rowid * c.fp16_sinks * D;
  kr.ring = static_cast<const __half*>(c.k_recent16) + rowid * c.fp16_recent * D;
  vr.ring = static_cast<const __half*>(c.v_recent16) + rowid * c.fp16_recent * D;
  const bool new_here = app && L_old >= 0 && L_old < L;  // the split kernel appended slot L_old
  kr.nw = new_here ? a.k_new + rowid * D : nullptr;
  vr.nw = new_here ? a.v_new + rowid * D : nullptr;
  const int nt = kr.ns + kr.nr, j0 = x * kTierTokens;

  // The appended token's tier rows: stored by the part that holds it (its
  // tier index is L_old when it is a sink, else the last one). No other part
  // reads those rows in this call (it reads them from k_new / v_new).
  if (new_here) {
    const int jn = L_old < kr.ns ? L_old : (L_old >= L - kr.nr ? kr.ns + (L_old - (L - kr.nr)) : -1);
    if (jn >= j0 && jn < j0 + kTierTokens && lane < NCH) {
      const u32x4 kx = *reinterpret_cast<const u32x4*>(kr.nw + lane * 8);
      const u32x4 vx = *reinterpret_cast<const u32x4*>(vr.nw + lane * 8);
      if (L_old < c.fp16_sinks) {
        const long long dst = (rowid * c.fp16_sinks + L_old) * D + lane * 8;
        *reinterpret_cast<u32x4*>(static_cast<__half*>(c.k_sink16) + dst) = kx;
        *reinterpret_cast<u32x4*>(static_cast<__half*>(c.v_sink16) + dst) = vx;
      }
      if (c.fp16_recent > 0) {
        const unsigned p = (unsigned)(seen - 1) % (unsigned)c.fp16_recent;
        const long long dst = (rowid * c.fp16_recent + p) * D + lane * 8;
        *reinterpret_cast<u32x4*>(static_cast<__half*>(c.k_recent16) + dst) = kx;
        *reinterpret_cast<u32x4*>(static_cast<__half*>(c.v_recent16) + dst) = vx;
      }
    }
  }

  // q of the group's heads, fp32 in LDS (padded heads are zero).
  __shared__ float qs[GM][D];
  for (int i = lane; i < GM * D; i += 64) {
    const int h = i / D;
    qs[h][i % D] = h < G ? __half2float(a.q[((long long)b * Hq + g * G) * D + i]) : 0.f;
  }
  __syncthreads();

  // ---- logits, one token per lane ----
  const int j = j0 + lane;
  const bool valid = j < nt;
  float s[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) s[h] = 0.f;
  if (valid) {
    const __half* k = kr.row(j, D);
#pragma unroll 4
    for (int ch = 0; ch < NCH; ++ch) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(k + ch * 8);
      float xe[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned u = w[e];  // a scalar first: a bit_cast of the vector element itself reads element 0
        const __half2 h2 = __builtin_bit_cast(__half2, u);
        xe[2 * e] = __low2float(h2);
        xe[2 * e + 1] = __high2float(h2);
      }
#pragma unroll
      for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[h] = fmaf(qs[h][ch * 8 + e], xe[e], s[h]);
    }
  }
  const int slot = j < kr.ns ? j : L - kr.nr + (j - kr.ns);
  float m[GM], l[GM], p[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    const float lg = valid ? s[h] * a.qk_log2 : -INFINITY;
    if (a.logits && valid && h < G) a.logits[((long long)b * Hq + g * G + h) * span + slot] = lg;
    m[h] = wave_max(lg);
    p[h] = valid ? __builtin_amdgcn_exp2f(lg - m[h]) : 0.f;
    l[h] = wave_sum(p[h]);
  }

  // ---- P.V over this part's tokens, channels across lanes ----
  float o[GM][CPL];
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < CPL; ++e) o[h][e] = 0.f;
  const int nv = min(kTierTokens, nt - j0);
#pragma unroll 4
  for (int t = 0; t < nv; ++t) {
    const __half* v = vr.row(j0 + t, D) + lane * CPL;
    float ve[CPL];
    if constexpr (CPL == 2) {
      const __half2 h2 = *reinterpret_cast<const __half2*>(v);
      ve[0] = __low2float(h2);
      ve[1] = __high2float(h2);
    } else {
      ve[0] = __half2float(*v);
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float ph = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[h]), t));
#pragma unroll
      for (int e = 0; e < CPL; ++e) o[h][e] = fmaf(ph, ve[e], o[h][e]);
    }
  }

  // ---- this part's state per head: (m, l, o) at part S + x ----
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) break;
    const long long pi = ((long long)b * Hq + g * G + h) * P + S + x;
#pragma unroll
    for (int e = 0; e < CPL; ++e) a.part_o[pi * D + lane * CPL + e] = o[h][e];
    if (lane == 0) {
      a.part_ml[pi * 2] = m[h];
      a.part_ml[pi * 2 + 1] = l[h];
    }
  }
}

template <int D>
hipError_t launch_tiers_d(const AttnLaunch& a, int G, hipStream_t st) {
  const dim3 grid(a.tier_parts, a.c.num_kv_heads, a.c.batch);
  if (G == 1) hipLaunchKernelGGL((attn_tier_kernel<D, 1>), grid, dim3(64), 0, st, a);
  else if (G == 2) hipLaunchKernelGGL((attn_tier_kernel<D, 2>), grid, dim3(64), 0, st, a);
  else if (G <= 4) hipLaunchKernelGGL((attn_tier_kernel<D, 4>), grid, dim3(64), 0, st, a);
  else if (G <= 8) hipLaunchKernelGGL((attn_tier_kernel<D, 8>), grid, dim3(64), 0, st, a);
  else hipLaunchKernelGGL((attn_tier_kernel<D, 16>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_tiers(const AttnLaunch& a, hipStream_t st) {
  if (a.tier_parts <= 0) return hipSuccess;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  return a.c.head_dim == 64 ? launch_tiers_d<64>(a, G, st) : launch_tiers_d<128>(a, G, st);
}

hipError_t launch_tier_append(const kvc_cache_t& c, const __half* kn, const __half* vn, int n_new,
                              hipStream_t st) {
  if (c.fp16_sinks <= 0 && c.fp16_recent <= 0) return hipSuccess;
  const long long threads = (long long)n_new * (c.head_dim / 8);
  const dim3 grid((unsigned)((threads + 255) / 256), c.num_kv_heads, c.batch);
  if (c.head_dim == 64) hipLaunchKernelGGL((tier_append_kernel<64>), grid, dim3(256), 0, st, c, kn, vn, n_new);
  else hipLaunchKernelGGL((tier_append_kernel<128>), grid, dim3(256), 0, st, c, kn, vn, n_new);
  return hipGetLastError();
}

}  // namespace kvc
