// Attention over the fp16 tiers of a cache (attn_tier_kernel, launched right
// after the split kernel; its own launch keeps the split kernel's registers
// as they are).
//
// "KV Cache Compression Report", section 3.2 keeps the attention sinks' K and
// V in fp16; the "KV Cache optimization techniques" tutorial, section 1.3
// keeps recent tokens at fp16 and older ones quantized. In a row of L slots
// the sink tier is slots [0, ns), ns = min(fp16_sinks, L), and the recent tier
// the newest nr = min(fp16_recent, L - ns) slots. The split workgroups mask
// those slots out; here each wave turns 64 tier tokens into one more partial
// softmax state per query head (part S + 4 x + wave), in the split states'
// convention (max in log2 units, sum, unnormalized o), so the merge folds the
// tiers in with the splits. The tier slots' H2O logits are spilled at their
// slots.
//
// Storage: sink rows by slot ([fp16_sinks][D] per row), recent rows in a ring
// by position % fp16_recent, slot i of the recent tier holding position
// num_seen - L + i. With an append in the same call, the new token's rows come
// from k_new / v_new, and the wave that holds it stores them in the tiers.
//
// Layout in a wave: LPT = D / 8 lanes per token (16 bytes each), TPI = 64 / LPT
// tokens per load, NI = 64 / TPI loads per lane for K and for V, issued half
// at a time (each half's loads together, before its arithmetic). Logits are
// LPT-lane dot products; the softmax runs online over the token groups; the
// groups' states are summed at the end. GP query heads per pass.
#pragma once

#include "kvc_internal.h"

namespace kvc {
namespace tier {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// qs: GP * D floats of LDS, free for this workgroup's use.
template <int D, int GP>
__device__ __forceinline__ void tier_parts(const AttnLaunch& a, int xt, float* qs) {
  constexpr int LPT = D / 8, TPI = 64 / LPT, NI = kTierTokens / TPI;
  const kvc_cache_t& c = a.c;
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.splits, P = a.parts;
  const long long span = attn_span(a);
  const bool app = a.k_new != nullptr;
  const int L_old = __builtin_amdgcn_readfirstlane(c.lengths[b]);
  const int L = max(0, __builtin_amdgcn_readfirstlane(min(min(L_old + (app ? 1 : 0), c.capacity), (int)span)));
  const int seen = __builtin_amdgcn_readfirstlane(c.num_seen[b]) + (app ? 1 : 0);
  const long long rowid = (long long)b * H + g;
  const int ns = min(c.fp16_sinks, L), nr = min(c.fp16_recent, L - ns), nt = ns + nr;
  const int part = 4 * xt + wave;  // parts past tier_parts idle (but join the barriers)
  const bool active = part < a.tier_parts;
  const int j0 = part * kTierTokens;
  const bool new_here = app && L_old >= 0 && L_old < L;  // slot L_old was appended in this call
  const __half* k_sink = static_cast<const __half*>(c.k_sink16) + rowid * c.fp16_sinks * D;
  const __half* v_sink = static_cast<const __half*>(c.v_sink16) + rowid * c.fp16_sinks * D;
  const __half* k_ring = static_cast<const __half*>(c.k_recent16) + rowid * c.fp16_recent * D;
  const __half* v_ring = static_cast<const __half*>(c.v_recent16) + rowid * c.fp16_recent * D;
  auto slot_of = [&](int j) { return j < ns ? j : L - nr + (j - ns); };
  // Element offset of tier token j's row in its buffer; -1: the appended row.
  auto row_off = [&](int j) -> long long {
    const int slot = slot_of(j);
    if (new_here && slot == L_old) return -1;
    if (j < ns) return (long long)slot * D;
    return (long long)((unsigned)(seen - L + slot) % (unsigned)c.fp16_recent) * D;
  };

  // The appended token's tier rows, stored by the wave that holds its tier
  // index; no other wave of this launch reads those rows (they read k_new).
  if (active && new_here) {
    const int jn = L_old < ns ? L_old : (L_old >= L - nr ? ns + (L_old - (L - nr)) : -1);
    if (jn >= j0 && jn < j0 + kTierTokens && lane < LPT) {
      const u32x4 kx = *reinterpret_cast<const u32x4*>(a.k_new + rowid * D + lane * 8);
      const u32x4 vx = *reinterpret_cast<const u32x4*>(a.v_new + rowid * D + lane * 8);
      if (L_old < c.fp16_sinks) {
        const long long dst = (rowid * c.fp16_sinks + L_old) * D + lane * 8;
        *reinterpret_cast<u32x4*>(static_cast<__half*>(c.k_sink16) + dst) = kx;
        *reinterpret_cast<u32x4*>(static_cast<__half*>(c.v_sink16) + dst) = vx;
      }
      if (c.fp16_recent > 0) {
        const long long dst = (rowid * c.fp16_recent + (unsigned)(seen - 1) % (unsigned)c.fp16_recent) * D + lane * 8;
        *reinterpret_cast<u32x4*>(static_cast<__half*>(c.k_recent16) + dst) = kx;
        *reinterpret_cast<u32x4*>(static_cast<__half*>(c.v_recent16) + dst) = vx;
      }
    }
  }

  // ---- per head pass: the wave's tokens in two halves, each half's K and V
  // loads issued together before its arithmetic; online softmax ----
  const int r = lane / LPT, cc = lane % LPT;  // token within a load, 16-byte chunk of the row
  constexpr int NH = NI / 2;
  for (int hp = 0; hp < G; hp += GP) {
    __syncthreads();  // the previous pass is done with qs
    for (int i = tid; i < GP * D; i += 256) {
      const int h = i / D;
      qs[i] = hp + h < G ? __half2float(a.q[((long long)b * Hq + g * G + hp) * D + i]) : 0.f;
    }
    __syncthreads();
    if (!active) continue;
    float m_run[GP], l_run[GP], o[GP][8];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      m_run[h] = -INFINITY;
      l_run[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      if (j0 + TPI * NH * half >= nt) break;  // no tier token left in this wave (uniform)
      u32x4 kx[NH], vx[NH];
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int j = j0 + TPI * (half * NH + i) + r;
        kx[i] = u32x4{0u, 0u, 0u, 0u};
        vx[i] = u32x4{0u, 0u, 0u, 0u};
        if (j < nt) {
          const long long off = row_off(j);
          const bool sink = j < ns;
          const __half* kr = off < 0 ? a.k_new + rowid * D : (sink ? k_sink : k_ring) + off;
          const __half* vr = off < 0 ? a.v_new + rowid * D : (sink ? v_sink : v_ring) + off;
          kx[i] = *reinterpret_cast<const u32x4*>(kr + cc * 8);
          vx[i] = *reinterpret_cast<const u32x4*>(vr + cc * 8);
        }
      }
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        if (j0 + TPI * (half * NH + i) >= nt) break;  // the rest of the groups are past the tier (uniform)
        const int j = j0 + TPI * (half * NH + i) + r;
        const bool ok = j < nt;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned uk = kx[i][e];  // a scalar first: a bit_cast of a vector element reads element 0
            const __half2 hk = __builtin_bit_cast(__half2, uk);
            d = fmaf(qs[h * D + cc * 8 + 2 * e], __low2float(hk), d);
            d = fmaf(qs[h * D + cc * 8 + 2 * e + 1], __high2float(hk), d);
          }
#pragma unroll
          for (int s = 1; s < LPT; s <<= 1) d += __shfl_xor(d, s);
          const bool real = ok && hp + h < G;
          const float lg = real ? d * a.qk_log2 : -INFINITY;
          if (a.logits && real && cc == 0) a.logits[((long long)b * Hq + g * G + hp + h) * span + slot_of(j)] = lg;
          float mb = lg;
#pragma unroll
          for (int s = LPT; s < 64; s <<= 1) mb = fmaxf(mb, __shfl_xor(mb, s));
          const float mn = fmaxf(m_run[h], mb);
          const float corr = m_run[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[h] - mn);
          const float p = lg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lg - mn);
          m_run[h] = mn;
          l_run[h] = fmaf(l_run[h], corr, p);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned uv = vx[i][e];
            const __half2 hv = __builtin_bit_cast(__half2, uv);
            o[h][2 * e] = fmaf(o[h][2 * e], corr, p * __low2float(hv));
            o[h][2 * e + 1] = fmaf(o[h][2 * e + 1], corr, p * __high2float(hv));
          }
        }
      }
    }
    // Sum the token groups (lanes equal mod LPT), then lanes 0..LPT-1 write
    // channels 8 cc .. 8 cc + 7 of each head's state.
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (hp + h >= G) break;
      float l = l_run[h];
#pragma unroll
      for (int s = LPT; s < 64; s <<= 1) l += __shfl_xor(l, s);
      const long long pi = ((long long)b * Hq + g * G + hp + h) * P + S + part;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = o[h][e];
#pragma unroll
        for (int s = LPT; s < 64; s <<= 1) v += __shfl_xor(v, s);
        if (r == 0) a.part_o[pi * D + cc * 8 + e] = v;
      }
      if (lane == 0) {
        a.part_ml[pi * 2] = m_run[h];
        a.part_ml[pi * 2 + 1] = l;
      }
    }
  }
}

}  // namespace tier
}  // namespace kvc
