// Attention over the fp16 tiers of a cache (attn_tier_kernel, launched right
// after the split kernel; its own launch keeps the split kernel's registers
// as they are).
//
// "KV Cache Compression Report", section 3.2 keeps the attention sinks' K and
// V in fp16; the "KV Cache optimization techniques" tutorial, section 1.3
// keeps recent tokens at fp16 and older ones quantized. In a row of L slots
// the sink tier is slots [0, ns), ns = min(fp16_sinks, L), and the recent tier
// the newest nr = min(fp16_recent, L - ns) slots. The split workgroups mask
// those slots out; here a two-wave workgroup turns 64 tier tokens into one
// more partial softmax state per query head (part S + x), in the split states'
// convention (max in log2 units, sum, unnormalized o), so the merge folds the
// tiers in with the splits. The tier slots' H2O logits are spilled at their
// slots.
//
// Storage: sink rows by slot ([fp16_sinks][D] per row), recent rows in a ring
// by position % fp16_recent, slot i of the recent tier holding position
// num_seen - L + i. With an append in the same call, the new token's rows come
// from k_new / v_new, and the wave that holds it stores them in the tiers.
//
// Layout in the wave: LPT = D / 8 lanes per token (16 bytes each), TPI = 64 /
// LPT tokens per load, NI = 64 / TPI = LPT loads per lane for K and for V.
// Wave w takes half w of the 64 tokens: its NH = LPT / 2 loads go out
// together, in one round, before its arithmetic; the two waves' states meet
// in LDS at the end. A lane's NH partial dot products are summed over the
// token's LPT lanes by a reduce-scatter (halve the list at each exchange, DPP
// lane moves), after which lane pair (2 i, 2 i + 1) of a token row holds the
// logit of group i: one exchange per value instead of a log2(LPT) butterfly
// per group, and one exp2 per lane. The probabilities go back to the lanes
// holding the V rows by lane-indexed reads. GP query heads per pass, their q
// rows in registers.
#pragma once

#include "kvc_internal.h"

namespace kvc {
namespace tier {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The value of the lane that differs from this one in bits 0..log2(S) (a
// mirror inside each half-row or row for S = 4, 8; xor 2, xor 1 below):
// DPP, no LDS round trip.
template <int S>
__device__ __forceinline__ float partner(float v) {
  if constexpr (S == 8) return dpp_f<0x140>(v, v);       // row mirror: lane ^ 15
  else if constexpr (S == 4) return dpp_f<0x141>(v, v);  // half-row mirror: lane ^ 7
  else if constexpr (S == 2) return dpp_f<0x4E>(v, v);   // lane ^ 2
  else return dpp_f<0xB1>(v, v);                         // lane ^ 1
}

// One exchange of the reduce-scatter: keep half of the list (the upper half
// where bit S of the lane is set), add the partner's copy of that half.
template <int S, int N>
__device__ __forceinline__ void scatter_step(float (&x)[N], int lane) {
  if constexpr (S >= 2) {
    constexpr int n = S / 2;
    const bool up = lane & S;
#pragma unroll
    for (int k = 0; k < n; ++k) {
      const float keep = up ? x[n + k] : x[k], give = up ? x[k] : x[n + k];
      x[k] = keep + partner<S>(give);
    }
    scatter_step<S / 2>(x, lane);
  }
}

// Sums x[0..N) over the 2 N lanes of an aligned group (N = 4 or 8): after
// it, lane l holds the total of list entry (l % (2 N)) / 2. Every partner
// shares the bits already used, so each exchange adds disjoint lane sets.
template <int N>
__device__ __forceinline__ float reduce_scatter(float (&x)[N], int lane) {
  static_assert(N == 4 || N == 8, "a row or half-row of lanes");
  scatter_step<N>(x, lane);
  return x[0] + partner<1>(x[0]);
}

// Sum over the wave, in every lane: DPP inside rows, row broadcasts, then
// lane 63 (the rows the broadcasts leave out hold partial values).
__device__ __forceinline__ float wave_total(float v) {
  v += dpp_f<0xB1>(v, v);
  v += dpp_f<0x4E>(v, v);
  v += dpp_f<0x141>(v, v);
  v += dpp_f<0x140>(v, v);
  v += dpp_f<0x142, 0xA>(v, v);
  v += dpp_f<0x143, 0xC>(v, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// xo: GP * D floats and xml: 2 * GP floats of LDS, this workgroup's (two
// waves, 128 threads).
template <int D, int GP>
__device__ __forceinline__ void tier_parts(const AttnLaunch& a, int part, float* xo, float* xml) {
  constexpr int LPT = D / 8, TPI = 64 / LPT, NI = kTierTokens / TPI, NH = NI / 2;
  static_assert(NI == LPT && NH * 2 == LPT, "one token group per lane pair after the reduce-scatter");
  const kvc_cache_t& c = a.c;
  const int g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63, half = threadIdx.x >> 6;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.splits, P = a.parts;
  const long long span = attn_span(a);
  const bool app = a.k_new != nullptr;
  const int L_old = __builtin_amdgcn_readfirstlane(c.lengths[b]);
  const int L = max(0, __builtin_amdgcn_readfirstlane(min(min(L_old + (app ? 1 : 0), c.capacity), (int)span)));
  const int seen = __builtin_amdgcn_readfirstlane(c.num_seen[b]) + (app ? 1 : 0);
  const long long rowid = (long long)b * H + g;
  const int ns = min(c.fp16_sinks, L), nr = min(c.fp16_recent, L - ns), nt = ns + nr;
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
  if (new_here) {
    const int jn = L_old < ns ? L_old : (L_old >= L - nr ? ns + (L_old - (L - nr)) : -1);
    const int h0 = j0 + half * (kTierTokens / 2);
    if (jn >= h0 && jn < h0 + kTierTokens / 2 && lane < LPT) {
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

  const int r = lane / LPT, cc = lane % LPT;  // token within a load, 16-byte chunk of the row
  const int gi = cc >> 1;                     // group whose logit the lane holds after the reduce-scatter
  constexpr int NO = 8 * LPT / 64;  // channels a lane ends with after the row reduce-scatter
  for (int hp = 0; hp < G; hp += GP) {
    float qv[GP][8];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      // q is only 2-byte aligned: element loads
      const __half* qr = a.q + ((long long)b * Hq + g * G + min(hp + h, G - 1)) * D + cc * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[h][e] = hp + h < G ? __half2float(qr[e]) : 0.f;
    }
    // This wave's final state per head: max, sum, and NO channels of o.
    float m_fin[GP], l_fin[GP], o_fin[GP][NO];
    int off = 0;  // the lane's first channel within its 8-channel chunk (set by the row reduce-scatter)
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      m_fin[h] = -INFINITY;
      l_fin[h] = 0.f;
#pragma unroll
      for (int k = 0; k < NO; ++k) o_fin[h][k] = 0.f;
    }
    if (j0 + TPI * NH * half < nt) {  // uniform per wave: the half holds tier tokens
      u32x4 kx[NH], vx[NH];
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int j = j0 + TPI * (half * NH + i) + r;
        kx[i] = u32x4{0u, 0u, 0u, 0u};
        vx[i] = u32x4{0u, 0u, 0u, 0u};
        if (j < nt) {
          const long long off_j = row_off(j);
          const bool sink = j < ns;
          const __half* kr = off_j < 0 ? a.k_new + rowid * D : (sink ? k_sink : k_ring) + off_j;
          const __half* vr = off_j < 0 ? a.v_new + rowid * D : (sink ? v_sink : v_ring) + off_j;
          kx[i] = *reinterpret_cast<const u32x4*>(kr + cc * 8);
          vx[i] = *reinterpret_cast<const u32x4*>(vr + cc * 8);
        }
      }
      const int jt = j0 + TPI * (half * NH + gi) + r;  // the token whose logit this lane ends with
      const bool ok = jt < nt;
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (hp + h >= G) break;  // uniform
        float dv[NH];
#pragma unroll
        for (int i = 0; i < NH; ++i) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned uk = kx[i][e];  // a scalar first: a bit_cast of a vector element reads element 0
            const __half2 hk = __builtin_bit_cast(__half2, uk);
            d = fmaf(qv[h][2 * e], __low2float(hk), d);
            d = fmaf(qv[h][2 * e + 1], __high2float(hk), d);
          }
          dv[i] = d;
        }
        const float dsum = reduce_scatter<NH>(dv, cc);  // every lane takes part in the exchanges
        const float lg = ok ? dsum * a.qk_log2 : -INFINITY;
        if (a.logits && ok && !(cc & 1)) a.logits[((long long)b * Hq + g * G + hp + h) * span + slot_of(jt)] = lg;
        // The half holds at least one tier token, so m is finite.
        const float m = wave_max(lg);
        const float p = ok ? __builtin_amdgcn_exp2f(lg - m) : 0.f;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
        for (int i = 0; i < NH; ++i) {
          const float pi = __shfl(p, r * LPT + 2 * i);  // probability of this lane's token in group i
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned uv = vx[i][e];
            const __half2 hv = __builtin_bit_cast(__half2, uv);
            o[2 * e] = fmaf(pi, __low2float(hv), o[2 * e]);
            o[2 * e + 1] = fmaf(pi, __high2float(hv), o[2 * e + 1]);
          }
        }
        m_fin[h] = m;
        l_fin[h] = wave_total((cc & 1) ? 0.f : p);  // lane pairs hold each token twice
        // Sum the TPI token rows (lanes equal mod LPT) by a reduce-scatter
        // over the 8 channels: the lane keeps NO consecutive ones.
        off = 0;
#pragma unroll
        for (int s = LPT; s < 64; s <<= 1) {
          const int n = 4 * LPT / s;  // entries kept after this exchange
          const bool up = lane & s;
          off += up ? n : 0;
#pragma unroll
          for (int k = 0; k < n; ++k) {
            const float keep = up ? o[n + k] : o[k], give = up ? o[k] : o[n + k];
            o[k] = keep + __shfl_xor(give, s);
          }
        }
#pragma unroll
        for (int k = 0; k < NO; ++k) o_fin[h][k] = o[k];
      }
    } else {
      // The lane's channel offset is the same whichever wave computes it.
#pragma unroll
      for (int s = LPT; s < 64; s <<= 1) off += (lane & s) ? 4 * LPT / s : 0;
    }
    // The two halves meet: wave 1 hands its states to wave 0 through LDS.
    if (half == 1) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
#pragma unroll
        for (int k = 0; k < NO; ++k) xo[h * D + cc * 8 + off + k] = o_fin[h][k];
        if (lane == 0) {
          xml[2 * h] = m_fin[h];
          xml[2 * h + 1] = l_fin[h];
        }
      }
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (hp + h >= G) break;
        const float m1 = xml[2 * h], l1 = xml[2 * h + 1];
        const float M = fmaxf(m_fin[h], m1);
        const float w0 = m_fin[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_fin[h] - M);
        const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
        const long long pi = ((long long)b * Hq + g * G + hp + h) * P + S + part;
#pragma unroll
        for (int k = 0; k < NO; ++k)
          a.part_o[pi * D + cc * 8 + off + k] = o_fin[h][k] * w0 + xo[h * D + cc * 8 + off + k] * w1;
        if (lane == 0) {
          a.part_ml[pi * 2] = M;
          a.part_ml[pi * 2 + 1] = l_fin[h] * w0 + l1 * w1;
        }
      }
    }
    __syncthreads();  // xo is free for the next pass
  }
}

}  // namespace tier
}  // namespace kvc
