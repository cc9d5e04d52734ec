// Merging the splits of decode attention: the per-head softmax statistics
// and the H2O update, shared by the merge kernel and the eviction kernel that
// takes the merge over in a one-call decode step (same code, same results).
//
// Per head: m = max_s m_s, l = sum_s l_s * exp2(m_s - m); a split's weight in
// the output is exp2(m_s - m) / l and a token's probability is
// exp2(s_i - m) / l (logits in log2 units). H2O ("KV Cache Compression
// Report", section 3.4; eviction-and-reuse survey, section 3.3) adds the sum
// of the group's probabilities to the token's score.
#pragma once

#include "kvc_internal.h"

namespace kvc {
namespace merge {

__device__ __forceinline__ float exp2_or_zero(float x) {
  return x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x);
}

// Weight of a partial softmax state with max m_part inside a merged state with
// max m_total >= m_part; an empty part (m_part = -inf) weighs 0, also when the
// merged state is empty too.
__device__ __forceinline__ float part_weight(float m_part, float m_total) {
  return m_part == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_part - m_total);
}

// Split states of one head as a wave holds them: lane l has splits
// l + 64 r, r < kStatRegs, as loaded (a clamped split past S; split_stats
// masks them); splits past 64 * kStatRegs are read again by split_stats.
// Nothing here uses the loaded values, so a caller's later loads are not held
// behind these.
constexpr int kStatRegs = 4;
struct SplitML {
  float m[kStatRegs], l[kStatRegs];
};

__device__ __forceinline__ SplitML load_split_ml(const float* ml, int S) {
  const int lane = threadIdx.x & 63;
  SplitML r;
#pragma unroll
  for (int q = 0; q < kStatRegs; ++q) {
    const int sp = min(lane + 64 * q, S - 1);
    r.m[q] = ml[2 * sp];
    r.l[q] = ml[2 * sp + 1];
  }
  return r;
}

// Statistics of one head from its S split states ml[2 s] = m_s, ml[2 s + 1] =
// l_s (the first 64 * kStatRegs already in `r`), computed by one wave, lanes
// over the splits: the global max m and 1/l (0 for an empty head); fac[s] (may
// be NULL) receives each split's output weight exp2(m_s - m) / l. Each lane
// accumulates its splits in increasing order; padded entries add exactly 0.
__device__ __forceinline__ void split_stats(const SplitML& raw, const float* ml, int S, float* fac, float& m_out,
                                            float& inv_out) {
  const int lane = threadIdx.x & 63;
  SplitML r;  // m = -inf and l = 0 past S
#pragma unroll
  for (int q = 0; q < kStatRegs; ++q) {
    const bool in = lane + 64 * q < S;
    r.m[q] = in ? raw.m[q] : -INFINITY;
    r.l[q] = in ? raw.l[q] : 0.f;
  }
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < kStatRegs; ++q) m = fmaxf(m, r.m[q]);
  for (int sp = lane + 64 * kStatRegs; sp < S; sp += 64) m = fmaxf(m, ml[2 * sp]);
  m = wave_max(m);
  float l = 0.f, f[kStatRegs];
#pragma unroll
  for (int q = 0; q < kStatRegs; ++q) {
    f[q] = part_weight(r.m[q], m);
    l = fmaf(r.l[q], f[q], l);
  }
  for (int sp = lane + 64 * kStatRegs; sp < S; sp += 64) l = fmaf(ml[2 * sp + 1], part_weight(ml[2 * sp], m), l);
  l = wave_sum(l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (fac) {
#pragma unroll
    for (int q = 0; q < kStatRegs; ++q)
      if (lane + 64 * q < S) fac[lane + 64 * q] = f[q] * inv;
    for (int sp = lane + 64 * kStatRegs; sp < S; sp += 64) fac[sp] = part_weight(ml[2 * sp], m) * inv;
  }
  m_out = m;
  inv_out = inv;
}

// One H2O step of a fma chain over the heads: add + p_i, p_i the head's
// probability of a token with logit lg, from the head's (m, 1/l).
__device__ __forceinline__ float h2o_add(float add, float lg, float m, float inv) {
  return fmaf(exp2_or_zero(lg - m), inv, add);
}

}  // namespace merge
}  // namespace kvc
