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

// Statistics of one head from its S split states ml[2 s] = m_s, ml[2 s + 1] =
// l_s, computed by one wave (lanes over the splits): the global max m and
// 1/l (0 for an empty head); fac[s] (may be NULL) receives each split's
// output weight exp2(m_s - m) / l.
__device__ __forceinline__ void split_stats(const float* ml, int S, float* fac, float& m_out, float& inv_out) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  for (int sp = lane; sp < S; sp += 64) m = fmaxf(m, ml[2 * sp]);
  m = wave_max(m);
  float l = 0.f;
  for (int sp = lane; sp < S; sp += 64) {
    const float f = part_weight(ml[2 * sp], m);
    if (fac) fac[sp] = f;
    l = fmaf(ml[2 * sp + 1], f, l);
  }
  l = wave_sum(l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (fac)
    for (int sp = lane; sp < S; sp += 64) fac[sp] *= inv;
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
