// Per-token symmetric quantization of one K or V row by one wave, shared by
// the append kernels and the decode-attention kernel that appends the new
// token itself.
//
// One fp32 scale per (sequence, KV head, token) = max-abs over head_dim / qmax,
// codes = round-half-even(x / scale) clamped to the code range ("KV Cache
// optimization techniques" tutorial, section 1.2; INT4 constants from section
// 1.1; "KV Cache Compression Report", section 3.2). Both divisions are
// correctly rounded fp32 divisions and the rounding is v_rndne (half to
// even), so codes and scales are reproducible bit for bit. Each lane holds one
// fp16 pair of the row (two for D = 256); the max-abs is a DPP wave reduction.
#pragma once

#include "kvc_internal.h"

namespace kvc {
namespace quant {

template <int BITS>
__device__ __forceinline__ int encode(float x, float s) {
  constexpr float kMax = BITS == 8 ? 127.f : 7.f;
  constexpr float kMin = BITS == 8 ? -127.f : -8.f;
  if (s == 0.f) return 0;
  float t = rintf(__fdiv_rn(x, s));
  t = fminf(fmaxf(t, kMin), kMax);
  return (int)t;
}

template <int BITS>
__device__ __forceinline__ void store_pair(uint8_t* codes, int p, int c0, int c1) {
  if (BITS == 8) {
    const unsigned short w = (unsigned short)((c0 & 0xFF) | ((c1 & 0xFF) << 8));
    reinterpret_cast<unsigned short*>(codes)[p] = w;
  } else {
    codes[p] = (uint8_t)((c0 & 0xF) | ((c1 & 0xF) << 4));
  }
}

// The fp16 pair(s) of one row a lane owns: pair `lane` (and `lane + 64` when
// D = 256); lanes past the row's D/2 pairs hold zeros.
template <int D>
struct RowVals {
  float2 v[D > 128 ? 2 : 1];
};

template <int D>
__device__ __forceinline__ RowVals<D> load_row(const __half* __restrict__ x, int lane) {
  constexpr int P = D / 2;
  const __half2* x2 = reinterpret_cast<const __half2*>(x);
  RowVals<D> r;
#pragma unroll
  for (int k = 0; k < (D > 128 ? 2 : 1); ++k) {
    const int p = lane + 64 * k;
    const float2 f = __half22float2(x2[min(p, P - 1)]);
    r.v[k] = p < P ? f : make_float2(0.f, 0.f);
  }
  return r;
}

// Quantize a loaded row: wave-wide max-abs, the scale, then each lane's codes.
template <int BITS, int D>
__device__ __forceinline__ void quant_vals(const RowVals<D>& r, uint8_t* __restrict__ codes,
                                           float* __restrict__ scale_out, int lane) {
  constexpr float kQmax = BITS == 8 ? 127.f : 7.f;
  constexpr int P = D / 2;
  constexpr int K = D > 128 ? 2 : 1;
  float a = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) a = fmaxf(a, fmaxf(fabsf(r.v[k].x), fabsf(r.v[k].y)));
  a = wave_max(a);
  const float s = __fdiv_rn(a, kQmax);
  if (lane == 0) *scale_out = s;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int p = lane + 64 * k;
    if (p < P) store_pair<BITS>(codes, p, encode<BITS>(r.v[k].x, s), encode<BITS>(r.v[k].y, s));
  }
}

}  // namespace quant
}  // namespace kvc
