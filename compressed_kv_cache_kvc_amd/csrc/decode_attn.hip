// Single-query decode attention over an INT8/INT4 KV cache, dequantization fused.
//
// Computes softmax(q K^T / sqrt(D)) V ("KV Cache Compression Report", section
// 1.1) reading the quantized cache directly; a key or value is code * scale
// (section 3.2 of the report), and the scale is applied once per token
// instead of per element: s_i = (q . code_i) * scale_i / sqrt(D) and
// o = sum_i (p_i * scale_i) * code_i.
//
// Split-K (flash-decoding) layout for gfx950:
//  * grid (splits, KV heads, sequences); a 256-thread workgroup (4 waves of 64)
//    owns 256 consecutive tokens of one (sequence, KV head) and serves all G
//    query heads that read that KV head (GQA);
//  * a token row (RB = D*bits/8 bytes) is read by LPT lanes, 16 bytes each for
//    INT8 and 8 bytes each for INT4 (16 elements per lane either way), and a
//    lane group owns IT consecutive tokens, so every load is a full row
//    segment and the group's scales are one or two 16-byte loads;
//  * every K and V load of the workgroup is issued before any arithmetic:
//    64 KB in flight per workgroup hides HBM latency;
//  * q.k uses v_dot2_f32_f16 on codes turned into fp16 exactly (byte | 0x6400
//    is 1024 + byte; subtracting 1024 + bias recovers the code), so the products
//    are exact and only the fp32 sums round;
//  * the split's softmax is exact within the workgroup (all 256 logits are
//    held in registers), so no online rescaling is needed inside a split; the
//    split writes (max, sum, o[D]) and the combine kernel merges splits in a
//    fixed order (deterministic results).
// Logits are kept in log2 units (scaled by log2(e)) and exponentiated with exp2.
//
// H2O (report section 3.4; eviction-and-reuse survey section 3.3): with a
// score array, each split also spills exp2(s_i - m_split); the combine kernel
// turns it into p_i = exp2(s_i - m) / l with the global (m, l) and adds the
// sum over the group's query heads to score[b][g][i].
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int TS = kSplitTokens;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int BITS>
struct Chunk;
template <>
struct Chunk<8> {
  using T = u32x4;  // 16 bytes = 16 INT8 codes
};
template <>
struct Chunk<4> {
  using T = u32x2;  // 8 bytes = 16 INT4 codes
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(unsigned w) { return __builtin_bit_cast(half2_t, w); }

// 4 INT8 codes (one dword) -> two fp16 pairs holding the exact code values,
// element order (0,1) and (2,3).
__device__ __forceinline__ void i8x4_to_h2(unsigned w, half2_t& a, half2_t& b) {
  const unsigned u = w ^ 0x80808080u;  // code + 128 in each byte
  const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias;
  b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias;
}

// 8 INT4 codes (one dword) -> four fp16 pairs, element order (0,4) (1,5) (2,6) (3,7).
__device__ __forceinline__ void i4x8_to_h2(unsigned w, half2_t* o) {
  const unsigned u = w ^ 0x88888888u;  // code + 8 in each nibble
  const half2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = as_h2(((u >> (4 * k)) & 0x000F000Fu) | 0x64006400u) - bias;
}

template <int BITS>
__device__ __forceinline__ float code_at(const unsigned* w, int e) {
  if (BITS == 8) return (float)(signed char)(w[e >> 2] >> (8 * (e & 3)));
  return (float)((int)(w[e >> 3] << (28 - 4 * (e & 7))) >> 28);  // sign-extended nibble
}

template <int BITS, int D, int HC, bool PAGED>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnLaunch a) {
  using CT = typename Chunk<BITS>::T;
  constexpr int RB = D * BITS / 8;
  constexpr int CB = (int)sizeof(CT);
  constexpr int EPL = 16;
  constexpr int NW = CB / 4;          // dwords per lane chunk
  constexpr int LPT = RB / CB;        // lanes per token
  constexpr int TPI = 64 / LPT;       // lane groups per wave
  constexpr int IT = 64 / TPI;        // tokens per lane group
  static_assert(RB % CB == 0 && 64 % LPT == 0 && IT >= 1, "layout");

  const kvc_cache_t& c = a.c;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPT, sub = lane - grp * LPT;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.splits;
  const int L = min(min(c.lengths[b], c.capacity), S * TS);
  const int tb = s * TS + wave * 64 + grp * IT;  // first token of this lane group
  const int nvalid = max(0, min(IT, L - tb));

  __shared__ float red_m[4][HC];
  __shared__ float red_l[4][HC];
  __shared__ float red_o[4][HC][D];

  // ---- issue all loads of this lane's K/V chunks and the group's scales ----
  CT kr[IT], vr[IT];
  float ks[IT], vs[IT];
  long long row0 = -1;
  if (nvalid > 0) {
    if (PAGED) {
      row0 = cache_row(c, b, g, tb);  // IT divides the block size: the group stays in one block
    } else {
      row0 = ((long long)b * H + g) * c.capacity + tb;
    }
  }
  const CT* kp = reinterpret_cast<const CT*>(static_cast<const uint8_t*>(c.k_codes) + (row0 < 0 ? 0 : row0) * RB) + sub;
  const CT* vp = reinterpret_cast<const CT*>(static_cast<const uint8_t*>(c.v_codes) + (row0 < 0 ? 0 : row0) * RB) + sub;
  const float* ksp = c.k_scale + (row0 < 0 ? 0 : row0);
  const float* vsp = c.v_scale + (row0 < 0 ? 0 : row0);
  if (row0 >= 0 && nvalid == IT) {
#pragma unroll
    for (int j = 0; j < IT; ++j) kr[j] = __builtin_nontemporal_load(kp + j * (RB / CB));
#pragma unroll
    for (int j = 0; j < IT; ++j) vr[j] = __builtin_nontemporal_load(vp + j * (RB / CB));
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      ks[j] = ksp[j];
      vs[j] = vsp[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      const bool ok = row0 >= 0 && j < nvalid;
      kr[j] = ok ? kp[j * (RB / CB)] : CT{};
      vr[j] = ok ? vp[j * (RB / CB)] : CT{};
      ks[j] = ok ? ksp[j] : 0.f;
      vs[j] = ok ? vsp[j] : 0.f;
    }
  }

  const float qk_scale = a.qk_log2;
  for (int hc = 0; hc < G; hc += HC) {
    // ---- q slice for this lane's 16 elements, as fp16 pairs in code order ----
    half2_t qv[HC][8];
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      const int h = g * G + hc + i;
      if (hc + i < G) {
        const __half* qh = a.q + ((long long)b * Hq + h) * D + sub * EPL;
        const uint4 q0 = reinterpret_cast<const uint4*>(qh)[0];
        const uint4 q1 = reinterpret_cast<const uint4*>(qh)[1];
        const unsigned qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        if (BITS == 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) qv[i][e] = as_h2(qw[e]);
        } else {
          // INT4 pairs are (k, k+4) within each group of 8 elements.
#pragma unroll
          for (int w8 = 0; w8 < 2; ++w8)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const unsigned lo = (qw[w8 * 4 + (k >> 1)] >> (16 * (k & 1))) & 0xFFFFu;
              const unsigned hi = (qw[w8 * 4 + 2 + (k >> 1)] >> (16 * (k & 1))) & 0xFFFFu;
              qv[i][w8 * 4 + k] = as_h2(lo | (hi << 16));
            }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[i][e] = half2_t{};
      }
    }

    // ---- logits ----
    float sl[HC][IT];
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      const unsigned* w = reinterpret_cast<const unsigned*>(&kr[j]);
      half2_t kh[8];
      if (BITS == 8) {
#pragma unroll
        for (int d = 0; d < NW; ++d) i8x4_to_h2(w[d], kh[2 * d], kh[2 * d + 1]);
      } else {
#pragma unroll
        for (int d = 0; d < NW; ++d) i4x8_to_h2(w[d], kh + 4 * d);
      }
#pragma unroll
      for (int i = 0; i < HC; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_fdot2(kh[e], qv[i][e], acc, false);
        sl[i][j] = acc;
      }
    }
#pragma unroll
    for (int i = 0; i < HC; ++i)
#pragma unroll
      for (int j = 0; j < IT; ++j) {
        float v = sl[i][j];
#pragma unroll
        for (int o = 1; o < LPT; o <<= 1) v += __shfl_xor(v, o);
        sl[i][j] = (j < nvalid) ? v * (ks[j] * qk_scale) : -INFINITY;
      }

    // ---- split max and sum per head ----
    float mloc[HC];
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < IT; ++j) m = fmaxf(m, sl[i][j]);
#pragma unroll
      for (int o = LPT; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      mloc[i] = m;
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < HC; ++i) red_m[wave][i] = mloc[i];
    }
    __syncthreads();
    float msplit[HC], lsum[HC];
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      msplit[i] = fmaxf(fmaxf(red_m[0][i], red_m[1][i]), fmaxf(red_m[2][i], red_m[3][i]));
      float l = 0.f;
#pragma unroll
      for (int j = 0; j < IT; ++j) {
        const float p = (msplit[i] == -INFINITY) ? 0.f : exp2f(sl[i][j] - msplit[i]);
        sl[i][j] = p;
        l += p;
      }
#pragma unroll
      for (int o = LPT; o < 64; o <<= 1) l += __shfl_xor(l, o);
      lsum[i] = l;
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < HC; ++i) red_l[wave][i] = lsum[i];
    }

    // ---- H2O spill of exp2(s - m_split) ----
    if (a.pexp != nullptr && sub == 0) {
#pragma unroll
      for (int i = 0; i < HC; ++i) {
        if (hc + i < G) {
          float* dst = a.pexp + ((long long)b * Hq + g * G + hc + i) * ((long long)S * TS) + tb;
#pragma unroll
          for (int j = 0; j < IT; ++j) dst[j] = sl[i][j];
        }
      }
    }

    // ---- P.V over this lane's 16 elements ----
    float acc[HC][EPL];
#pragma unroll
    for (int i = 0; i < HC; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      const unsigned* w = reinterpret_cast<const unsigned*>(&vr[j]);
      float wt[HC];
#pragma unroll
      for (int i = 0; i < HC; ++i) wt[i] = sl[i][j] * vs[j];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float v = code_at<BITS>(w, e);
#pragma unroll
        for (int i = 0; i < HC; ++i) acc[i][e] = fmaf(wt[i], v, acc[i][e]);
      }
    }
#pragma unroll
    for (int i = 0; i < HC; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float v = acc[i][e];
#pragma unroll
        for (int o = LPT; o < 64; o <<= 1) v += __shfl_xor(v, o);
        acc[i][e] = v;
      }
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < HC; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) red_o[wave][i][sub * EPL + e] = acc[i][e];
    }
    __syncthreads();

    // ---- write this split's partials ----
    for (int idx = tid; idx < HC * D; idx += 256) {
      const int i = idx / D, d = idx - i * D;
      if (hc + i < G) {
        const int h = g * G + hc + i;
        const float o = red_o[0][i][d] + red_o[1][i][d] + red_o[2][i][d] + red_o[3][i][d];
        a.part_o[(((long long)b * Hq + h) * S + s) * D + d] = o;
      }
    }
    if (tid < HC && hc + tid < G) {
      const int h = g * G + hc + tid;
      float* ml = a.part_ml + (((long long)b * Hq + h) * S + s) * 2;
      ml[0] = msplit[tid];
      ml[1] = red_l[0][tid] + red_l[1][tid] + red_l[2][tid] + red_l[3][tid];
    }
    __syncthreads();
  }
}

// Merge the splits of every query head of one (sequence, KV head) and, with
// H2O, accumulate attention mass into the score row.
//   blockIdx.x == 0      : out[b][h][:] for the G heads of KV head g
//   blockIdx.x == 1 + k  : score slots [k * 1024, (k + 1) * 1024)
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnLaunch a) {
  extern __shared__ float fac[];  // [G][S]: exp2(m_s - m) / l
  const kvc_cache_t& c = a.c;
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.splits;
  const int L = min(min(c.lengths[b], c.capacity), S * TS);
  __shared__ float red[8];
  for (int i = 0; i < G; ++i) {
    const int h = g * G + i;
    const float* ml = a.part_ml + ((long long)b * Hq + h) * S * 2;
    float m = -INFINITY;
    for (int sp = tid; sp < S; sp += 256) m = fmaxf(m, ml[2 * sp]);
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float l = 0.f;
    for (int sp = tid; sp < S; sp += 256) {
      const float ms = ml[2 * sp];
      const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - m);
      fac[i * S + sp] = f;
      l += ml[2 * sp + 1] * f;
    }
    l = wave_sum(l);
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = l;
    __syncthreads();
    l = red[4] + red[5] + red[6] + red[7];
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    for (int sp = tid; sp < S; sp += 256) fac[i * S + sp] *= inv;
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    for (int idx = tid; idx < G * D; idx += 256) {
      const int i = idx / D, d = idx - i * D;
      const int h = g * G + i;
      const float* po = a.part_o + ((long long)b * Hq + h) * S * D + d;
      float o = 0.f;
      for (int sp = 0; sp < S; ++sp) o = fmaf(po[(long long)sp * D], fac[i * S + sp], o);
      a.out[((long long)b * Hq + h) * D + d] = o;
    }
    return;
  }
  if (a.score == nullptr) return;
  const int base = (blockIdx.x - 1) * 1024;
  float* srow = a.score + ((long long)b * H + g) * c.capacity;
  for (int t = base + tid; t < min(base + 1024, L); t += 256) {
    const int sp = t / TS;
    float sum = 0.f;
    for (int i = 0; i < G; ++i) {
      const float pe = a.pexp[((long long)b * Hq + g * G + i) * ((long long)S * TS) + t];
      sum = fmaf(pe, fac[i * S + sp], sum);
    }
    srow[t] += sum;
  }
}

template <int BITS, int D, int HC, bool PAGED>
hipError_t launch_split(const AttnLaunch& a, hipStream_t st) {
  hipLaunchKernelGGL((attn_split_kernel<BITS, D, HC, PAGED>), dim3(a.splits, a.c.num_kv_heads, a.c.batch),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int BITS, int D, bool PAGED>
hipError_t launch_hc(const AttnLaunch& a, int G, hipStream_t st) {
  if (G == 1) return launch_split<BITS, D, 1, PAGED>(a, st);
  if (G == 2) return launch_split<BITS, D, 2, PAGED>(a, st);
  return launch_split<BITS, D, 4, PAGED>(a, st);
}

template <int BITS, int D>
hipError_t launch_paged(const AttnLaunch& a, int G, hipStream_t st) {
  return a.c.block_size ? launch_hc<BITS, D, true>(a, G, st) : launch_hc<BITS, D, false>(a, G, st);
}

}  // namespace

hipError_t launch_decode_attn(const AttnLaunch& a, hipStream_t st) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  hipError_t e;
  if (a.c.bits == 8)
    e = a.c.head_dim == 64 ? launch_paged<8, 64>(a, G, st) : launch_paged<8, 128>(a, G, st);
  else
    e = a.c.head_dim == 64 ? launch_paged<4, 64>(a, G, st) : launch_paged<4, 128>(a, G, st);
  if (e != hipSuccess) return e;
  const int h2o_blocks = a.score ? (a.splits * TS + 1023) / 1024 : 0;
  const size_t lds = (size_t)G * a.splits * sizeof(float);
  if (a.c.head_dim == 64)
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(1 + h2o_blocks, a.c.num_kv_heads, a.c.batch), dim3(256),
                       lds, st, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(1 + h2o_blocks, a.c.num_kv_heads, a.c.batch), dim3(256),
                       lds, st, a);
  return hipGetLastError();
}

}  // namespace kvc
