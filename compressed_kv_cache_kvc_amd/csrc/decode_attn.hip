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
//    owns `tiles` consecutive 256-token tiles of one (sequence, KV head) and
//    serves the query heads that read that KV head (GQA), HC at a time;
//  * a token row (RB = D*bits/8 bytes) is read by LPT lanes, 16 bytes each for
//    INT8 and 8 bytes each for INT4 (16 elements per lane either way); a lane
//    group owns IT consecutive tokens of a tile, so each load is a full row
//    segment;
//  * loads are raw buffer loads: K and V share one 32-bit lane offset, the
//    bases sit in scalar registers, and reads past the sequence length return
//    zeros, so the ragged tail needs no branches;
//  * all K and V loads of a tile are issued before any arithmetic (64 KB in
//    flight per workgroup), and the kernel is shaped to keep 4 workgroups per
//    CU resident for the single-head case;
//  * q.k uses v_dot2_f32_f16 on codes turned into fp16 exactly (byte | 0x6400
//    is 1024 + byte; subtracting 1024 + the code bias recovers the code), so
//    the products are exact and only the fp32 sums round;
//  * each wave keeps its own online softmax (running max, sum, output) over
//    its tokens of every tile, so the tile loop has no barrier; the four waves
//    merge once at the end and the split writes (max, sum, o[D]);
//  * a second kernel merges the splits in a fixed order (deterministic).
// Logits are kept in log2 units (scaled by log2(e)) and exponentiated with exp2.
//
// H2O (report section 3.4; eviction-and-reuse survey section 3.3): with a
// score array, the split kernel also spills each logit; the merge kernel turns
// it into p_i = exp2(s_i - m) / l with the global (m, l) of its query head and
// adds the sum over the group's query heads to score[b][g][i].
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int TS = kSplitTokens;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

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

// Buffer resource word 3 for gfx9-family raw buffers (32-bit dword format).
constexpr int kBufferFlags = 0x00020000;

template <typename CT>
__device__ __forceinline__ CT load_chunk(__amdgpu_buffer_rsrc_t r, unsigned off) {
  if constexpr (sizeof(CT) == 16)
    return __builtin_bit_cast(CT, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  else
    return __builtin_bit_cast(CT, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of LPT consecutive lanes (LPT = 2, 4, 8 or 16), with
// DPP lane permutes: xor 1, xor 2, then the half-row and row mirrors.
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  if (LPT >= 2) v += dpp<0xB1>(v);
  if (LPT >= 4) v += dpp<0x4E>(v);
  if (LPT >= 8) v += dpp<0x141>(v);
  if (LPT >= 16) v += dpp<0x140>(v);
  return v;
}

// Sum (or max) over the lanes of a wave that share lane % LPT: DPP row
// rotations inside each 16-lane row, then cross-row exchanges.
template <int LPT, bool MAX>
__device__ __forceinline__ float stride_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  if (LPT <= 2) v = op(v, dpp<0x122>(v));
  if (LPT <= 4) v = op(v, dpp<0x124>(v));
  if (LPT <= 8) v = op(v, dpp<0x128>(v));
  v = op(v, __shfl_xor(v, 16));
  v = op(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float exp2_or_zero(float x) {
  return x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x);
}

// Weight of a partial softmax state with max m_part inside a merged state with
// max m_total >= m_part; an empty part (m_part = -inf) weighs 0, also when the
// merged state is empty too.
__device__ __forceinline__ float part_weight(float m_part, float m_total) {
  return m_part == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_part - m_total);
}

template <int BITS, int D, int HC, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HC == 1 ? 4 : 2)))
void attn_split_kernel(AttnLaunch a) {
  using CT = typename Chunk<BITS>::T;
  constexpr int RB = D * BITS / 8;
  constexpr int CB = (int)sizeof(CT);
  constexpr int EPL = 16;
  constexpr int NW = CB / 4;          // dwords per lane chunk
  constexpr int LPT = RB / CB;        // lanes per token
  constexpr int TPI = 64 / LPT;       // lane groups per wave
  constexpr int IT = 64 / TPI;        // tokens per lane group per tile
  static_assert(RB % CB == 0 && 64 % LPT == 0 && IT >= 1 && 16 % IT == 0, "layout");

  const kvc_cache_t& c = a.c;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPT, sub = lane - grp * LPT;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.splits, NT = a.tiles;
  const long long span = (long long)S * NT * TS;  // logit slots per query head
  // Uniform by construction; readfirstlane keeps it (and the buffer resources
  // built from it) in scalar registers.
  const int L = __builtin_amdgcn_readfirstlane(min(min(c.lengths[b], c.capacity), (int)span));

  __shared__ float red_m[4][HC];
  __shared__ float red_l[4][HC];
  __shared__ float red_o[4][HC][D];

  // Contiguous: one resource per (sequence, KV head) row limited to L tokens.
  // Paged: one resource over the whole pool (the host checks it is below
  // 4 GiB) and a block lookup per lane group; IT divides the block size, so a
  // group's IT tokens of a tile sit in one block.
  __amdgpu_buffer_rsrc_t rk, rv, rks, rvs;
  unsigned pool_rows = 0;
  if (PAGED) {
    pool_rows = (unsigned)c.num_blocks * H * c.block_size;
    rk = __builtin_amdgcn_make_buffer_rsrc(c.k_codes, 0, pool_rows * RB, kBufferFlags);
    rv = __builtin_amdgcn_make_buffer_rsrc(c.v_codes, 0, pool_rows * RB, kBufferFlags);
    rks = __builtin_amdgcn_make_buffer_rsrc(c.k_scale, 0, pool_rows * 4, kBufferFlags);
    rvs = __builtin_amdgcn_make_buffer_rsrc(c.v_scale, 0, pool_rows * 4, kBufferFlags);
  } else {
    const long long base = ((long long)b * H + g) * c.capacity;
    const unsigned valid = (unsigned)max(L, 0);
    rk = __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(c.k_codes) + base * RB, 0, valid * RB, kBufferFlags);
    rv = __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(c.v_codes) + base * RB, 0, valid * RB, kBufferFlags);
    rks = __builtin_amdgcn_make_buffer_rsrc(c.k_scale + base, 0, valid * 4, kBufferFlags);
    rvs = __builtin_amdgcn_make_buffer_rsrc(c.v_scale + base, 0, valid * 4, kBufferFlags);
  }
  const float qk_scale = a.qk_log2;

  for (int hc = 0; hc < G; hc += HC) {
    // ---- q slice for this lane's 16 elements, as fp16 pairs in code order ----
    half2_t qv[HC][8];
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      if (hc + i < G) {
        const __half* qh = a.q + ((long long)b * Hq + g * G + hc + i) * D + sub * EPL;
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

    float m_run[HC], l_run[HC], acc[HC][EPL];
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      m_run[i] = -INFINITY;
      l_run[i] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;
    }

    for (int tile = 0; tile < NT; ++tile) {
      const int tb = (s * NT + tile) * TS + wave * 64 + grp * IT;  // first token of this lane group
      const int nvalid = max(0, min(IT, L - tb));
      unsigned row;
      if (PAGED) {
        const long long r = nvalid > 0 ? cache_row(c, b, g, tb) : -1;
        row = r < 0 ? pool_rows : (unsigned)r;  // no block: every read returns zero
      } else {
        row = (unsigned)tb;
      }

      // ---- issue every load of the tile ----
      CT kr[IT], vr[IT];
      float ks[IT], vs[IT];
      const unsigned off = row * RB + sub * CB;
#pragma unroll
      for (int j = 0; j < IT; ++j) kr[j] = load_chunk<CT>(rk, off + j * RB);
#pragma unroll
      for (int j = 0; j < IT; ++j) vr[j] = load_chunk<CT>(rv, off + j * RB);
      // One dword per scale: each read is bounds-checked on its own.
#pragma unroll
      for (int j = 0; j < IT; ++j) {
        ks[j] = load_f32(rks, (row + j) * 4);
        vs[j] = load_f32(rvs, (row + j) * 4);
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
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) dot = __builtin_amdgcn_fdot2(kh[e], qv[i][e], dot, false);
          sl[i][j] = dot;
        }
      }
#pragma unroll
      for (int i = 0; i < HC; ++i)
#pragma unroll
        for (int j = 0; j < IT; ++j) {
          const float v = group_sum<LPT>(sl[i][j]);
          sl[i][j] = (j < nvalid) ? v * (ks[j] * qk_scale) : -INFINITY;
        }

      // ---- H2O: spill the logits ----
      if (a.logits != nullptr && sub == 0) {
#pragma unroll
        for (int i = 0; i < HC; ++i) {
          if (hc + i < G) {
            float* dst = a.logits + ((long long)b * Hq + g * G + hc + i) * span + tb;
#pragma unroll
            for (int j = 0; j < IT; ++j) dst[j] = sl[i][j];
          }
        }
      }

      // ---- online softmax, one running state per wave ----
#pragma unroll
      for (int i = 0; i < HC; ++i) {
        float mt = sl[i][0];
#pragma unroll
        for (int j = 1; j < IT; ++j) mt = fmaxf(mt, sl[i][j]);
        mt = stride_reduce<LPT, true>(mt);
        const float m_new = fmaxf(m_run[i], mt);
        const float corr = (m_new == -INFINITY) ? 1.f : exp2_or_zero(m_run[i] - m_new);
        m_run[i] = m_new;
        l_run[i] *= corr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[i][e] *= corr;
#pragma unroll
        for (int j = 0; j < IT; ++j) {
          const float p = (m_new == -INFINITY) ? 0.f : exp2_or_zero(sl[i][j] - m_new);
          sl[i][j] = p;
          l_run[i] += p;
        }
      }

      // ---- P.V over this lane's 16 elements ----
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
    }

    // ---- merge the lane groups of each wave, then the four waves ----
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      const float l = stride_reduce<LPT, false>(l_run[i]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = stride_reduce<LPT, false>(acc[i][e]);
      if (lane == 0) {
        red_m[wave][i] = m_run[i];
        red_l[wave][i] = l;
      }
      if (grp == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) red_o[wave][i][sub * EPL + e] = acc[i][e];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < HC * D; idx += 256) {
      const int i = idx / D, d = idx - i * D;
      if (hc + i < G) {
        const float M = fmaxf(fmaxf(red_m[0][i], red_m[1][i]), fmaxf(red_m[2][i], red_m[3][i]));
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) o = fmaf(red_o[w][i][d], part_weight(red_m[w][i], M), o);
        a.part_o[(((long long)b * Hq + g * G + hc + i) * S + s) * D + d] = o;
        if (d == 0) {
          float l = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) l = fmaf(red_l[w][i], part_weight(red_m[w][i], M), l);
          float* ml = a.part_ml + (((long long)b * Hq + g * G + hc + i) * S + s) * 2;
          ml[0] = M;
          ml[1] = l;
        }
      }
    }
    __syncthreads();
  }
}

// Merge the splits of the query heads of one (sequence, KV head).
//   blockIdx.x <  G : out[b][g*G + x][:]
//   blockIdx.x >= G : H2O update of score slots [k * 1024, (k + 1) * 1024),
//                     k = blockIdx.x - G
// Per head: m = max_s m_s, l = sum_s l_s * exp2(m_s - m); a split's weight in
// the output is exp2(m_s - m) / l and a token's probability is exp2(s_i - m) / l.
constexpr int kH2oChunk = 1024;
// GMAX: logits of up to GMAX heads are prefetched into registers; heads past
// GMAX (G > 8) are read after the statistics.
template <int D, int GMAX>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnLaunch a) {
  constexpr int kPrefetchHeads = GMAX;
  extern __shared__ float fac[];  // [heads][S] split weights, then [heads] m and 1/l
  const kvc_cache_t& c = a.c;
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.splits;
  const long long span = (long long)S * a.tiles * TS;
  const int L = __builtin_amdgcn_readfirstlane(min(min(c.lengths[b], c.capacity), (int)span));
  const bool out_block = x < G;
  const int h_lo = out_block ? x : 0, nh = out_block ? 1 : G;
  float* minv = fac + nh * S;  // [nh][2]: m, 1/l

  // H2O blocks: fetch the score slots and the first heads' logits before the
  // split statistics, so both memory round trips overlap.
  const int t0 = (x - G) * kH2oChunk + tid * 4;
  float sc[4] = {0.f, 0.f, 0.f, 0.f};
  float lg[kPrefetchHeads][4];
  float* srow = a.score ? a.score + ((long long)b * H + g) * c.capacity : nullptr;
  const float* lrow = a.logits + ((long long)b * Hq + g * G) * span;
  if (!out_block && srow) {
    // Unconditional loads from clamped slots, so that they are all in flight
    // together; slot 0 always exists, and values past L are never used.
    const int tl = max(L - 1, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) sc[k] = srow[min(t0 + k, tl)];
#pragma unroll
    for (int i = 0; i < kPrefetchHeads; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) lg[i][k] = lrow[min(i, G - 1) * span + min(t0 + k, tl)];
  }

  // Split statistics: one wave per head, lanes over the splits.
  for (int i = wave; i < nh; i += 4) {
    const float* ml = a.part_ml + ((long long)b * Hq + g * G + h_lo + i) * S * 2;
    float m = -INFINITY;
    for (int sp = lane; sp < S; sp += 64) m = fmaxf(m, ml[2 * sp]);
    m = wave_max(m);
    float l = 0.f;
    for (int sp = lane; sp < S; sp += 64) {
      const float f = part_weight(ml[2 * sp], m);
      fac[i * S + sp] = f;
      l = fmaf(ml[2 * sp + 1], f, l);
    }
    l = wave_sum(l);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int sp = lane; sp < S; sp += 64) fac[i * S + sp] *= inv;
    if (lane == 0) {
      minv[2 * i] = m;
      minv[2 * i + 1] = inv;
    }
  }
  __syncthreads();

  if (out_block) {
    // 256 / D threads per output element, each over every (256 / D)-th split.
    constexpr int PARTS = 256 / D;
    __shared__ float part[PARTS][D];
    const int d = tid % D, pi = tid / D;
    const int h = g * G + x;
    const float* po = a.part_o + ((long long)b * Hq + h) * S * D + d;
    float o = 0.f;
#pragma unroll 8
    for (int sp = pi; sp < S; sp += PARTS) o = fmaf(po[(long long)sp * D], fac[sp], o);
    part[pi][d] = o;
    __syncthreads();
    if (pi == 0) {
      float r = part[0][d];
#pragma unroll
      for (int p = 1; p < PARTS; ++p) r += part[p][d];
      a.out[((long long)b * Hq + h) * D + d] = r;
    }
    return;
  }
  if (!srow) return;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = t0 + k;
    if (t < L) {
      float add = 0.f;
#pragma unroll
      for (int i = 0; i < kPrefetchHeads; ++i)
        if (i < G) add = fmaf(exp2_or_zero(lg[i][k] - minv[2 * i]), minv[2 * i + 1], add);
      for (int i = kPrefetchHeads; i < G; ++i)
        add = fmaf(exp2_or_zero(lrow[i * span + t] - minv[2 * i]), minv[2 * i + 1], add);
      srow[t] = sc[k] + add;
    }
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

int attn_heads_per_pass(int G) { return G == 1 ? 1 : G == 2 ? 2 : 4; }

hipError_t launch_decode_attn(const AttnLaunch& a, hipStream_t st) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  hipError_t e;
  if (a.c.bits == 8)
    e = a.c.head_dim == 64 ? launch_paged<8, 64>(a, G, st) : launch_paged<8, 128>(a, G, st);
  else
    e = a.c.head_dim == 64 ? launch_paged<4, 64>(a, G, st) : launch_paged<4, 128>(a, G, st);
  if (e != hipSuccess) return e;
  const long long span = (long long)a.splits * a.tiles * TS;
  const int h2o_blocks = a.score ? (int)((span + kH2oChunk - 1) / kH2oChunk) : 0;
  const int nh = G;  // the H2O blocks need every head's statistics
  const size_t lds = (size_t)nh * (a.splits + 2) * sizeof(float);
  const dim3 grid(G + h2o_blocks, a.c.num_kv_heads, a.c.batch);
  const int gmax = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
#define KVC_COMBINE(DD, GG) \
  hipLaunchKernelGGL((attn_combine_kernel<DD, GG>), grid, dim3(256), lds, st, a)
  if (a.c.head_dim == 64) {
    if (gmax == 1) KVC_COMBINE(64, 1);
    else if (gmax == 2) KVC_COMBINE(64, 2);
    else if (gmax == 4) KVC_COMBINE(64, 4);
    else KVC_COMBINE(64, 8);
  } else {
    if (gmax == 1) KVC_COMBINE(128, 1);
    else if (gmax == 2) KVC_COMBINE(128, 2);
    else if (gmax == 4) KVC_COMBINE(128, 4);
    else KVC_COMBINE(128, 8);
  }
#undef KVC_COMBINE
  return hipGetLastError();
}

}  // namespace kvc
