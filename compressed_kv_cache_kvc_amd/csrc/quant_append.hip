// Quantize-on-write of new K/V tokens into the compressed cache, with the
// per-token symmetric quantizer of quant_row.h (one wave per row).
//
// Loads are unconditional (clamped addresses, masked values), so a wave's
// rows are all in flight at once.
#include "quant_row.h"

namespace kvc {
namespace {

using quant::load_row;
using quant::quant_vals;
using quant::RowVals;

// Decode-sized appends: one workgroup per sequence does every row of that
// sequence and then advances its length, so a single launch suffices. Each
// wave loads R rows (row indices clamped, so the loads are unconditional)
// before reducing any of them; the first batch is issued before the lengths
// are read, so one memory latency covers both.
template <int KBITS, int VBITS, int D>
__global__ __launch_bounds__(1024) void quant_append_seq_kernel(kvc_cache_t c, const __half* __restrict__ kn,
                                                                const __half* __restrict__ vn, int n_new,
                                                                float* __restrict__ score) {
  constexpr int R = 4;
  constexpr int RBK = D * KBITS / 8, RBV = D * VBITS / 8;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = c.num_kv_heads;
  const int rows = H * n_new * 2;
  RowVals<D> vals[R];
  auto load_batch = [&](int r0) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int r = min(r0 + 16 * q, rows - 1);
      const int kv = r & 1, ht = r >> 1, h = ht / n_new, t = ht - h * n_new;
      vals[q] = load_row<D>((kv ? vn : kn) + (((long long)b * H + h) * n_new + t) * D, lane);
    }
  };
  load_batch(wave);
  const int L0 = __builtin_amdgcn_readfirstlane(c.lengths[b]);
  const int seen = __builtin_amdgcn_readfirstlane(c.num_seen[b]);
  for (int r0 = wave; r0 < rows; r0 += 16 * R) {
    if (r0 != wave) load_batch(r0);
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int r = r0 + 16 * q;
      if (r >= rows) continue;
      const int kv = r & 1, ht = r >> 1, h = ht / n_new, t = ht - h * n_new;
      const long long row = cache_row(c, b, h, L0 + t);
      if (row < 0) continue;
      if (kv)  // uniform per wave: rows alternate K, V and a wave's rows differ by 16
        quant_vals<VBITS, D>(vals[q], static_cast<uint8_t*>(c.v_codes) + row * RBV, c.v_scale + row, lane);
      else
        quant_vals<KBITS, D>(vals[q], static_cast<uint8_t*>(c.k_codes) + row * RBK, c.k_scale + row, lane);
      if (kv == 0 && lane == 0) {
        if (c.positions) c.positions[row] = seen + t;
        if (score) score[((long long)b * H + h) * c.capacity + L0 + t] = 0.f;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    c.lengths[b] = L0 + n_new;
    c.num_seen[b] = seen + n_new;
  }
}

// Prefill-sized appends: every K row, then every V row, of the whole append
// as one flat list over the grid. A row of D fp16 values is D/8 lanes of 16
// bytes, so one wave instruction loads 64 / (D/8) consecutive rows (1 KB,
// contiguous); each wave keeps U such loads in flight. The max-abs is a DPP
// reduction over the row's lanes; each lane then quantizes its 8 values with
// correctly rounded quotients (one division per row, then three operations
// per value) and the rounding of quant_row.h (the codes are identical
// whichever kernel writes them) and stores them with one 8-byte
// (INT8) or 4-byte (INT4) store. The lengths advance in a second launch once
// every row has read them.
template <int D>
__device__ __forceinline__ float row_lanes_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v, v));   // quad: xor 1
  v = fmaxf(v, dpp_f<0x4E>(v, v));   // quad: xor 2
  v = fmaxf(v, dpp_f<0x141>(v, v));  // half-row mirror: 8 lanes
  if (D == 128) v = fmaxf(v, dpp_f<0x140>(v, v));  // row mirror: 16 lanes
  return v;
}

template <int KBITS, int VBITS, int D>
__global__ __launch_bounds__(256) void quant_append_bulk_kernel(kvc_cache_t c, const __half* __restrict__ kn,
                                                                const __half* __restrict__ vn, int n_new,
                                                                float* __restrict__ score, long long tokens) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int LPR = D / 8;     // lanes per row, 8 fp16 values each
  constexpr int RPI = 64 / LPR;  // rows per wave instruction
  constexpr int U = 4;           // loads in flight per wave
  const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
  // Row indices in 32 bits (the launcher takes this kernel only for fewer
  // than 2^31 rows): K rows [0, tokens), V rows [tokens, 2 tokens).
  const unsigned ntok = (unsigned)tokens, rows = 2u * ntok, nn = (unsigned)n_new, H = (unsigned)c.num_kv_heads;
  const unsigned nwaves = gridDim.x * 4u;
  for (unsigned r0 = (blockIdx.x * 4u + (threadIdx.x >> 6)) * (RPI * U); r0 < rows; r0 += nwaves * (RPI * U)) {
    // The rows' values, then their sequences' lengths and counts (clamped
    // rows, so every load is unconditional and all are in flight together).
    uint4 x[U];
    unsigned rtu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const unsigned r = min(r0 + u * RPI + sub, rows - 1);
      rtu[u] = r >= ntok ? r - ntok : r;  // (b, h, t) flattened
      x[u] = *reinterpret_cast<const uint4*>((r >= ntok ? vn : kn) + (size_t)rtu[u] * D + part * 8);
    }
    int len0[U], seen0[U], tt[U], hh[U], bb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const unsigned bh = rtu[u] / nn;
      tt[u] = (int)(rtu[u] - bh * nn);
      bb[u] = (int)(bh / H);
      hh[u] = (int)(bh - (unsigned)bb[u] * H);
      len0[u] = c.lengths[bb[u]];
      seen0[u] = c.num_seen[bb[u]];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const unsigned r = r0 + u * RPI + sub;
      const bool valid = r < rows, kv = r >= ntok;
      const int t = tt[u], h = hh[u], b = bb[u];
      const long long bh = (long long)b * H + h;
      const __half2* hv = reinterpret_cast<const __half2*>(&x[u]);
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 f = __half22float2(hv[i]);
        v[2 * i] = f.x;
        v[2 * i + 1] = f.y;
      }
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      amax = row_lanes_max<D>(amax);
      if (!valid) continue;
      const int bits = kv ? VBITS : KBITS;
      const float qmax = bits == 8 ? 127.f : 7.f, qmin = bits == 8 ? -127.f : -8.f;
      const float sc = __fdiv_rn(amax, qmax);
      // The row's quotients v / sc, correctly rounded, by Markstein's
      // correction of a product with the correctly rounded reciprocal: with
      // y = RN(1 / sc), q0 = RN(v y) and r = v - q0 sc (exact, by fma),
      // RN(q0 + r y) = RN(v / sc). tests/test_quotient_sequence.py checks this
      // for every fp16 v and every fp16 max-abs >= |v|, at both code widths,
      // so the codes equal those of quant_row.h's divisions.
      const float y = __fdiv_rn(1.f, sc);
      int code[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q0 = __fmul_rn(v[i], y);
        const float q1 = fmaf(fmaf(-q0, sc, v[i]), y, q0);
        const float q = sc == 0.f ? 0.f : rintf(q1);
        code[i] = (int)fminf(fmaxf(q, qmin), qmax);
      }
      const int L0 = len0[u];
      const long long row = cache_row(c, b, h, L0 + t);
      if (row < 0) continue;
      if (bits == 8) {
        unsigned w0 = 0, w1 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w0 |= (unsigned)(code[i] & 0xFF) << (8 * i);
          w1 |= (unsigned)(code[4 + i] & 0xFF) << (8 * i);
        }
        uint8_t* dst = static_cast<uint8_t*>(kv ? c.v_codes : c.k_codes) + row * D + part * 8;
        *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
      } else {
        unsigned w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= (unsigned)(code[i] & 0xF) << (4 * i);
        uint8_t* dst = static_cast<uint8_t*>(kv ? c.v_codes : c.k_codes) + row * (D / 2) + part * 4;
        *reinterpret_cast<unsigned*>(dst) = w;
      }
      if (part == 0) {
        (kv ? c.v_scale : c.k_scale)[row] = sc;
        if (!kv) {
          if (c.positions) c.positions[row] = seen0[u] + t;
          if (score) score[bh * c.capacity + L0 + t] = 0.f;
        }
      }
    }
  }
}

// Prefill-sized appends whose inputs or codes are not aligned for the bulk
// kernel, or of 2^31 rows or more: four rows per workgroup, one wave per row.
template <int KBITS, int VBITS, int D>
__global__ __launch_bounds__(256) void quant_append_rows_kernel(kvc_cache_t c, const __half* __restrict__ kn,
                                                                const __half* __restrict__ vn, int n_new,
                                                                float* __restrict__ score, long long total) {
  constexpr int RBK = D * KBITS / 8, RBV = D * VBITS / 8;
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= total) return;
  const int H = c.num_kv_heads;
  const int kv = (int)(r & 1);
  const long long rest = r >> 1;
  const int t = (int)(rest % n_new);
  const long long bh = rest / n_new;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const RowVals<D> vals = load_row<D>((kv ? vn : kn) + rest * D, lane);
  const int L0 = c.lengths[b];
  const long long row = cache_row(c, b, h, L0 + t);
  if (row < 0) return;
  if (kv)
    quant_vals<VBITS, D>(vals, static_cast<uint8_t*>(c.v_codes) + row * RBV, c.v_scale + row, lane);
  else
    quant_vals<KBITS, D>(vals, static_cast<uint8_t*>(c.k_codes) + row * RBK, c.k_scale + row, lane);
  if (kv == 0 && lane == 0) {
    if (c.positions) c.positions[row] = c.num_seen[b] + t;
    if (score) score[bh * c.capacity + L0 + t] = 0.f;
  }
}

__global__ void advance_lengths_kernel(int32_t* lengths, int32_t* num_seen, int B, int n) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    lengths[b] += n;
    num_seen[b] += n;
  }
}

template <int KBITS, int VBITS, int D>
hipError_t launch_bits(const kvc_cache_t& c, const __half* kn, const __half* vn, int n_new, float* score,
                       hipStream_t st) {
  const long long rows_per_seq = (long long)c.num_kv_heads * n_new * 2;
  if (rows_per_seq <= 256) {
    hipLaunchKernelGGL((quant_append_seq_kernel<KBITS, VBITS, D>), dim3(c.batch), dim3(1024), 0, st, c, kn, vn, n_new,
                       score);
    return hipGetLastError();
  }
  const long long tokens = (long long)c.batch * c.num_kv_heads * n_new;
  const uintptr_t align = (uintptr_t)kn | (uintptr_t)vn | (uintptr_t)c.k_codes | (uintptr_t)c.v_codes;
  if (align % 16 || 2 * tokens >= (1LL << 31)) {
    const long long total = rows_per_seq * c.batch;
    hipLaunchKernelGGL((quant_append_rows_kernel<KBITS, VBITS, D>), dim3((unsigned)((total + 3) / 4)), dim3(256), 0,
                       st, c, kn, vn, n_new, score, total);
  } else {
    // The bulk kernel: one pass of U loads per wave (2^31 rows make at most
    // 2^25 workgroups), so that no wave's loads wait behind its own earlier
    // stores, which gfx9 counts with them.
    const long long rows_per_wg = 4LL * (64 / (D / 8)) * 4;
    const long long blocks = std::max(1LL, (2 * tokens + rows_per_wg - 1) / rows_per_wg);
    hipLaunchKernelGGL((quant_append_bulk_kernel<KBITS, VBITS, D>), dim3((unsigned)blocks), dim3(256), 0, st, c, kn,
                       vn, n_new, score, tokens);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(advance_lengths_kernel, dim3((c.batch + 255) / 256), dim3(256), 0, st, c.lengths,
                     c.num_seen, c.batch, n_new);
  return hipGetLastError();
}

template <int KBITS, int VBITS>
hipError_t launch_dim(const kvc_cache_t& c, const __half* kn, const __half* vn, int n_new, float* score,
                      hipStream_t st) {
  return c.head_dim == 64 ? launch_bits<KBITS, VBITS, 64>(c, kn, vn, n_new, score, st)
                          : launch_bits<KBITS, VBITS, 128>(c, kn, vn, n_new, score, st);
}

}  // namespace

hipError_t launch_quant_append(const kvc_cache_t& c, const __half* kn, const __half* vn, int n_new,
                               float* score, hipStream_t st) {
  // fp16 tiers first: that kernel reads the lengths before this append.
  const hipError_t e = launch_tier_append(c, kn, vn, n_new, st);
  if (e != hipSuccess) return e;
  const int vb = vbits_of(c);
  if (c.bits == 8)
    return vb == 8 ? launch_dim<8, 8>(c, kn, vn, n_new, score, st) : launch_dim<8, 4>(c, kn, vn, n_new, score, st);
  return vb == 8 ? launch_dim<4, 8>(c, kn, vn, n_new, score, st) : launch_dim<4, 4>(c, kn, vn, n_new, score, st);
}

}  // namespace kvc
