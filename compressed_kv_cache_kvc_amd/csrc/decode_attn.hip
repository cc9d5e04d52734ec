// Single-query decode attention over an INT8/INT4 KV cache, dequantization fused.
//
// Computes softmax(q K^T / sqrt(D)) V ("KV Cache Compression Report", section
// 1.1) straight from the quantized cache. A key or value is code * scale
// (section 3.2 of the report), and the scale is applied once per token rather
// than per element: s_i = (q . code_i) * kscale_i / sqrt(D) and
// o = sum_i (p_i * vscale_i) * code_i.
//
// Both contractions run on the int8 matrix cores (v_mfma_i32_16x16x64_i8),
// with the cache codes as one operand, unconverted:
//  * q . code: q (fp16) is split per head into four int8 limbs,
//    q = 2^-E (a0 + a1/2^7 + a2/2^14 + a3/2^21), exact to 2^-27 of max|q|.
//    Rows of the A operand are (head, limb) pairs, the B operand is 16 tokens
//    x 64 codes read straight from HBM, and the integer sums are exact, so
//    the only roundings are the final combination of the four limb sums;
//  * p . V: the weights w_i = p_i * vscale_i of a 64-token block are split
//    into four limbs the same way (exponent from the block maximum; being
//    non-negative, as the base-128 digits of one integer), and V, staged in LDS, is read
//    transposed (ds_read_b64_tr_b8) so that each lane holds 16 tokens of one
//    channel, the layout of the B operand.
// INT4 codes are widened to bytes holding code + 8; the +8 is taken out of
// the integer sums (q side) or as 8 * sum(w) (V side).
//
// Split-K (flash-decoding) layout for gfx950:
//  * grid (splits, KV heads, sequences); a 256-thread workgroup owns `tiles`
//    256-token tiles of one (sequence, KV head) row (the last split may own a
//    few more, so the grid stays within one round of resident workgroups)
//    and serves every query head of that KV head (GQA), up to 8 per pass;
//  * each wave owns one 64-token block of every tile. It issues the block's
//    loads at once, raw buffer loads bounded by the cache capacity: scales,
//    then K codes (registers, in the B-operand layout), then V codes, which
//    INT8 caches move straight into the wave's LDS staging area (LDS DMA).
//    The first block's loads go out before the sequence length is known;
//    tokens past it are masked by selects;
//  * V rows are staged token-major with their 16-byte chunks XOR-swizzled per
//    row, so that every transposed read touches each LDS bank exactly twice;
//  * the online softmax keeps one token per lane, so exp2 runs once per
//    (head, token);
//  * the four waves merge once at the end and the split writes (max, sum,
//    o[D]); a second kernel merges the splits in a fixed order (deterministic).
// Logits are kept in log2 units (scaled by log2(e)) and exponentiated with exp2.
//
// fp16 tiers (report section 3.2: fp16 sinks; tutorial section 1.3: recent
// tokens at fp16): the split kernel masks the tier slots and skips the recent
// tier's blocks; attn_tier_kernel (tiers.h) adds them as extra partial states.
//
// H2O (report section 3.4; eviction-and-reuse survey section 3.3): with a
// score array, the split kernel also spills each logit; the merge kernel turns
// it into p_i = exp2(s_i - m) / l with the global (m, l) of its query head and
// adds the sum over the group's query heads to score[b][g][i].
#include <type_traits>

#include "kvc_internal.h"
#include "merge.h"
#include "quant_row.h"
#include "tiers.h"

namespace kvc {
namespace {

constexpr int TS = kSplitTokens;  // tokens per tile: 4 blocks of 64

// Waves per workgroup of the split kernel, by query heads per pass.
#ifndef KVC_SPLIT_WAVES
#define KVC_SPLIT_WAVES 4
#endif
template <int GP>
constexpr int kSplitWaves = GP == 1 ? KVC_SPLIT_WAVES : 4;
// 64-token blocks per chunk: a wave issues a chunk's loads together and takes
// one softmax rescale and one P.V limb combination per chunk (its blocks'
// integer P.V sums add up in the MFMA accumulators). Two for one head per pass
// on a contiguous cache (two waves per SIMD at the grid's size, so the second
// block's registers and staging area cost no occupancy), one otherwise.
template <int GP, bool PAGED, int NW>
constexpr int kChunk = 1;
// One head per pass on a contiguous cache: the grid holds two waves per SIMD,
// so the kernel may use 256 registers per lane at no cost in occupancy; it
// keeps the masked QK operands, issues a block's P.V MFMAs before reading
// any of their sums, and gives the wave merge its own LDS.
template <int GP, bool PAGED, int NW>
constexpr bool kLean = GP == 1 && !PAGED && NW == 4;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Buffer resource word 3 for gfx9-family raw buffers (32-bit dword format).
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ i32x4 load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ i32x2 load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ i32x4 mfma(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16 INT4 codes (8 bytes, element 2j in the low nibble of byte j) -> 16 bytes
// holding code + 8 (0..15). Byte i of the result holds element
// int4_elem(i): bytes 0-3 elements 0,2,4,6; 4-7 1,3,5,7; 8-11 8,10,12,14;
// 12-15 9,11,13,15.
__device__ __forceinline__ i32x4 widen_int4(i32x2 w) {
  const unsigned u0 = (unsigned)w[0] ^ 0x88888888u, u1 = (unsigned)w[1] ^ 0x88888888u;
  return i32x4{(int)(u0 & 0x0F0F0F0Fu), (int)((u0 >> 4) & 0x0F0F0F0Fu), (int)(u1 & 0x0F0F0F0Fu),
               (int)((u1 >> 4) & 0x0F0F0F0Fu)};
}
__device__ __forceinline__ int int4_elem(int i) { return (i & 8) | ((i & 3) << 1) | ((i >> 2) & 1); }
__device__ __forceinline__ int int4_byte(int e) { return (e & 8) | ((e & 1) << 2) | ((e >> 1) & 3); }

// a0 + a1 / 2^7 + a2 / 2^14 + a3 / 2^21 for the four limb sums of one MFMA
// output row group (each below 2^24 in magnitude, so exact in fp32).
__device__ __forceinline__ float limb_sum(i32x4 c) {
  float t = (float)c[3] * 0x1p-21f;
  t = fmaf((float)c[2], 0x1p-14f, t);
  t = fmaf((float)c[1], 0x1p-7f, t);
  return t + (float)c[0];
}

// Split y (|y| < 64) into four limbs: y = a0 + a1/2^7 + a2/2^14 + a3/2^21 + r,
// |r| <= 2^-22, each |a| <= 64. Every step is exact in fp32.
__device__ __forceinline__ void to_limbs(float y, int* l) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = rintf(y);
    l[k] = (int)a;
    y = (y - a) * 128.f;
  }
}

// The same for a non-negative y (< 64), given as y * 2^21: the limbs are the
// base-128 digits of n = RNE(y * 2^21), a0 = n >> 21 (at most 64) and a1..a3
// in [0, 127]. Their weighted sum n / 2^21 equals to_limbs' (which also
// rounds y to the nearest multiple of 2^-21, ties to even), in 6 operations
// instead of 16; only the split of n into digits differs.
__device__ __forceinline__ void to_limbs_nonneg(float y21, int* l) {
  const unsigned n = (unsigned)rintf(y21);
  l[0] = (int)(n >> 21);
  l[1] = (int)((n >> 14) & 127u);
  l[2] = (int)((n >> 7) & 127u);
  l[3] = (int)(n & 127u);
}

// Exponent E with max * 2^E in [32, 64): then every scaled value is below 64
// in magnitude and its leading limb fits the int8 range. 0 for max == 0.
__device__ __forceinline__ int limb_exponent(float mx) {
  int ex = 0;
  frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
  return mx > 0.f ? 6 - ex : 0;
}

template <bool MAX>
__device__ __forceinline__ float op2(float a, float b) {
  return MAX ? fmaxf(a, b) : a + b;
}

// Reduction over the lanes that hold one query head in the logit layout:
// all 64 lanes (GP = 1), lane rows r and r ^ 2 (GP = 2) or one 16-lane row
// (GP >= 4). Every lane receives the result of its head.
template <int GP, bool MAX>
__device__ __forceinline__ float head_reduce(float v) {
  v = op2<MAX>(v, dpp_f<0xB1>(v, v));
  v = op2<MAX>(v, dpp_f<0x4E>(v, v));
  v = op2<MAX>(v, dpp_f<0x141>(v, v));
  v = op2<MAX>(v, dpp_f<0x140>(v, v));
  if (GP == 1) {
    const float id = MAX ? v : 0.f;  // what the masked-off rows of a broadcast combine with
    v = op2<MAX>(v, dpp_f<0x142, 0xA>(id, v));
    v = op2<MAX>(v, dpp_f<0x143, 0xC>(id, v));
    v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  } else if (GP == 2) {
    v = op2<MAX>(v, __shfl_xor(v, 32));
  }
  return v;
}

using merge::exp2_or_zero;
using merge::part_weight;

__device__ __forceinline__ unsigned sel4(const unsigned* v, int i) {
  return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// GP: query heads served per pass, padded to 1, 2, 4 or 8.
//
// Logit layout of a 64-token block: NC = GP accumulators; lane l of
// accumulator c holds (head, token) = (j % GP, 16 * (j / GP) + l % 16) with
// j = 4c + l / 16, i.e. one token per lane for GP = 1 and one head per 16-lane
// row for GP >= 4. The PV output of row set rs holds head 4 rs + l / 16 (the
// same head as the lane's logits) and channel 16 m + l % 16 of block m.
//
// KBITS and VBITS: the K and V code widths (8 or 4), set apart so a cache can
// hold K and V at different precisions.
//
// FOLD (one-head contiguous kernel only): the first split's workgroups also
// compute a one-part fp16 tier (AttnLaunch::fold_tier); a separate instance,
// so the kernel without tiers keeps its code and registers.
template <int KBITS, int VBITS, int D, int GP, bool PAGED, int NW, bool FOLD = false>
__global__ __launch_bounds__(64 * NW) __attribute__((
    amdgpu_waves_per_eu(NW == 8 ? 4 : (kChunk<GP, PAGED, NW> == 2 || kLean<GP, PAGED, NW>) ? 2 : GP <= 2 ? 3 : 2)))
    void attn_split_kernel(AttnLaunch a) {
  constexpr int CH = kChunk<GP, PAGED, NW>;
  constexpr bool LEAN = kLean<GP, PAGED, NW>;
  constexpr int RBK = D * KBITS / 8;        // bytes per K token row in HBM
  constexpr int RBV = D * VBITS / 8;        // bytes per V token row in HBM
  constexpr int KB = KBITS == 8 ? 16 : 8;   // HBM bytes per lane per K load (16 elements)
  constexpr int VKB = VBITS == 8 ? 16 : 8;  // the same for V
  constexpr int NDH = D / 64;               // 64-element halves of a row (QK k = 64)
  constexpr int NCB = D / 16;               // 16-channel blocks (PV n = 16) = lanes per V row
  constexpr int TPV = 64 / NCB;             // tokens per V load instruction
  constexpr int NC = GP;                    // logit accumulators per block
  constexpr int NRS = GP > 4 ? GP / 4 : 1;  // PV row sets (4 heads each)
  constexpr int NQ = GP > 4 ? GP / 4 : 1;   // q limb rows held per lane (one per row set)
  constexpr int NSC = GP >= 4 ? 4 : GP;     // scale loads per block
  constexpr int VROW = D;                   // staged V row stride in LDS (chunks XOR-swizzled, see vchunk)
  // INT4 at D = 128: 16-byte loads, each lane taking two 16-element slices at
  // once (K: its slices of both 64-element halves, elements 32 quad + 16 dh +
  // 0..15; V: two adjacent 16-channel chunks of one token).
  constexpr bool K16 = KBITS == 4 && D == 128;
  constexpr bool V16 = VBITS == 4 && D == 128;
  static_assert(GP == 1 || GP == 2 || GP == 4 || GP == 8, "GP");
  static_assert(NW == 4 || NW == 8, "NW");
  // LDS chunk (16 bytes) of staged token row t that holds V chunk m: the XOR
  // makes the 64 lanes of a transposed read (tokens 16 q + 0..7 or 8..15 of
  // one chunk, q = 0..3) touch every LDS bank exactly twice.
  auto vchunk = [](int t, int m) -> int {
    return NCB == 8 ? (m ^ (((t >> 1) ^ ((t >> 4) << 2)) & 7)) : (m ^ (((t >> 2) ^ (t >> 4)) & 3));
  };

  const kvc_cache_t& c = a.c;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int quad = lane >> 4, col = lane & 15;
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.splits, NT = a.tiles;
  const long long span = attn_span(a);  // logit slots per query head
  const int NTs = s == S - 1 ? a.last_tiles : NT;  // tiles of this split
  const bool app = a.k_new != nullptr;
  // The sequence length is loaded first and used only once this wave's first
  // block of loads has gone out (below): loads return in order, so waiting
  // for it does not wait for the block, and no wave holds its cache reads
  // back for a dependent load (which, with the memory system full, takes as
  // long as the reads queued before it).
  const int len_raw = c.lengths[b];

  __shared__ __align__(16) uint8_t v_stage[CH][NW][64 * VROW];
  __shared__ __align__(16) int8_t w_limb[NW][CH][NRS][16][64];
  __shared__ __align__(16) int8_t q_limb[GP][4][D];
  __shared__ float q_fac[GP], q_off[GP];
  __shared__ float red_m[NW][GP], red_l[NW][GP];
  // The waves' partial outputs [NW][GP][D]: they reuse the staging area once
  // every wave is done with it, or have their own (no barrier before they are
  // written).
  constexpr bool OWN_RED = CH == 2 || LEAN;
  __shared__ float red_o_own[OWN_RED ? NW * GP * D : 1];
  float* red_o = OWN_RED ? red_o_own : reinterpret_cast<float*>(&v_stage[0][0][0]);
  static_assert(NW * GP * D * 4 <= NW * 64 * VROW, "merge buffer fits the staging area");

  // Contiguous: one resource per (sequence, KV head) row of `capacity` tokens;
  // rows past the capacity read 0. Paged: one resource over the whole pool
  // (the host checks it is below 4 GiB); a 16-token page of a missing block
  // maps past the end and reads 0. Neither depends on the sequence length, so
  // the first loads go out before it is known; slots in [L, capacity) hold
  // stale but finite codes, and every token past L is masked by selects.
  __amdgpu_buffer_rsrc_t rk, rv, rks, rvs;
  unsigned pool_rows = 0;
  if (PAGED) {
    pool_rows = (unsigned)c.num_blocks * H * c.block_size;
    rk = __builtin_amdgcn_make_buffer_rsrc(c.k_codes, 0, pool_rows * RBK, kBufferFlags);
    rv = __builtin_amdgcn_make_buffer_rsrc(c.v_codes, 0, pool_rows * RBV, kBufferFlags);
    rks = __builtin_amdgcn_make_buffer_rsrc(c.k_scale, 0, pool_rows * 4, kBufferFlags);
    rvs = __builtin_amdgcn_make_buffer_rsrc(c.v_scale, 0, pool_rows * 4, kBufferFlags);
  } else {
    const long long base = ((long long)b * H + g) * c.capacity;
    const unsigned valid = (unsigned)c.capacity;
    rk = __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(c.k_codes) + base * RBK, 0, valid * RBK,
                                           kBufferFlags);
    rv = __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(c.v_codes) + base * RBV, 0, valid * RBV,
                                           kBufferFlags);
    rks = __builtin_amdgcn_make_buffer_rsrc(c.k_scale + base, 0, valid * 4, kBufferFlags);
    rvs = __builtin_amdgcn_make_buffer_rsrc(c.v_scale + base, 0, valid * 4, kBufferFlags);
  }

  // This wave's blocks: the split's 64-token blocks j = NW it + wave (4 per
  // tile); block `it` starts at token t0(it) and holds tokens below L only
  // for it < nb.
  auto block_t0 = [&](int it) { return (s * NT * 4 + it * NW + wave) * 64; };
  // Registers of one block's loads (a chunk holds CH sets).
  using KT = typename std::conditional<KBITS == 8, i32x4, i32x2>::type;
  struct Regs {
    KT kq[4][NDH];
    i32x2 vq[VBITS == 8 ? 1 : NCB];  // V16: pairs (2 j, 2 j + 1) hold one 16-byte load
    float ksv[NSC], vsv[NSC];
  };
  // Issue every load of block `it`: K and V scales, then K codes into `r`,
  // then V codes (INT8: straight into this wave's LDS staging area `vs`,
  // swizzled; INT4: into `r`). Waiting for the scales and K (loads return in
  // order) does not wait for V. Rows of contiguous caches are tokens; paged
  // rows come from the block's four 16-token pages.
  auto issue = [&](Regs& r, int it, int vs) {
    // INT8 V: the lane-dependent offsets are recomputed at every issue (a few
    // adds) rather than kept live across the block loop, where at 8 heads per
    // pass they would be spilled to scratch.
    int lane = threadIdx.x & 63;
    if constexpr (VBITS == 8) asm volatile("" : "+v"(lane));
    const int quad = lane >> 4, col = lane & 15;
    unsigned pb[4];
    const int t0 = block_t0(it);
    if (PAGED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * i;
        const int blk = t < c.capacity ? c.block_table[(long long)b * c.max_blocks_per_seq + t / 16] : -1;
        pb[i] = __builtin_amdgcn_readfirstlane((unsigned)blk < (unsigned)c.num_blocks ? (unsigned)((blk * H + g) * 16)
                                                                                     : pool_rows);
      }
    }
    auto row_static = [&](int page, int t) -> unsigned {  // page known at compile time
      return PAGED ? pb[page] + (unsigned)(t & 15) : (unsigned)(t0 + t);
    };
#pragma unroll
    for (int si = 0; si < NSC; ++si) {
      const int t = GP >= 8 ? 16 * si + col : 16 * ((4 * si + quad) / GP) + col;
      const unsigned row = PAGED ? sel4(pb, t >> 4) + (unsigned)(t & 15) : (unsigned)(t0 + t);
      r.ksv[si] = load_f32(rks, row * 4);
      r.vsv[si] = load_f32(rvs, row * 4);
    }
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      if constexpr (K16) {
        const i32x4 w = load16(rk, row_static(tg, 16 * tg + col) * RBK + quad * 16);
        r.kq[tg][0] = i32x2{w[0], w[1]};
        r.kq[tg][1] = i32x2{w[2], w[3]};
      } else {
#pragma unroll
        for (int dh = 0; dh < NDH; ++dh) {
          const unsigned off = row_static(tg, 16 * tg + col) * RBK + dh * (RBK / NDH) + quad * KB;
          if constexpr (KBITS == 8) r.kq[tg][dh] = load16(rk, off); else r.kq[tg][dh] = load8(rk, off);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      // Lane l fills LDS chunk l % NCB of token row TPV j + l / NCB (DMA
      // writes lane l at 16 l), so it fetches the V chunk that belongs there.
      const int t = TPV * j + lane / NCB;
      if constexpr (VBITS == 8) {
        const unsigned off = row_static((TPV * j) >> 4, t) * RBV + vchunk(t, lane % NCB) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)&v_stage[vs][wave][j * 1024], 16, off, 0, 0, 0);
      } else if constexpr (V16) {
        // 4 lanes per token, 16 tokens per load: lane l takes chunks
        // 2 (l % 4) and 2 (l % 4) + 1 of token 16 (j / 2) + l / 4.
        if (j % 2 == 0) {
          const int tv = 16 * (j / 2) + lane / 4;
          const i32x4 w = load16(rv, row_static(j / 2, tv) * RBV + (lane % 4) * 16);
          r.vq[j] = i32x2{w[0], w[1]};
          r.vq[j + 1] = i32x2{w[2], w[3]};
        }
      } else {
        const unsigned off = row_static((TPV * j) >> 4, t) * RBV + (lane % NCB) * VKB;
        r.vq[j] = load8(rv, off);
      }
    }
  };

  // ---- q of a pass (wave w reads heads w, w + NW, ...), then the pass's
  // first block: q returns first, so the q setup waits for q alone ----
  constexpr int EPL = D / 64, HPW = (GP + NW - 1) / NW;
  // Raw fp16 bits, converted where used, so nothing waits for them here.
  unsigned short xq[HPW][EPL];
  const unsigned short* qbits = reinterpret_cast<const unsigned short*>(a.q);
  auto load_q = [&](int hp, int gh) {
#pragma unroll
    for (int hi = 0; hi < HPW; ++hi)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int h = wave + NW * hi;
        xq[hi][e] = qbits[((long long)b * Hq + g * G + hp + min(h, gh - 1)) * D + lane * EPL + e];
      }
  };
  Regs rg[CH];
  load_q(0, min(GP, G));
  issue(rg[0], 0, 0);  // block 0 of every wave exists; tokens past the length are masked

  // ---- the length (uniform; readfirstlane keeps it in scalar registers) ----
  // With an append, the new token is slot L_old and the attention covers it.
  const int L_old = __builtin_amdgcn_readfirstlane(len_raw);
  const int L = __builtin_amdgcn_readfirstlane(min(min(L_old + (app ? 1 : 0), c.capacity), (int)span));
  // fp16 tiers: slots [t_lo, t_hi) are read from the codes; the sink tier
  // below and the recent tier above are attended by attn_tier_kernel (their
  // logits are masked here and not spilled, and blocks past t_hi not read).
  // Without tiers t_lo = 0 and t_hi = L.
  const int t_lo = max(0, min(c.fp16_sinks, L));
  const int t_hi = L - max(0, min(c.fp16_recent, L - t_lo));
  const int blocks_hi = min(4 * NTs, (t_hi - s * NT * kSplitTokens + 63) / 64) - wave;
  const int nb = blocks_hi > 0 ? (blocks_hi + NW - 1) / NW : 0;

  // Append: the wave whose block `it_new` holds slot L_old quantizes the new
  // token's K and V rows into the cache (the quantizer of the append kernels,
  // so the codes are identical), sets its position and zeroes its score, then
  // waits for those stores; no other wave reads the slot, so no barrier is
  // needed. If the slot is in its block 0, whose loads went out before the
  // length was known, it loads that block again. Workgroup (0, 0) of each
  // sequence keeps the old length and count for the merge kernel (at the
  // end), which advances them once no workgroup reads them.
  if (app) {
    const int qb = L_old >> 6;           // 64-token block of the new slot
    const int jb = qb - s * NT * 4;      // its block index within this split
    if (L_old >= 0 && L_old < c.capacity && L_old < span && min((qb >> 2) / NT, S - 1) == s && jb % NW == wave) {
      const long long row = cache_row(c, b, g, L_old);
      if (row >= 0) {
        const long long src = ((long long)b * H + g) * D;
        const quant::RowVals<D> kx = quant::load_row<D>(a.k_new + src, lane);
        const quant::RowVals<D> vx = quant::load_row<D>(a.v_new + src, lane);
        quant::quant_vals<KBITS, D>(kx, static_cast<uint8_t*>(c.k_codes) + row * RBK, c.k_scale + row, lane);
        quant::quant_vals<VBITS, D>(vx, static_cast<uint8_t*>(c.v_codes) + row * RBV, c.v_scale + row, lane);
        if (lane == 0) {
          if (c.positions) c.positions[row] = c.num_seen[b];
          if (a.score) a.score[((long long)b * H + g) * c.capacity + L_old] = 0.f;
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores have completed (gfx9 counts them with loads)
      if (jb / NW == 0) issue(rg[0], 0, 0);
    }
  }

  for (int hp = 0; hp < G; hp += GP) {
    const int gh = min(GP, G - hp);  // real heads in this pass
    if (hp > 0) {
      load_q(hp, gh);
      issue(rg[0], 0, 0);
    }
#pragma unroll
    for (int cc = 1; cc < CH; ++cc)
      if (cc < nb) issue(rg[cc], cc, cc);
    // ---- q as int8 limbs, per head: wave w takes heads w, w + NW, ... ----
#pragma unroll
    for (int hi = 0; hi < HPW; ++hi) {
      const int h = wave + NW * hi;
      if (h >= GP) break;
      float x[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = h < gh ? __half2float(__ushort_as_half(xq[hi][e])) : 0.f;
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) mx = fmaxf(mx, fabsf(x[e]));
      mx = wave_max(mx);
      const int E = limb_exponent(mx);
      int lsum[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = lane * EPL + e;
        int lm[4];
        to_limbs(ldexpf(x[e], E), lm);
        // Position of element d in a limb row: the A operand of MFMA dh reads
        // bytes 64 dh + 16 quad .. + 15, which must hold the elements lane
        // group quad's K slice holds (INT4: in widened byte order).
        const int pos = KBITS == 8 ? d
                        : K16      ? ((d >> 4) & 1) * 64 + (d >> 5) * 16 + int4_byte(d & 15)
                                   : ((d & ~15) | int4_byte(d & 15));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          q_limb[h][k][pos] = (int8_t)lm[k];
          lsum[k] += lm[k];
        }
      }
      if (KBITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) lsum[k] = wave_sum_i(lsum[k]);
      }
      if (lane == 0) {
        q_fac[h] = mx > 0.f ? ldexpf(a.qk_log2, -E) : 0.f;
        // INT4: the codes enter as code + 8, so each limb sum carries 8 * sum(limb).
        q_off[h] = KBITS == 4 ? 8.f * ((float)lsum[0] + (float)lsum[1] * 0x1p-7f + (float)lsum[2] * 0x1p-14f +
                                      (float)lsum[3] * 0x1p-21f)
                             : 0.f;
      }
    }
    if (GP < 4) {  // limb rows of heads that do not exist stay zero
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) {
        int* z = reinterpret_cast<int*>(&w_limb[wave][cc][0][4 * GP][0]);
        for (int i = lane; i < (16 - 4 * GP) * 16; i += 64) z[i] = 0;
      }
    }
    __syncthreads();

    // ---- QK A operands: lane row 4 * slot + r holds limb r of one head ----
    // GP <= 4: the MFMA of token group tg uses slots tg % (4 / GP) * GP ...
    // + GP - 1 (head = slot % GP), the others are zero; GP = 8: row set rs
    // holds heads 4 rs + slot.
    const int slot = col >> 2;
    i32x4 qrow[NQ][NDH];
#pragma unroll
    for (int v = 0; v < NQ; ++v) {
      const int h = GP > 4 ? 4 * v + slot : slot % GP;
#pragma unroll
      for (int dh = 0; dh < NDH; ++dh)
        qrow[v][dh] = *reinterpret_cast<const i32x4*>(&q_limb[h][col & 3][dh * 64 + quad * 16]);
    }
    // GP < 4: the masked variants of the operand, built once and kept when
    // registers allow (LEAN), else rebuilt per use, which keeps 32 registers
    // free.
    constexpr int NVAR = GP < 4 ? 4 / GP : 1;
    constexpr bool KEEP_VAR = CH == 2 || LEAN;
    i32x4 qvar[KEEP_VAR ? NVAR : 1][NDH];
    if constexpr (KEEP_VAR) {
#pragma unroll
      for (int vi = 0; vi < NVAR; ++vi)
#pragma unroll
        for (int dh = 0; dh < NDH; ++dh) {
          const bool on = slot / GP == vi;
          const i32x4 q = qrow[0][dh];
          qvar[vi][dh] = i32x4{on ? q[0] : 0, on ? q[1] : 0, on ? q[2] : 0, on ? q[3] : 0};
        }
    }
    auto a_operand = [&](int tg, int v, int dh) -> i32x4 {
      if (GP >= 4) return qrow[v][dh];
      if constexpr (KEEP_VAR) return qvar[tg % NVAR][dh];
      const bool on = slot / GP == tg % NVAR;
      i32x4 q = qrow[0][dh];
      asm volatile("" : "+v"(q));  // rebuilt per use
      return i32x4{on ? q[0] : 0, on ? q[1] : 0, on ? q[2] : 0, on ? q[3] : 0};
    };
    float qf[NC], qo[NC];
    bool hv[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int h = (4 * cc + quad) % GP;
      qf[cc] = q_fac[h];
      qo[cc] = q_off[h];
      hv[cc] = h < gh;
    }

    float m_run[NRS], l_part[NRS], w_part[NRS], o_acc[NRS][NCB];
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
      m_run[rs] = -INFINITY;
      l_part[rs] = 0.f;
      w_part[rs] = 0.f;
#pragma unroll
      for (int m = 0; m < NCB; ++m) o_acc[rs][m] = 0.f;
    }

    // Logits of one 64-token block: int8 MFMA on raw K codes, scaled by the
    // token's K scale; tokens off the coded range get -inf. With H2O each
    // logit is spilled to its slot.
    auto logits = [&](Regs& r, int it, float* sv) {
      const int t0 = block_t0(it);
      i32x4 acc[NC], acc2[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) acc[cc] = acc2[cc] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int dh = 0; dh < NDH; ++dh) {
          i32x4 kb;
          if constexpr (KBITS == 8) kb = r.kq[tg][dh]; else kb = widen_int4(r.kq[tg][dh]);
          if (GP <= 4) {
            const int cc = tg * GP / 4;
            // Two accumulator chains (by half row) when one head is served,
            // so consecutive MFMAs do not wait for each other.
            if (GP == 1 && dh == 1) acc2[cc] = mfma(a_operand(tg, 0, dh), kb, acc2[cc]);
            else acc[cc] = mfma(a_operand(tg, 0, dh), kb, acc[cc]);
          } else {
#pragma unroll
            for (int rs = 0; rs < NRS; ++rs) acc[tg * NRS + rs] = mfma(a_operand(tg, rs, dh), kb, acc[tg * NRS + rs]);
          }
        }
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        if (GP == 1 && NDH > 1) acc[cc] = acc[cc] + acc2[cc];
        const int j = 4 * cc + quad, tok = 16 * (j / GP) + col;
        float x = (limb_sum(acc[cc]) - qo[cc]) * qf[cc] * r.ksv[GP >= 8 ? cc / 2 : cc];
        const int ti = t0 + tok;
        const bool coded = ti >= t_lo && ti < t_hi;
        if (!coded || !hv[cc]) x = -INFINITY;
        sv[cc] = x;
      }
    };
    // H2O: spill a block's logits (tier slots: their kernel). Issued after the
    // block's P.V, so the wait for the V loads does not also wait for them.
    auto spill = [&](int it, const float* sv) {
      if (a.logits == nullptr) return;
      int lane = threadIdx.x & 63;  // recomputed addresses, as in issue
      if constexpr (VBITS == 8) asm volatile("" : "+v"(lane));
      const int quad = lane >> 4, col = lane & 15;
      const int t0 = block_t0(it);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int j = 4 * cc + quad, ti = t0 + 16 * (j / GP) + col;
        const bool coded = ti >= t_lo && ti < t_hi;
        if (hv[cc] && (coded || ti >= L)) a.logits[((long long)b * Hq + g * G + hp + j % GP) * span + ti] = sv[cc];
      }
    };

    // One chunk of `ncur` blocks (ncur <= CH): logits, one online-softmax
    // step over the chunk, the weights as int8 limbs with one exponent per
    // chunk, then P.V with the blocks' integer sums added in the accumulators.
    auto process = [&](int it0, int ncur) {
      float sv[CH][NC];
#pragma unroll
      for (int ci = 0; ci < CH; ++ci) {
        if (ci < ncur) {
          logits(rg[ci], it0 + ci, sv[ci]);
        } else {
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) sv[ci][cc] = -INFINITY;
        }
      }

      // ---- online softmax, one running state per (wave, head) ----
      float corr[NRS], wscale[NRS];
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        float mb = -INFINITY;
#pragma unroll
        for (int ci = 0; ci < CH; ++ci)
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
            if ((GP >= 8 ? cc % NRS : 0) == rs) mb = fmaxf(mb, sv[ci][cc]);
        mb = head_reduce<GP, true>(mb);
        const float mn = fmaxf(m_run[rs], mb);
        corr[rs] = m_run[rs] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rs] - mn);
        m_run[rs] = mn;
        l_part[rs] *= corr[rs];
        w_part[rs] *= corr[rs];
      }
      float wv[CH][NC];
#pragma unroll
      for (int ci = 0; ci < CH; ++ci)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          const int rs = GP >= 8 ? cc % NRS : 0;
          const float p = sv[ci][cc] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[ci][cc] - m_run[rs]);
          l_part[rs] += p;
          // a masked slot's scale may be stale
          wv[ci][cc] = sv[ci][cc] == -INFINITY ? 0.f : p * rg[ci].vsv[GP >= 8 ? cc / 2 : cc];
          w_part[rs] += wv[ci][cc];
        }

      // ---- weights as int8 limbs, rows (head, limb) x 64 tokens, in LDS ----
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        float wm = 0.f;
#pragma unroll
        for (int ci = 0; ci < CH; ++ci)
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
            if ((GP >= 8 ? cc % NRS : 0) == rs) wm = fmaxf(wm, wv[ci][cc]);
        wm = head_reduce<GP, true>(wm);
        const int E = limb_exponent(wm);
        wscale[rs] = ldexpf(1.f, -E);
#pragma unroll
        for (int ci = 0; ci < CH; ++ci) {
          if (ci >= ncur) continue;
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) {
            if ((GP >= 8 ? cc % NRS : 0) != rs) continue;
            const int j = 4 * cc + quad, h = j % GP, tok = 16 * (j / GP) + col;
            int lm[4];
            to_limbs_nonneg(ldexpf(wv[ci][cc], E + 21), lm);  // weights are >= 0
#pragma unroll
            for (int k = 0; k < 4; ++k) w_limb[wave][ci][rs][4 * (h & 3) + k][tok] = (int8_t)lm[k];
          }
        }
      }
      // ---- V rows in LDS: INT8 came by DMA; INT4 is widened here ----
      if constexpr (VBITS == 4) {
#pragma unroll
        for (int ci = 0; ci < CH; ++ci) {
          if (ci >= ncur) continue;
#pragma unroll
          for (int j = 0; j < NCB; ++j) {
            const int t = V16 ? 16 * (j / 2) + lane / 4 : TPV * j + lane / NCB;
            const int m = V16 ? 2 * (lane % 4) + (j % 2) : lane % NCB;
            const i32x4 val = widen_int4(rg[ci].vq[j]);
            i32x2* dst = reinterpret_cast<i32x2*>(&v_stage[ci][wave][t * VROW + vchunk(t, m) * 16]);
            dst[0] = i32x2{val[0], val[1]};
            dst[1] = i32x2{val[2], val[3]};
          }
        }
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the V DMA of this chunk has landed
      }
      asm volatile("" ::: "memory");

      // ---- p . V: A = weight limbs, B = V transposed by ds_read_b64_tr_b8 ----
      // Within each 16-lane group, source lane 2b + h reads token 16 quad + b
      // (+ 8), channels 8h..8h+7 of the block; lane col then holds channel col
      // of those 8 tokens.
      const int tr_row = quad * 16 + (col >> 1), tr_col = (col & 1) * 8;
      i32x4 aw[NRS][CH];
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs)
#pragma unroll
        for (int ci = 0; ci < CH; ++ci)
          aw[rs][ci] = *reinterpret_cast<const i32x4*>(&w_limb[wave][ci][rs][col][quad * 16]);
      // Each channel block's V is read once and serves every row set. LEAN:
      // every channel block's MFMA is issued before the first sum is read, so
      // no MFMA result is waited for right after its issue.
      constexpr int NPV = LEAN ? NCB : 1;
      i32x4 pvs[NPV];
#pragma unroll
      for (int m = 0; m < NCB; ++m) {
        i32x4 pv[NRS];
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) pv[rs] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int ci = 0; ci < CH; ++ci) {
          if (ci >= ncur) continue;
          uint8_t* p0 = &v_stage[ci][wave][tr_row * VROW + vchunk(tr_row, m) * 16 + tr_col];
          uint8_t* p1 = &v_stage[ci][wave][(tr_row + 8) * VROW + vchunk(tr_row + 8, m) * 16 + tr_col];
          const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p0);
          const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p1);
          const i32x4 vb = i32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int rs = 0; rs < NRS; ++rs) pv[rs] = mfma(aw[rs][ci], vb, pv[rs]);
        }
        if constexpr (LEAN) {
          pvs[m] = pv[0];
        } else {
#pragma unroll
          for (int rs = 0; rs < NRS; ++rs) o_acc[rs][m] = fmaf(o_acc[rs][m], corr[rs], wscale[rs] * limb_sum(pv[rs]));
        }
      }
      if constexpr (LEAN) {
#pragma unroll
        for (int m = 0; m < NCB; ++m) o_acc[0][m] = fmaf(o_acc[0][m], corr[0], wscale[0] * limb_sum(pvs[m]));
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int ci = 0; ci < CH; ++ci)
        if (ci < ncur) spill(it0 + ci, sv[ci]);
    };
    for (int it0 = 0; it0 < nb; it0 += CH) {
      const int ncur = min(CH, nb - it0);
      if (it0 > 0) {
#pragma unroll
        for (int ci = 0; ci < CH; ++ci)
          if (ci < ncur) issue(rg[ci], it0 + ci, ci);
      }
      process(it0, ncur);
    }

    // ---- merge the waves ----
    // A wave with no block of this split still issued block 0's loads (some
    // into the staging area): they complete before any LDS is reused.
    if (nb == 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    float l_tot[NRS], w_tot[NRS];
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
      l_tot[rs] = head_reduce<GP, false>(l_part[rs]);
      w_tot[rs] = VBITS == 4 ? head_reduce<GP, false>(w_part[rs]) : 0.f;
    }
    if (!OWN_RED) __syncthreads();  // every wave is done with v_stage, which red_o reuses
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
      const int hh = (GP >= 8 ? 4 * rs : 0) + quad;  // head of this lane's PV rows
      if (quad < (GP < 4 ? GP : 4) && hh < gh) {
        if (col == 0) {
          red_m[wave][hh] = m_run[rs];
          red_l[wave][hh] = l_tot[rs];
        }
#pragma unroll
        for (int m = 0; m < NCB; ++m) {
          const int ch = m * 16 + (VBITS == 8 ? col : int4_elem(col));
          red_o[(wave * GP + hh) * D + ch] = o_acc[rs][m] - 8.f * w_tot[rs];
        }
      }
    }
    __syncthreads();
    for (int idx = tid; idx < gh * D; idx += 64 * NW) {
      const int i = idx / D, d = idx - i * D;
      float M = red_m[0][i];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, red_m[w][i]);
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o = fmaf(red_o[(w * GP + i) * D + d], part_weight(red_m[w][i], M), o);
      const long long hq = (long long)b * Hq + g * G + hp + i;
      a.part_o[(hq * a.parts + s) * D + d] = o;
      if (d == 0) {
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) l = fmaf(red_l[w][i], part_weight(red_m[w][i], M), l);
        a.part_ml[(hq * a.parts + s) * 2] = M;
        a.part_ml[(hq * a.parts + s) * 2 + 1] = l;
      }
    }
    if (hp + GP < G) __syncthreads();  // the next pass rewrites the LDS this one read
  }
  // A one-part fp16 tier: the first split's workgroup adds it after its own
  // work (tiers.h; a workgroup of this kernel's waves runs it as two working
  // waves and idle ones, all reaching its barriers). Its exchange area is the
  // staging area, free now: every DMA into it has been waited for, and the
  // barrier below orders the last reads of it before the first writes.
  // Only in the one-head contiguous kernel, which has registers to spare at
  // two waves per SIMD: elsewhere the tier code's registers would raise the
  // kernel's (those launches keep the tier kernel).
  static_assert(!FOLD || LEAN, "the tier is folded into the one-head contiguous kernel only");
  if constexpr (FOLD) if (s == 0) {
    constexpr int TGT = 1;  // the tier launch's query heads per pass at one head
    static_assert(TGT * D * 4 <= CH * NW * 64 * VROW, "the tier's exchange fits the staging area");
    __shared__ float tier_ml[2 * TGT];
    __syncthreads();
    tier::tier_parts<D, TGT>(a, 0, reinterpret_cast<float*>(&v_stage[0][0][0]), tier_ml);
  }
  if (app && s == 0 && g == 0 && tid == 0) {
    a.stash[b] = L_old;
    a.stash[c.batch + b] = c.num_seen[b];
  }
  // Control words of a later in-place eviction in the same step: cleared
  // last, after every load this workgroup waits for.
  if (a.zero_count) {
    const long long nthreads = (long long)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
    const long long flat =
        ((long long)(blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    for (long long i = flat; i < a.zero_count; i += nthreads) a.zero_words[i] = 0;
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
  constexpr int PARTS = 256 / D;  // threads per output element
  constexpr int kPre = 8;         // split partials per thread read before the statistics
  extern __shared__ float fac[];  // [heads][S] split weights, then [heads] m and 1/l
  const kvc_cache_t& c = a.c;
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // S: the partial states per head (the splits and the fp16-tier parts).
  const int H = c.num_kv_heads, Hq = a.num_q_heads, G = Hq / H, S = a.parts;
  const long long span = attn_span(a);
  // With an append, the length before it comes from the split kernel (the
  // cache's own length is advanced here, by one workgroup).
  const bool app = a.append != 0;
  // The length is used last (H2O blocks): loaded now, read after the loads
  // below have gone out.
  const int len_raw = app ? a.stash[b] + 1 : c.lengths[b];
  const bool out_block = x < G;
  const int h_lo = out_block ? x : 0, nh = out_block ? 1 : G;
  float* minv = fac + nh * S;  // [nh][2]: m, 1/l

  // Every read below comes from a clamped, always valid address and does not
  // wait for the sequence length or the statistics, so all of them are in
  // flight together; values past L are never used.
  const int tl = (int)min(span, (long long)c.capacity) - 1;
  const int t0 = (x - G) * kH2oChunk + tid * 4;
  float sc[4] = {0.f, 0.f, 0.f, 0.f};
  float lg[kPrefetchHeads][4];
  float* srow = a.score ? a.score + ((long long)b * H + g) * c.capacity : nullptr;
  const float* lrow = a.logits + ((long long)b * Hq + g * G) * span;
  if (!out_block && srow) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sc[k] = srow[min(t0 + k, tl)];
    // A logit row is span floats (a multiple of 256) in a 256-byte aligned
    // workspace, so a thread's 4 slots are one 16-byte load; a chunk past the
    // row reads the row's last 4 slots instead (slots past L are not used).
    const long long t4 = min((long long)t0, span - 4);
#pragma unroll
    for (int i = 0; i < kPrefetchHeads; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(lrow + min(i, G - 1) * span + t4);
      lg[i][0] = v.x;
      lg[i][1] = v.y;
      lg[i][2] = v.z;
      lg[i][3] = v.w;
    }
  }
  const int d = tid % D, pi = tid / D;
  const float* po = a.part_o + ((long long)b * Hq + g * G + h_lo) * S * D + d;
  float pre[kPre];
  if (out_block) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) pre[k] = po[(long long)min(pi + k * PARTS, S - 1) * D];
  }

  // Split statistics: one wave per head, lanes over the splits.
  for (int i = wave; i < nh; i += 4) {
    const float* ml = a.part_ml + ((long long)b * Hq + g * G + h_lo + i) * S * 2;
    float m, inv;
    merge::split_stats(merge::load_split_ml(ml, S), ml, S, fac + i * S, m, inv);
    if (lane == 0) {
      minv[2 * i] = m;
      minv[2 * i + 1] = inv;
    }
  }
  __syncthreads();

  if (out_block) {
    // PARTS threads per output element, each over every PARTS-th split.
    __shared__ float part[PARTS][D];
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < kPre; ++k)
      if (pi + k * PARTS < S) o = fmaf(pre[k], fac[pi + k * PARTS], o);
    for (int sp = pi + kPre * PARTS; sp < S; sp += PARTS) o = fmaf(po[(long long)sp * D], fac[sp], o);
    part[pi][d] = o;
    __syncthreads();
    if (pi == 0) {
      float r = part[0][d];
#pragma unroll
      for (int p = 1; p < PARTS; ++p) r += part[p][d];
      a.out[((long long)b * Hq + g * G + x) * D + d] = r;
    }
    if (app && x == 0 && g == 0 && tid == 0) {
      c.lengths[b] = a.stash[b] + 1;
      c.num_seen[b] = a.stash[c.batch + b] + 1;
    }
    return;
  }
  if (!srow) return;
  const int L = __builtin_amdgcn_readfirstlane(min(min(len_raw, c.capacity), (int)span));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = t0 + k;
    if (t < L) {
      float add = 0.f;
#pragma unroll
      for (int i = 0; i < kPrefetchHeads; ++i)
        if (i < G) add = merge::h2o_add(add, lg[i][k], minv[2 * i], minv[2 * i + 1]);
      for (int i = kPrefetchHeads; i < G; ++i) add = merge::h2o_add(add, lrow[i * span + t], minv[2 * i], minv[2 * i + 1]);
      srow[t] = sc[k] + add;
    }
  }
}

// Attention over the fp16 tiers (tiers.h): the two waves of workgroup x make
// part S + x of each query head, GT heads per pass.
template <int D, int GT>
__global__ __launch_bounds__(128) void attn_tier_kernel(AttnLaunch a) {
  __shared__ float xo[GT * D], xml[2 * GT];
  tier::tier_parts<D, GT>(a, blockIdx.x, xo, xml);
}

template <int KBITS, int VBITS, int D, int GP, bool PAGED>
hipError_t launch_split(const AttnLaunch& a, hipStream_t st) {
  constexpr int NW = kSplitWaves<GP>;
  if constexpr (kLean<GP, PAGED, NW>) {
    if (a.fold_tier) {
      hipLaunchKernelGGL((attn_split_kernel<KBITS, VBITS, D, GP, PAGED, NW, true>),
                         dim3(a.splits, a.c.num_kv_heads, a.c.batch), dim3(64 * NW), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_split_kernel<KBITS, VBITS, D, GP, PAGED, NW>), dim3(a.splits, a.c.num_kv_heads, a.c.batch),
                     dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

template <int KBITS, int VBITS, int D, bool PAGED>
hipError_t launch_gp(const AttnLaunch& a, int G, hipStream_t st) {
  if (G == 1) return launch_split<KBITS, VBITS, D, 1, PAGED>(a, st);
  if (G == 2) return launch_split<KBITS, VBITS, D, 2, PAGED>(a, st);
  if (G <= 4) return launch_split<KBITS, VBITS, D, 4, PAGED>(a, st);
  return launch_split<KBITS, VBITS, D, 8, PAGED>(a, st);  // more than 8: passes of 8
}

template <int KBITS, int VBITS, int D>
hipError_t launch_paged(const AttnLaunch& a, int G, hipStream_t st) {
  return a.c.block_size ? launch_gp<KBITS, VBITS, D, true>(a, G, st) : launch_gp<KBITS, VBITS, D, false>(a, G, st);
}

template <int KBITS, int VBITS>
hipError_t launch_dim(const AttnLaunch& a, int G, hipStream_t st) {
  return a.c.head_dim == 64 ? launch_paged<KBITS, VBITS, 64>(a, G, st) : launch_paged<KBITS, VBITS, 128>(a, G, st);
}

}  // namespace

hipError_t launch_attn_split(const AttnLaunch& a0, hipStream_t st) {
  // The tier is folded only where the one-head contiguous kernel has the
  // folding instance (four waves per workgroup); otherwise the tier kernel runs.
  AttnLaunch a = a0;
  a.fold_tier = a0.fold_tier && kLean<1, false, kSplitWaves<1>>;
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const int vb = vbits_of(a.c);
  hipError_t e;
  if (a.c.bits == 8) e = vb == 8 ? launch_dim<8, 8>(a, G, st) : launch_dim<8, 4>(a, G, st);
  else e = vb == 8 ? launch_dim<4, 8>(a, G, st) : launch_dim<4, 4>(a, G, st);
  if (e != hipSuccess || a.tier_parts <= 0 || a.fold_tier) return e;
  // The fp16 tiers: one two-wave workgroup per part, right after the splits.
  const dim3 grid(a.tier_parts, a.c.num_kv_heads, a.c.batch);
  const int gt = G == 1 ? 1 : G == 2 ? 2 : 4;
#define KVC_TIER(DD, GG) hipLaunchKernelGGL((attn_tier_kernel<DD, GG>), grid, dim3(128), 0, st, a)
  if (a.c.head_dim == 64) {
    if (gt == 1) KVC_TIER(64, 1);
    else if (gt == 2) KVC_TIER(64, 2);
    else KVC_TIER(64, 4);
  } else {
    if (gt == 1) KVC_TIER(128, 1);
    else if (gt == 2) KVC_TIER(128, 2);
    else KVC_TIER(128, 4);
  }
#undef KVC_TIER
  return hipGetLastError();
}

hipError_t launch_decode_attn(const AttnLaunch& a, hipStream_t st) {
  const hipError_t e = launch_attn_split(a, st);
  if (e != hipSuccess) return e;
  return launch_attn_merge(a, st);
}

hipError_t launch_attn_merge(const AttnLaunch& a, hipStream_t st) {
  const int G = a.num_q_heads / a.c.num_kv_heads;
  const long long span = attn_span(a);
  const int h2o_blocks = a.score ? (int)((span + kH2oChunk - 1) / kH2oChunk) : 0;
  const int nh = G;  // the H2O blocks need every head's statistics
  const size_t lds = (size_t)nh * (a.parts + 2) * sizeof(float);
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
