// Stable out-of-place compaction of the kept cache slots.
//
// The kept slots keep their relative (ascending) order and carry their scores
// with them ("KV Cache optimization techniques" tutorial, section 2.2; "KV
// Cache Compression Report", section 3.4). The destination of a kept slot is
// the number of kept slots before it: an exclusive prefix sum of the mask.
//
// A 256-thread workgroup owns a 256-slot chunk of one (sequence, KV head) row,
// one slot per thread. Its offset is the count of kept slots in the chunks
// before it: for rows of up to 64 chunks the workgroup counts them straight
// from the mask (one launch); longer rows get a first launch that writes
// per-chunk counts. A block scan of the chunk's flags gives each kept slot its
// destination and lists the kept slots in LDS; the rows are then copied
// cooperatively, RB/16 lanes per row with 16-byte accesses (RB the wider of
// the K and V rows; lanes past the narrower row's end idle for it), and every
// load of the chunk is issued before the first store so that the copy is
// bound by bandwidth rather than latency. Reading src and writing dst, which may not
// overlap, removes every race.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int CH = kCompactChunk;
constexpr int NT = CH;  // one slot per thread

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int block_sum(int v, int* tmp) {
  v = wave_sum_i(v);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) r += tmp[w];
  __syncthreads();
  return r;
}

// Number of nonzero bytes in a 32-bit word.
__device__ __forceinline__ int nonzero_bytes(unsigned x) {
  return __popc((((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u);
}

__device__ __forceinline__ int row_length(const kvc_cache_t& c, int b, int chunks) {
  return __builtin_amdgcn_readfirstlane(min(min(c.lengths[b], c.capacity), chunks * CH));
}

__global__ __launch_bounds__(NT) void compact_count_kernel(kvc_cache_t src, const uint8_t* __restrict__ mask,
                                                           int32_t* __restrict__ counts, int chunks) {
  const int ch = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = row_length(src, b, chunks);
  const uint8_t* m = mask + ((long long)b * src.num_kv_heads + g) * src.capacity;
  const int i = ch * CH + threadIdx.x;
  __shared__ int tmp[NT / 64];
  const int n = block_sum(i < L && m[i] != 0, tmp);
  if (threadIdx.x == 0) counts[((long long)b * src.num_kv_heads + g) * chunks + ch] = n;
}

// Copy `total` kept rows of one (sequence, KV head) row: kept row q (source
// slot list[q], in LDS) goes to destination slot off + q. K and V rows move
// cooperatively, RB/16 lanes per row with 16-byte accesses; every load of a
// batch is issued before its stores. Lanes past the last kept row reload that
// row (a cache hit) rather than branch, and only their stores are skipped.
// Thread t also moves the scales, position and score of kept row t.
template <int RBK, int RBV, int NT>
__device__ __forceinline__ void copy_rows(const kvc_cache_t& src, const float* __restrict__ src_score,
                                          const kvc_cache_t& dst, float* __restrict__ dst_score, long long rowoff,
                                          const int* list, int total, int off) {
  constexpr int RB = RBK > RBV ? RBK : RBV;
  constexpr int LPR = RB / 16;        // lanes per row
  constexpr int RPP = NT / LPR;       // rows per pass
  constexpr int BATCH = 8;  // every pass of a 256-row chunk in flight at once (RB <= 128)
  const int tid = threadIdx.x;
  const uint8_t* sk = static_cast<const uint8_t*>(src.k_codes) + rowoff * RBK;
  const uint8_t* sv = static_cast<const uint8_t*>(src.v_codes) + rowoff * RBV;
  uint8_t* dk = static_cast<uint8_t*>(dst.k_codes) + rowoff * RBK;
  uint8_t* dv = static_cast<uint8_t*>(dst.v_codes) + rowoff * RBV;
  const int part = tid % LPR, r0 = tid / LPR;
  const bool kpart = RBK == RB || part * 16 < RBK, vpart = RBV == RB || part * 16 < RBV;
  const bool mine = tid < total;
  const long long si = rowoff + list[mine ? tid : 0], di = rowoff + off + tid;
  float ksv = 0.f, vsv = 0.f, scv = 0.f;
  int pos = 0;
  if (mine) {
    ksv = src.k_scale[si];
    vsv = src.v_scale[si];
    if (src.positions && dst.positions) pos = src.positions[si];
    if (src_score && dst_score) scv = src_score[si];
  }
  const int npass = (total + RPP - 1) / RPP;
  for (int p0 = 0; p0 < npass; p0 += BATCH) {
    u32x4 kx[BATCH], vx[BATCH];
#pragma unroll
    for (int p = 0; p < BATCH; ++p) {
      const long long s_row = list[min(r0 + (p0 + p) * RPP, total - 1)];
      if (kpart) kx[p] = *reinterpret_cast<const u32x4*>(sk + s_row * RBK + part * 16);
      if (vpart) vx[p] = *reinterpret_cast<const u32x4*>(sv + s_row * RBV + part * 16);
    }
#pragma unroll
    for (int p = 0; p < BATCH; ++p) {
      const int q = r0 + (p0 + p) * RPP;
      if (q < total) {
        const long long d = off + q;
        // Streaming stores: the compacted rows are not read again by this
        // launch, so they should not sit dirty in L2 until the kernel ends.
        if (kpart) __builtin_nontemporal_store(kx[p], reinterpret_cast<u32x4*>(dk + d * RBK + part * 16));
        if (vpart) __builtin_nontemporal_store(vx[p], reinterpret_cast<u32x4*>(dv + d * RBV + part * 16));
      }
    }
  }
  if (mine) {
    dst.k_scale[di] = ksv;
    dst.v_scale[di] = vsv;
    if (src.positions && dst.positions) dst.positions[di] = pos;
    if (src_score && dst_score) dst_score[di] = scv;
  }
}

template <int RBK, int RBV, bool RECOUNT>
__global__ __launch_bounds__(NT) void compact_move_kernel(kvc_cache_t src, const float* __restrict__ src_score,
                                                          const uint8_t* __restrict__ mask, kvc_cache_t dst,
                                                          float* __restrict__ dst_score,
                                                          const int32_t* __restrict__ counts, int chunks) {
  const int ch = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int H = src.num_kv_heads;
  const int L = row_length(src, b, chunks);
  const long long rowoff = ((long long)b * H + g) * src.capacity;
  const uint8_t* mrow = mask + rowoff;
  __shared__ int tmp[2 * (NT / 64)];
  __shared__ int list[CH];

  if (ch * CH >= L) {
    if (ch == 0 && g == 0 && tid == 0) {
      dst.lengths[b] = 0;
      dst.num_seen[b] = src.num_seen[b];
    }
    return;
  }
  const int i = ch * CH + tid;
  // Clamped to the capacity (a kernel argument), not to L, so that this load
  // does not wait for the length.
  const int f = (i < L) & (mrow[min(i, src.capacity - 1)] != 0);
  // Kept slots in the chunks before this one: `pre` is this thread's share.
  int pre = 0;
  if (RECOUNT) {
    if (ch > 0) {
      if (rowoff % 16 == 0) {
        // 16 mask bytes per load, at most four loads per thread, all issued
        // together (clamped index, masked count).
        const int words = ch * (CH / 16);
#pragma unroll
        for (int q = 0; q < kCompactRecountChunks * (CH / 16) / NT; ++q) {
          const int w = tid + q * NT;
          const uint4 v = reinterpret_cast<const uint4*>(mrow)[min(w, words - 1)];
          const int nzb = nonzero_bytes(v.x) + nonzero_bytes(v.y) + nonzero_bytes(v.z) + nonzero_bytes(v.w);
          pre += w < words ? nzb : 0;
        }
      } else {
#pragma unroll 8
        for (int q = 0; q < ch; ++q) pre += mrow[tid + q * NT] != 0;
      }
    }
  } else {
    const int32_t* cr = counts + ((long long)b * H + g) * chunks;
    for (int q = tid; q < ch; q += NT) pre += cr[q];
  }

  // One block scan gives both the chunk's rank of each kept slot (low 16 bits:
  // the flags) and, from its total, the offset (high bits: the earlier counts;
  // at most 16384 with RECOUNT). Long rows sum their offset separately.
  const int lane = tid & 63, wave = tid >> 6;
  int incl = wave_inclusive_scan(RECOUNT ? (pre << 16) | f : f);
  int* wt = tmp + NT / 64;
  if (lane == 63) wt[wave] = incl;
  int off;
  if (!RECOUNT) off = block_sum(pre, tmp);  // barriers inside also publish wt
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) incl += wt[w];
    total += wt[w];
  }
  if (RECOUNT) {
    off = total >> 16;
    total &= 0xFFFF;
    incl &= 0xFFFF;
  }
  if (f) list[incl - 1] = i;
  __syncthreads();

  copy_rows<RBK, RBV, NT>(src, src_score, dst, dst_score, rowoff, list, total, off);
  // The chunk holding the row's last slot knows the row's total.
  if (g == 0 && ch == (L - 1) / CH && tid == 0) {
    dst.lengths[b] = off + total;
    dst.num_seen[b] = src.num_seen[b];
  }
}


// Compaction from a sorted gather list (the kept slots of each row in
// ascending order, as kvc_h2o_select emits): destination slot j of row (b, g)
// takes source slot keep_index[b][g][j] for j < min(length, n_keep). No scan
// is needed. The flat list [B][Hkv][n_keep] is split evenly over the grid, so
// every CU moves the same number of rows: a workgroup takes `per_wg` (at most
// NT) consecutive entries, one entry per thread for the index, scales,
// position and score, and LPR lanes per entry for the codes, with every load
// in flight before the first store.
template <int RBK, int RBV>
__global__ __launch_bounds__(NT) void compact_gather_kernel(kvc_cache_t src, const float* __restrict__ src_score,
                                                            const int32_t* __restrict__ keep_index, int n_keep,
                                                            kvc_cache_t dst, float* __restrict__ dst_score,
                                                            long long entries, int per_wg) {
  constexpr int RB = RBK > RBV ? RBK : RBV;
  constexpr int LPR = RB / 16;        // lanes per row
  constexpr int RPP = NT / LPR;       // rows per pass
  constexpr int NPASS = NT / RPP;     // passes for NT rows
  const int tid = threadIdx.x, H = src.num_kv_heads;
  const long long cap = src.capacity;
  __shared__ long long s_row[NT], d_row[NT];  // source / destination row of each entry; -1: not copied
  const long long e = (long long)blockIdx.x * per_wg + tid;
  const bool mine = tid < per_wg && e < entries;
  long long si = -1, di = 0;
  if (mine) {
    const long long bg = e / n_keep;
    const int j = (int)(e - bg * n_keep), b = (int)(bg / H);
    const int idx = keep_index[e];
    const int count = min(min(src.lengths[b], src.capacity), n_keep);
    if (j < count) {
      si = bg * cap + min(max(idx, 0), src.capacity - 1);  // a bad index cannot leave the row
      di = bg * cap + j;
    }
  }
  s_row[tid] = si;
  d_row[tid] = di;
  float ksv = 0.f, vsv = 0.f, scv = 0.f;
  int pos = 0;
  if (si >= 0) {
    ksv = src.k_scale[si];
    vsv = src.v_scale[si];
    if (src.positions && dst.positions) pos = src.positions[si];
    if (src_score && dst_score) scv = src_score[si];
  }
  if (blockIdx.x == 0) {
    for (int b = tid; b < src.batch; b += NT) {
      dst.lengths[b] = min(min(src.lengths[b], src.capacity), n_keep);
      dst.num_seen[b] = src.num_seen[b];
    }
  }
  __syncthreads();
  const uint8_t* sk = static_cast<const uint8_t*>(src.k_codes);
  const uint8_t* sv = static_cast<const uint8_t*>(src.v_codes);
  uint8_t* dk = static_cast<uint8_t*>(dst.k_codes);
  uint8_t* dv = static_cast<uint8_t*>(dst.v_codes);
  const int part = tid % LPR, r0 = tid / LPR;
  const bool kpart = RBK == RB || part * 16 < RBK, vpart = RBV == RB || part * 16 < RBV;
  u32x4 kx[NPASS], vx[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const long long r = s_row[r0 + p * RPP];
    const long long row = r < 0 ? 0 : r;  // every load valid; unused rows are not stored
    if (kpart) kx[p] = *reinterpret_cast<const u32x4*>(sk + row * RBK + part * 16);
    if (vpart) vx[p] = *reinterpret_cast<const u32x4*>(sv + row * RBV + part * 16);
  }
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int q = r0 + p * RPP;
    if (s_row[q] >= 0) {
      // Streaming stores: the compacted rows are not read again by this launch.
      if (kpart) __builtin_nontemporal_store(kx[p], reinterpret_cast<u32x4*>(dk + d_row[q] * RBK + part * 16));
      if (vpart) __builtin_nontemporal_store(vx[p], reinterpret_cast<u32x4*>(dv + d_row[q] * RBV + part * 16));
    }
  }
  if (si >= 0) {
    dst.k_scale[di] = ksv;
    dst.v_scale[di] = vsv;
    if (src.positions && dst.positions) dst.positions[di] = pos;
    if (src_score && dst_score) dst_score[di] = scv;
  }
}

template <int RBK, int RBV>
hipError_t launch_rb(const kvc_cache_t& src, const float* ss, const uint8_t* mask, const kvc_cache_t& dst,
                     float* ds, int32_t* counts, int chunks, hipStream_t st) {
  const dim3 grid(chunks, src.num_kv_heads, src.batch);
  if (chunks <= kCompactRecountChunks) {
    hipLaunchKernelGGL((compact_move_kernel<RBK, RBV, true>), grid, dim3(NT), 0, st, src, ss, mask, dst, ds, counts,
                       chunks);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(compact_count_kernel, grid, dim3(NT), 0, st, src, mask, counts, chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((compact_move_kernel<RBK, RBV, false>), grid, dim3(NT), 0, st, src, ss, mask, dst, ds, counts,
                     chunks);
  return hipGetLastError();
}

template <int RBK, int RBV>
hipError_t launch_gather_rb(const kvc_cache_t& src, const float* ss, const int32_t* keep_index, int n_keep,
                            const kvc_cache_t& dst, float* ds, hipStream_t st) {
  // About 2 workgroups per CU for the flat list, at most NT entries each.
  const long long entries = (long long)src.batch * src.num_kv_heads * n_keep;
  const long long target = 2LL * device_cus();
  const int per_wg = (int)std::min<long long>(NT, std::max<long long>(1, (entries + target - 1) / target));
  const long long wgs = (entries + per_wg - 1) / per_wg;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((compact_gather_kernel<RBK, RBV>), dim3((unsigned)wgs), dim3(NT), 0, st, src, ss, keep_index, n_keep,
                     dst, ds, entries, per_wg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compact_gather(const kvc_cache_t& src, const float* src_score, const int32_t* keep_index,
                                 int n_keep, const kvc_cache_t& dst, float* dst_score, hipStream_t st) {
  return with_row_bytes(src, [&](auto rbk, auto rbv) {
    return launch_gather_rb<decltype(rbk)::value, decltype(rbv)::value>(src, src_score, keep_index, n_keep, dst, dst_score, st);
  });
}

hipError_t launch_compact(const kvc_cache_t& src, const float* src_score, const uint8_t* mask,
                          const kvc_cache_t& dst, float* dst_score, int32_t* counts, int chunks, hipStream_t st) {
  return with_row_bytes(src, [&](auto rbk, auto rbv) {
    return launch_rb<decltype(rbk)::value, decltype(rbv)::value>(src, src_score, mask, dst, dst_score, counts, chunks, st);
  });
}

}  // namespace kvc
