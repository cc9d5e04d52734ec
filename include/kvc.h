/*
 * kvc.h - C ABI of libkvc: compressed-KV single-query decode attention on
 * AMD Instinct MI355X (gfx950).
 *
 * A decode step over a compressed KV cache has four parts, each one call:
 *   kvc_quant_append  per-token symmetric INT8/INT4 quantize-on-write of K, V
 *   kvc_decode_attn   softmax(q K^T / sqrt(D)) V with dequantization fused in,
 *                     plus optional H2O accumulation of attention mass
 *                     (kvc_append_decode_attn: the one-token append and the
 *                     attention in one call)
 *   kvc_h2o_select    sink + recent-window + top-k heavy-hitter keep mask
 *   kvc_compact       stable out-of-place compaction of the kept slots
 *                     (kvc_compact_gather: from the keep list instead;
 *                     kvc_h2o_evict: selection and compaction in one call)
 *   kvc_decode_step   the whole step (append, attention, H2O, eviction) in
 *                     one call of two launches, into another cache or in
 *                     place
 * and a host-side paged block pool (kvc_pool_*) that yields block tables.
 *
 * Conventions shared by every call:
 *  - Plain C types only. Device pointers are raw addresses of device memory
 *    the caller allocated (e.g. from torch tensors); host pointers are named
 *    "_host". `stream` is a hipStream_t passed as void* (NULL = default stream).
 *  - The library never allocates or frees device memory, keeps no pointer
 *    after a call returns, and never synchronizes: a device call validates its
 *    arguments on the host, enqueues kernels on `stream` and returns. KVC_OK
 *    means "validated and enqueued". A fault inside a kernel surfaces at the
 *    caller's next synchronization.
 *  - Errors are status codes; nothing throws or exits across the ABI.
 *    kvc_last_error() returns a message for the calling thread's last failure.
 *    On any error status nothing was enqueued.
 *  - `max_len_hint` is the caller's upper bound on the cache lengths the call
 *    will see (device lengths are not read on the host). It sizes the launch
 *    grid and the workspace and is checked against the capacity. Kernels also
 *    clamp every device length to the capacity, so a wrong hint cannot make
 *    them access memory out of bounds; it can only make results wrong.
 *  - Calls on one stream run in order; calls that write the same buffers must
 *    not overlap on different streams.
 *  - Head dimension: the kernels are built for head_dim 64 and 128. Every
 *    other multiple of 16 up to 256 is a well-formed descriptor that every
 *    device call refuses with KVC_ERR_UNSUPPORTED (nothing enqueued); other
 *    values are KVC_ERR_INVALID_ARG.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 4

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = 1,  /* bad pointer, size, shape or aliasing */
  KVC_ERR_CAPACITY = 2,     /* not enough cache slots or pool blocks */
  KVC_ERR_UNSUPPORTED = 3,  /* valid request outside what this build implements */
  KVC_ERR_DEVICE = 4        /* a HIP runtime call failed; see kvc_last_error() */
} kvc_status;

/*
 * Descriptor of one compressed cache (one layer). Plain old data; the caller
 * owns every buffer it points to.
 *
 * Layout (row = one token of one KV head, RB = head_dim * bits / 8 bytes):
 *  contiguous (block_size == 0):
 *    k_codes, v_codes  uint8 [batch][num_kv_heads][capacity][RB]
 *    k_scale, v_scale  fp32  [batch][num_kv_heads][capacity]
 *    positions         int32 [batch][num_kv_heads][capacity] or NULL
 *  paged (block_size == 16):
 *    k_codes, v_codes  uint8 [num_blocks][num_kv_heads][block_size][RB]
 *    k_scale, v_scale  fp32  [num_blocks][num_kv_heads][block_size]
 *    block_table       int32 [batch][max_blocks_per_seq], -1 = no block;
 *                      logical token t of sequence b lives in slot
 *                      t % block_size of block block_table[b][t / block_size]
 *    positions         must be NULL; capacity = max_blocks_per_seq * block_size
 *  both:
 *    lengths   int32 [batch]  tokens currently held per sequence (all KV heads
 *                             of a sequence hold the same count)
 *    num_seen  int32 [batch]  tokens ever appended per sequence
 *
 * INT8 codes are two's-complement bytes in [-127, 127]. INT4 codes are
 * two's-complement nibbles in [-7, 7], element 2j in the low nibble of byte j
 * and element 2j+1 in the high nibble. A token's value is code * scale.
 *
 * fp16 tiers (optional; "KV Cache Compression Report", section 3.2: the
 * attention-sink tokens keep fp16 K and V; "KV Cache optimization techniques"
 * tutorial, section 1.3: recent tokens at fp16, older ones quantized). In a row
 * of L slots, the sink tier is slots [0, ns) with ns = min(fp16_sinks, L) and
 * the recent tier the last nr = min(fp16_recent, L - ns) slots; attention
 * reads tier slots at their fp16 values and every other slot from its codes.
 * Codes are still written for every token.
 *    k_sink16, v_sink16      fp16 [batch][num_kv_heads][fp16_sinks][head_dim]:
 *                            the row of slot j < fp16_sinks
 *    k_recent16, v_recent16  fp16 [batch][num_kv_heads][fp16_recent][head_dim]:
 *                            a ring, the row of position p at p % fp16_recent,
 *                            where slot i of the recent tier holds position
 *                            num_seen - L + i
 * The appends fill them. The tiers stay valid through eviction only while it
 * keeps slots [0, fp16_sinks) and the newest fp16_recent slots: the eviction
 * calls require n_sink >= fp16_sinks and n_recent >= fp16_recent, and a
 * caller-made keep mask or list must keep those slots. A compaction's
 * destination names the same tier buffers as its source (they are indexed by
 * slot or position, both unchanged by a stable compaction).
 */
typedef struct kvc_cache {
  int32_t bits;                /* 8 or 4: K code width (and V's unless v_bits is set) */
  int32_t batch;               /* sequences, >= 1 */
  int32_t num_kv_heads;        /* >= 1 */
  int32_t head_dim;            /* 64 or 128 (other multiples of 16 up to 256: UNSUPPORTED) */
  int32_t capacity;            /* slots per (sequence, KV head) */
  int32_t block_size;          /* 0 = contiguous, 16 = paged */
  int32_t max_blocks_per_seq;  /* paged only */
  int32_t num_blocks;          /* paged only: blocks in the pool arrays */
  void* k_codes;
  void* v_codes;
  float* k_scale;
  float* v_scale;
  int32_t* lengths;
  int32_t* num_seen;
  int32_t* positions;
  const int32_t* block_table;
  int32_t v_bits;              /* 0 (V as K), 8 or 4: V code width; K and V at different
                                  widths ("KV Cache optimization techniques" tutorial,
                                  section 1.1: the quantizer's K-V mode, keys and values at
                                  different precision) */
  int32_t fp16_sinks;          /* >= 0: slots of the fp16 sink tier (0 = none) */
  int32_t fp16_recent;         /* >= 0: slots of the fp16 recent tier (0 = none) */
  void* k_sink16;              /* fp16 tier buffers, layouts above; NULL when the tier is 0 */
  void* v_sink16;
  void* k_recent16;
  void* v_recent16;
} kvc_cache_t;

/* ABI version compiled into the library (KVC_ABI_VERSION). */
int32_t kvc_abi_version(void);

/* Static name of a status code ("KVC_OK", ...); "KVC_UNKNOWN" otherwise. */
const char* kvc_status_str(int32_t status);

/* Message of the calling thread's last failed call ("" if none). The pointer
 * stays valid until the thread's next libkvc call. */
const char* kvc_last_error(void);

/*
 * Quantize-on-write (per-token symmetric quantization).
 * Sources: "KV Cache optimization techniques" tutorial, section 1.2 (one scale
 * per token over head_dim, max-abs / 127) and section 1.1 (INT4: / 7, clamp
 * [-8, 7]); "KV Cache Compression Report", section 3.2 (quantize K and V when
 * they are written, never recompute).
 *
 * For each sequence b, KV head h and new token t < n_new, with x = the fp16 row
 * k_new[b][h][t][:] (and likewise v_new):
 *   scale = amax_d |x_d| / qmax   (qmax 127 or 7; correctly rounded fp32 division)
 *   code_d = round-half-even(x_d / scale)  (correctly rounded fp32 division),
 *            clamped to [-127, 127] or [-8, 7]; an all-zero row gets scale 0
 *            and codes 0.
 * The row is written at slot lengths[b] + t; positions (if not NULL) get
 * num_seen[b] + t; h2o_score (if not NULL, [batch][num_kv_heads][capacity]
 * fp32) is set to 0 at the new slots. lengths[b] and num_seen[b] then advance
 * by n_new, on the device, in stream order. With fp16 tiers the new fp16 rows
 * are also stored for them: slot lengths[b] + t < fp16_sinks goes to the sink
 * buffer, and the newest fp16_recent new tokens go to the recent ring.
 *
 * k_new, v_new: device fp16 [batch][num_kv_heads][n_new][head_dim].
 * Errors: INVALID_ARG for a bad descriptor (including negative fp16 tier
 * sizes, NULL or non-16-byte-aligned tier buffers), NULL inputs, n_new < 1,
 * max_len_hint < 0, or k_new / v_new not 16-byte aligned on a tiered cache;
 * CAPACITY if max_len_hint + n_new > capacity. Paged: the
 * blocks for the new slots must already be in the table; slots whose block is
 * missing are skipped by the kernel.
 */
int32_t kvc_quant_append(const kvc_cache_t* cache, const void* k_new, const void* v_new,
                         int32_t n_new, float* h2o_score, int32_t max_len_hint,
                         void* stream);

/*
 * Workspace bytes kvc_decode_attn needs for this cache, head count and length
 * bound (with_h2o != 0 when an H2O score array will be passed). 0 on invalid
 * arguments.
 */
size_t kvc_decode_attn_workspace_bytes(const kvc_cache_t* cache, int32_t num_q_heads,
                                       int32_t max_len_hint, int32_t with_h2o);

/*
 * Decode attention over the compressed cache, dequantization fused.
 * Sources: "KV Cache Compression Report", section 1.1 (attention =
 * softmax(Q K^T / sqrt(d)) V) and section 3.2 (the attention kernel reads
 * K_q * scale_k and V_q * scale_v, dequantizing inside the kernel); section 3.4
 * (H2O: accumulated attention per token); eviction-and-reuse survey, section
 * 3.3 (a token's score is the attention it receives from later tokens) and
 * section 6 (GQA: query heads share KV heads).
 *
 * For sequence b and query head h, with G = num_q_heads / num_kv_heads, KV head
 * g = h / G and L = lengths[b]:
 *   s_i = (q[b][h] . code^K_i) * scale^K_i / sqrt(head_dim),   i < L
 *   p_i = exp(s_i - max_j s_j) / sum_j exp(s_j - max_j s_j)
 *   out[b][h][:] = sum_i p_i * scale^V_i * code^V_i
 * If h2o_score is not NULL ([batch][num_kv_heads][capacity] fp32):
 *   h2o_score[b][g][i] += sum over the G query heads of g of p_i.
 * With fp16 tiers, the key and value of a tier slot are its fp16 rows instead
 * of code * scale (the tier slots' logits and values are computed in fp32 from
 * fp16; the codes of the recent tier are not read).
 *
 * q: device fp16 [batch][num_q_heads][head_dim]; out: device fp32
 * [batch][num_q_heads][head_dim]. workspace: device memory of at least
 * kvc_decode_attn_workspace_bytes(...) bytes, 256-byte aligned, owned by the
 * caller; its contents on entry do not matter. One workspace serves one call
 * at a time.
 * Errors: INVALID_ARG for a bad descriptor, NULL q/out, num_q_heads not a
 * multiple of num_kv_heads, G > 16, max_len_hint < 1 or a workspace that is
 * NULL or too small; CAPACITY if max_len_hint > capacity.
 */
int32_t kvc_decode_attn(const kvc_cache_t* cache, const void* q, int32_t num_q_heads,
                        float* out, float* h2o_score, int32_t max_len_hint,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step's append and attention in one call: kvc_quant_append of one
 * token per sequence (n_new = 1), then kvc_decode_attn over the cache that
 * includes it. Sources: those of the two calls ("KV Cache optimization
 * techniques" tutorial, sections 1.1 and 1.2; "KV Cache Compression Report",
 * sections 1.1, 3.2 and 3.4).
 *
 * k_new, v_new: device fp16 [batch][num_kv_heads][head_dim], the new token of
 * each sequence; it goes to slot lengths[b] (codes, scale, position =
 * num_seen[b], and score 0 before the H2O update), then lengths[b] and
 * num_seen[b] advance by one, exactly as kvc_quant_append does. The cache's
 * codes, scales, positions, lengths, scores and `out` equal those of the two
 * separate calls bit for bit. max_len_hint bounds the lengths before the
 * append; the workspace needs kvc_decode_attn_workspace_bytes(cache,
 * num_q_heads, max_len_hint + 1, with_h2o) bytes. The append happens inside
 * the attention kernels (the wave that reads the new slot writes it first), so
 * the step takes two launches instead of three.
 * Errors: those of both calls; CAPACITY if max_len_hint + 1 > capacity.
 */
int32_t kvc_append_decode_attn(const kvc_cache_t* cache, const void* k_new, const void* v_new,
                               const void* q, int32_t num_q_heads, float* out, float* h2o_score,
                               int32_t max_len_hint, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * The two phases of the attention calls, for callers that schedule them
 * apart (flash-decoding split and merge; same sources as kvc_decode_attn):
 * kvc_decode_attn_split runs the split kernel (with k_new and v_new, both
 * non-NULL, it first appends the new token, as kvc_append_decode_attn does)
 * and leaves its partial results in the workspace; kvc_decode_attn_merge
 * (appended = whether the split appended) merges them into `out`, applies the
 * H2O update and, after an append, advances lengths and num_seen. The pair,
 * with the same cache, heads, h2o_score (NULL or not), max_len_hint and
 * workspace, and nothing between them that touches those, equals
 * kvc_decode_attn (or kvc_append_decode_attn) bit for bit. max_len_hint is as
 * in those calls (the length before the append, if any).
 * Errors: as kvc_decode_attn / kvc_append_decode_attn; INVALID_ARG if only
 * one of k_new, v_new is given.
 */
int32_t kvc_decode_attn_split(const kvc_cache_t* cache, const void* k_new, const void* v_new,
                              const void* q, int32_t num_q_heads, float* h2o_score,
                              int32_t max_len_hint, void* workspace, size_t workspace_bytes,
                              void* stream);
int32_t kvc_decode_attn_merge(const kvc_cache_t* cache, int32_t appended, int32_t num_q_heads,
                              float* out, float* h2o_score, int32_t max_len_hint, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Keep-set selection: attention sinks + recent window + heavy hitters.
 * Sources: "KV Cache Compression Report", section 3.3 (the first 4 tokens
 * are permanent attention sinks, a window keeps the most recent tokens) and
 * section 3.4 (keep the top-scoring tokens plus the recent ones, kept indices
 * sorted); "KV Cache optimization techniques" tutorial, sections 2.2 and 2.4.
 *
 * For each (b, g) row with L = lengths[b]:
 *   L <= budget: keep every slot < L.
 *   otherwise:   keep slots [0, n_sink) and [L - n_recent, L), plus the
 *                k = budget - n_sink - n_recent slots of [n_sink, L - n_recent)
 *                with the largest h2o_score; equal scores go to the lower slot.
 * keep_mask: device uint8 [batch][num_kv_heads][capacity]; slots < L get 1 or 0,
 * slots >= L are left untouched. keep_index (may be NULL): device int32
 * [batch][num_kv_heads][budget]; entries j < min(L, budget) receive the kept
 * slots in ascending order (the gather list kvc_compact_gather takes); later
 * entries are left untouched. h2o_score must hold non-negative, non-NaN values
 * (attention mass always is).
 * Errors: INVALID_ARG for a bad descriptor, NULL score or mask, budget < 1,
 * n_sink < 0, n_recent < 0, n_sink + n_recent > budget, or a tiered cache with
 * n_sink < fp16_sinks or n_recent < fp16_recent; CAPACITY if budget or
 * max_len_hint > capacity.
 */
int32_t kvc_h2o_select(const kvc_cache_t* cache, const float* h2o_score, int32_t budget,
                       int32_t n_sink, int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index,
                       int32_t max_len_hint, void* stream);

/* Workspace bytes kvc_compact needs. */
size_t kvc_compact_workspace_bytes(const kvc_cache_t* src, int32_t max_len_hint);

/*
 * Stable out-of-place compaction of the kept slots.
 * Sources: "KV Cache optimization techniques" tutorial, section 2.2 (kept
 * indices sorted, and the attention scores move with the kept K/V); "KV Cache
 * Compression Report", section 3.4 (the kept list is sorted).
 *
 * For each (b, g) row, the slots i < lengths[b] with keep_mask[b][g][i] != 0
 * are copied, in ascending order, to slots 0, 1, ... of dst: K and V codes and
 * scales, positions (when both src and dst have them) and h2o scores (when
 * src_score and dst_score are both given). dst->lengths[b] is set to the count
 * kept by KV head 0 (every head of a sequence must keep the same count, as
 * kvc_h2o_select guarantees) and dst->num_seen[b] to src->num_seen[b].
 * Slots of dst at or beyond the new length are left untouched.
 *
 * src and dst must be contiguous caches with the same bits, batch,
 * num_kv_heads, head_dim and capacity; no dst buffer may overlap a src buffer,
 * the mask or the src scores (INVALID_ARG otherwise); paged caches give
 * UNSUPPORTED. With fp16 tiers, dst must name src's tier sizes and buffers
 * (INVALID_ARG otherwise), and the mask must keep slots [0, fp16_sinks) and
 * the newest fp16_recent slots of each row (not checked: the tiers would then
 * describe other tokens). workspace: device memory of
 * kvc_compact_workspace_bytes(...).
 */
int32_t kvc_compact(const kvc_cache_t* src, const float* src_score, const uint8_t* keep_mask,
                    const kvc_cache_t* dst, float* dst_score, int32_t max_len_hint,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Compaction from a gather list, the form kvc_h2o_select emits in keep_index.
 * Same result and sources as kvc_compact: for each (b, g) row, destination
 * slot j takes source slot keep_index[b][g][j] (K and V codes and scales,
 * positions when both caches have them, scores when both score arrays are
 * given) for j < min(lengths[b], n_keep); dst->lengths[b] is set to that count
 * and dst->num_seen[b] to src->num_seen[b]. keep_index: device int32
 * [batch][num_kv_heads][n_keep], ascending within a row; an index outside
 * [0, capacity) is clamped into it (no out-of-bounds access, a wrong result).
 * No workspace and no scan: one launch that starts copying at once.
 * Errors: as kvc_compact, plus INVALID_ARG for a NULL list or n_keep < 1 and
 * CAPACITY for n_keep > capacity.
 */
int32_t kvc_compact_gather(const kvc_cache_t* src, const float* src_score, const int32_t* keep_index,
                           int32_t n_keep, const kvc_cache_t* dst, float* dst_score, void* stream);

/*
 * Eviction in one call: the keep set of kvc_h2o_select, moved to dst as
 * kvc_compact_gather moves it. Sources: those two calls ("KV Cache
 * Compression Report", sections 3.3 and 3.4; "KV Cache optimization
 * techniques" tutorial, sections 2.2 and 2.4).
 *
 * For each (b, g) row with L = src->lengths[b], the slots kvc_h2o_select would
 * keep (with the same budget, n_sink, n_recent and h2o_score) are copied in
 * ascending order to slots 0 .. min(L, budget) - 1 of dst: K and V codes and
 * scales, positions when both caches have them, and scores into dst_score
 * when it is not NULL. dst->lengths[b] = min(L, budget), dst->num_seen[b] =
 * src->num_seen[b]; slots of dst at or beyond the new length are left
 * untouched. keep_index (required, device int32 [batch][num_kv_heads][budget])
 * and keep_mask (may be NULL, device uint8 [batch][num_kv_heads][capacity])
 * receive exactly what kvc_h2o_select writes into them.
 * When max_len_hint - n_sink - n_recent <= 8192, one launch does both steps
 * (each row's workgroups select redundantly and each copies a share of the
 * kept rows); longer rows take the two launches of the separate calls.
 * h2o_score must hold non-negative, non-NaN values.
 * Errors: those of kvc_h2o_select and kvc_compact_gather: INVALID_ARG for bad
 * descriptors, differing src/dst geometries, NULL h2o_score or keep_index,
 * budget < 1, n_sink or n_recent < 0, n_sink + n_recent > budget, or a dst
 * buffer overlapping src, h2o_score, keep_mask or keep_index; CAPACITY if
 * budget or max_len_hint > capacity; UNSUPPORTED for paged caches.
 */
int32_t kvc_h2o_evict(const kvc_cache_t* src, const float* h2o_score, int32_t budget, int32_t n_sink,
                      int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index, const kvc_cache_t* dst,
                      float* dst_score, int32_t max_len_hint, void* stream);

/*
 * A whole decode step in one call: kvc_append_decode_attn (with H2O) followed
 * by kvc_h2o_evict from `cache` into `dst`. Sources: those of the two calls
 * (tutorial sections 1.1, 1.2, 2.2, 2.4; report sections 1.1, 3.2 to 3.4;
 * eviction-and-reuse survey, section 3.3).
 *
 * Results: `out`, the cache's codes, scales, positions, lengths and num_seen,
 * keep_index, keep_mask (may be NULL) and every buffer of dst including
 * dst_score (required: the kept tokens' accumulated scores) equal those of the
 * two calls bit for bit. The source scores h2o_score are input to the step;
 * afterwards they hold, for slots below the new length, either the old or the
 * updated values (the new token's slot holds 0 or its mass), since the
 * one-launch path below does not write them back: dst_score is the state a
 * decode loop continues from.
 *
 * When num_q_heads / num_kv_heads <= 4 and max_len_hint + 1 - n_sink -
 * n_recent <= 8192, the step is two launches: the split attention kernel
 * (appending the new token) and the eviction kernel, which also merges the
 * splits (the output and the H2O update of the scores it selects on and
 * copies). Otherwise it runs the separate calls' launches. max_len_hint
 * bounds the lengths before the append; the workspace is that of
 * kvc_append_decode_attn (kvc_decode_attn_workspace_bytes(cache, num_q_heads,
 * max_len_hint + 1, 1)) and must not overlap any cache buffer.
 *
 * In place: `dst` may describe `cache` itself (every buffer the same, and
 * dst_score == h2o_score). The kept tokens then keep their order and move
 * down to their rank inside the cache, so only those past the first evicted
 * slot are rewritten (a decode loop that evicts one token per step moves
 * about half a row instead of copying all of it; tutorial section 2.2's
 * sorted keep, applied where the tokens are). Output, keep_index, keep_mask,
 * lengths, num_seen and, below the new length, codes, scales, positions and
 * scores equal those of the same step into a separate dst bit for bit; slots
 * at or past the new length hold stale tokens. Launches: the split kernel,
 * then one in-place eviction kernel that merges the splits (up to 8 query
 * heads per KV head), selects and moves; with more query heads the merge
 * kernel runs first, and with more than 8192 candidates the selection kernel
 * too. Its workgroups order their reads and writes of the cache through flags
 * in the workspace, so the workspace must not be shared with a concurrent
 * call.
 * Errors: those of kvc_append_decode_attn and kvc_h2o_evict (with
 * max_len_hint + 1 as the eviction's hint), and INVALID_ARG for a NULL
 * h2o_score or dst_score, a dst that shares some but not all of the cache's
 * buffers, an in-place dst_score other than h2o_score, or a keep_index or
 * keep_mask that overlaps a cache buffer, the scores or each other.
 */
int32_t kvc_decode_step(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                        int32_t num_q_heads, float* out, float* h2o_score, int32_t budget,
                        int32_t n_sink, int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index,
                        const kvc_cache_t* dst, float* dst_score, int32_t max_len_hint,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same step with the same results; its workspace is a static device
 * array inside the library (one per GPU, kvc_decode_step_noalloc_max_bytes()
 * bytes = 16 MiB, held until the process ends) instead of a caller buffer.
 * The call allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine); on its first call on a device it looks up that device's copy of
 * the array. Nothing in the array needs clearing between calls: every byte a
 * step reads was written by the same step.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from different threads without stream
 * order between them) race. Issue them on one stream.
 *
 * Errors: those of kvc_decode_step, and KVC_ERR_CAPACITY (nothing enqueued)
 * when the step's workspace, kvc_decode_attn_workspace_bytes(cache,
 * num_q_heads, max_len_hint + 1, 1), exceeds the array; KVC_ERR_DEVICE when
 * the array's device address cannot be obtained.
 */
size_t kvc_decode_step_noalloc_max_bytes(void);
int32_t kvc_decode_step_noalloc(const kvc_cache_t* cache, const void* k_new, const void* v_new, const void* q,
                                int32_t num_q_heads, float* out, float* h2o_score, int32_t budget,
                                int32_t n_sink, int32_t n_recent, uint8_t* keep_mask, int32_t* keep_index,
                                const kvc_cache_t* dst, float* dst_score, int32_t max_len_hint, void* stream);

/*
 * Block-granular H2O eviction on a paged cache: whole 16-token blocks are
 * evicted and compaction is a rewrite of the block table (no codes move).
 * Sources: eviction-and-reuse survey, section 4 (evict blocks by attention
 * score: sort by mean score, lowest first, stable, and evict the first
 * int(n * (1 - retention)); evicted blocks release their reference) and
 * "KV Cache optimization techniques" tutorial, section 3.2 (block table,
 * reference counts).
 *
 * For each sequence b with L = min(src->lengths[b], max_len_hint) and
 * n = ceil(L / 16) blocks: a block's score is the mean of h2o_score over its
 * filled slots and all KV heads (an fp32 sum in a fixed order, so blocks
 * holding equal scores get equal means); with
 * n_evict = (int)(n * (1 - retention)) in double arithmetic, the n_evict
 * blocks first in ascending order of score (equal scores: lower block index
 * first) are evicted. dst's table row b lists the kept physical blocks in
 * their order, then -1; dst->lengths[b] counts their tokens (the last block
 * may be partial and stays last); dst->num_seen[b] = src->num_seen[b];
 * dst_score[b][h] holds the kept blocks' scores at their new slots (slots at
 * or past the new length untouched); freed[b][0..n_evict) lists the evicted
 * physical blocks in block order and freed_count[b] = n_evict (give them back
 * with kvc_pool_release).
 *
 * src and dst are paged caches with the same geometry that share the code and
 * scale pools; dst's block table, lengths and num_seen are its own (device
 * buffers the call writes). workspace: device memory of
 * kvc_paged_block_evict_workspace_bytes(src) bytes, 256-byte aligned, disjoint
 * from every other buffer (the block means). Cost: two launches; n^2
 * comparisons per sequence, sized for decode-length tables.
 * Errors: INVALID_ARG for bad or contiguous descriptors, different
 * geometries or pools, NULL arrays, retention outside [0, 1], overlapping
 * inputs and outputs, a missing, small or unaligned workspace; CAPACITY if max_len_hint > capacity; UNSUPPORTED above
 * 8192 blocks per sequence, or for caches with fp16 tiers (block eviction
 * keeps no sinks or window, so it cannot keep the tiers).
 */
size_t kvc_paged_block_evict_workspace_bytes(const kvc_cache_t* src);
int32_t kvc_paged_block_evict(const kvc_cache_t* src, const float* h2o_score, double retention,
                              const kvc_cache_t* dst, float* dst_score, int32_t* freed,
                              int32_t* freed_count, int32_t max_len_hint, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Per-layer keep budgets (host only): the pyramid schedules of the pages.
 * Sources: "KV Cache optimization techniques" tutorial, section 2.3
 * (PyramidKV, linear: layer l of n keeps the fraction 1 - 0.8 l / n, shallow
 * layers keep more) and the eviction-and-reuse survey, section 4 (quadratic:
 * r + (1 - r)(l / n)^2 from a base ratio r, deep layers keep more; the page
 * assumes n = 80, here n = num_layers).
 *
 * budgets_host[l] = max(min_budget, (int32)(base * ratio_l)) for l <
 * num_layers, the product truncated toward zero, in double arithmetic. Layer
 * l's budget is then the `budget` argument of kvc_h2o_select,
 * kvc_h2o_evict or kvc_decode_step for that layer (min_budget =
 * n_sink + n_recent keeps their precondition). base_ratio is used by the
 * quadratic schedule only.
 * Errors: INVALID_ARG for a NULL output, num_layers < 1, base < 1,
 * min_budget < 0, an unknown schedule or a base_ratio outside [0, 1].
 */
enum { KVC_SCHEDULE_LINEAR = 0, KVC_SCHEDULE_QUADRATIC = 1 };
int32_t kvc_layer_budgets(int32_t schedule, int32_t num_layers, int32_t base, double base_ratio,
                          int32_t min_budget, int32_t* budgets_host);

/*
 * K/V-separated attention (top-k V).
 * Source: "KV Cache Compression Report", section 3.5 (K/V stored apart: the
 * quantized K of every token stays on the GPU to score the query; full-
 * precision V is kept hot on the GPU or cold in host memory and fetched for
 * the top-scored tokens only).
 *
 * For sequence b and KV head g with L = lengths[b]: the logits s_{h,i} and
 * probabilities p_{h,i} of kvc_decode_attn (every cached token, each key as
 * that call reads it: from the codes, or the fp16 row on a tier); the kept set = the min(top_k, L) slots with the largest group mass
 * sum over the G query heads of g of p_{h,i} (equal mass: lower slot); then
 * for each query head h of g:
 *   out[b][h][:] = sum over kept i of exp(s_{h,i}) / sum over kept j of
 *                  exp(s_{h,j}) * V_i
 * where V_i is slot i's fp16 row: from the cache's fp16 tiers when slot i is
 * on one (hot), else from v_host (cold).
 *
 * q: device fp16 [batch][num_q_heads][head_dim]; out: device fp32
 * [batch][num_q_heads][head_dim]. v_host: pinned host memory (hipHostMalloc,
 * or a pinned torch CPU tensor), fp16 [batch][num_kv_heads][capacity][head_dim]
 * indexed by slot, owned and kept current by the caller (the row of every
 * cold slot < L must hold that token's V); the device reads it directly, so
 * each call moves min(top_k, L) rows per (sequence, KV head) over the host
 * link. workspace: kvc_decode_attn_kvsep_workspace_bytes(...) bytes, 256-byte
 * aligned. The cache's H2O scores are not touched.
 * Errors: those of kvc_decode_attn, plus INVALID_ARG for top_k < 1, a NULL or
 * unaligned v_host, or v_host not pinned device-readable host memory;
 * CAPACITY if top_k > capacity.
 */
size_t kvc_decode_attn_kvsep_workspace_bytes(const kvc_cache_t* cache, int32_t num_q_heads,
                                             int32_t top_k, int32_t max_len_hint);
int32_t kvc_decode_attn_kvsep(const kvc_cache_t* cache, const void* q, int32_t num_q_heads,
                              int32_t top_k, const void* v_host, float* out,
                              int32_t max_len_hint, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Measurement helper (not a step of the method): one streaming read of
 * `bytes` bytes of device memory at `src` (16-byte aligned, bytes a positive
 * multiple of 16) with the decode-attention kernel's 16-byte load width, 4096
 * workgroups. It gives the HBM read ceiling one launch reaches, the
 * practical reference next to the nominal 8 TB/s for the attention's roofline.
 * `sink` (device, kvc_bw_probe_sink_bytes() bytes, disjoint from src) receives
 * one word per workgroup. Errors: INVALID_ARG for NULL pointers, a bad size or
 * alignment, a small or overlapping sink.
 */
size_t kvc_bw_probe_sink_bytes(void);
int32_t kvc_bw_probe(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/*
 * Paged block pool (host only; no device memory is touched).
 * Source: "KV Cache optimization techniques" tutorial, section 3.2
 * (PagedAttention): fixed-size blocks, a per-sequence block list, a reference
 * count per block and a free set; allocation fails without side effects when
 * blocks run short; freeing an unknown sequence does nothing; an unknown
 * sequence is an error when its blocks are asked for.
 *
 * The free list is shuffled with `shuffle_seed` (0 = identity order), so block
 * placement is a seeded permutation of the pool. Pools are not thread-safe.
 */
typedef struct kvc_pool kvc_pool_t;

/* NULL on num_blocks < 1, block_size < 1 or allocation failure. */
kvc_pool_t* kvc_pool_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed);
void kvc_pool_destroy(kvc_pool_t* pool);

/* Make sequence seq_id (>= 0) hold at least num_tokens tokens, growing an
 * existing reservation. All or nothing: CAPACITY and no change if free blocks
 * are short; INVALID_ARG for seq_id < 0 or num_tokens < 0. */
int32_t kvc_pool_reserve(kvc_pool_t* pool, int32_t seq_id, int32_t num_tokens);

/* Drop the sequence's reference on each of its blocks; blocks whose count
 * reaches 0 return to the free list. OK (no-op) for an unknown seq_id. */
int32_t kvc_pool_free(kvc_pool_t* pool, int32_t seq_id);

/* Give back blocks of sequence seq_id (the blocks kvc_paged_block_evict frees):
 * each is removed from the sequence's list, whose other blocks keep their
 * order, and its reference count drops; at zero it returns to the free set
 * (tutorial section 3.2; eviction-and-reuse survey, section 4: evicted blocks
 * release their reference). All or nothing: INVALID_ARG and no change for an
 * unknown sequence, a NULL list with n > 0, n < 0, or a block the sequence
 * does not hold (each listed once). */
int32_t kvc_pool_release(kvc_pool_t* pool, int32_t seq_id, const int32_t* blocks_host, int32_t n);

/* Blocks on the free list (-1 for a NULL pool). */
int32_t kvc_pool_num_free(const kvc_pool_t* pool);

/* Blocks held by seq_id, or -1 if it is unknown. */
int32_t kvc_pool_num_blocks(const kvc_pool_t* pool, int32_t seq_id);

/* Fill table_host [batch][max_blocks] with each listed sequence's blocks in
 * logical order, padded with -1. INVALID_ARG for an unknown seq_id, NULL
 * pointers or batch < 1; CAPACITY if a sequence holds more than max_blocks. */
int32_t kvc_pool_block_table(const kvc_pool_t* pool, const int32_t* seq_ids_host,
                             int32_t batch, int32_t max_blocks, int32_t* table_host);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
