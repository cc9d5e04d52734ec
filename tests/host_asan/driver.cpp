// Drives libkvc's host code (entry-point validation, workspace geometry,
// overlap checks, the block pool, the budget schedules) for a build under
// AddressSanitizer and UndefinedBehaviorSanitizer. Kernels are stubbed
// (stubs.cpp): "device" buffers are fake, distinct addresses that the host
// code compares but never dereferences. Exits 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <random>
#include <set>
#include <vector>

#include "kvc.h"

extern "C" int kvc_stub_launches;

static int g_fail = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #c, kvc_last_error()); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

// Fake device address space: every buffer gets its own 1 GiB-aligned region.
static uintptr_t g_next = uintptr_t(1) << 40;
static void* fake(size_t = 0) {
  g_next += uintptr_t(1) << 30;
  return reinterpret_cast<void*>(g_next);
}

static kvc_cache_t cache(int bits, int B, int H, int D, int cap) {
  kvc_cache_t c;
  memset(&c, 0, sizeof c);
  c.bits = bits;
  c.batch = B;
  c.num_kv_heads = H;
  c.head_dim = D;
  c.capacity = cap;
  c.k_codes = fake();
  c.v_codes = fake();
  c.k_scale = (float*)fake();
  c.v_scale = (float*)fake();
  c.lengths = (int32_t*)fake();
  c.num_seen = (int32_t*)fake();
  c.positions = (int32_t*)fake();
  return c;
}

static void test_attention() {
  kvc_cache_t c = cache(8, 2, 4, 128, 4096);
  const int Hq = 16;
  const size_t need = kvc_decode_attn_workspace_bytes(&c, Hq, 4000, 1);
  CHECK(need > 0);
  void* ws = fake();
  void *q = fake(), *out = fake(), *score = fake(), *kn = fake(), *vn = fake();
  int before = kvc_stub_launches;
  CHECK(kvc_decode_attn(&c, q, Hq, (float*)out, (float*)score, 4000, ws, need, nullptr) == KVC_OK);
  CHECK(kvc_stub_launches > before);
  CHECK(kvc_append_decode_attn(&c, kn, vn, q, Hq, (float*)out, (float*)score, 3999, ws, need, nullptr) == KVC_OK);
  CHECK(kvc_decode_attn_split(&c, kn, vn, q, Hq, (float*)score, 3999, ws, need, nullptr) == KVC_OK);
  CHECK(kvc_decode_attn_merge(&c, 1, Hq, (float*)out, (float*)score, 3999, ws, need, nullptr) == KVC_OK);
  before = kvc_stub_launches;
  CHECK(kvc_decode_attn(&c, q, Hq, (float*)out, (float*)score, 4000, ws, need - 1, nullptr) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_decode_attn(&c, q, 6, (float*)out, (float*)score, 4000, ws, need, nullptr) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_decode_attn(&c, q, Hq, (float*)out, (float*)score, 4097, ws, need, nullptr) == KVC_ERR_CAPACITY);
  CHECK(kvc_decode_attn(&c, q, Hq, (float*)out, (float*)score, 4000, (char*)ws + 4, need, nullptr) ==
        KVC_ERR_INVALID_ARG);
  CHECK(kvc_stub_launches == before);  // nothing enqueued on an error
  // Every descriptor field that validation reads, out of range.
  for (int f = 0; f < 8; ++f) {
    kvc_cache_t d = c;
    switch (f) {
      case 0: d.bits = 5; break;
      case 1: d.batch = 0; break;
      case 2: d.head_dim = 96; break;
      case 3: d.capacity = 0; break;
      case 4: d.k_codes = nullptr; break;
      case 5: d.block_size = 8; break;
      case 6: d.v_bits = 3; break;
      case 7: d.fp16_sinks = 4; break;  // a tier without its buffers
    }
    CHECK(kvc_decode_attn(&d, q, Hq, (float*)out, nullptr, 16, ws, need, nullptr) != KVC_OK);
    CHECK(strlen(kvc_last_error()) > 0);
    CHECK(kvc_quant_append(&d, kn, vn, 1, nullptr, 0, nullptr) != KVC_OK);
  }
  CHECK(kvc_quant_append(&c, kn, vn, 96, (float*)score, 4000, nullptr) == KVC_OK);
  CHECK(kvc_quant_append(&c, kn, vn, 97, (float*)score, 4000, nullptr) == KVC_ERR_CAPACITY);
  // fp16 tiers, mixed widths, paged.
  kvc_cache_t t = c;
  t.v_bits = 4;
  t.fp16_sinks = 4;
  t.fp16_recent = 1000;
  t.k_sink16 = fake();
  t.v_sink16 = fake();
  t.k_recent16 = fake();
  t.v_recent16 = fake();
  const size_t tneed = kvc_decode_attn_workspace_bytes(&t, Hq, 4000, 1);
  CHECK(tneed > need);
  CHECK(kvc_decode_attn(&t, q, Hq, (float*)out, (float*)score, 4000, ws, tneed, nullptr) == KVC_OK);
  kvc_cache_t p = cache(8, 3, 4, 64, 512);
  p.block_size = 16;
  p.max_blocks_per_seq = 32;
  p.num_blocks = 50;
  p.positions = nullptr;
  p.block_table = (const int32_t*)fake();
  const size_t pneed = kvc_decode_attn_workspace_bytes(&p, 8, 512, 0);
  CHECK(kvc_decode_attn(&p, q, 8, (float*)out, nullptr, 512, ws, pneed, nullptr) == KVC_OK);
  // K/V separation.
  const size_t kneed = kvc_decode_attn_kvsep_workspace_bytes(&c, Hq, 1000, 4000);
  CHECK(kneed > 0);
  std::vector<char> host(64);
  CHECK(kvc_decode_attn_kvsep(&c, q, Hq, 1000, host.data(), (float*)out, 4000, ws, kneed, nullptr) == KVC_OK);
  CHECK(kvc_decode_attn_kvsep(&c, q, Hq, 0, host.data(), (float*)out, 4000, ws, kneed, nullptr) ==
        KVC_ERR_INVALID_ARG);
  // Bandwidth probe.
  void* sink = fake();
  CHECK(kvc_bw_probe(fake(), 1 << 20, sink, kvc_bw_probe_sink_bytes(), nullptr) == KVC_OK);
  CHECK(kvc_bw_probe(fake(), (1 << 20) + 3, sink, kvc_bw_probe_sink_bytes(), nullptr) == KVC_ERR_INVALID_ARG);
}

static void test_eviction() {
  const int B = 2, H = 4, cap = 9000, budget = 2457;
  kvc_cache_t s = cache(8, B, H, 128, cap), d = cache(8, B, H, 128, cap);
  void *score = fake(), *dscore = fake(), *kidx = fake(), *mask = fake();
  CHECK(kvc_h2o_select(&s, (float*)score, budget, 4, 1024, (uint8_t*)mask, (int32_t*)kidx, 8192, nullptr) == KVC_OK);
  CHECK(kvc_h2o_select(&s, (float*)score, 1000, 4, 1024, (uint8_t*)mask, nullptr, 8192, nullptr) ==
        KVC_ERR_INVALID_ARG);  // sinks + window above the budget
  CHECK(kvc_h2o_evict(&s, (float*)score, budget, 4, 1024, (uint8_t*)mask, (int32_t*)kidx, &d, (float*)dscore, 8192,
                      nullptr) == KVC_OK);
  CHECK(kvc_h2o_evict(&s, (float*)score, budget, 4, 1024, (uint8_t*)mask, (int32_t*)kidx, &d, (float*)dscore, 8999,
                      nullptr) == KVC_OK);  // past 8192 candidates: select + gather
  kvc_cache_t alias = d;
  alias.v_codes = s.k_codes;  // dst overlapping src
  const int before = kvc_stub_launches;
  CHECK(kvc_h2o_evict(&s, (float*)score, budget, 4, 1024, (uint8_t*)mask, (int32_t*)kidx, &alias, (float*)dscore,
                      8192, nullptr) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_stub_launches == before);
  const size_t cneed = kvc_compact_workspace_bytes(&s, 8192);
  CHECK(kvc_compact(&s, (float*)score, (uint8_t*)mask, &d, (float*)dscore, 8192, fake(), cneed, nullptr) == KVC_OK);
  CHECK(kvc_compact_gather(&s, (float*)score, (int32_t*)kidx, budget, &d, (float*)dscore, nullptr) == KVC_OK);
  // The whole step, with and without a caller workspace.
  const int Hq = 8;
  const size_t need = kvc_decode_attn_workspace_bytes(&s, Hq, 8192, 1);
  void *q = fake(), *out = fake(), *kn = fake(), *vn = fake();
  CHECK(kvc_decode_step(&s, kn, vn, q, Hq, (float*)out, (float*)score, budget, 4, 1024, (uint8_t*)mask,
                        (int32_t*)kidx, &d, (float*)dscore, 8191, fake(), need, nullptr) == KVC_OK);
  CHECK(kvc_decode_step_noalloc(&s, kn, vn, q, Hq, (float*)out, (float*)score, budget, 4, 1024, (uint8_t*)mask,
                                (int32_t*)kidx, &d, (float*)dscore, 8191, nullptr) == KVC_OK);
  CHECK(kvc_decode_step_noalloc(&s, kn, vn, q, Hq, (float*)out, (float*)score, budget, 4, 1024, (uint8_t*)mask,
                                (int32_t*)kidx, &d, (float*)dscore, 9000, nullptr) == KVC_ERR_CAPACITY);
  // In place (the cache is its own destination): one launch after the split
  // when the rows fit it, else the merge and selection kernels first.
  int n0 = kvc_stub_launches;
  CHECK(kvc_decode_step(&s, kn, vn, q, Hq, (float*)out, (float*)score, budget, 4, 1024, (uint8_t*)mask,
                        (int32_t*)kidx, &s, (float*)score, 8191, fake(), need, nullptr) == KVC_OK);
  CHECK(kvc_stub_launches == n0 + 2);
  n0 = kvc_stub_launches;
  kvc_cache_t big = cache(8, B, H, 128, 12000);
  const size_t need_long = kvc_decode_attn_workspace_bytes(&big, Hq, 11000, 1);
  void *bscore = fake(), *bmask = fake();
  CHECK(kvc_decode_step(&big, kn, vn, q, Hq, (float*)out, (float*)bscore, budget, 4, 1024, (uint8_t*)bmask,
                        (int32_t*)kidx, &big, (float*)bscore, 10999, fake(), need_long, nullptr) == KVC_OK);
  CHECK(kvc_stub_launches == n0 + 3);
  CHECK(kvc_decode_step_noalloc(&s, kn, vn, q, Hq, (float*)out, (float*)score, budget, 4, 1024, (uint8_t*)mask,
                                (int32_t*)kidx, &s, (float*)score, 8191, nullptr) == KVC_OK);
  kvc_cache_t part = s;
  part.v_codes = d.v_codes;  // shares only some buffers with the cache
  n0 = kvc_stub_launches;
  CHECK(kvc_decode_step(&s, kn, vn, q, Hq, (float*)out, (float*)score, budget, 4, 1024, (uint8_t*)mask,
                        (int32_t*)kidx, &part, (float*)score, 8191, fake(), need, nullptr) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_stub_launches == n0);
  // Block eviction on a paged cache.
  kvc_cache_t p = cache(8, 3, 4, 128, 512), pd;
  p.block_size = 16;
  p.max_blocks_per_seq = 32;
  p.num_blocks = 96;
  p.positions = nullptr;
  p.block_table = (const int32_t*)fake();
  pd = p;
  pd.block_table = (const int32_t*)fake();
  pd.lengths = (int32_t*)fake();
  pd.num_seen = (int32_t*)fake();
  const size_t bneed = kvc_paged_block_evict_workspace_bytes(&p);
  CHECK(kvc_paged_block_evict(&p, (float*)score, 0.5, &pd, (float*)dscore, (int32_t*)fake(), (int32_t*)fake(), 512,
                              fake(), bneed, nullptr) == KVC_OK);
  CHECK(kvc_paged_block_evict(&p, (float*)score, 1.5, &pd, (float*)dscore, (int32_t*)fake(), (int32_t*)fake(), 512,
                              fake(), bneed, nullptr) == KVC_ERR_INVALID_ARG);
}

// The pool against a plain model: per-sequence block lists and a free set.
static void test_pool() {
  CHECK(kvc_pool_create(0, 16, 1) == nullptr);
  const int NB = 200;
  kvc_pool_t* pool = kvc_pool_create(NB, 16, 12345);
  CHECK(pool != nullptr);
  std::map<int, std::vector<int32_t>> model;
  std::mt19937 rng(7);
  int free_blocks = NB;
  for (int step = 0; step < 20000; ++step) {
    const int op = rng() % 5, seq = rng() % 12;
    if (op == 0 || op == 1) {
      const int tokens = rng() % 400;
      const int have = model.count(seq) ? (int)model[seq].size() : 0;
      const int want = std::max(have, (tokens + 15) / 16);
      const int32_t st = kvc_pool_reserve(pool, seq, tokens);
      if (want - have <= free_blocks) {
        CHECK(st == KVC_OK);
        free_blocks -= want - have;
        std::vector<int32_t> t(64);
        int32_t id = seq;
        CHECK(kvc_pool_block_table(pool, &id, 1, 64, t.data()) == (want <= 64 ? KVC_OK : KVC_ERR_CAPACITY));
        std::vector<int32_t> blocks;
        for (int i = 0; i < want && i < 64; ++i) blocks.push_back(t[i]);
        if (want <= 64) {
          for (int i = 0; i < have; ++i) CHECK(blocks[i] == model[seq][i]);  // growth keeps the old blocks
          model[seq] = blocks;
        }
      } else {
        CHECK(st == KVC_ERR_CAPACITY);
      }
    } else if (op == 2) {
      CHECK(kvc_pool_free(pool, seq) == KVC_OK);
      if (model.count(seq)) {
        free_blocks += (int)model[seq].size();
        model.erase(seq);
      }
    } else if (op == 3 && model.count(seq) && !model[seq].empty()) {
      // Release a random subset (each block once).
      std::vector<int32_t> give;
      for (int32_t b : model[seq])
        if (rng() % 3 == 0) give.push_back(b);
      CHECK(kvc_pool_release(pool, seq, give.data(), (int32_t)give.size()) == KVC_OK);
      std::set<int32_t> g(give.begin(), give.end());
      std::vector<int32_t> left;
      for (int32_t b : model[seq])
        if (!g.count(b)) left.push_back(b);
      model[seq] = left;
      free_blocks += (int)give.size();
      int32_t bogus = NB + 5;
      CHECK(kvc_pool_release(pool, seq, &bogus, 1) == KVC_ERR_INVALID_ARG);
    } else {
      CHECK(kvc_pool_num_blocks(pool, seq) == (model.count(seq) ? (int)model[seq].size() : -1));
    }
    CHECK(kvc_pool_num_free(pool) == free_blocks);
  }
  // Every held block is distinct across sequences.
  std::set<int32_t> seen;
  for (auto& kv : model)
    for (int32_t b : kv.second) {
      CHECK(b >= 0 && b < NB);
      CHECK(seen.insert(b).second);
    }
  int32_t ids[2] = {0, 999};
  std::vector<int32_t> t(2 * 64);
  CHECK(kvc_pool_block_table(pool, ids, 2, 64, t.data()) == KVC_ERR_INVALID_ARG);  // unknown id
  CHECK(kvc_pool_reserve(pool, -1, 10) == KVC_ERR_INVALID_ARG);
  kvc_pool_destroy(pool);
  kvc_pool_destroy(nullptr);
  CHECK(kvc_pool_num_free(nullptr) == -1);
}

static void test_budgets() {
  std::vector<int32_t> b(80);
  CHECK(kvc_layer_budgets(KVC_SCHEDULE_LINEAR, 80, 8192, 0.0, 1028, b.data()) == KVC_OK);
  CHECK(b[0] == 8192);
  for (int l = 1; l < 80; ++l) CHECK(b[l] <= b[l - 1] && b[l] >= 1028);
  CHECK(kvc_layer_budgets(KVC_SCHEDULE_QUADRATIC, 80, 8192, 0.2, 1028, b.data()) == KVC_OK);
  for (int l = 1; l < 80; ++l) CHECK(b[l] >= b[l - 1]);
  CHECK(kvc_layer_budgets(KVC_SCHEDULE_QUADRATIC, 80, 8192, 1.5, 1028, b.data()) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_layer_budgets(7, 80, 8192, 0.2, 1028, b.data()) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_layer_budgets(KVC_SCHEDULE_LINEAR, 0, 8192, 0.2, 1028, b.data()) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_layer_budgets(KVC_SCHEDULE_LINEAR, 80, 8192, 0.2, 1028, nullptr) == KVC_ERR_INVALID_ARG);
}

int main() {
  CHECK(kvc_abi_version() == 4);
  CHECK(strcmp(kvc_status_str(KVC_ERR_CAPACITY), "KVC_ERR_CAPACITY") == 0);
  test_attention();
  test_eviction();
  test_pool();
  test_budgets();
  printf("host checks: %d failures, %d stub launches\n", g_fail, kvc_stub_launches);
  return g_fail ? 1 : 0;
}
