// Host logic of the library (lora_host.cpp: validation, the segment/index
// builder of [TGI] step 4 and the tile plan) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Built with g++ on the CPU by
// tests/test_host_sanitize.py together with lora_host.cpp only (no HIP code).
//
// Every output buffer is allocated with exactly the size the header promises
// (lora_apply_host_meta_bytes, T entries per metadata array, max_loras per
// segment array), so a write past any of them is reported by the sanitizer.
// The outputs are also checked for what the header states: each set sorted by
// (id, token) and stable, segments the maximal runs, every v row in exactly one
// tile record whose slot and tokens agree with the metadata, and every error
// reported before anything is written.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "lora_pool.h"

static int g_fail = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);    \
      if (++g_fail > 20) std::exit(1);                                        \
    }                                                                         \
  } while (0)

// exact-size heap copy, so the sanitizer sees the true bounds
template <typename T> static T* exact(size_t n) {
  return static_cast<T*>(std::malloc(n ? n * sizeof(T) : 1));
}

struct Batch {
  std::vector<int32_t> ids;
  std::vector<uint8_t> prefill;
};

static Batch draw_batch(std::mt19937_64& rng, int32_t T, int32_t max_loras) {
  Batch b;
  b.ids.resize(T);
  b.prefill.resize(T);
  std::uniform_int_distribution<int32_t> id(-1, max_loras - 1);
  const int kind = (int)(rng() % 4);
  int32_t t = 0;
  while (t < T) {
    // runs of one id: single rows (decode), short or long runs (prefill)
    int32_t len = kind == 0 ? 1 : 1 + (int32_t)(rng() % (kind == 1 ? 8 : kind == 2 ? 200 : 3000));
    len = std::min(len, T - t);
    const int32_t a = id(rng);
    // flags other than 0/1 count as prefill
    const uint8_t p = (rng() % 3 == 0) ? 0 : (uint8_t)(1 + rng() % 255);
    const bool per_row = rng() % 4 == 0;
    for (int32_t i = 0; i < len; ++i) {
      b.ids[t + i] = a;
      b.prefill[t + i] = per_row ? (uint8_t)(rng() % 2) : p;
    }
    t += len;
  }
  if (rng() % 5 == 0) std::sort(b.ids.begin(), b.ids.end());
  return b;
}

// lora_build_meta on exact-size arrays; returns the status, checks invariants
static int32_t run_meta(const Batch& b, int32_t max_loras, int32_t R, int32_t bgmv_max_rank,
                        bool null_prefill) {
  const int32_t T = (int32_t)b.ids.size();
  int32_t* ids = exact<int32_t>(T);
  uint8_t* pre = null_prefill ? nullptr : exact<uint8_t>(T);
  if (T > 0) std::memcpy(ids, b.ids.data(), sizeof(int32_t) * T);
  if (pre && T > 0) std::memcpy(pre, b.prefill.data(), T);
  lora_meta m;
  m.sgmv_perm = exact<int32_t>(T);
  m.bgmv_tok = exact<int32_t>(T);
  m.bgmv_ids = exact<int32_t>(T);
  m.seg_starts = exact<int32_t>(max_loras);
  m.seg_lens = exact<int32_t>(max_loras);
  m.seg_ids = exact<int32_t>(max_loras);
  const int32_t st = lora_build_meta(ids, pre, T, max_loras, R, bgmv_max_rank, &m);
  if (st == LORA_OK) {
    const int32_t limit = bgmv_max_rank > 0 ? bgmv_max_rank : LORA_BGMV_MAX_RANK_DEFAULT;
    std::vector<int32_t> sg, bg;
    for (int32_t t = 0; t < T; ++t) {
      if (ids[t] < 0) continue;
      ((R > limit || (pre && pre[t])) ? sg : bg).push_back(t);
    }
    auto key = [&](int32_t u, int32_t v) { return ids[u] != ids[v] ? ids[u] < ids[v] : u < v; };
    std::sort(sg.begin(), sg.end(), key);
    std::sort(bg.begin(), bg.end(), key);
    CHECK(m.num_sgmv_rows == (int32_t)sg.size() && m.num_bgmv_rows == (int32_t)bg.size());
    for (size_t i = 0; i < sg.size(); ++i) CHECK(m.sgmv_perm[i] == sg[i]);
    for (size_t i = 0; i < bg.size(); ++i) CHECK(m.bgmv_tok[i] == bg[i] && m.bgmv_ids[i] == ids[bg[i]]);
    int32_t pos = 0;
    for (int32_t s = 0; s < m.num_segs; ++s) {
      CHECK(m.seg_starts[s] == pos && m.seg_lens[s] > 0);
      CHECK(s == 0 || m.seg_ids[s] > m.seg_ids[s - 1]);
      for (int32_t i = 0; i < m.seg_lens[s]; ++i) CHECK(ids[m.sgmv_perm[pos + i]] == m.seg_ids[s]);
      pos += m.seg_lens[s];
    }
    CHECK(pos == m.num_sgmv_rows);
  }
  std::free(ids);
  std::free(pre);
  for (int32_t* p : {m.sgmv_perm, m.bgmv_tok, m.bgmv_ids, m.seg_starts, m.seg_lens, m.seg_ids})
    std::free(p);
  return st;
}

// lora_apply_plan(_ranked) into an exact-size staging buffer; checks coverage
static int32_t run_plan(const lora_pool_desc& d, const Batch& b, int32_t bgmv_max_rank,
                        const int32_t* slot_ranks) {
  const int32_t T = (int32_t)b.ids.size();
  const int64_t bytes = lora_apply_host_meta_bytes(&d, T);
  CHECK(bytes > 0);
  // 16-byte aligned, exactly `bytes` long
  void* stage = std::aligned_alloc(16, (size_t)((bytes + 15) / 16 * 16));
  int32_t* ids = exact<int32_t>(T);
  uint8_t* pre = exact<uint8_t>(T);
  if (T > 0) {
    std::memcpy(ids, b.ids.data(), sizeof(int32_t) * T);
    std::memcpy(pre, b.prefill.data(), T);
  }
  lora_plan p;
  const int32_t st = slot_ranks
      ? lora_apply_plan_ranked(&d, T, ids, pre, bgmv_max_rank, slot_ranks, stage, bytes, &p)
      : lora_apply_plan(&d, T, ids, pre, bgmv_max_rank, stage, bytes, &p);
  if (st == LORA_OK) {
    CHECK(p.image_offset % 16 == 0 && p.image_offset + p.image_bytes <= bytes);
    const int32_t* img = (const int32_t*)((const char*)stage + p.image_offset);
    const int32_t rows = p.num_sgmv_rows + p.num_bgmv_rows;
    std::vector<int> covered(rows, 0);
    const int32_t R = d.max_lora_rank;
    for (int32_t w = 0; w < p.wave_tiles; ++w) {
      const int32_t* r = img + p.off_wave + (int64_t)w * LORA_PLAN_WAVE_WORDS;
      CHECK(r[1] >= 1 && r[1] <= LORA_PLAN_WAVE_ROWS && r[2] >= 0 && r[2] + r[1] <= rows);
      CHECK(r[3] == 0 || (r[3] % 8 == 0 && r[3] < R));
      for (int32_t i = 0; i < r[1] && r[2] + i < rows; ++i) {
        ++covered[r[2] + i];
        CHECK(r[4 + i] == img[p.off_perm + r[2] + i] && ids[r[4 + i]] == r[0]);
      }
    }
    for (int32_t w = 0; w < p.mfma_tiles; ++w) {
      const int32_t* r = img + p.off_mfma + (int64_t)w * LORA_PLAN_MFMA_WORDS;
      const int32_t n = r[1] & 0xffff, rk = r[1] >> 16;
      CHECK(n >= 1 && n <= LORA_PLAN_MFMA_ROWS && r[2] >= 0 && r[2] + n <= rows);
      CHECK(rk == 0 || (rk % 8 == 0 && rk < R));
      bool consecutive = true;
      for (int32_t i = 0; i < n && r[2] + i < rows; ++i) {
        ++covered[r[2] + i];
        const int32_t t = img[p.off_perm + r[2] + i];
        CHECK(ids[t] == r[0]);
        consecutive &= t == img[p.off_perm + r[2]] + i;
      }
      CHECK(r[3] == (consecutive ? img[p.off_perm + r[2]] : -1));
    }
    for (int32_t i = 0; i < rows; ++i) CHECK(covered[i] == 1);
    CHECK(p.ksplit >= 1 && p.ksplit <= LORA_PLAN_MAX_KSPLIT_MFMA);
    CHECK(p.ksplit_wave >= 1 && p.ksplit_wave <= LORA_PLAN_MAX_KSPLIT);
    CHECK(lora_apply_workspace_bytes(&d, T) > 0);
    CHECK(lora_apply_device_workspace_bytes(&d, T) > 0);
  }
  std::free(stage);
  std::free(ids);
  std::free(pre);
  return st;
}

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 400;
  std::mt19937_64 rng(20260);
  const int32_t ranks[] = {8, 16, 24, 32, 64, 72, 128};
  int ok = 0, rejected = 0;
  for (int c = 0; c < cases; ++c) {
    lora_pool_desc d{};
    d.dtype = rng() % 3 ? LORA_BF16 : LORA_F32;
    d.max_loras = 1 + (int32_t)(rng() % (c % 10 == 0 ? 5000 : 300));
    d.max_lora_rank = ranks[rng() % 7];
    d.in_features = 8 * (1 + (int32_t)(rng() % 1024));
    d.num_slices = 1 + (int32_t)(rng() % 3);
    for (int s = 0; s < d.num_slices; ++s) d.out_features[s] = 8 * (1 + (int32_t)(rng() % 2048));
    CHECK(lora_pool_validate(&d) == LORA_OK);
    const int32_t T = c % 7 == 0 ? 0 : (int32_t)(rng() % (c % 13 == 0 ? 70000 : 5000));
    Batch b = draw_batch(rng, T, d.max_loras);
    const bool bad = T > 0 && rng() % 8 == 0;
    if (bad) b.ids[rng() % T] = (rng() % 2) ? d.max_loras + (int32_t)(rng() % 5) : -2 - (int32_t)(rng() % 5);
    const int32_t bmr = rng() % 4 == 0 ? (int32_t)(8 * (rng() % 20)) : 0;
    const int32_t s1 = run_meta(b, d.max_loras, d.max_lora_rank, bmr, rng() % 5 == 0);
    CHECK(bad ? s1 == LORA_E_ID : s1 == LORA_OK);
    std::vector<int32_t> sr;
    const bool ranked = rng() % 2;
    if (ranked) {
      sr.resize(d.max_loras);
      for (auto& r : sr) r = (int32_t)(rng() % (d.max_lora_rank + 1));
    }
    int32_t* srp = nullptr;
    if (ranked) {
      srp = exact<int32_t>(d.max_loras);
      std::memcpy(srp, sr.data(), sizeof(int32_t) * d.max_loras);
    }
    const int32_t s2 = run_plan(d, b, bmr, srp);
    CHECK(bad ? s2 == LORA_E_ID : s2 == LORA_OK);
    if (ranked && d.max_loras > 0 && !bad) {  // a rank above R is rejected
      srp[rng() % d.max_loras] = d.max_lora_rank + 1;
      CHECK(run_plan(d, b, bmr, srp) == LORA_E_RANK);
    }
    std::free(srp);
    (bad ? rejected : ok) += 1;
  }
  // malformed descriptors and arguments: rejected, nothing dereferenced
  lora_pool_desc d{};
  CHECK(lora_pool_validate(nullptr) != LORA_OK);
  CHECK(lora_pool_validate(&d) != LORA_OK);
  d.dtype = LORA_BF16;
  d.max_loras = 2;
  d.max_lora_rank = 12;  // not a multiple of 8
  d.in_features = 64;
  d.num_slices = 1;
  d.out_features[0] = 64;
  CHECK(lora_pool_validate(&d) != LORA_OK);
  d.max_lora_rank = 16;
  d.num_slices = LORA_MAX_SLICES + 1;
  CHECK(lora_pool_validate(&d) != LORA_OK);
  d.num_slices = 1;
  CHECK(lora_build_meta(nullptr, nullptr, 4, 2, 16, 0, nullptr) != LORA_OK);
  lora_plan p;
  CHECK(lora_apply_plan(&d, 4, nullptr, nullptr, 0, nullptr, 0, &p) != LORA_OK);
  int32_t ids4[4] = {0, 1, -1, 0};
  alignas(16) int32_t small[4];
  CHECK(lora_apply_plan(&d, 4, ids4, nullptr, 0, small, sizeof(small), &p) == LORA_E_WORKSPACE);
  CHECK(lora_scaling(16, 32.0f, 0) == 2.0f && lora_scaling(16, 16.0f, 1) == 4.0f);
  std::printf("host_sanitize: %d batches planned, %d rejected ids, %d failed checks\n", ok,
              rejected, g_fail);
  return g_fail ? 1 : 0;
}
