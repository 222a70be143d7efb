// Host-side logic of the C ABI: error state, descriptor validation, pool sizing,
// scaling, the SGMV/BGMV metadata builder and workspace sizing.  Nothing here
// touches the GPU, so every path is testable on a machine without one.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "lora_internal.h"

namespace lora {

static thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

bool log_enabled() {
  const char* e = std::getenv("LORA_POOL_LOG");
  return e && e[0] && e[0] != '0';
}

int32_t check_desc(const lora_pool_desc* d, Geo* g) {
  if (!d) return fail(LORA_E_ARG, "descriptor is NULL");
  if (d->dtype != LORA_F32 && d->dtype != LORA_BF16)
    return fail(LORA_E_DTYPE, "unknown dtype %d (0 = fp32, 1 = bf16)", d->dtype);
  if (d->max_loras < 1) return fail(LORA_E_SHAPE, "max_loras must be >= 1, got %d", d->max_loras);
  if (d->num_slices < 1 || d->num_slices > LORA_MAX_SLICES)
    return fail(LORA_E_SHAPE, "num_slices must be in [1, %d], got %d", LORA_MAX_SLICES,
                d->num_slices);
  if (d->max_lora_rank < 8) return fail(LORA_E_RANK, "max_lora_rank must be >= 8, got %d",
                                         d->max_lora_rank);
  if (d->max_lora_rank % 8)
    return fail(LORA_E_ALIGN, "max_lora_rank must be a multiple of 8, got %d", d->max_lora_rank);
  if (d->in_features < 8 || d->in_features % 8)
    return fail(d->in_features < 8 ? LORA_E_SHAPE : LORA_E_ALIGN,
                "in_features must be a positive multiple of 8, got %d", d->in_features);
  int64_t O = 0;
  for (int s = 0; s < d->num_slices; ++s) {
    int32_t o = d->out_features[s];
    if (o < 8 || o % 8)
      return fail(o < 8 ? LORA_E_SHAPE : LORA_E_ALIGN,
                  "out_features[%d] must be a positive multiple of 8, got %d", s, o);
    O += o;
  }
  if (O > (int64_t)1 << 30) return fail(LORA_E_SHAPE, "total out_features too large");
  const int64_t eb = elem_bytes(d->dtype);
  const int64_t a_bytes = (int64_t)d->max_loras * d->num_slices * d->max_lora_rank *
                          (int64_t)d->in_features * eb;
  const int64_t b_bytes = (int64_t)d->max_loras * O * d->max_lora_rank * eb;
  if (a_bytes <= 0 || b_bytes <= 0 || a_bytes > ((int64_t)1 << 40) || b_bytes > ((int64_t)1 << 40))
    return fail(LORA_E_SHAPE, "pool too large");
  if (g) {
    g->dtype = d->dtype;
    g->max_loras = d->max_loras;
    g->R = d->max_lora_rank;
    g->K = d->in_features;
    g->S = d->num_slices;
    g->O = (int32_t)O;
    g->T = 0;
    int32_t acc = 0;
    for (int s = 0; s < LORA_MAX_SLICES; ++s) {
      g->out[s] = s < d->num_slices ? d->out_features[s] : 0;
      g->off[s] = acc;
      acc += g->out[s];
    }
  }
  return LORA_OK;
}

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

StageLayout stage_layout(int32_t T, int32_t max_loras) {
  StageLayout m;
  const int64_t t = T, ml = max_loras;
  m.perm = 0;
  m.seg_starts = m.perm + t;
  m.seg_lens = m.seg_starts + ml;
  m.seg_ids = m.seg_lens + ml;
  m.bgmv_tok = m.seg_ids + ml;
  m.bgmv_ids = m.bgmv_tok + t;
  m.image = align_up(m.bgmv_ids + t, 4);
  // Every segment (at most max_loras) and every run of equal BGMV ids (at most
  // max_loras) adds at most one partial tile: wave tiles <= ceil(T / 8) +
  // 2 max_loras, MFMA tiles <= ceil(T / 64) + 2 max_loras.
  const int64_t wave = (t + LORA_PLAN_WAVE_ROWS - 1) / LORA_PLAN_WAVE_ROWS + 2 * ml;
  const int64_t mfma = (t + LORA_PLAN_MFMA_ROWS - 1) / LORA_PLAN_MFMA_ROWS + 2 * ml;
  m.image_max_words = align_up(t, 4) + LORA_PLAN_WAVE_WORDS * wave + LORA_PLAN_MFMA_WORDS * mfma;
  m.total_words = m.image + m.image_max_words;
  return m;
}

static int32_t env_rows(const char* name, long dflt) {
  const char* e = std::getenv(name);
  const long x = e ? std::strtol(e, nullptr, 10) : dflt;
  return (int32_t)(x < 1 ? 1 : x > INT32_MAX ? INT32_MAX : x);
}

WorkspaceLayout workspace_layout(const Geo& g, int32_t T) {
  WorkspaceLayout w;
  w.v = align_up(stage_layout(T, g.max_loras).image_max_words * 4, 256);
  w.total = w.v + (int64_t)LORA_PLAN_MAX_KSPLIT * T * g.S * g.R * 4;
  return w;
}

DeviceLayout device_layout(const Geo& g, int32_t T) {
  DeviceLayout d;
  const int64_t rows = T > 0 ? T : 1, ml = g.max_loras;
  int64_t o = 0;
  d.counts = o;
  o = align_up(o + 4 * 4, 256);
  d.sgmv_perm = o;
  o = align_up(o + rows * 4, 16);
  d.bgmv_tok = o;
  o = align_up(o + rows * 4, 16);
  d.bgmv_ids = o;
  o = align_up(o + rows * 4, 16);
  d.seg_starts = o;
  o = align_up(o + ml * 4, 16);
  d.seg_lens = o;
  o = align_up(o + ml * 4, 16);
  d.seg_ids = o;
  o = align_up(o + ml * 4, 16);
  d.perm = o;
  o = align_up(o + rows * 4, 256);
  d.tiles = o;
  o = align_up(o + (int64_t)device_tile_cap(T, g.max_loras) * LORA_PLAN_WAVE_WORDS * 4, 256);
  d.mtiles = o;
  o = align_up(o + (int64_t)device_mfma_cap(g, T, true) * LORA_PLAN_MFMA_WORDS * 4, 256);
  d.v = o;
  d.total = o + (int64_t)LORA_PLAN_MAX_KSPLIT * rows * g.S * g.R * 4;
  return d;
}

int32_t device_mfma_cap(const Geo& g, int32_t T, bool sgmv) {
  const int64_t ml = g.max_loras, t = T > 0 ? T : 0;
  const int64_t pieces = (t + LORA_PLAN_MFMA_ROWS - 1) / LORA_PLAN_MFMA_ROWS;
  const int64_t slot_bound = pieces + 2 * std::min(t, ml);
  int64_t runs = sgmv ? std::min(ml, t / sgmv_mfma_min_rows()) : 0;
  if (t >= bgmv_mfma_min_total(g.R)) runs += std::min(ml, t / bgmv_mfma_min_rows());
  const int64_t cap = runs > 0 ? std::min(slot_bound, pieces + runs) : 0;
  return (int32_t)cap;
}

int32_t sgmv_mfma_min_rows() {
  static const int32_t v = env_rows("LORA_SGMV_MFMA_MIN_ROWS", 16);
  return v;
}

int32_t bgmv_mfma_min_rows() {
  static const int32_t v = env_rows("LORA_BGMV_MFMA_MIN_ROWS", 48);
  return v;
}

int32_t bgmv_mfma_min_total(int32_t R) {
  // 0: no override; a 64-row tile reads each adapter row once where eight
  // 8-row tiles read it eight times, which pays sooner the more ranks there are
  static const int32_t v = env_rows("LORA_BGMV_MFMA_MIN_TOTAL", INT32_MAX);
  if (v != INT32_MAX) return v;
  return R <= 16 ? 2048 : 1024;
}

// Every id in [-1, max_loras): a min / max pass (vectorisable), then the
// first offending row for the message.
static int32_t check_ids(const int32_t* ids, int32_t T, int32_t max_loras) {
  int32_t lo = -1, hi = -1;
  for (int32_t t = 0; t < T; ++t) {
    lo = std::min(lo, ids[t]);
    hi = std::max(hi, ids[t]);
  }
  if (lo >= -1 && hi < max_loras) return LORA_OK;
  for (int32_t t = 0; t < T; ++t) {
    if (ids[t] < -1 || ids[t] >= max_loras)
      return fail(LORA_E_ID, "ids[%d] = %d is outside [-1, %d)", t, ids[t], max_loras);
  }
  return LORA_OK;
}

// Stable counting sort of the two row sets by adapter id.  Bucket sizes are a
// histogram over max_loras slots; an exclusive scan gives each id's first
// position; tokens are then placed in increasing index order, which keeps the
// sort stable.  SGMV segments are the non-empty buckets of the SGMV set.
int32_t build_meta_core(const int32_t* ids, const uint8_t* prefill, int32_t T,
                        int32_t max_loras, int32_t max_lora_rank, int32_t bgmv_max_rank,
                        lora_meta* out) {
  const int32_t limit = bgmv_max_rank > 0 ? bgmv_max_rank : LORA_BGMV_MAX_RANK_DEFAULT;
  const bool all_sgmv = max_lora_rank > limit;
  // per-slot counters and positions, kept per thread and reused, so a call
  // allocates nothing once it has seen its pool size: up to four interleaved
  // count tables of 2 max_loras + 1 keys (key 2 a + set, or 2 max_loras for a
  // row without adapter), then the SGMV and BGMV positions
  const size_t nk = 2 * (size_t)max_loras + 1;
  static thread_local std::vector<int32_t> scratch;
  if (scratch.size() < 4 * nk + 2 * (size_t)max_loras) scratch.resize(4 * nk + 2 * (size_t)max_loras);
  int32_t* cnt4 = scratch.data();
  int32_t* pos_s = cnt4 + 4 * nk;
  int32_t* pos_b = pos_s + max_loras;
  const bool per_row_set = !all_sgmv && prefill != nullptr;
  auto in_sgmv = [&](int32_t t) { return all_sgmv || (prefill && prefill[t]); };
  auto key_of = [&](int32_t t) {
    const int32_t a = ids[t];
    return a >= 0 ? 2 * a + (in_sgmv(t) ? 1 : 0) : 2 * max_loras;
  };
  // end of the run of rows with row t's key: once a run's second row matches,
  // the rest of the run is found 16 rows at a time (a compare the compiler
  // vectorises), so long runs cost little and runs of one row cost one test
  auto run_end = [&](int32_t t) {
    const int32_t a = ids[t];
    const bool sg = in_sgmv(t);
    int32_t u = t + 1;
    if (u < T && ids[u] == a && in_sgmv(u) == sg) {
      ++u;
      while (u + 16 <= T) {
        int32_t diff = 0;
        for (int i = 0; i < 16; ++i) diff |= ids[u + i] ^ a;
        if (per_row_set) {  // 16 flag bytes: all nonzero (SGMV run) or all zero
          uint64_t w[2];
          std::memcpy(w, prefill + u, sizeof(w));
          const uint64_t ones = 0x0101010101010101ull, highs = 0x8080808080808080ull;
          const bool any_zero_byte = (((w[0] - ones) & ~w[0]) | ((w[1] - ones) & ~w[1])) & highs;
          diff |= sg ? any_zero_byte : ((w[0] | w[1]) != 0);
        }
        if (diff) break;
        u += 16;
      }
      while (u < T && ids[u] == a && in_sgmv(u) == sg) ++u;
    }
    return u;
  };
  // The first rows decide how the batch is walked.  Long runs of one key (a
  // sorted prefill batch) go run by run: one counter or position update per
  // run, where one per row would make a store-to-load chain on a single
  // counter.  Short runs (mixed decode ids) go row by row, the run search
  // being pure overhead there; in a batch that is large next to its count
  // table the histogram then counts row t in table t % 4, so equal neighbours
  // do not chain either.
  bool by_runs;
  {
    const int32_t n = std::min<int32_t>(T, 512);
    int32_t changes = 0;
    for (int32_t t = 1, prev = n > 0 ? key_of(0) : 0; t < n; ++t) {
      const int32_t k = key_of(t);
      changes += k != prev;
      prev = k;
    }
    by_runs = (int64_t)changes * 8 < n;
  }
  // 1. histogram (four tables only for batches large next to them: clearing
  //    and summing them costs more than the chains they break in small ones)
  const int32_t ntab = !by_runs && (int64_t)T >= 8 * (int64_t)nk ? 4 : 1;
  std::fill(cnt4, cnt4 + ntab * nk, 0);
  if (by_runs) {
    for (int32_t t = 0; t < T;) {
      const int32_t u = run_end(t);
      cnt4[key_of(t)] += u - t;
      t = u;
    }
  } else if (ntab == 4) {
    for (int32_t t = 0; t < T; ++t) ++cnt4[(size_t)(t & 3) * nk + key_of(t)];
  } else {
    for (int32_t t = 0; t < T; ++t) ++cnt4[key_of(t)];
  }
  int32_t ns = 0, nb = 0, nseg = 0;
  for (int32_t a = 0; a < max_loras; ++a) {
    int32_t cs = 0, cb = 0;
    for (int i = 0; i < ntab; ++i) {
      cs += cnt4[(size_t)i * nk + 2 * a + 1];
      cb += cnt4[(size_t)i * nk + 2 * a];
    }
    pos_s[a] = ns;
    pos_b[a] = nb;
    if (cs > 0) {
      out->seg_starts[nseg] = ns;
      out->seg_lens[nseg] = cs;
      out->seg_ids[nseg] = a;
      ++nseg;
    }
    ns += cs;
    nb += cb;
  }
  int32_t* const perm = out->sgmv_perm;
  int32_t* const btok = out->bgmv_tok;
  int32_t* const bids = out->bgmv_ids;
  // 2. placement in token order, which keeps the sort stable
  if (by_runs) {
    for (int32_t t = 0; t < T;) {
      const int32_t u = run_end(t);
      const int32_t a = ids[t];
      if (a >= 0) {
        if (in_sgmv(t)) {
          const int32_t p = pos_s[a];
          for (int32_t v = t; v < u; ++v) perm[p + (v - t)] = v;
          pos_s[a] = p + (u - t);
        } else {
          const int32_t p = pos_b[a];
          for (int32_t v = t; v < u; ++v) {
            btok[p + (v - t)] = v;
            bids[p + (v - t)] = a;
          }
          pos_b[a] = p + (u - t);
        }
      }
      t = u;
    }
  } else {
    // short runs (mixed decode ids): row by row
    for (int32_t t = 0; t < T; ++t) {
      const int32_t a = ids[t];
      if (a < 0) continue;
      if (in_sgmv(t)) {
        perm[pos_s[a]++] = t;
      } else {
        const int32_t p = pos_b[a]++;
        btok[p] = t;
        bids[p] = a;
      }
    }
  }
  out->num_sgmv_rows = ns;
  out->num_segs = nseg;
  out->num_bgmv_rows = nb;
  out->reserved = 0;
  return LORA_OK;
}

// Tile plan ([TGI] step 4: rows grouped by adapter, one adapter per tile).
// Runs of rows of one adapter (SGMV segments, and the runs of equal ids among
// the BGMV rows, which the builder sorts by id) are cut into tiles:
//   - MFMA tiles of LORA_PLAN_MFMA_ROWS rows (bf16 pools): SGMV segments of at
//     least sgmv_mfma_min_rows rows, and BGMV runs of at least
//     bgmv_mfma_min_rows rows when such runs hold at least bgmv_mfma_min_total
//     rows of the batch (a large decode batch; in a small one the extra MFMA
//     launches cost more than the dense tiles save);
//   - wavefront tiles of LORA_PLAN_WAVE_ROWS rows: every other run.
// v row numbering: SGMV rows first, then BGMV rows; perm holds the token of
// every v row.
// K split of the MFMA shrink: doubled while the launch has fewer than two
// workgroups per compute unit (256 CUs) and every split keeps at least four
// 64-wide K steps, up to 8 for pools of rank <= 32 (whose partials of v are
// small next to x) and 4 above
int32_t mfma_ksplit_max(const Geo& g) {
  return g.R > 32 ? LORA_PLAN_MAX_KSPLIT_MFMA_WIDE : LORA_PLAN_MAX_KSPLIT_MFMA;
}

int32_t mfma_ksplit(const Geo& g, int64_t nm, bool four_stages) {
  int32_t ksplit = 1;
  if (nm > 0) {
    const int64_t wgs = nm * g.S * ((g.R + 63) / 64);
    const int64_t ksteps = (g.K + 63) / 64;
    const int32_t top = mfma_ksplit_max(g);
    // a workgroup's rate is bounded by what its compute unit can pull, so the
    // time follows the compute unit with the most workgroups: ceil(wgs k /
    // kComputeUnits) workgroups of 1/k of a tile's K each.  Of the splits
    // that start below 512 workgroups (k - 1 parts of each tile fewer than
    // 512) and keep at least 4 K steps per part, take the one with the least
    // such load, the most parts on a tie (shorter workgroups)
    int64_t best_num = -1, best_den = 1;
    int32_t lone = 0;  // the most parts of a tie at one workgroup per compute unit
    for (int32_t k = 1; k <= top; ++k) {
      if (k > 1 && (wgs * (k - 1) >= 512 || ksteps / k < 4)) break;
      const int64_t num = (wgs * k + kComputeUnits - 1) / kComputeUnits;  // load num / k
      if (best_num >= 0 && num * best_den < best_num * k) lone = 0;  // a better load
      if (best_num < 0 || num * best_den <= best_num * k) {
        best_num = num;
        best_den = k;
        ksplit = k;
        if (wgs * k <= kComputeUnits) lone = k;
      }
    }
    // where the DMA-staged shrink runs four stages at one workgroup per unit,
    // such a split beats a tie at two workgroups per unit, and its expand sums
    // fewer partials (the 4096-row rank-16 decode: K split 8 -> 4, kernels
    // 28.0 -> 27.0 us); at three per unit the concurrent workgroups win
    // (gate_up: split 1 against 3, shrink 30.4 against 27.7 us)
    if (four_stages && lone > 0 && wgs * ksplit <= 2 * kComputeUnits) ksplit = lone;
    if (const char* e = std::getenv("LORA_MFMA_KSPLIT")) {  // tuning override: 1 .. top
      const long o = std::strtol(e, nullptr, 10);
      if (o >= 1 && o <= top) ksplit = (int32_t)o;
    }
  }
  return ksplit;
}

int32_t wave_ksplit(const Geo& g, int64_t nw) {
  int32_t ksplit_wave = 1;
  if (g.dtype == LORA_BF16 && nw > 0 && g.R <= 64) {
    const int64_t nk = (g.K + 31) / 32;
    const int64_t batch = (int64_t)kTileShrinkWaves * tile_shrink_cb(g.R);
    const int64_t wgs = nw * g.S;
    // a workgroup's rate is bounded by what its compute unit can pull, so the
    // time follows the compute unit with the most workgroups: ceil(wgs k /
    // kComputeUnits) workgroups of 1/k of a tile's K each.  Take the split
    // with the least such load (the fewest parts on a tie), among those that
    // keep at most four workgroups per compute unit and a full load batch per
    // wave in every part
    int64_t best_num = -1, best_den = 1;
    for (int32_t k = 1; k <= tile_kparts_max(g.R); ++k) {
      if (k > 1 && (wgs * k > 4 * kComputeUnits || nk / k < batch)) break;
      const int64_t num = (wgs * k + kComputeUnits - 1) / kComputeUnits;  // load num / k
      if (best_num < 0 || num * best_den < best_num * k) {
        best_num = num;
        best_den = k;
        ksplit_wave = k;
      }
    }
    if (const char* e = std::getenv("LORA_WAVE_KSPLIT")) {  // tuning override
      const long o = std::strtol(e, nullptr, 10);
      if (o >= 1 && o <= tile_kparts_max(g.R)) ksplit_wave = (int32_t)o;
    }
  }
  return ksplit_wave;
}

int32_t check_slot_ranks(const Geo& g, const int32_t* slot_ranks) {
  if (!slot_ranks) return LORA_OK;
  for (int32_t a = 0; a < g.max_loras; ++a) {
    if (slot_ranks[a] < 0 || slot_ranks[a] > g.R)
      return fail(LORA_E_RANK, "slot_ranks[%d] = %d is outside [0, max_lora_rank = %d]", a,
                  slot_ranks[a], g.R);
  }
  return LORA_OK;
}

int32_t plan_core(const Geo& g, int32_t T, const int32_t* ids, const uint8_t* prefill,
                  int32_t bgmv_max_rank, int32_t* stage, lora_plan* p,
                  const int32_t* slot_ranks) {
  // rank a tile record carries: 0 = the pool's R, else the slot's rank
  // rounded up to 8 (the kernels' vector width), below R
  auto rank_of = [&](int32_t slot) -> int32_t {
    if (!slot_ranks || slot_ranks[slot] <= 0) return 0;
    const int32_t r8 = (slot_ranks[slot] + 7) / 8 * 8;
    return r8 < g.R ? r8 : 0;
  };
  const StageLayout sl = stage_layout(T, g.max_loras);
  lora_meta m;
  m.sgmv_perm = stage + sl.perm;
  m.seg_starts = stage + sl.seg_starts;
  m.seg_lens = stage + sl.seg_lens;
  m.seg_ids = stage + sl.seg_ids;
  m.bgmv_tok = stage + sl.bgmv_tok;
  m.bgmv_ids = stage + sl.bgmv_ids;
  if (int32_t e = build_meta_core(ids, prefill, T, g.max_loras, g.R, bgmv_max_rank, &m)) return e;
  const int32_t ns = m.num_sgmv_rows, nb = m.num_bgmv_rows;
  const bool bf = g.dtype == LORA_BF16;
  const int32_t thr = bf ? sgmv_mfma_min_rows() : INT32_MAX;
  // end of the BGMV run starting at row i: the builder sorts the BGMV rows by
  // id, so past its first 16 rows (short runs of mixed decode ids end there,
  // where a search's unpredictable branches would cost more) a binary search
  // finds it
  auto run_end = [&](int32_t i) {
    const int32_t a = m.bgmv_ids[i];
    const int32_t lin = std::min(nb, i + 16);
    int32_t j = i + 1;
    while (j < lin && m.bgmv_ids[j] == a) ++j;
    if (j < lin || j == nb) return j;
    return (int32_t)(std::upper_bound(m.bgmv_ids + j, m.bgmv_ids + nb, a) - m.bgmv_ids);
  };
  int32_t bthr = INT32_MAX;
  if (bf) {
    int64_t long_rows = 0;
    for (int32_t i = 0; i < nb;) {
      const int32_t j = run_end(i);
      if (j - i >= bgmv_mfma_min_rows()) long_rows += j - i;
      i = j;
    }
    if (long_rows > 0 && long_rows >= bgmv_mfma_min_total(g.R)) bthr = bgmv_mfma_min_rows();
  }
  int32_t* img = stage + sl.image;
  const int64_t off_wave = align_up((int64_t)ns + nb, 4);
  std::memcpy(img, m.sgmv_perm, sizeof(int32_t) * (size_t)ns);
  std::memcpy(img + ns, m.bgmv_tok, sizeof(int32_t) * (size_t)nb);
  for (int64_t i = (int64_t)ns + nb; i < off_wave; ++i) img[i] = -1;
  int32_t* wave = img + off_wave;
  int64_t nw = 0;
  auto emit_wave = [&](int32_t slot, int32_t first, int32_t rows, const int32_t* tok) {
    int32_t* r = wave + nw * LORA_PLAN_WAVE_WORDS;
    r[0] = slot;
    r[1] = rows;
    r[2] = first;
    r[3] = rank_of(slot);
    for (int i = 4; i < LORA_PLAN_WAVE_WORDS; ++i) r[i] = -1;
    for (int i = 0; i < rows; ++i) r[4 + i] = tok[i];
    ++nw;
  };
  for (int32_t s = 0; s < m.num_segs; ++s) {
    const int32_t st = m.seg_starts[s], ln = m.seg_lens[s];
    if (ln >= thr) continue;
    for (int32_t j = 0; j < ln; j += LORA_PLAN_WAVE_ROWS)
      emit_wave(m.seg_ids[s], st + j, std::min(LORA_PLAN_WAVE_ROWS, ln - j), m.sgmv_perm + st + j);
  }
  for (int32_t i = 0; i < nb;) {
    const int32_t j = run_end(i);
    if (j - i < bthr) {
      for (int32_t k = i; k < j; k += LORA_PLAN_WAVE_ROWS)
        emit_wave(m.bgmv_ids[i], ns + k, std::min(LORA_PLAN_WAVE_ROWS, j - k), m.bgmv_tok + k);
    }
    i = j;
  }
  const int64_t off_mfma = off_wave + nw * LORA_PLAN_WAVE_WORDS;
  int32_t* mt = img + off_mfma;
  int64_t nm = 0;
  // word 3: the tile's first token when its tokens are consecutive (a prefill
  // sequence usually is), so the kernels need not read them from perm; else -1.
  // A run's tokens increase (the sort is stable), so they are consecutive
  // exactly when last - first = rows - 1
  auto emit_mfma = [&](int32_t slot, int32_t first, int32_t len) {
    for (int32_t j = 0; j < len; j += LORA_PLAN_MFMA_ROWS) {
      int32_t* r = mt + nm * LORA_PLAN_MFMA_WORDS;
      const int32_t rows = std::min(LORA_PLAN_MFMA_ROWS, len - j);
      const int32_t* tok = img + first + j;
      const bool consecutive = tok[rows - 1] - tok[0] == rows - 1;
      r[0] = slot;
      r[1] = rows | (rank_of(slot) << 16);
      r[2] = first + j;
      r[3] = consecutive ? tok[0] : -1;
      ++nm;
    }
  };
  for (int32_t s = 0; s < m.num_segs; ++s) {
    if (m.seg_lens[s] >= thr) emit_mfma(m.seg_ids[s], m.seg_starts[s], m.seg_lens[s]);
  }
  for (int32_t i = 0; i < nb;) {
    const int32_t j = run_end(i);
    if (j - i >= bthr) emit_mfma(m.bgmv_ids[i], ns + i, j - i);
    i = j;
  }
  const int64_t words = off_mfma + nm * LORA_PLAN_MFMA_WORDS;
  const int32_t ksplit = mfma_ksplit(g, nm, g.K % 64 == 0 && g.K <= kDmaShrinkMaxK);
  const int32_t ksplit_wave = wave_ksplit(g, nw);
  if (words > sl.image_max_words)  // cannot happen: the bounds above hold for any batch
    return fail(LORA_E_WORKSPACE, "tile plan overflow (%lld words > %lld)", (long long)words,
                (long long)sl.image_max_words);
  p->num_sgmv_rows = ns;
  p->num_bgmv_rows = nb;
  p->num_segs = m.num_segs;
  p->wave_tiles = (int32_t)nw;
  p->mfma_tiles = (int32_t)nm;
  p->mfma_min_rows = thr;
  p->ksplit = ksplit;
  p->bgmv_mfma_min_rows = bthr;
  p->ksplit_wave = ksplit_wave;
  p->reserved = 0;
  p->image_offset = sl.image * 4;
  p->image_bytes = words * 4;
  p->off_perm = 0;
  p->off_wave = off_wave;
  p->off_mfma = off_mfma;
  return LORA_OK;
}

}  // namespace lora

using namespace lora;

extern "C" {

const char* lora_last_error(void) { return g_last_error.c_str(); }

int32_t lora_abi_version(void) { return LORA_POOL_ABI_VERSION; }

int32_t lora_pool_validate(const lora_pool_desc* desc) {
  clear_error();
  return check_desc(desc, nullptr);
}

int64_t lora_pool_bytes_A(const lora_pool_desc* desc) {
  clear_error();
  Geo g;
  int32_t st = check_desc(desc, &g);
  if (st) return st;
  return (int64_t)g.max_loras * g.S * g.R * (int64_t)g.K * elem_bytes(g.dtype);
}

int64_t lora_pool_bytes_B(const lora_pool_desc* desc) {
  clear_error();
  Geo g;
  int32_t st = check_desc(desc, &g);
  if (st) return st;
  return (int64_t)g.max_loras * g.O * (int64_t)g.R * elem_bytes(g.dtype);
}

float lora_scaling(int32_t r, float alpha, int32_t use_rslora) {
  if (r <= 0) return NAN;
  const double dr = (double)r;
  const double s = use_rslora ? (double)alpha / std::sqrt(dr) : (double)alpha / dr;
  return (float)s;
}

int32_t lora_build_meta(const int32_t* ids, const uint8_t* prefill, int32_t T,
                        int32_t max_loras, int32_t max_lora_rank, int32_t bgmv_max_rank,
                        lora_meta* out) {
  clear_error();
  if (!out) return fail(LORA_E_ARG, "out is NULL");
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  if (max_loras < 1) return fail(LORA_E_SHAPE, "max_loras must be >= 1, got %d", max_loras);
  if (T > 0 && !ids) return fail(LORA_E_ARG, "ids is NULL");
  if (!out->seg_starts || !out->seg_lens || !out->seg_ids)
    return fail(LORA_E_ARG, "segment arrays must not be NULL");
  if (T > 0 && (!out->sgmv_perm || !out->bgmv_tok || !out->bgmv_ids))
    return fail(LORA_E_ARG, "row arrays must not be NULL");
  if (int32_t e = check_ids(ids, T, max_loras)) return e;
  return build_meta_core(ids, prefill, T, max_loras, max_lora_rank, bgmv_max_rank, out);
}

int64_t lora_apply_host_meta_bytes(const lora_pool_desc* desc, int32_t T) {
  clear_error();
  Geo g;
  int32_t st = check_desc(desc, &g);
  if (st) return st;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  return stage_layout(T, g.max_loras).total_words * 4;
}

int64_t lora_apply_device_workspace_bytes(const lora_pool_desc* desc, int32_t T) {
  clear_error();
  Geo g;
  int32_t st = check_desc(desc, &g);
  if (st) return st;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  if (g.max_loras > LORA_META_DEVICE_MAX_LORAS)
    return fail(LORA_E_SHAPE, "max_loras must be <= %d for the device plan, got %d",
                LORA_META_DEVICE_MAX_LORAS, g.max_loras);
  return device_layout(g, T).total;
}

int64_t lora_apply_workspace_bytes(const lora_pool_desc* desc, int32_t T) {
  clear_error();
  Geo g;
  int32_t st = check_desc(desc, &g);
  if (st) return st;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  return workspace_layout(g, T).total;
}

int32_t lora_apply_plan(const lora_pool_desc* desc, int32_t T, const int32_t* ids_host,
                        const uint8_t* prefill_host, int32_t bgmv_max_rank, void* meta_host,
                        int64_t meta_host_bytes, lora_plan* plan) {
  return lora_apply_plan_ranked(desc, T, ids_host, prefill_host, bgmv_max_rank, nullptr,
                                meta_host, meta_host_bytes, plan);
}

int32_t lora_apply_plan_ranked(const lora_pool_desc* desc, int32_t T, const int32_t* ids_host,
                               const uint8_t* prefill_host, int32_t bgmv_max_rank,
                               const int32_t* slot_ranks, void* meta_host,
                               int64_t meta_host_bytes, lora_plan* plan) {
  clear_error();
  Geo g;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  if (!plan) return fail(LORA_E_ARG, "plan is NULL");
  if (T > 0 && !ids_host) return fail(LORA_E_ARG, "ids_host is NULL");
  if (!meta_host) return fail(LORA_E_ARG, "meta_host is NULL");
  if ((uintptr_t)meta_host % 16) return fail(LORA_E_ALIGN, "meta_host is not 16-byte aligned");
  const int64_t need = stage_layout(T, g.max_loras).total_words * 4;
  if (meta_host_bytes < need)
    return fail(LORA_E_WORKSPACE, "meta_host has %lld bytes, needs %lld",
                (long long)meta_host_bytes, (long long)need);
  if (int32_t e = check_ids(ids_host, T, g.max_loras)) return e;
  if (int32_t e = check_slot_ranks(g, slot_ranks)) return e;
  return plan_core(g, T, ids_host, prefill_host, bgmv_max_rank, (int32_t*)meta_host, plan,
                   slot_ranks);
}

}  // extern "C"
