// Host-side logic of the C ABI: error state, descriptor validation, pool sizing,
// scaling, the SGMV/BGMV metadata builder and workspace sizing.  Nothing here
// touches the GPU, so every path is testable on a machine without one.
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

MetaLayout meta_layout(int32_t T, int32_t max_loras) {
  MetaLayout m;
  m.perm = 0;
  m.seg_starts = m.perm + T;
  m.seg_lens = m.seg_starts + max_loras;
  m.seg_ids = m.seg_lens + max_loras;
  m.bgmv_tok = m.seg_ids + max_loras;
  m.bgmv_ids = m.bgmv_tok + T;
  m.total_ints = m.bgmv_ids + T;
  return m;
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
  std::vector<int32_t> cnt_s(max_loras, 0), cnt_b(max_loras, 0);
  for (int32_t t = 0; t < T; ++t) {
    const int32_t a = ids[t];
    if (a < 0) continue;
    const bool sg = all_sgmv || (prefill && prefill[t]);
    (sg ? cnt_s : cnt_b)[a]++;
  }
  std::vector<int32_t> pos_s(max_loras), pos_b(max_loras);
  int32_t ns = 0, nb = 0, nseg = 0;
  for (int32_t a = 0; a < max_loras; ++a) {
    pos_s[a] = ns;
    pos_b[a] = nb;
    if (cnt_s[a] > 0) {
      out->seg_starts[nseg] = ns;
      out->seg_lens[nseg] = cnt_s[a];
      out->seg_ids[nseg] = a;
      ++nseg;
    }
    ns += cnt_s[a];
    nb += cnt_b[a];
  }
  for (int32_t t = 0; t < T; ++t) {
    const int32_t a = ids[t];
    if (a < 0) continue;
    const bool sg = all_sgmv || (prefill && prefill[t]);
    if (sg) {
      out->sgmv_perm[pos_s[a]++] = t;
    } else {
      const int32_t p = pos_b[a]++;
      out->bgmv_tok[p] = t;
      out->bgmv_ids[p] = a;
    }
  }
  out->num_sgmv_rows = ns;
  out->num_segs = nseg;
  out->num_bgmv_rows = nb;
  out->reserved = 0;
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
  for (int32_t t = 0; t < T; ++t) {
    if (ids[t] < -1 || ids[t] >= max_loras)
      return fail(LORA_E_ID, "ids[%d] = %d is outside [-1, %d)", t, ids[t], max_loras);
  }
  return build_meta_core(ids, prefill, T, max_loras, max_lora_rank, bgmv_max_rank, out);
}

int64_t lora_apply_host_meta_bytes(const lora_pool_desc* desc, int32_t T) {
  clear_error();
  Geo g;
  int32_t st = check_desc(desc, &g);
  if (st) return st;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  return meta_layout(T, g.max_loras).total_ints * 4;
}

int64_t lora_apply_workspace_bytes(const lora_pool_desc* desc, int32_t T) {
  clear_error();
  Geo g;
  int32_t st = check_desc(desc, &g);
  if (st) return st;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  const int64_t meta = align_up(meta_layout(T, g.max_loras).total_ints * 4, 256);
  return meta + (int64_t)T * g.S * g.R * 4;
}

}  // extern "C"
