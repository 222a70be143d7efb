// C ABI entry points that touch the GPU: pool load / clear, the four grouped
// shrink / expand operations and the lora_apply dispatcher.  Every argument is
// validated before the first HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "lora_internal.h"
#include "lora_kernels.h"

using namespace lora;

namespace {

uint16_t host_f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float host_bf16_to_f32(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int32_t hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LORA_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return LORA_OK;
}

int32_t need_ptr(const void* p, const char* name) {
  if (!p) return fail(LORA_E_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(LORA_E_ALIGN, "%s is not 16-byte aligned", name);
  return LORA_OK;
}

int32_t check_rows(int32_t n, int32_t T, const char* what) {
  if (n < 0) return fail(LORA_E_ARG, "%s must be >= 0, got %d", what, n);
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  return LORA_OK;
}

int32_t check_common(const lora_pool_desc* desc, Geo* g, const void* act, const char* act_name,
                     const void* pool, const char* pool_name, const void* v) {
  if (int32_t e = check_desc(desc, g)) return e;
  if (int32_t e = need_ptr(act, act_name)) return e;
  if (int32_t e = need_ptr(pool, pool_name)) return e;
  if (int32_t e = need_ptr(v, "v")) return e;
  return LORA_OK;
}

int32_t sgmv_args(const int32_t* perm, const int32_t* seg_starts, const int32_t* seg_lens,
                  const int32_t* seg_ids, int32_t num_segs) {
  if (num_segs < 0) return fail(LORA_E_ARG, "num_segs must be >= 0, got %d", num_segs);
  if (num_segs > (1 << 20)) return fail(LORA_E_SHAPE, "num_segs too large (%d)", num_segs);
  if (!perm || !seg_starts || !seg_lens || !seg_ids)
    return fail(LORA_E_ARG, "SGMV metadata pointers must not be NULL");
  return LORA_OK;
}

// Validates a caller's plan against its image(s) and builds the device view.
// `image` is the device copy; `image_host` (nullable) the host copy, which lets
// a small plan travel in the kernel arguments, in which case `image` is not
// read and may be NULL.
int32_t plan_view(const Geo& g, const lora_plan* p, const void* image, const void* image_host,
                  TilePlan* tp) {
  if (!p) return fail(LORA_E_ARG, "plan is NULL");
  const int32_t kmax = g.R > 32 ? LORA_PLAN_MAX_KSPLIT_MFMA_WIDE : LORA_PLAN_MAX_KSPLIT_MFMA;
  if (p->ksplit < 1 || p->ksplit > kmax)
    return fail(LORA_E_ARG, "malformed plan (ksplit %d outside [1, %d] for max_lora_rank %d)",
                p->ksplit, kmax, g.R);
  if (p->ksplit_wave < 1 || p->ksplit_wave > LORA_PLAN_MAX_KSPLIT)
    return fail(LORA_E_ARG, "malformed plan (ksplit_wave %d outside [1, %d])", p->ksplit_wave,
                LORA_PLAN_MAX_KSPLIT);
  if (p->num_sgmv_rows < 0 || p->num_bgmv_rows < 0 || p->wave_tiles < 0 || p->mfma_tiles < 0 ||
      p->off_perm < 0 || p->off_wave < 0 || p->off_mfma < 0 || p->image_bytes < 0)
    return fail(LORA_E_ARG, "malformed plan (negative count or offset)");
  if ((int64_t)p->num_sgmv_rows + p->num_bgmv_rows > INT32_MAX)
    return fail(LORA_E_ARG, "malformed plan (row count)");
  if (p->off_wave % 4 || p->off_mfma % 4)
    return fail(LORA_E_ALIGN, "plan sections must start on 16-byte boundaries");
  const int64_t words = p->image_bytes / 4;
  if (p->off_perm + p->num_sgmv_rows + p->num_bgmv_rows > words ||
      p->off_wave + (int64_t)LORA_PLAN_WAVE_WORDS * p->wave_tiles > words ||
      p->off_mfma + (int64_t)LORA_PLAN_MFMA_WORDS * p->mfma_tiles > words)
    return fail(LORA_E_ARG, "malformed plan (sections exceed image_bytes)");
  if (p->mfma_tiles > 0 && g.dtype != LORA_BF16)
    return fail(LORA_E_DTYPE, "MFMA tiles need a bf16 pool");
  const int32_t* host = (const int32_t*)image_host;
  const bool small = host && p->mfma_tiles == 0 && p->wave_tiles <= kArgTilesL &&
                     g.max_loras <= (1 << 28);
  if ((p->wave_tiles > 0 || p->mfma_tiles > 0) && !small) {
    if (int32_t e = need_ptr(image, "image")) return e;
  }
  const int32_t* img = (const int32_t*)image;
  *tp = TilePlan{img ? img + p->off_perm : nullptr, img ? img + p->off_wave : nullptr,
                 p->wave_tiles, img ? img + p->off_mfma : nullptr, p->mfma_tiles,
                 host ? host + p->off_wave : nullptr, p->ksplit,
                 p->num_sgmv_rows + p->num_bgmv_rows, p->ksplit_wave, nullptr, nullptr, nullptr,
                 /*walk=*/0};
  return LORA_OK;
}

}  // namespace

extern "C" {

int32_t lora_pool_load(const lora_pool_desc* desc, void* A_pool, void* B_pool, int32_t slot,
                       int32_t slice, const void* A_src, const void* B_src, int32_t r,
                       float alpha, int32_t use_rslora, int32_t src_on_device, void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (int32_t e = need_ptr(A_pool, "A_pool")) return e;
  if (int32_t e = need_ptr(B_pool, "B_pool")) return e;
  if (!A_src || !B_src) return fail(LORA_E_ARG, "A_src / B_src must not be NULL");
  if (slot < 0 || slot >= g.max_loras)
    return fail(LORA_E_ID, "slot %d is outside [0, %d)", slot, g.max_loras);
  if (slice < 0 || slice >= g.S) return fail(LORA_E_ID, "slice %d is outside [0, %d)", slice, g.S);
  if (r <= 0 || r > g.R)
    return fail(LORA_E_RANK, "adapter rank %d must be in [1, max_lora_rank = %d]", r, g.R);
  if (src_on_device != 0 && src_on_device != 1)
    return fail(LORA_E_ARG, "src_on_device must be 0 or 1");
  const float scale = lora_scaling(r, alpha, use_rslora);
  if (!std::isfinite(scale)) return fail(LORA_E_ARG, "scale alpha/r is not finite");
  const int64_t eb = elem_bytes(g.dtype);
  const int out_s = g.out[slice];
  char* Ad = (char*)A_pool + ((int64_t)slot * g.S + slice) * g.R * (int64_t)g.K * eb;
  char* Bd = (char*)B_pool + ((int64_t)slot * g.O + g.off[slice]) * (int64_t)g.R * eb;
  hipStream_t st = (hipStream_t)stream;
  if (log_enabled())
    std::fprintf(stderr, "lora_pool: loading adapter into slot %d slice %d (rank %d, scale %g)\n",
                 slot, slice, r, (double)scale);
  if (src_on_device) return run_pool_load(g, Ad, Bd, A_src, B_src, r, out_s, scale, st);

  // host sources: pad and fold on the host, then copy
  const size_t na = (size_t)g.R * g.K, nb = (size_t)out_s * g.R;
  std::vector<unsigned char> Ah(na * eb, 0), Bh(nb * eb, 0);
  std::memcpy(Ah.data(), A_src, (size_t)r * g.K * eb);
  if (g.dtype == LORA_BF16) {
    const uint16_t* Bs = (const uint16_t*)B_src;
    uint16_t* Bo = (uint16_t*)Bh.data();
    for (int j = 0; j < out_s; ++j)
      for (int k = 0; k < r; ++k)
        Bo[(size_t)j * g.R + k] = host_f32_to_bf16(host_bf16_to_f32(Bs[(size_t)j * r + k]) * scale);
  } else {
    const float* Bs = (const float*)B_src;
    float* Bo = (float*)Bh.data();
    for (int j = 0; j < out_s; ++j)
      for (int k = 0; k < r; ++k) Bo[(size_t)j * g.R + k] = Bs[(size_t)j * r + k] * scale;
  }
  if (int32_t e = hip_ok(hipMemcpyAsync(Ad, Ah.data(), Ah.size(), hipMemcpyHostToDevice, st),
                         "copy A slice")) return e;
  if (int32_t e = hip_ok(hipMemcpyAsync(Bd, Bh.data(), Bh.size(), hipMemcpyHostToDevice, st),
                         "copy B slice")) return e;
  return hip_ok(hipStreamSynchronize(st), "pool load sync");
}

int32_t lora_pool_clear(const lora_pool_desc* desc, void* A_pool, void* B_pool, int32_t slot,
                        void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (int32_t e = need_ptr(A_pool, "A_pool")) return e;
  if (int32_t e = need_ptr(B_pool, "B_pool")) return e;
  if (slot < 0 || slot >= g.max_loras)
    return fail(LORA_E_ID, "slot %d is outside [0, %d)", slot, g.max_loras);
  const int64_t eb = elem_bytes(g.dtype);
  const int64_t abytes = (int64_t)g.S * g.R * g.K * eb, bbytes = (int64_t)g.O * g.R * eb;
  hipStream_t st = (hipStream_t)stream;
  if (int32_t e = hip_ok(hipMemsetAsync((char*)A_pool + slot * abytes, 0, abytes, st), "clear A"))
    return e;
  return hip_ok(hipMemsetAsync((char*)B_pool + slot * bbytes, 0, bbytes, st), "clear B");
}

int32_t lora_build_meta_device(const int32_t* ids, const uint8_t* prefill, int32_t T,
                               int32_t max_loras, int32_t max_lora_rank,
                               int32_t bgmv_max_rank, const lora_meta* out, int32_t* counts,
                               void* stream) {
  clear_error();
  if (!out || !counts) return fail(LORA_E_ARG, "out / counts must not be NULL");
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  if (max_loras < 1 || max_loras > LORA_META_DEVICE_MAX_LORAS)
    return fail(LORA_E_SHAPE, "max_loras must be in [1, %d], got %d", LORA_META_DEVICE_MAX_LORAS,
                max_loras);
  if (!out->seg_starts || !out->seg_lens || !out->seg_ids)
    return fail(LORA_E_ARG, "segment arrays must not be NULL");
  if (T > 0 && (!ids || !out->sgmv_perm || !out->bgmv_tok || !out->bgmv_ids))
    return fail(LORA_E_ARG, "ids and row arrays must not be NULL");
  const int32_t limit = bgmv_max_rank > 0 ? bgmv_max_rank : LORA_BGMV_MAX_RANK_DEFAULT;
  return run_build_meta_device(ids, prefill, T, max_loras, max_lora_rank > limit, *out, counts,
                               (hipStream_t)stream);
}

int32_t lora_sgmv_shrink(const lora_pool_desc* desc, const void* x, const void* A_pool, float* v,
                         const int32_t* perm, const int32_t* seg_starts, const int32_t* seg_lens,
                         const int32_t* seg_ids, int32_t num_segs, int32_t num_rows, int32_t T,
                         void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_rows(num_rows, T, "num_rows")) return e;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (num_rows == 0 || num_segs == 0 || T == 0) return LORA_OK;
  if (int32_t e = check_common(desc, &g, x, "x", A_pool, "A_pool", v)) return e;
  if (int32_t e = sgmv_args(perm, seg_starts, seg_lens, seg_ids, num_segs)) return e;
  g.T = T;
  return run_shrink(g, x, A_pool, v,
                    segments_list(perm, seg_starts, seg_lens, seg_ids, num_segs, num_rows),
                    (hipStream_t)stream);
}

int32_t lora_sgmv_expand(const lora_pool_desc* desc, const float* v, const void* B_pool, void* y,
                         const int32_t* perm, const int32_t* seg_starts, const int32_t* seg_lens,
                         const int32_t* seg_ids, int32_t num_segs, int32_t num_rows, int32_t T,
                         void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_rows(num_rows, T, "num_rows")) return e;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (num_rows == 0 || num_segs == 0 || T == 0) return LORA_OK;
  if (int32_t e = check_common(desc, &g, y, "y", B_pool, "B_pool", v)) return e;
  if (int32_t e = sgmv_args(perm, seg_starts, seg_lens, seg_ids, num_segs)) return e;
  g.T = T;
  return run_expand(g, v, B_pool, y,
                    segments_list(perm, seg_starts, seg_lens, seg_ids, num_segs, num_rows),
                    (hipStream_t)stream);
}

int32_t lora_bgmv_shrink(const lora_pool_desc* desc, const void* x, const void* A_pool, float* v,
                         const int32_t* tok, const int32_t* ids, int32_t n, int32_t T,
                         void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_rows(n, T, "n")) return e;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (n == 0 || T == 0) return LORA_OK;
  if (int32_t e = check_common(desc, &g, x, "x", A_pool, "A_pool", v)) return e;
  if (!tok || !ids) return fail(LORA_E_ARG, "tok / ids must not be NULL");
  g.T = T;
  return run_shrink(g, x, A_pool, v, rows_list(tok, ids, n), (hipStream_t)stream);
}

int32_t lora_bgmv_expand(const lora_pool_desc* desc, const float* v, const void* B_pool, void* y,
                         const int32_t* tok, const int32_t* ids, int32_t n, int32_t T,
                         void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_rows(n, T, "n")) return e;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (n == 0 || T == 0) return LORA_OK;
  if (int32_t e = check_common(desc, &g, y, "y", B_pool, "B_pool", v)) return e;
  if (!tok || !ids) return fail(LORA_E_ARG, "tok / ids must not be NULL");
  g.T = T;
  return run_expand(g, v, B_pool, y, rows_list(tok, ids, n), (hipStream_t)stream);
}

int32_t lora_plan_shrink(const lora_pool_desc* desc, const void* x, const void* A_pool, float* v,
                         int32_t T, const lora_plan* plan, const void* image,
                         const void* image_host, void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  TilePlan tp;
  if (int32_t e = plan_view(g, plan, image, image_host, &tp)) return e;
  if (T == 0 || (tp.wave_tiles == 0 && tp.mfma_tiles == 0)) return LORA_OK;
  if (int32_t e = check_common(desc, &g, x, "x", A_pool, "A_pool", v)) return e;
  g.T = T;
  return run_plan_shrink(g, x, A_pool, v, tp, (hipStream_t)stream);
}

int32_t lora_plan_expand(const lora_pool_desc* desc, const float* v, const void* B_pool, void* y,
                         int32_t T, const lora_plan* plan, const void* image,
                         const void* image_host, void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  TilePlan tp;
  if (int32_t e = plan_view(g, plan, image, image_host, &tp)) return e;
  if (T == 0 || (tp.wave_tiles == 0 && tp.mfma_tiles == 0)) return LORA_OK;
  if (int32_t e = check_common(desc, &g, y, "y", B_pool, "B_pool", v)) return e;
  g.T = T;
  return run_plan_expand(g, v, B_pool, y, tp, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// lora_plan_apply, plus: with copy_to set (device memory of at least
// plan->image_bytes, the workspace's image region) the shrink launches copy
// the plan records and MFMA-tile tokens they read into copy_to (the image's
// offsets) and the expand launches read that copy.
int32_t plan_apply_impl(const lora_pool_desc* desc, const void* x, const void* A_pool,
                        const void* B_pool, void* y, int32_t T, const lora_plan* plan,
                        const void* image, const void* image_host, void* ws, int64_t ws_bytes,
                        void* stream, int32_t* copy_to) {
  Geo g;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  TilePlan tp;
  if (int32_t e = plan_view(g, plan, image, image_host, &tp)) return e;
  if (T == 0 || (tp.wave_tiles == 0 && tp.mfma_tiles == 0)) return LORA_OK;
  if (int32_t e = need_ptr(A_pool, "A_pool")) return e;
  if (int32_t e = need_ptr(B_pool, "B_pool")) return e;
  if (int32_t e = need_ptr(x, "x")) return e;
  if (int32_t e = need_ptr(y, "y")) return e;
  if (int32_t e = need_ptr(ws, "ws")) return e;
  const WorkspaceLayout wl = workspace_layout(g, T);
  if (ws_bytes < wl.total)
    return fail(LORA_E_WORKSPACE, "workspace has %lld bytes, needs %lld", (long long)ws_bytes,
                (long long)wl.total);
  if ((int64_t)std::max(tp.ksplit, tp.ksplit_wave) * tp.num_rows >
      (int64_t)LORA_PLAN_MAX_KSPLIT * T)
    return fail(LORA_E_ARG, "malformed plan (%d rows for %d tokens)", tp.num_rows, T);
  if (copy_to) {
    tp.copy_perm = copy_to + plan->off_perm;
    tp.copy_wave = copy_to + plan->off_wave;
    tp.copy_mfma = copy_to + plan->off_mfma;
  }
  g.T = T;
  return run_plan_apply(g, x, A_pool, B_pool, y, tp, (float*)((char*)ws + wl.v),
                        (hipStream_t)stream);
}

}  // namespace

extern "C" {

int32_t lora_plan_apply(const lora_pool_desc* desc, const void* x, const void* A_pool,
                        const void* B_pool, void* y, int32_t T, const lora_plan* plan,
                        const void* image, const void* image_host, void* ws, int64_t ws_bytes,
                        void* stream) {
  clear_error();
  return plan_apply_impl(desc, x, A_pool, B_pool, y, T, plan, image, image_host, ws, ws_bytes,
                         stream, nullptr);
}

// `host` itself when it is pinned host memory (hipHostMalloc) that the device
// reaches at the same address, else nullptr (pageable memory, or a mapping at
// another address: the caller then copies).  Kernels that read a plan there
// see every write the host made before their launch.
static const void* device_alias(const void* host) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, host) != hipSuccess) {
    (void)hipGetLastError();  // pageable memory is not an error here
    return nullptr;
  }
  return a.type == hipMemoryTypeHost && a.devicePointer == host ? host : nullptr;
}

int32_t lora_apply(const lora_pool_desc* desc, const void* A_pool, const void* B_pool,
                   const void* x, void* y, int32_t T, const int32_t* ids_host,
                   const uint8_t* prefill_host, int32_t bgmv_max_rank, void* ws,
                   int64_t ws_bytes, void* meta_host, int64_t meta_host_bytes, void* stream) {
  return lora_apply_ranked(desc, A_pool, B_pool, x, y, T, ids_host, prefill_host, bgmv_max_rank,
                           nullptr, ws, ws_bytes, meta_host, meta_host_bytes, stream);
}

int32_t lora_apply_device(const lora_pool_desc* desc, const void* A_pool, const void* B_pool,
                          const void* x, void* y, int32_t T, const int32_t* ids,
                          const uint8_t* prefill, int32_t bgmv_max_rank, void* ws,
                          int64_t ws_bytes, void* stream) {
  return lora_apply_device_ranked(desc, A_pool, B_pool, x, y, T, ids, prefill, bgmv_max_rank,
                                  nullptr, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Checks of lora_apply_device's arguments other than the workspace; fills g
// (g.T = T).  Sets *noop for an empty batch.  No HIP call.
int32_t device_args(const lora_pool_desc* desc, const void* A_pool, const void* B_pool,
                    const void* x, const void* y, int32_t T, const int32_t* ids, Geo* g,
                    bool* noop) {
  *noop = false;
  if (int32_t e = check_desc(desc, g)) return e;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  if (g->max_loras > LORA_META_DEVICE_MAX_LORAS)
    return fail(LORA_E_SHAPE, "max_loras must be <= %d for the device plan, got %d",
                LORA_META_DEVICE_MAX_LORAS, g->max_loras);
  if (T == 0) {
    *noop = true;
    return LORA_OK;
  }
  if (int32_t e = need_ptr(A_pool, "A_pool")) return e;
  if (int32_t e = need_ptr(B_pool, "B_pool")) return e;
  if (int32_t e = need_ptr(x, "x")) return e;
  if (int32_t e = need_ptr(y, "y")) return e;
  if (int32_t e = need_ptr(ids, "ids")) return e;
  g->T = T;
  return LORA_OK;
}

// lora_apply_device on validated arguments and a workspace of at least
// device_layout(g, T).total bytes at `ws` (256-byte aligned).  Every byte of
// the workspace the kernels read is written earlier in the same call (the
// builder writes the metadata and every tile record up to the capacities, the
// shrink every v row the expand reads), so it needs no clearing between calls.
int32_t apply_device_run(const Geo& g, const void* A_pool, const void* B_pool, const void* x,
                         void* y, int32_t T, const int32_t* ids, const uint8_t* prefill,
                         int32_t bgmv_max_rank, const int32_t* slot_ranks, void* ws,
                         hipStream_t st) {
  const DeviceLayout d = device_layout(g, T);
  char* w = (char*)ws;
  lora_meta m;
  m.num_sgmv_rows = m.num_segs = m.num_bgmv_rows = m.reserved = 0;
  m.sgmv_perm = (int32_t*)(w + d.sgmv_perm);
  m.bgmv_tok = (int32_t*)(w + d.bgmv_tok);
  m.bgmv_ids = (int32_t*)(w + d.bgmv_ids);
  m.seg_starts = (int32_t*)(w + d.seg_starts);
  m.seg_lens = (int32_t*)(w + d.seg_lens);
  m.seg_ids = (int32_t*)(w + d.seg_ids);
  int32_t* counts = (int32_t*)(w + d.counts);
  int32_t* tiles = (int32_t*)(w + d.tiles);
  int32_t* mtiles = (int32_t*)(w + d.mtiles);
  int32_t* perm = (int32_t*)(w + d.perm);
  const int32_t limit = bgmv_max_rank > 0 ? bgmv_max_rank : LORA_BGMV_MAX_RANK_DEFAULT;
  // the plan's shape is known on the host only as capacities: cap 8-row
  // records and mcap 64-row records (surplus ones have 0 rows), T v rows.
  // Small plans take the one-launch kernel, which reads 8-row records only;
  // other bf16 plans put long SGMV segments and, in large decode batches, long
  // BGMV runs on 64-row MFMA tiles by the host plan's rules
  const int32_t cap = device_tile_cap(T, g.max_loras);
  const bool onepass = device_plan_is_onepass(g, cap);
  const bool mfma = g.dtype == LORA_BF16 && !onepass;
  const bool all_sgmv = g.R > limit;
  // no flags and no forced SGMV: every row is a BGMV row
  const int32_t mcap = mfma ? device_mfma_cap(g, T, prefill != nullptr || all_sgmv) : 0;
  const DevicePlanOut po{tiles,
                         cap,
                         mtiles,
                         mcap,
                         mfma ? sgmv_mfma_min_rows() : INT32_MAX,
                         mfma ? bgmv_mfma_min_rows() : INT32_MAX,
                         bgmv_mfma_min_total(g.R),
                         perm,
                         slot_ranks,
                         g.R};
  if (int32_t e = run_build_meta_device(ids, prefill, T, g.max_loras, all_sgmv, m, counts, st,
                                        &po))
    return e;
  // the 8-row K split is chosen for the records such a batch typically makes,
  // not for the capacity: with 64-row tiles about two partial tiles per slot
  // (long runs take 64-row tiles, as the rest of a flagged batch's rows
  // mostly do), else one per slot besides the full tiles of every row.  The
  // split changes only how the work is spread
  const int64_t wave_est =
      mfma ? std::min<int64_t>(cap, 2 * std::min<int64_t>(g.max_loras, T))
           : std::min<int64_t>(cap, ((int64_t)T + LORA_PLAN_WAVE_ROWS - 1) / LORA_PLAN_WAVE_ROWS +
                                        std::min<int64_t>(g.max_loras, T));
  const int32_t kw = std::min(wave_ksplit(g, wave_est), walk_kparts_max(g.R));
  TilePlan tp{perm, tiles, cap, mtiles, mcap, nullptr, mfma_ksplit(g, mcap), T, kw, nullptr,
              nullptr, nullptr, /*walk=*/1};
  if (onepass) return run_plan_onepass_list(g, x, A_pool, B_pool, y, tp, st);
  float* v = (float*)(w + d.v);
  if (int32_t e = run_plan_shrink(g, x, A_pool, v, tp, st)) return e;
  return run_plan_expand(g, v, B_pool, y, tp, st);
}

// Workspace of lora_apply_device_noalloc: one array per GPU, allocated with
// the code object when the library is first used on that GPU and held until
// the process ends.  Host code never passes `scratch` itself to a kernel (on
// the host that name is a stand-in, not a device address): it uses the
// address hipGetSymbolAddress returns, looked up once per device with that
// device current and kept in scratch_addr.
__device__ __align__(256) unsigned char scratch[LORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

int32_t scratch_addr(void** out) {
  int dev = -1;
  if (int32_t e = hip_ok(hipGetDevice(&dev), "hipGetDevice")) return e;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LORA_E_ARG, "device %d is outside the %d devices the scratch table covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (int32_t e = hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address"))
      return e;
    if (!p || ((uintptr_t)p & 255u))
      return fail(LORA_E_HIP, "scratch address %p is not 256-byte aligned", p);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return LORA_OK;
}

}  // namespace

extern "C" {

int32_t lora_apply_device_ranked(const lora_pool_desc* desc, const void* A_pool,
                                 const void* B_pool, const void* x, void* y, int32_t T,
                                 const int32_t* ids, const uint8_t* prefill,
                                 int32_t bgmv_max_rank, const int32_t* slot_ranks, void* ws,
                                 int64_t ws_bytes, void* stream) {
  clear_error();
  Geo g;
  bool noop;
  if (int32_t e = device_args(desc, A_pool, B_pool, x, y, T, ids, &g, &noop)) return e;
  if (noop) return LORA_OK;
  if (int32_t e = need_ptr(ws, "ws")) return e;
  if (!aligned16(x) || !aligned16(y) || !aligned16(A_pool) || !aligned16(B_pool) ||
      ((uintptr_t)ws & 255u))
    return fail(LORA_E_ALIGN, "x, y and the pool must be 16-byte aligned, ws 256-byte aligned");
  const DeviceLayout d = device_layout(g, T);
  if (ws_bytes < d.total)
    return fail(LORA_E_WORKSPACE, "workspace has %lld bytes, needs %lld", (long long)ws_bytes,
                (long long)d.total);
  return apply_device_run(g, A_pool, B_pool, x, y, T, ids, prefill, bgmv_max_rank, slot_ranks,
                          ws, (hipStream_t)stream);
}

int32_t lora_apply_device_noalloc(const lora_pool_desc* desc, const void* A_pool,
                                  const void* B_pool, const void* x, void* y, int32_t T,
                                  const int32_t* ids, const uint8_t* prefill,
                                  int32_t bgmv_max_rank, void* stream) {
  clear_error();
  Geo g;
  bool noop;
  if (int32_t e = device_args(desc, A_pool, B_pool, x, y, T, ids, &g, &noop)) return e;
  if (noop) return LORA_OK;
  if (!aligned16(x) || !aligned16(y) || !aligned16(A_pool) || !aligned16(B_pool))
    return fail(LORA_E_ALIGN, "x, y and the pool must be 16-byte aligned");
  const DeviceLayout d = device_layout(g, T);
  if (d.total > (int64_t)LORA_NOALLOC_SCRATCH_BYTES)
    return fail(LORA_E_WORKSPACE,
                "the batch needs %lld bytes of workspace; the no-alloc scratch holds %lld "
                "(use lora_apply_device with a workspace of the caller's)",
                (long long)d.total, (long long)LORA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int32_t e = scratch_addr(&ws)) return e;
  return apply_device_run(g, A_pool, B_pool, x, y, T, ids, prefill, bgmv_max_rank, nullptr, ws,
                          (hipStream_t)stream);
}

int32_t lora_apply_ranked(const lora_pool_desc* desc, const void* A_pool, const void* B_pool,
                          const void* x, void* y, int32_t T, const int32_t* ids_host,
                          const uint8_t* prefill_host, int32_t bgmv_max_rank,
                          const int32_t* slot_ranks, void* ws, int64_t ws_bytes,
                          void* meta_host, int64_t meta_host_bytes, void* stream) {
  clear_error();
  Geo g;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (T < 0) return fail(LORA_E_ARG, "T must be >= 0, got %d", T);
  if (T == 0) return LORA_OK;
  if (int32_t e = need_ptr(A_pool, "A_pool")) return e;
  if (int32_t e = need_ptr(B_pool, "B_pool")) return e;
  if (int32_t e = need_ptr(x, "x")) return e;
  if (int32_t e = need_ptr(y, "y")) return e;
  if (int32_t e = need_ptr(ws, "ws")) return e;
  const WorkspaceLayout wl = workspace_layout(g, T);
  if (ws_bytes < wl.total)
    return fail(LORA_E_WORKSPACE, "workspace has %lld bytes, needs %lld", (long long)ws_bytes,
                (long long)wl.total);
  lora_plan p;
  if (int32_t e = lora_apply_plan_ranked(desc, T, ids_host, prefill_host, bgmv_max_rank,
                                         slot_ranks, meta_host, meta_host_bytes, &p))
    return e;
  const int32_t rows = p.num_sgmv_rows + p.num_bgmv_rows;
  if (rows == 0) return LORA_OK;
  const char* image_host = (const char*)meta_host + p.image_offset;
  const bool small = p.mfma_tiles == 0 && p.wave_tiles <= kArgTilesL && g.max_loras <= (1 << 28);
  const void* image = ws;
  int32_t* copy_to = nullptr;
  if (!small) {  // small plans travel in the kernel arguments instead
    if (const void* mapped = device_alias(image_host)) {
      // pinned staging: the shrink launches read the plan where it lies and
      // leave a copy in the workspace's image region for the expand launches
      image = mapped;
      copy_to = (int32_t*)ws;
    } else if (int32_t e = hip_ok(hipMemcpyAsync(ws, image_host, (size_t)p.image_bytes,
                                                 hipMemcpyHostToDevice, (hipStream_t)stream),
                                  "plan copy")) {
      return e;
    }
  }
  return plan_apply_impl(desc, x, A_pool, B_pool, y, T, &p, image, image_host, ws, ws_bytes,
                         stream, copy_to);
}

}  // extern "C"
