/*
 * lora_pool.h - C ABI of the MI355X (gfx950) multi-LoRA delta library.
 *
 * For a batch whose rows each name an adapter slot (or none), one shared base
 * projection output y = W x is updated in place:
 *
 *     y[t, off_s : off_s + out_s] += s_a * B_{a,s} (A_{a,s} x_t)   for a = ids[t] >= 0
 *
 * as a two-stage grouped computation: shrink (x -> v, length R per slice) then
 * expand (v -> out).  SGMV handles contiguous segments of tokens sharing an
 * adapter (prefill), BGMV per-token adapter indices (decode).
 *
 * Pages this follows (cited by title and section):
 *  [TGI]  "Text Generation Inference 多 LoRA 适配器服务实战: LORA_ADAPTERS 配置与
 *         SGMV/BGMV 内核加速原理": implementation step 3 (scale alpha/r or
 *         alpha/sqrt(r) for rsLoRA, folded into lora_B at load; rank padding for
 *         the kernels' vector width), step 4 (prefill -> SGMV segments, decode ->
 *         BGMV per token; SGMV whenever the rank exceeds the BGMV limit; the four
 *         shrink/expand operations), step 5 (uneven q/k/v output slices).
 *  [vLLM] "vLLM 怎么在离线推理中为单次请求挂载不同 LoRA 适配器": step 2
 *         (max_loras pre-allocated slots, max_lora_rank slot size), LoRARequest
 *         rules (a None request runs the base model), limits (the slot rank
 *         must cover every adapter's rank).
 *  [QA]   "Multi-LoRA serving: 一基座, 多 adapter": direct answer (delta W = B A;
 *         the base GEMM runs once per batch and a grouped kernel adds each
 *         row's B(Ax) by adapter id).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Ownership: every device buffer (pool, x, y, v, metadata, workspace) is
 *    allocated and freed by the caller.  The library allocates no device
 *    memory and keeps no device state between calls.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream).  Device work
 *    is enqueued asynchronously on it; no call synchronises except
 *    lora_pool_load with host sources (documented there).
 *  - Errors: functions return LORA_OK (0) or a negative lora_status; the
 *    message of the last failure on the calling thread is returned by
 *    lora_last_error().  All argument validation happens before any HIP call,
 *    so every error path can be exercised without a GPU.  Device-resident
 *    metadata cannot be validated on the host: kernels skip (never read or
 *    write) rows whose token index is outside [0, T) or whose adapter slot is
 *    outside [0, max_loras), and clamp segments to the row list.
 *  - Aliasing: y is updated in place; x must not overlap y; v must not overlap
 *    x, y or the pool.
 *  - Alignment: in_features, every out_features[s] and max_lora_rank must be
 *    multiples of 8; every device pointer must be 16-byte aligned.
 *  - dtype: x, y, A_pool and B_pool share one element type (fp32 or bf16);
 *    v and all accumulation are fp32; y is rounded once (nearest-even) to its
 *    dtype after adding the fp32 delta to the fp32 value of y.
 *
 * Layouts (row-major; R = max_lora_rank, K = in_features, S = num_slices,
 * O = sum of out_features, off_s = sum of out_features[0..s-1]):
 *    x       [T][K]
 *    y       [T][O]               slice s occupies columns off_s .. off_s+out_s-1
 *    A_pool  [max_loras][S][R][K] rows r..R-1 of a slot/slice are zero
 *    B_pool  [max_loras][O][R]    row off_s+j of slot a holds s_a * B_{a,s}[j][:]
 *                                 (columns r..R-1 zero), i.e. the peft lora_B
 *                                 [out, r] layout, scaled and zero-padded
 *    v       [rows][S][R] fp32    row i belongs to the i-th entry of the row list
 */
#ifndef LORA_POOL_H
#define LORA_POOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_POOL_ABI_VERSION 3
#define LORA_MAX_SLICES 8
/* [TGI] step 4 names a BGMV rank limit without a value; 64 covers the ranks
 * the kernels are built for.  Pass bgmv_max_rank <= 0 to lora_build_meta /
 * lora_apply to use it. */
#define LORA_BGMV_MAX_RANK_DEFAULT 64

typedef enum {
  LORA_OK = 0,
  LORA_E_ARG = -1,        /* null pointer, negative size, bad flag */
  LORA_E_DTYPE = -2,      /* unknown dtype */
  LORA_E_SHAPE = -3,      /* inconsistent sizes, too many slices, capacity too small */
  LORA_E_ALIGN = -4,      /* size not a multiple of 8 or pointer not 16-byte aligned */
  LORA_E_RANK = -5,       /* adapter rank > max_lora_rank ([vLLM] limits) or <= 0 */
  LORA_E_ID = -6,         /* adapter id < -1 or >= max_loras, or bad slot index */
  LORA_E_WORKSPACE = -7,  /* workspace or staging buffer too small */
  LORA_E_HIP = -8         /* a HIP runtime call failed */
} lora_status;

typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/* Geometry of one adapter pool (one projection, possibly fused slices). */
typedef struct {
  int32_t dtype;                             /* lora_dtype */
  int32_t max_loras;                         /* slots ([vLLM] step 2), >= 1 */
  int32_t max_lora_rank;                     /* R: rank every slot is padded to */
  int32_t in_features;                       /* K */
  int32_t num_slices;                        /* S in [1, LORA_MAX_SLICES] */
  int32_t out_features[LORA_MAX_SLICES];     /* out_s, s < S */
} lora_pool_desc;

/* Host-side metadata produced by lora_build_meta ([TGI] step 4).  The caller
 * owns all arrays; capacities: sgmv_perm, bgmv_tok, bgmv_ids >= T entries;
 * seg_starts, seg_lens, seg_ids >= max_loras entries (one segment per distinct
 * adapter at most, since a segment is a maximal run of equal id). */
typedef struct {
  int32_t num_sgmv_rows;  /* out: entries of sgmv_perm */
  int32_t num_segs;       /* out: entries of seg_* */
  int32_t num_bgmv_rows;  /* out: entries of bgmv_tok / bgmv_ids */
  int32_t reserved;
  int32_t* sgmv_perm;     /* token indices of SGMV rows sorted by (id, token) */
  int32_t* seg_starts;    /* offset of each segment into sgmv_perm */
  int32_t* seg_lens;      /* rows per segment (> 0) */
  int32_t* seg_ids;       /* adapter slot per segment, strictly increasing */
  int32_t* bgmv_tok;      /* token indices of BGMV rows sorted by (id, token) */
  int32_t* bgmv_ids;      /* adapter slot per BGMV row */
} lora_meta;

/* ------------------------------------------------------------------ misc */

/* Message of the last failure on this thread ("" if none).  Never NULL. */
const char* lora_last_error(void);
/* LORA_POOL_ABI_VERSION of the loaded library. */
int32_t lora_abi_version(void);

/* ------------------------------------------------------------------ pool */

/* Check a descriptor: dtype, max_loras >= 1, 1 <= S <= 8, K, out_s and R
 * positive multiples of 8.  Returns LORA_OK or an error. */
int32_t lora_pool_validate(const lora_pool_desc* desc);

/* Bytes of A_pool (max_loras*S*R*K*e) and B_pool (max_loras*O*R*e) for a valid
 * descriptor ([vLLM] step 2: every slot is pre-allocated at the slot rank); a
 * negative lora_status for an invalid one. */
int64_t lora_pool_bytes_A(const lora_pool_desc* desc);
int64_t lora_pool_bytes_B(const lora_pool_desc* desc);

/* The scale an adapter's B is multiplied by at load ([TGI] step 3):
 * alpha / r, or alpha / sqrt(r) with use_rslora, evaluated in double and
 * rounded to float.  r is the adapter's own rank, never the padded rank.
 * Returns NaN for r <= 0. */
float lora_scaling(int32_t r, float alpha, int32_t use_rslora);

/* Load one slice of one adapter into slot `slot` ([TGI] step 3; [vLLM] limits).
 *   A_src  [r][K] in the pool dtype (peft lora_A.weight layout)
 *   B_src  [out_s][r] in the pool dtype (peft lora_B.weight layout)
 * Writes A_pool[slot][slice][0:r][:] = A_src and rows r..R-1 = 0;
 * B_pool[slot][off_s + j][k] = round_dtype((float)B_src[j][k] * lora_scaling())
 * for k < r (one fp32 multiply, one nearest-even rounding), 0 for k >= r.
 * src_on_device = 1: A_src/B_src are device pointers; the work is one kernel
 * on `stream` (asynchronous).  src_on_device = 0: host pointers; the padded,
 * folded slices are staged in host memory and copied; the call returns after
 * the copy has completed.  Errors: LORA_E_RANK if r <= 0 or r > R, LORA_E_ID if
 * slot/slice is out of range, LORA_E_ARG on null pointers. */
int32_t lora_pool_load(const lora_pool_desc* desc, void* A_pool, void* B_pool,
                       int32_t slot, int32_t slice, const void* A_src, const void* B_src,
                       int32_t r, float alpha, int32_t use_rslora, int32_t src_on_device,
                       void* stream);

/* Zero every slice of slot `slot` in A_pool and B_pool (asynchronous, on
 * stream).  A cleared slot adds nothing. */
int32_t lora_pool_clear(const lora_pool_desc* desc, void* A_pool, void* B_pool,
                        int32_t slot, void* stream);

/* Merged-weight mode ([QA] "Multi-LoRA serving", the follow-up on merging an
 * adapter into the base: a server running one fine-tune merges it and pays no
 * per-request delta; serving many adapters keeps the runtime path).  For slot
 * `slot`, slice `slice` (width out_s = out_features[slice]):
 *   W_out[o][k] = round(W[o][k] + sum_{r<R} B_pool[slot][off_s + o][r] *
 *                                           A_pool[slot][slice][r][k])
 * i.e. W + s_a B A with the scale already folded into the pool's B; fp32
 * accumulation and one rounding to the pool dtype (nearest, ties to even).
 *   W, W_out: device [out_s][in_features] of the pool dtype, row-major (the
 *             base projection's weight rows for this slice), 16-byte aligned.
 *             W_out == W merges in place; other overlaps are rejected.  Merging
 *             is not undone by subtracting (the rounding is not invertible):
 *             keep the base W and merge the next adapter from it.
 * One kernel on `stream` (asynchronous; bf16 pools use MFMA).  Errors:
 * LORA_E_ID for slot / slice out of range, LORA_E_RANK if max_lora_rank >
 * LORA_MERGE_MAX_RANK, LORA_E_ALIGN, LORA_E_ARG on NULL or overlapping
 * buffers, all before any HIP call. */
#define LORA_MERGE_MAX_RANK 512
int32_t lora_merge_weights(const lora_pool_desc* desc, const void* A_pool, const void* B_pool,
                           int32_t slot, int32_t slice, const void* W, void* W_out,
                           void* stream);

/* ------------------------------------------------------------- metadata */

/* Host-only, bit-exact metadata builder ([TGI] step 4).
 *   ids[T]      adapter slot per token, -1 = no adapter ([vLLM] None request)
 *   prefill[T]  1 for prefill tokens, 0 for decode tokens (may be NULL = all 0)
 * A token with id >= 0 goes to SGMV if prefill[t] != 0 or
 * max_lora_rank > bgmv_max_rank (<= 0 selects LORA_BGMV_MAX_RANK_DEFAULT),
 * otherwise to BGMV.  Each set is ordered by (id, token index) (a stable
 * counting sort); SGMV segments are maximal runs of equal id.
 * Errors: LORA_E_ID for an id < -1 or >= max_loras (nothing is written),
 * LORA_E_ARG for null arrays with T > 0.  T = 0 gives empty sets. */
int32_t lora_build_meta(const int32_t* ids, const uint8_t* prefill, int32_t T,
                        int32_t max_loras, int32_t max_lora_rank, int32_t bgmv_max_rank,
                        lora_meta* out);

/* Most adapter slots lora_build_meta_device handles (its per-slot counters
 * live in LDS). */
#define LORA_META_DEVICE_MAX_LORAS 8192

/* The same metadata built on the GPU ([TGI] step 4), asynchronously on
 * `stream`, so a batch needs no host round trip (and the delta path can be
 * captured in a graph).
 *   ids, prefill  device arrays of T entries (prefill may be NULL = all 0)
 *   out           device arrays with the capacities of lora_build_meta; the
 *                 num_* fields of *out are not read or written
 *   counts        device int32[4]: num_sgmv_rows, num_segs, num_bgmv_rows and
 *                 the number of ids < -1 or >= max_loras (those rows are
 *                 left out, as if their id were -1)
 * The arrays equal lora_build_meta's bit for bit up to those counts, and are
 * padded behind them so the grouped entry points can take upper-bound sizes
 * (num_segs = max_loras, num_rows = n = T): seg_lens = 0 past num_segs,
 * bgmv_ids = -1 (and bgmv_tok = 0) past num_bgmv_rows, sgmv_perm = 0 past
 * num_sgmv_rows.  Errors (before any HIP call): LORA_E_ARG for null pointers
 * or T < 0, LORA_E_SHAPE for max_loras outside [1, LORA_META_DEVICE_MAX_LORAS].
 * One workgroup does the work: a histogram, scans over the slots, then one
 * wavefront places the rows in token order. */
int32_t lora_build_meta_device(const int32_t* ids, const uint8_t* prefill, int32_t T,
                               int32_t max_loras, int32_t max_lora_rank,
                               int32_t bgmv_max_rank, const lora_meta* out, int32_t* counts,
                               void* stream);

/* ----------------------------------------------------- grouped kernels */
/* All four take device pointers for x/y/v/pools/metadata and host scalars.
 * T is the number of rows of x and y (bounds for token indices).
 * n / num_rows = 0 is a no-op returning LORA_OK. */

/* SGMV shrink ([TGI] step 4, prefill): for every segment g and row i in
 * [seg_starts[g], seg_starts[g] + seg_lens[g]) (clamped to num_rows) with
 * t = perm[i], a = seg_ids[g]:  v[i][s][k] = sum_j A_pool[a][s][k][j] * x[t][j]
 * for all slices s and k < R (fp32 accumulation).  Long segments of a bf16
 * pool run on MFMA tiles, short ones on the wavefront path. */
int32_t lora_sgmv_shrink(const lora_pool_desc* desc, const void* x, const void* A_pool,
                         float* v, const int32_t* perm, const int32_t* seg_starts,
                         const int32_t* seg_lens, const int32_t* seg_ids, int32_t num_segs,
                         int32_t num_rows, int32_t T, void* stream);

/* SGMV expand: for the same rows, y[t][off_s + j] = round_dtype((float)y[t][off_s + j]
 * + sum_k B_pool[a][off_s + j][k] * v[i][s][k]) for every slice s, j < out_s. */
int32_t lora_sgmv_expand(const lora_pool_desc* desc, const float* v, const void* B_pool,
                         void* y, const int32_t* perm, const int32_t* seg_starts,
                         const int32_t* seg_lens, const int32_t* seg_ids, int32_t num_segs,
                         int32_t num_rows, int32_t T, void* stream);

/* BGMV shrink ([TGI] step 4, decode): for every row i < n with t = tok[i],
 * a = ids[i] (a = -1 rows are skipped and their v left untouched):
 * v[i][s][k] = sum_j A_pool[a][s][k][j] * x[t][j].  Rows sorted by id (as
 * lora_build_meta emits them) share each adapter's weight reads. */
int32_t lora_bgmv_shrink(const lora_pool_desc* desc, const void* x, const void* A_pool,
                         float* v, const int32_t* tok, const int32_t* ids, int32_t n,
                         int32_t T, void* stream);

/* BGMV expand: y[t][off_s + j] += sum_k B_pool[a][off_s + j][k] * v[i][s][k]
 * (rounded as above); rows with a = -1 are never read or written. */
int32_t lora_bgmv_expand(const lora_pool_desc* desc, const float* v, const void* B_pool,
                         void* y, const int32_t* tok, const int32_t* ids, int32_t n,
                         int32_t T, void* stream);

/* ------------------------------------------------------------ dispatcher */

/* Device workspace lora_apply needs for a batch of T tokens (the device copy
 * of the tile plan, then v for every row and K split), and the host staging
 * size for the plan.  Negative lora_status on an invalid descriptor or T < 0. */
int64_t lora_apply_workspace_bytes(const lora_pool_desc* desc, int32_t T);
int64_t lora_apply_host_meta_bytes(const lora_pool_desc* desc, int32_t T);

/* Rows per wavefront-path tile and per MFMA tile of a plan. */
#define LORA_PLAN_WAVE_ROWS 8
#define LORA_PLAN_MFMA_ROWS 64
/* most K-split partials of v a plan uses (LORA_PLAN_MAX_KSPLIT_MFMA for MFMA
 * tiles, at most LORA_PLAN_MAX_KSPLIT_MFMA_WIDE of them when max_lora_rank >
 * 32; LORA_PLAN_MAX_KSPLIT for wavefront tiles) */
#define LORA_PLAN_MAX_KSPLIT 8
#define LORA_PLAN_MAX_KSPLIT_MFMA 8
#define LORA_PLAN_MAX_KSPLIT_MFMA_WIDE 4
/* int32 words per tile record of a plan */
#define LORA_PLAN_WAVE_WORDS 16
#define LORA_PLAN_MFMA_WORDS 4

/* Tile plan of one batch, as lora_apply_plan lays it out in meta_host.
 *
 * The rows of the batch are the rows of lora_build_meta: the SGMV rows
 * (sgmv_perm order) are v rows 0 .. num_sgmv_rows - 1 and the BGMV rows
 * (bgmv_tok order, sorted by id) follow them.  Every tile covers consecutive v
 * rows of one adapter, cut from a run of rows of that adapter (an SGMV
 * segment or a run of equal ids among the BGMV rows):
 *   - MFMA tiles (bf16 pools only), pieces of LORA_PLAN_MFMA_ROWS rows: SGMV
 *     segments of at least mfma_min_rows rows, and BGMV runs of at least
 *     bgmv_mfma_min_rows rows (a threshold the plan sets only for batches in
 *     which such runs hold many rows);
 *   - wavefront tiles, pieces of LORA_PLAN_WAVE_ROWS rows: every other run.
 *
 * The device image starts image_offset bytes into meta_host and is
 * image_bytes long; offsets below count int32 words from its start:
 *   perm [num_sgmv_rows + num_bgmv_rows]  token of each v row
 *   wave [wave_tiles][16]             slot, rows, first v row, rank (0 =
 *                                     max_lora_rank; see lora_apply_plan_ranked),
 *                                     token of each row (-1 past the last
 *                                     row), -1 ...
 *   mfma [mfma_tiles][4]              slot, rows | rank << 16 (rank as
 *                                     above), first v row, first token
 *                                     when the tile's tokens are consecutive
 *                                     (perm[first + i] = first token + i),
 *                                     else -1
 *
 * ksplit: the shrink of the MFMA tiles splits K into this many contiguous
 * ranges and writes one partial of v per range (the expand sums them in order
 * 0, 1, ...); ksplit_wave does the same for the wavefront tiles (bf16 pools
 * with R <= 64; 1 otherwise).  The plan picks both so that the launches fill
 * the GPU. */
typedef struct {
  int32_t num_sgmv_rows;
  int32_t num_bgmv_rows;
  int32_t num_segs;
  int32_t wave_tiles;
  int32_t mfma_tiles;
  int32_t mfma_min_rows;   /* INT32_MAX when no segment uses MFMA tiles */
  int32_t ksplit;          /* in [1, LORA_PLAN_MAX_KSPLIT_MFMA]; at most
                              LORA_PLAN_MAX_KSPLIT_MFMA_WIDE when
                              max_lora_rank > 32 */
  int32_t bgmv_mfma_min_rows;  /* INT32_MAX when no BGMV run uses MFMA tiles */
  int32_t ksplit_wave;     /* in [1, LORA_PLAN_MAX_KSPLIT] */
  int32_t reserved;        /* 0 */
  int64_t image_offset;    /* bytes from meta_host to the device image (16-byte aligned) */
  int64_t image_bytes;
  int64_t off_perm;        /* int32 offsets inside the image */
  int64_t off_wave;
  int64_t off_mfma;
} lora_plan;

/* Host half of lora_apply: validates the arguments, builds the metadata
 * (lora_build_meta's arrays, in the front of meta_host) and packs the tile
 * plan's device image behind it.  No HIP call; deterministic.  Returns
 * LORA_OK, LORA_E_ID for an id outside [-1, max_loras), LORA_E_WORKSPACE if
 * meta_host_bytes < lora_apply_host_meta_bytes(desc, T), LORA_E_ARG for NULL
 * pointers or T < 0. */
int32_t lora_apply_plan(const lora_pool_desc* desc, int32_t T, const int32_t* ids_host,
                        const uint8_t* prefill_host, int32_t bgmv_max_rank, void* meta_host,
                        int64_t meta_host_bytes, lora_plan* plan);

/* lora_apply_plan for pools whose slots hold adapters of smaller rank than
 * max_lora_rank ([TGI] step 3 pads every adapter to the slot rank; this
 * variant skips the padding).  slot_ranks: host int32[max_loras], the rank of
 * the adapter in each slot, 0 = max_lora_rank; the tile records then carry it
 * (rounded up to 8) and the bf16 MFMA kernels skip the padded ranks' weight
 * loads and products, which are zero: the result equals lora_apply_plan's.
 * Plans that travel in the kernel arguments (at most 48 wavefront tiles) and
 * the fp32 and R > 64 kernels use max_lora_rank.  LORA_E_RANK for an entry
 * outside [0, max_lora_rank]; otherwise as lora_apply_plan. */
int32_t lora_apply_plan_ranked(const lora_pool_desc* desc, int32_t T, const int32_t* ids_host,
                               const uint8_t* prefill_host, int32_t bgmv_max_rank,
                               const int32_t* slot_ranks, void* meta_host,
                               int64_t meta_host_bytes, lora_plan* plan);

/* Device half of a plan, so one plan can serve every layer of a batch.
 *   image:      device copy of the plan's image (16-byte aligned,
 *               plan->image_bytes long), or NULL when image_host is given and
 *               the plan is small.
 *   image_host: host copy of the image (as lora_apply_plan leaves it in
 *               meta_host), or NULL.  A small plan (no MFMA tiles, at most 48
 *               wavefront tiles, max_loras <= 2^28) with a host copy travels
 *               in the kernel arguments and `image` is not read; otherwise
 *               `image` is used.
 *   v:          device fp32 [max(ksplit, ksplit_wave)][num_sgmv_rows +
 *               num_bgmv_rows][S][R]
 *               (plan row order; partial p of row i at
 *               ((p * rows + i) * S + s) * R + k).
 *   lora_plan_shrink:  v[row][s][k] = sum_j A_pool[a][s][k][j] * x[t][j] for
 *                      every row of every tile ([TGI] step 4, shrink)
 *   lora_plan_expand:  y[t][off_s + j] = round_dtype((float)y[t][off_s + j] +
 *                      sum_k B_pool[a][off_s + j][k] * v[row][s][k])
 * Rows whose token, slot or row index is out of range are skipped.  Returns
 * LORA_E_ARG for NULL pointers or a malformed plan, LORA_E_ALIGN for a
 * misaligned image, LORA_E_DTYPE for MFMA tiles on an fp32 pool.  The host
 * image is read before the call returns. */
int32_t lora_plan_shrink(const lora_pool_desc* desc, const void* x, const void* A_pool, float* v,
                         int32_t T, const lora_plan* plan, const void* image,
                         const void* image_host, void* stream);
int32_t lora_plan_expand(const lora_pool_desc* desc, const float* v, const void* B_pool, void* y,
                         int32_t T, const lora_plan* plan, const void* image,
                         const void* image_host, void* stream);

/* Both stages of a plan on `stream` ([TGI] step 4: shrink, then expand), so
 * one plan serves every layer of a batch: y[t] += B_a (A_a x[t]) for every
 * row of every tile, the result of lora_plan_shrink followed by
 * lora_plan_expand.
 *   image, image_host: as for lora_plan_shrink.
 *   ws: device workspace of >= lora_apply_workspace_bytes(desc, T) bytes,
 *     16-byte aligned (v of the two-launch form).
 * A plan of at most 12 wavefront tiles (and no MFMA tiles) on a bf16 pool with
 * max_lora_rank <= 32 runs as ONE launch in which every workgroup computes
 * its tile's v (MFMA) and applies it to its output columns; otherwise the stages are lora_plan_shrink and
 * lora_plan_expand.  LORA_ONEPASS_DECODE=0 in the environment turns the
 * one-launch form off.  Returns as lora_plan_shrink, plus LORA_E_WORKSPACE
 * for a short ws. */
int32_t lora_plan_apply(const lora_pool_desc* desc, const void* x, const void* A_pool,
                        const void* B_pool, void* y, int32_t T, const lora_plan* plan,
                        const void* image, const void* image_host, void* ws, int64_t ws_bytes,
                        void* stream);

/* The whole delta path for one batch ([TGI] step 4; [QA] direct answer):
 * lora_apply_plan into meta_host, then lora_plan_apply on `stream`, updating y
 * in place.  Rows with id -1 are never read or written.
 * The plan reaches the kernels in one of three ways: a small plan goes in the
 * kernel arguments; otherwise, if meta_host is pinned (hipHostMalloc), the
 * kernels read the plan's image from meta_host itself; otherwise the image is
 * copied into ws.
 *   ids_host[T], prefill_host[T] (NULL = all decode): host arrays.
 *   ws: device workspace of >= lora_apply_workspace_bytes(desc, T) bytes.
 *   meta_host: host staging of >= lora_apply_host_meta_bytes(desc, T) bytes,
 *     16-byte aligned.  If it is pinned the caller must not rewrite it until
 *     the stream has passed this call; pageable memory may be reused as soon
 *     as the call returns.
 * Returns without synchronising.  T = 0 is a no-op. */
int32_t lora_apply(const lora_pool_desc* desc, const void* A_pool, const void* B_pool,
                   const void* x, void* y, int32_t T, const int32_t* ids_host,
                   const uint8_t* prefill_host, int32_t bgmv_max_rank, void* ws,
                   int64_t ws_bytes, void* meta_host, int64_t meta_host_bytes, void* stream);

/* The whole delta path from device ids, with no host work that depends on
 * the batch (so the calls can be captured in a graph and replayed with new ids
 * and flags written into the same buffers): lora_build_meta_device's
 * metadata ([TGI] step 4), then a device-built plan of 8-row tiles of one
 * adapter, then the tile kernels' shrink and expand, all on `stream`.
 *   ids, prefill  device arrays of T entries (prefill may be NULL = all 0);
 *                 ids outside [-1, max_loras) are skipped like -1 (the host
 *                 path rejects them with LORA_E_ID; here no host code sees
 *                 the ids), and counted: see ws
 *   ws            device workspace of lora_apply_device_workspace_bytes(desc,
 *                 T) bytes, 256-byte aligned: metadata, the tile records, v.
 *                 Once the stream has passed the call, its first four int32
 *                 words hold the batch's SGMV rows, SGMV segments, BGMV rows
 *                 and the number of rows whose id was outside [-1, max_loras):
 *                 a caller that must not serve such rows from the base model
 *                 alone reads word 3 back and treats non-zero as an error
 * The result is lora_apply's (within rounding: the K split may differ).
 * The plan follows the host plan's rules except that decode rows always take
 * 8-row tiles; its record counts are known on the host only as capacities
 * (surplus records have 0 rows).  The metadata is built by one workgroup, so
 * large prefill batches are faster through lora_apply.  Errors (before any
 * HIP call): LORA_E_SHAPE if
 * max_loras > LORA_META_DEVICE_MAX_LORAS, LORA_E_WORKSPACE, LORA_E_ALIGN,
 * LORA_E_ARG; T = 0 is a no-op. */
int64_t lora_apply_device_workspace_bytes(const lora_pool_desc* desc, int32_t T);
int32_t lora_apply_device(const lora_pool_desc* desc, const void* A_pool, const void* B_pool,
                          const void* x, void* y, int32_t T, const int32_t* ids,
                          const uint8_t* prefill, int32_t bgmv_max_rank, void* ws,
                          int64_t ws_bytes, void* stream);

/* lora_apply_device with each slot's true rank, as lora_apply_ranked:
 * slot_ranks is a device int32[max_loras] (0 = max_lora_rank; read by the
 * GPU, so it is not validated on the host: a value outside [0,
 * max_lora_rank] acts as max_lora_rank).  The tile records carry the ranks
 * and the bf16 MFMA kernels skip the padded ones; plans small enough for the
 * one-launch decode kernel use max_lora_rank.  Same result as
 * lora_apply_device. */
int32_t lora_apply_device_ranked(const lora_pool_desc* desc, const void* A_pool,
                                 const void* B_pool, const void* x, void* y, int32_t T,
                                 const int32_t* ids, const uint8_t* prefill,
                                 int32_t bgmv_max_rank, const int32_t* slot_ranks, void* ws,
                                 int64_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * path and result as lora_apply_device (bit for bit: the same kernels, plan
 * and K splits), but the workspace is the library's own: a file-scope device
 * array of LORA_NOALLOC_SCRATCH_BYTES bytes per GPU, created with the
 * library's code object the first time the library runs on that GPU and held
 * until the process ends.  The call allocates and frees nothing (no
 * hipMalloc, no allocating library routine); the caller passes the pool, x, y,
 * ids and prefill as for lora_apply_device.
 *   Size limit: a batch whose lora_apply_device_workspace_bytes(desc, T)
 *   exceeds LORA_NOALLOC_SCRATCH_BYTES is rejected with LORA_E_WORKSPACE
 *   before any HIP call (for S * R = 16 that is about 130 000 rows, for
 *   S * R = 128 about 16 000).
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the
 *   previous call's contents; nothing in it needs clearing (each call writes
 *   every byte it reads before reading it).  Calls on one stream are ordered
 *   and safe; calls that overlap on one GPU (other streams, other threads)
 *   race on the array and give undefined results.
 *   Errors: as lora_apply_device, plus LORA_E_WORKSPACE for the size limit and
 *   LORA_E_HIP if the array's address cannot be obtained.  T = 0 is a no-op. */
#define LORA_NOALLOC_SCRATCH_BYTES (64u << 20)
int32_t lora_apply_device_noalloc(const lora_pool_desc* desc, const void* A_pool,
                                  const void* B_pool, const void* x, void* y, int32_t T,
                                  const int32_t* ids, const uint8_t* prefill,
                                  int32_t bgmv_max_rank, void* stream);

/* lora_apply with each slot's true rank (slot_ranks as in
 * lora_apply_plan_ranked, nullable): same result, padded ranks skipped. */
int32_t lora_apply_ranked(const lora_pool_desc* desc, const void* A_pool, const void* B_pool,
                          const void* x, void* y, int32_t T, const int32_t* ids_host,
                          const uint8_t* prefill_host, int32_t bgmv_max_rank,
                          const int32_t* slot_ranks, void* ws, int64_t ws_bytes,
                          void* meta_host, int64_t meta_host_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_POOL_H */
