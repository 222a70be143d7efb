// Internal declarations shared by the host logic and the HIP launchers.
#pragma once

#include <cstdint>
#include <cstddef>

#include "lora_pool.h"

namespace lora {

// Geometry derived from a validated lora_pool_desc.
struct Geo {
  int32_t dtype;
  int32_t max_loras;
  int32_t R;         // padded slot rank
  int32_t K;         // in_features
  int32_t S;         // slices
  int32_t O;         // sum of out_features
  int32_t T;         // rows of x and y for the current call
  int32_t out[LORA_MAX_SLICES];
  int32_t off[LORA_MAX_SLICES];
};

// Records a thread-local message and returns `code`.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Validates a descriptor and fills `g` (g->T is set to 0).
int32_t check_desc(const lora_pool_desc* desc, Geo* g);

inline int64_t elem_bytes(int32_t dtype) { return dtype == LORA_BF16 ? 2 : 4; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// lora_apply's host staging (int32 words): the builder's arrays, then the
// plan's device image (16-byte aligned), which is what gets copied to the GPU.
struct StageLayout {
  int64_t perm, seg_starts, seg_lens, seg_ids, bgmv_tok, bgmv_ids;
  int64_t image;            // first word of the device image
  int64_t image_max_words;  // capacity of the device image
  int64_t total_words;
};
StageLayout stage_layout(int32_t T, int32_t max_loras);

// lora_apply's device workspace (byte offsets): the plan image (when it is
// copied), then v (LORA_PLAN_MAX_KSPLIT partials of T rows x S x R fp32).
struct WorkspaceLayout {
  int64_t v, total;
};
WorkspaceLayout workspace_layout(const Geo& g, int32_t T);
int64_t align_up(int64_t v, int64_t a);

// SGMV segments at least this long run on MFMA tiles (bf16 pools); the
// environment variable LORA_SGMV_MFMA_MIN_ROWS overrides the default of 16.
int32_t sgmv_mfma_min_rows();
// BGMV runs of one adapter at least bgmv_mfma_min_rows long (default 48,
// LORA_BGMV_MFMA_MIN_ROWS) run on 64-row MFMA tiles when such runs hold at
// least bgmv_mfma_min_total(R) rows of the batch (default 2048 for pools of
// rank R <= 16, else 1024; LORA_BGMV_MFMA_MIN_TOTAL overrides both).
int32_t bgmv_mfma_min_rows();
int32_t bgmv_mfma_min_total(int32_t R);

// MFMA shrink of wavefront tiles (bf16 pools, R <= 64): rank tiles of 16 it
// computes (R = 48 takes 4) and the 32-wide K chunks each wave loads per batch.
constexpr int32_t tile_shrink_rank_tiles(int32_t R) { return R <= 16 ? 1 : R <= 32 ? 2 : 4; }
constexpr int32_t tile_shrink_cb(int32_t R) {
  return tile_shrink_rank_tiles(R) == 1 ? 8 : tile_shrink_rank_tiles(R) == 2 ? 6 : 4;
}
constexpr int32_t kTileShrinkWaves = 4;  // waves per workgroup of that shrink
// Most partials of v that shrink writes: 8 (LORA_PLAN_MAX_KSPLIT).
constexpr int32_t tile_kparts_max(int32_t R) { return R <= 64 ? LORA_PLAN_MAX_KSPLIT : 4; }
// Compute units of an MI355X (the K splits balance workgroups over them).
constexpr int64_t kComputeUnits = 256;
// ... for a device-built plan (its 8-row kernels walk their records), whose
// walking expand sums at most this many partials for pools of rank above 32
constexpr int32_t kMaxWalkKpartsWide = 2;
constexpr int32_t walk_kparts_max(int32_t R) {
  return R > 32 ? kMaxWalkKpartsWide : tile_kparts_max(R);
}

// K split of the wavefront tiles' MFMA shrink for a plan of nw such tiles
// (bf16, R <= 64; else 1): the split that leaves the least work on the
// busiest compute unit, with at most four workgroups per compute unit and one
// full load batch per wave in every part.
int32_t wave_ksplit(const Geo& g, int64_t nw);
// K split of the 64-row MFMA tiles' shrink for a plan of nm such tiles: the
// split that leaves the least work on the busiest compute unit (the most
// parts on a tie), among those up to mfma_ksplit_max(g) that start below 512
// workgroups and keep four 64-wide K steps per part.  four_stages (a host
// plan whose shrink is DMA-staged): a tie between at most one workgroup per
// compute unit and at most two goes to the former.
int32_t mfma_ksplit(const Geo& g, int64_t nm, bool four_stages = false);
// Widest K of the DMA-staged 64-row MFMA shrink (K a multiple of 64).
constexpr int32_t kDmaShrinkMaxK = 8192;
// most partials that split may use for this pool: LORA_PLAN_MAX_KSPLIT_MFMA
// for R <= 32, LORA_PLAN_MAX_KSPLIT_MFMA_WIDE above
int32_t mfma_ksplit_max(const Geo& g);

// Device-built plan of lora_apply_device: capacities of its 8-row tile
// records (each slot adds at most one partial tile to each of its two row
// sets) and of its 64-row MFMA tile records, and its workspace (byte
// offsets): the metadata arrays, the v-row -> token map, both record arrays,
// then v (LORA_PLAN_MAX_KSPLIT partials of T rows x S x R fp32).
inline int32_t device_tile_cap(int32_t T, int32_t max_loras) {
  return (T + LORA_PLAN_WAVE_ROWS - 1) / LORA_PLAN_WAVE_ROWS + 2 * (T < max_loras ? T : max_loras);
}
// Every MFMA record is a piece of a run of one slot's rows that takes MFMA
// tiles: its SGMV rows when there are at least sgmv_mfma_min_rows() of them
// (possible only when `sgmv` says the batch can hold SGMV rows) and, in
// batches of at least bgmv_mfma_min_total(R) rows, its BGMV rows when there
// are at least bgmv_mfma_min_rows().  The pieces of runs holding n rows in all
// number at most ceil(n / 64) + runs, and at most min(max_loras, T / min rows)
// runs of each kind exist; the count never exceeds the per-slot bound
// ceil(T / 64) + 2 min(T, max_loras) either.
int32_t device_mfma_cap(const Geo& g, int32_t T, bool sgmv);
struct DeviceLayout {
  int64_t counts, sgmv_perm, bgmv_tok, bgmv_ids, seg_starts, seg_lens, seg_ids, perm, tiles,
      mtiles, v, total;
};
DeviceLayout device_layout(const Geo& g, int32_t T);

// Builder core (no argument checks beyond what lora_build_meta does).
int32_t build_meta_core(const int32_t* ids, const uint8_t* prefill, int32_t T,
                        int32_t max_loras, int32_t max_lora_rank, int32_t bgmv_max_rank,
                        lora_meta* out);

// Host half of lora_apply on validated arguments: metadata and tile plan into
// `stage` (stage_layout(T, g.max_loras).total_words words).  slot_ranks
// (nullable, max_loras entries in [0, R], 0 = R) gives each slot's true rank:
// tile records then carry it (rounded up to 8) so the MFMA kernels skip the
// padded ranks.
int32_t plan_core(const Geo& g, int32_t T, const int32_t* ids, const uint8_t* prefill,
                  int32_t bgmv_max_rank, int32_t* stage, lora_plan* plan,
                  const int32_t* slot_ranks = nullptr);
// slot_ranks entries in [0, R]
int32_t check_slot_ranks(const Geo& g, const int32_t* slot_ranks);

bool log_enabled();

}  // namespace lora
