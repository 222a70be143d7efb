// Launch-side declarations of the gfx950 kernels (used by the C ABI layer).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdlib>

#include "lora_internal.h"

namespace lora {

constexpr int kNumXcd = 8;             // XCDs on MI355X; workgroups are dealt round-robin
constexpr int kWaveTileRows = LORA_PLAN_WAVE_ROWS;  // rows per tile of the VALU kernels
constexpr int kMfmaTileRows = LORA_PLAN_MFMA_ROWS;  // rows per tile of the MFMA kernels
constexpr int kExpandCols = 256;       // output columns per VALU expand workgroup
constexpr int kExpandMfmaCols = 128;   // output columns per MFMA expand workgroup
// Plans of wavefront tiles only go by value in the kernel arguments: packed
// records of kArgWords words, up to kArgTilesS (480 bytes) or kArgTilesL tiles.
constexpr int kArgWords = 2 + LORA_PLAN_WAVE_ROWS;
constexpr int kArgTilesS = 12;
constexpr int kArgTilesL = 48;
constexpr int kMaxKsplit = LORA_PLAN_MAX_KSPLIT_MFMA;  // K splits of the MFMA shrink (R <= 32)
constexpr int kMaxKsplitWide = LORA_PLAN_MAX_KSPLIT_MFMA_WIDE;  // ... for R > 32
constexpr int kMaxKsplitWave = LORA_PLAN_MAX_KSPLIT;   // K splits of the wavefront tiles

// A list of rows to process.  Row i reads token tok[i] of x / y and writes row i
// of v.  Three ways to cut it into tiles, one adapter per tile:
//   segments  (ids == tiles == nullptr): [seg_starts[g], + seg_lens[g]) share
//             seg_ids[g]; a launch covers the segments whose clamped length is
//             in [seg_min, seg_max]; tiles are found on the device.
//   rows      (ids != nullptr): fixed ranges of rows; ids[i] is row i's adapter.
//   tile list (tiles != nullptr): num_tiles host-built records (the plan's
//             layout); tok is the plan's perm (used by the MFMA kernels).
// In tile-list mode the shrink kernels can also copy what they read of the
// list into device memory (copy_tiles: the records; copy_tok: the tokens of
// MFMA tile rows) so that the expand launch reads the copy instead: lora_apply
// passes a list that lives in pinned host memory, where every read crosses
// PCIe.
struct RowList {
  const int32_t* tok;
  const int32_t* ids;
  const int32_t* seg_starts;
  const int32_t* seg_lens;
  const int32_t* seg_ids;
  const int32_t* tiles;
  int32_t num_segs;
  int32_t num_rows;
  int32_t num_tiles;
  int32_t seg_min;
  int32_t seg_max;
  int32_t* copy_tiles;
  int32_t* copy_tok;
};

inline RowList segments_list(const int32_t* perm, const int32_t* starts, const int32_t* lens,
                             const int32_t* sids, int32_t num_segs, int32_t num_rows) {
  return RowList{perm, nullptr, starts, lens, sids, nullptr, num_segs, num_rows, 0, 0, INT32_MAX};
}

inline RowList rows_list(const int32_t* tok, const int32_t* ids, int32_t n) {
  return RowList{tok, ids, nullptr, nullptr, nullptr, nullptr, 0, n, 0, 0, INT32_MAX};
}

// Column chunks of the fused output: chunk c belongs to slice s when
// start[s] <= c < start[s + 1].
struct Chunks {
  int32_t total;
  int32_t start[LORA_MAX_SLICES + 1];
};

// Device copy of a lora_plan image (pointers into the workspace).
struct TilePlan {
  const int32_t* perm;
  const int32_t* wave;
  int32_t wave_tiles;
  const int32_t* mfma;
  int32_t mfma_tiles;
  const int32_t* wave_host;  // host copy of the wave records, or nullptr
  int32_t ksplit;            // partials of the MFMA tiles' shrink
  int32_t num_rows;          // v rows (SGMV rows, then BGMV rows) = entries of perm
  int32_t ksplit_wave;       // partials of the wavefront tiles' shrink (bf16, R <= 64)
  // device copy of the image (same offsets) that the shrink launches write and
  // the expand launches read, or nullptr: the expand reads perm / wave / mfma
  int32_t* copy_perm;
  int32_t* copy_wave;
  int32_t* copy_mfma;
  // 1 when wave_tiles (and mfma_tiles) are capacities (a device-built plan):
  // its records come first, then records without rows
  int32_t walk;
};

// Enqueue the shrink / expand of one row list (segments or rows) on `st`;
// grids are upper bounds, surplus workgroups exit after the tile lookup.
int32_t run_shrink(const Geo& g, const void* x, const void* A, float* v, RowList L,
                   hipStream_t st);
int32_t run_expand(const Geo& g, const float* v, const void* B, void* y, RowList L,
                   hipStream_t st);
// The shrink (MFMA tiles, then wavefront tiles) or expand launches of a tile
// plan, exact grids.
int32_t run_plan_shrink(const Geo& g, const void* x, const void* A, float* v, const TilePlan& p,
                        hipStream_t st);
int32_t run_plan_expand(const Geo& g, const float* v, const void* B, void* y, const TilePlan& p,
                        hipStream_t st);
// Both stages of a plan: one launch (each workgroup computes its tile's v with
// MFMA and applies it to its columns) for bf16 decode plans of at most
// kArgTilesS tiles with R <= 32, else run_plan_shrink then run_plan_expand
// (v: the plan's rows).
bool plan_is_onepass(const Geo& g, const TilePlan& p);
// A device-built plan of at most kDeviceOnepassCap records (bf16, R <= 32)
// runs as that one launch too, reading its records from device memory
// (records with 0 rows exit at once).
constexpr int32_t kDeviceOnepassCap = 24;
bool device_plan_is_onepass(const Geo& g, int32_t cap);
int32_t run_plan_onepass_list(const Geo& g, const void* x, const void* A, const void* B, void* y,
                              const TilePlan& p, hipStream_t st);
int32_t run_plan_apply(const Geo& g, const void* x, const void* A, const void* B, void* y,
                       const TilePlan& p, float* v, hipStream_t st);
// Outputs of a device-built plan (lora_apply_device): cap 8-row tile records,
// mcap 64-row MFMA tile records and the v-row -> token map perm[T] (written
// during placement; entries past the batch's rows are left as they were and
// no record reaches them).  A slot's
// SGMV rows take MFMA tiles when there are at least mfma_min of them; its BGMV
// rows when there are at least bgmv_min of them and such runs hold at least
// bgmv_total rows of the batch (values above T disable either).  Records past
// the last tile have 0 rows.
struct DevicePlanOut {
  int32_t* tiles;
  int32_t cap;
  int32_t* mtiles;
  int32_t mcap;
  int32_t mfma_min;
  int32_t bgmv_min;
  int32_t bgmv_total;
  int32_t* perm;
  const int32_t* slot_ranks;  // device int32[max_loras] or nullptr: records carry ranks
  int32_t R;                  // the pool's rank (records carry 0 for it)
};
// Device-side builder (csrc/lora_meta.hip): lora_build_meta's arrays from
// device ids, one workgroup on `st`; counts[4] = rows, segments, BGMV rows,
// rejected ids.  With `plan` it writes a device-built plan (its v-row -> token
// map and tile records) instead of those arrays, which m then need not hold.
int32_t run_build_meta_device(const int32_t* ids, const uint8_t* prefill, int32_t T,
                              int32_t max_loras, bool all_sgmv, const lora_meta& m,
                              int32_t* counts, hipStream_t st,
                              const DevicePlanOut* plan = nullptr);
int32_t run_pool_load(const Geo& g, void* A_slot_slice, void* B_slot_slice, const void* Asrc,
                      const void* Bsrc, int r, int out_s, float scale, hipStream_t st);

}  // namespace lora
