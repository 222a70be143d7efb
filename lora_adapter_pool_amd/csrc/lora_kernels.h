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
constexpr int kWaveTileRows = 8;       // rows per tile of the VALU kernels
constexpr int kExpandCols = 256;       // output columns per VALU expand workgroup
constexpr int kExpandMfmaCols = 128;   // output columns per MFMA expand workgroup
constexpr int kSgmvMfmaMinRows = 16;   // SGMV segments this long or longer use MFMA (bf16)

// A list of rows to process.  Row i reads token tok[i] of x / y and writes row i
// of v.  BGMV: ids != nullptr gives the adapter slot of every row.  SGMV:
// ids == nullptr; segments give [start, start + len) ranges of rows sharing
// seg_ids[g]; only segments whose clamped length is in [seg_min, seg_max] are
// covered by a given launch.
struct RowList {
  const int32_t* tok;
  const int32_t* ids;
  const int32_t* seg_starts;
  const int32_t* seg_lens;
  const int32_t* seg_ids;
  int32_t num_segs;
  int32_t num_rows;
  int32_t seg_min;
  int32_t seg_max;
};

// Column chunks of the fused output: chunk c belongs to slice s when
// start[s] <= c < start[s + 1].
struct Chunks {
  int32_t total;
  int32_t start[LORA_MAX_SLICES + 1];
};

// Enqueue the shrink / expand of one row list on `st`.  host_seg_* (nullable)
// are host copies of the segment arrays; with them the grids are exact.
int32_t run_shrink(const Geo& g, const void* x, const void* A, float* v, RowList L,
                   const int32_t* host_seg_starts, const int32_t* host_seg_lens, hipStream_t st);
int32_t run_expand(const Geo& g, const float* v, const void* B, void* y, RowList L,
                   const int32_t* host_seg_starts, const int32_t* host_seg_lens, hipStream_t st);
int32_t run_pool_load(const Geo& g, void* A_slot_slice, void* B_slot_slice, const void* Asrc,
                      const void* Bsrc, int r, int out_s, float scale, hipStream_t st);

}  // namespace lora
