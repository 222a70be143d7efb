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

// Host metadata staging layout used by lora_apply (int32 offsets).
struct MetaLayout {
  int64_t perm, seg_starts, seg_lens, seg_ids, bgmv_tok, bgmv_ids, total_ints;
};
MetaLayout meta_layout(int32_t T, int32_t max_loras);
int64_t align_up(int64_t v, int64_t a);

// Builder core (no argument checks beyond what lora_build_meta does).
int32_t build_meta_core(const int32_t* ids, const uint8_t* prefill, int32_t T,
                        int32_t max_loras, int32_t max_lora_rank, int32_t bgmv_max_rank,
                        lora_meta* out);

bool log_enabled();

}  // namespace lora
