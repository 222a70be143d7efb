// gfx950 (MI355X) kernels of the multi-LoRA delta path.
//
// Two stages per row list (step 4 of the TGI multi-LoRA article: shrink
// x -> r, then expand r -> out, grouped by adapter):
//   shrink: v[i][s][k]   = sum_j A_pool[a][s][k][j] * x[t][j]          (fp32 acc)
//   expand: y[t][off_s+j] = rne(y[t][off_s+j] + sum_k B_pool[a][off_s+j][k] * v[i][s][k])
//
// Work is cut into tiles of consecutive rows of one adapter.  Three ways to
// find a workgroup's tile: a host-built tile list (lora_apply's plan: one
// 64-byte record load), SGMV segments (block-parallel prefix sum over the
// segment arrays on the device) or BGMV rows with per-row ids (fixed row
// ranges; a tile then processes each distinct adapter once).
//
// Kernels:
//   shrink_wave   VALU, up to 16 waves split K, 8 contiguous elements per
//                 lane (16-byte loads), rank chunks across workgroups; the K
//                 reduction is a wavefront transpose-reduce plus a fixed-order
//                 sum of the waves' partials in LDS (deterministic).
//   expand_wave   VALU, one output column per thread; the B block of the tile
//                 is copied from HBM into LDS with contiguous 16-byte loads and
//                 read back row-per-thread (padded rows, no bank conflicts);
//                 v rows are LDS broadcasts.
//   shrink_mfma   bf16 MFMA 16x16x32 for long SGMV segments: x rows are the
//                 A operand, adapter A rows the B operand, fp32 accumulators.
//   expand_mfma   bf16 MFMA 16x16x32 computing (B_pool tile) x v^T so that each
//                 lane ends with 8 consecutive output columns of one token
//                 (16-byte y read-modify-write); fp32 v enters as a hi + lo
//                 bf16 pair (two MFMAs), keeping ~16 mantissa bits of v.
//
// Workgroup ids are remapped so that consecutive tiles (which share adapter
// weights and, across rank chunks, x rows) land on the same XCD's L2: the
// hardware deals workgroups round-robin over the 8 XCDs.
//
// Every token index, adapter slot and row index read from device metadata is
// bounds-checked against T, max_loras and the row count; rows that fail are
// skipped, never dereferenced.
#include <hip/hip_runtime.h>

#include "lora_internal.h"
#include "lora_kernels.h"

namespace lora {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32 converts two values per instruction; lo lands in bits
// 0..15, hi in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming (non-temporal) forms for data a kernel touches once: the x rows
// of a long segment, y rows of a read-modify-write.  On MI355X they sustain
// about a tenth more HBM bandwidth than the default cache policy (6.9 against
// 6.2 TB/s streaming reads, 6.0 against 5.4 TB/s in-place updates).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3..0 and 15..14,
// expcnt 6..4, lgkmcnt 11..8): at most 4 vector memory operations and no LDS
// operation outstanding; no vector memory operation outstanding; no LDS
// operation outstanding (vector memory operations may be)
constexpr int kWaitVm4Lgkm0 = 0x0074;
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// A workgroup barrier for the reuse of LDS only: each wave's LDS accesses
// are complete, its global stores may still be in flight.  __syncthreads also
// orders global memory at workgroup scope, so every wave would first wait for
// its stores to land, a memory round trip per barrier.  (The empty asm
// statements keep the compiler from moving LDS accesses across the barrier.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// All-ones or all-zeros, to zero a loaded value with a bit-AND: a select on a
// loaded value lets the compiler sink the load under a branch, after which it
// has to drain every outstanding load before continuing.
__device__ __forceinline__ uint32_t all_or_none(bool b) { return b ? 0xffffffffu : 0u; }

// Raw buffer over `bytes` bytes at `base` (gfx9 descriptor word 3: 32-bit
// untyped data, no swizzle).  A 16-byte store at a byte offset at or past the
// end is dropped by the hardware, so lanes with nothing to write still issue
// the store instruction: the compiler can then count outstanding memory
// operations exactly across a loop instead of draining them all.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kDropOffset = 0x80000000u;  // past every buffer made by make_rsrc
__device__ __forceinline__ void st16_buf(u32x4 val, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(val, r, (int)off, 0, 0);
}
// the same store with the non-temporal cache policy (aux bit 1)
__device__ __forceinline__ void st16_buf_nt(u32x4 val, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(val, r, (int)off, 0, 2);
}
// 16-byte loads through a raw buffer: a 32-bit offset per lane instead of a
// 64-bit address (fewer registers); the caller keeps every offset in bounds
__device__ __forceinline__ u32x4 ld16_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x4 ld16_buf_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}

// Element access: 8 consecutive elements travel as one Raw (16 bytes of bf16
// or 32 bytes of fp32) and are widened to fp32 only where they are used.
template <typename E> struct El;

template <> struct El<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  struct Raw { u32x4 a, b; };
  static __device__ __forceinline__ Raw raw8(const float* p) { return {ld16(p), ld16(p + 4)}; }
  static __device__ __forceinline__ void mask(Raw& r, uint32_t m) { r.a &= m; r.b &= m; }
  static __device__ __forceinline__ void unpack(const Raw& r, float (&o)[8]) {
    o[0] = __uint_as_float(r.a.x); o[1] = __uint_as_float(r.a.y);
    o[2] = __uint_as_float(r.a.z); o[3] = __uint_as_float(r.a.w);
    o[4] = __uint_as_float(r.b.x); o[5] = __uint_as_float(r.b.y);
    o[6] = __uint_as_float(r.b.z); o[7] = __uint_as_float(r.b.w);
  }
  static __device__ __forceinline__ void load8(const float* p, float (&o)[8]) { unpack(raw8(p), o); }
  static __device__ __forceinline__ float get(float v) { return v; }
  static __device__ __forceinline__ float put(float v) { return v; }
};

template <> struct El<uint16_t> {
  static constexpr int kVec = 8;
  struct Raw { u32x4 a; };
  static __device__ __forceinline__ Raw raw8(const uint16_t* p) { return {ld16(p)}; }
  static __device__ __forceinline__ void mask(Raw& r, uint32_t m) { r.a &= m; }
  static __device__ __forceinline__ void unpack(const Raw& r, float (&o)[8]) {
    o[0] = __uint_as_float(r.a.x << 16); o[1] = __uint_as_float(r.a.x & 0xffff0000u);
    o[2] = __uint_as_float(r.a.y << 16); o[3] = __uint_as_float(r.a.y & 0xffff0000u);
    o[4] = __uint_as_float(r.a.z << 16); o[5] = __uint_as_float(r.a.z & 0xffff0000u);
    o[6] = __uint_as_float(r.a.w << 16); o[7] = __uint_as_float(r.a.w & 0xffff0000u);
  }
  static __device__ __forceinline__ void load8(const uint16_t* p, float (&o)[8]) { unpack(raw8(p), o); }
  static __device__ __forceinline__ float get(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  static __device__ __forceinline__ uint16_t put(float v) {
    return static_cast<uint16_t>(f32_to_bf16_bits(v));
  }
};

// Lane i of each row of 16 lanes takes the value of lane (i + 8) % 16 (DPP
// row_ror:8).  A DPP move reads its source lane whether or not that lane is
// active, and an inactive source gives no defined value, so the moves must run
// with every lane active: results are combined with pick() (bit masks), never
// with a conditional the compiler could turn into a branch around the move.
__device__ __forceinline__ u32x4 rot8_rows16(u32x4 v) {
  return u32x4{(uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, 0x128, 0xf, 0xf, false),
               (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, 0x128, 0xf, 0xf, false),
               (uint32_t)__builtin_amdgcn_mov_dpp((int)v.z, 0x128, 0xf, 0xf, false),
               (uint32_t)__builtin_amdgcn_mov_dpp((int)v.w, 0x128, 0xf, 0xf, false)};
}
// a where the lane mask m is all ones, b where it is zero (no branch)
__device__ __forceinline__ u32x4 pick(uint32_t m, u32x4 a, u32x4 b) { return (a & m) | (b & ~m); }

// Workgroups are dealt round-robin over the XCDs; give each XCD a contiguous
// range of logical ids (a bijection on [0, n)).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n / kNumXcd, r = n % kNumXcd;
  const int x = bid % kNumXcd, k = bid / kNumXcd;
  return x * q + min(x, r) + k;
}
// The same dealing in chunks of c consecutive logical ids, chunk j to XCD
// j % 8 (ids past the last whole round of 8 chunks keep their place): a
// bijection on [0, n) that spreads any prefix of the ids over every XCD.
__device__ __forceinline__ int xcd_remap_chunks(int bid, int n, int c) {
  if (c <= 0) return xcd_remap(bid, n);
  const int n0 = n / (kNumXcd * c) * (kNumXcd * c);
  if (bid >= n0) return bid;
  const int x = bid % kNumXcd, k = bid / kNumXcd;
  return ((k / c) * kNumXcd + x) * c + k % c;
}

// Segments mode: locate tile `f` (tiles of TM rows inside each segment whose
// clamped length lies in [seg_min, seg_max], in segment order).  Called by
// every thread of a workgroup of up to 1024 threads.  The segment arrays are
// read in parallel, one segment per thread per pass, and a block-wide prefix
// sum of tile counts finds the segment holding tile f, so the lookup costs one
// memory round trip rather than one per segment.  Returns false (uniformly)
// past the last tile; the results are the same in every lane.  The barrier at
// entry keeps the reset of s_found from racing with waves that still read the
// result of an earlier call, so a workgroup may call it more than once.
template <int TM>
__device__ __forceinline__ bool find_tile(const RowList& L, int f, int& r0, int& cnt, int& sid) {
  __shared__ int s_found[4];
  __shared__ int s_wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nthr = blockDim.x, nw = nthr >> 6;
  __syncthreads();
  if (tid == 0) s_found[3] = 0;
  int base = 0;
  bool found = false;
  for (int c0 = 0; c0 < L.num_segs; c0 += nthr) {
    const int gi = c0 + tid;
    int nt = 0, st = 0, ln = 0, id = -1;
    if (gi < L.num_segs) {
      st = L.seg_starts[gi];
      ln = L.seg_lens[gi];
      id = L.seg_ids[gi];
      if (st >= 0 && st < L.num_rows && ln > 0) {
        ln = min(ln, L.num_rows - st);
        if (ln >= L.seg_min && ln <= L.seg_max) nt = (ln + TM - 1) / TM;
      }
    }
    int inc = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    if (lane == 63) s_wsum[wv] = inc;
    __syncthreads();
    int wbase = 0, total = 0;
    for (int w = 0; w < nw; ++w) {
      const int ws = s_wsum[w];
      wbase += w < wv ? ws : 0;
      total += ws;
    }
    const int excl = base + wbase + inc - nt;
    if (nt > 0 && f >= excl && f < excl + nt) {
      const int j = f - excl;
      s_found[0] = st + j * TM;
      s_found[1] = min(TM, ln - j * TM);
      s_found[2] = id;
      s_found[3] = 1;
    }
    __syncthreads();
    found = s_found[3] != 0;
    base += total;
    if (found || f < base) break;
    __syncthreads();  // s_wsum is rewritten by the next pass
  }
  if (!found) return false;
  r0 = s_found[0];
  cnt = s_found[1];
  sid = s_found[2];
  return true;
}

// The same lookup within one wavefront (every wavefront of the workgroup
// computes it for itself, 64 segments per pass, a shuffle prefix sum and a
// ballot): no LDS and no barrier.  The 64-row MFMA kernels use it: beside
// the block-wide lookup's LDS array the compiler drains every outstanding
// load before each LDS read of the DMA-staged shrink's loop, which cannot
// then keep loads in flight across its steps.
template <int TM>
__device__ __forceinline__ bool find_tile_wave(const RowList& L, int f, int& r0, int& cnt,
                                               int& sid) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int c0 = 0; c0 < L.num_segs; c0 += 64) {
    const int gi = c0 + lane;
    int nt = 0, st = 0, ln = 0, id = -1;
    if (gi < L.num_segs) {
      st = L.seg_starts[gi];
      ln = L.seg_lens[gi];
      id = L.seg_ids[gi];
      if (st >= 0 && st < L.num_rows && ln > 0) {
        ln = min(ln, L.num_rows - st);
        if (ln >= L.seg_min && ln <= L.seg_max) nt = (ln + TM - 1) / TM;
      }
    }
    int inc = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    const int excl = base + inc - nt;
    const unsigned long long hit = __ballot(nt > 0 && f >= excl && f < excl + nt);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int j = f - __shfl(excl, src, 64);
      r0 = __builtin_amdgcn_readfirstlane(__shfl(st, src, 64) + j * TM);
      cnt = __builtin_amdgcn_readfirstlane(min(TM, __shfl(ln, src, 64) - j * TM));
      sid = __builtin_amdgcn_readfirstlane(__shfl(id, src, 64));
      return true;
    }
    base += __shfl(inc, 63, 64);
    if (f < base) break;
  }
  return false;
}

// How a kernel finds its tile: device segments, device rows with ids, the
// plan's device image, or records passed by value in two capacities.
// kListWalk: the plan's device image, like kList, for a plan whose record
// count is a capacity (a device-built plan: its records first, then empty
// ones); the 8-row tile kernels then walk several records per workgroup.
enum { kSegs = 0, kRows = 1, kList = 2, kArg = 3, kArgL = 4, kArgC = 5, kListWalk = 6 };

// Tile records passed by value (kArg, kArgL): a small plan travels in the
// kernel arguments, which the wavefronts read with scalar loads, so no copy of
// the plan precedes the launch.  Records are packed to kArgWords words (slot
// in bits 0..27 and rows in bits 28..31 of word 0, first v row, tokens), and
// the smaller capacity keeps the arguments short: the launch cost grows with
// their size.  Other modes carry an empty struct.
template <int MODE> struct PlanArg {};
template <> struct PlanArg<kArg> { int32_t w[kArgTilesS * kArgWords]; };
template <> struct PlanArg<kArgL> { int32_t w[kArgTilesL * kArgWords]; };
// Compact records for the one-launch decode kernel, which never touches v:
// word 0 as above, then the tokens as 16-bit halves (batches of T < 65536),
// 20 bytes a tile instead of 40.
constexpr int kArgCWords = 1 + kWaveTileRows / 2;
template <> struct PlanArg<kArgC> { uint32_t w[kArgTilesS * kArgCWords]; };
template <int MODE> constexpr int arg_tiles() { return MODE == kArgL ? kArgTilesL : kArgTilesS; }

// Rows of one tile, the same in every lane (scalar registers).  Row r is v row
// vrow0 + r, reads token tok[r] and uses adapter aid[r]; bit r of `valid` is
// set when the row exists and its token and adapter are in range.
template <int TM> struct TileRows {
  int vrow0;
  int cnt;
  int rank;  // ranks the tile's adapter uses: the record's rank, else the pool's R
  uint32_t valid;
  int tok[TM];
  int aid[TM];
};

// Tile f of a row list.  Lane r (< TM) fetches row r with one unconditional
// load (a clamped index for lanes past the last row) and the values are
// broadcast with readlane, so all rows cost one memory round trip.
//   kList: the host-built record (slot, rows, first v row, 0, tokens...) is
//          one 64-byte load, 16 lanes one word each.
//   kSegs: find_tile, then the tokens from tok[].
//   kRows: rows f*TM .. of the list, tokens and adapters from tok[] / ids[].
template <int TM, int MODE>
__device__ __forceinline__ bool tile_rows(const RowList& L, const Geo& g, int f,
                                          const PlanArg<MODE>& pa, TileRows<TM>& tr,
                                          bool copy = false, bool pre = false, int prew = 0) {
  static_assert(TM <= LORA_PLAN_WAVE_WORDS - 4, "a tile record holds at most 12 tokens");
  const int lane = threadIdx.x & 63;
  tr.rank = g.R;
  if constexpr (MODE == kArg || MODE == kArgL) {
    static_assert(TM <= kArgWords - 2, "a packed record holds kArgWords - 2 tokens");
    if (f >= L.num_tiles || f >= arg_tiles<MODE>()) return false;
    const int32_t* rec = pa.w + f * kArgWords;
    const int sid = rec[0] & 0x0fffffff;
    tr.cnt = (int)((uint32_t)rec[0] >> 28);
    tr.vrow0 = rec[1];
#pragma unroll
    for (int r = 0; r < TM; ++r) {
      tr.tok[r] = rec[2 + r];
      tr.aid[r] = sid;
    }
  } else if constexpr (MODE == kArgC) {
    static_assert(TM <= 2 * (kArgCWords - 1), "a compact record holds 2 tokens a word");
    if (f >= L.num_tiles || f >= arg_tiles<MODE>()) return false;
    const uint32_t* rec = pa.w + f * kArgCWords;
    const int sid = (int)(rec[0] & 0x0fffffffu);
    tr.cnt = (int)(rec[0] >> 28);
    tr.vrow0 = 0;  // no v rows: the kernel reading this form keeps v on chip
#pragma unroll
    for (int r = 0; r < TM; ++r) {
      tr.tok[r] = (int)((rec[1 + r / 2] >> (16 * (r & 1))) & 0xffffu);  // 0xffff: past T
      tr.aid[r] = sid;
    }
  } else if constexpr (MODE == kList || MODE == kListWalk) {
    if (f >= L.num_tiles) return false;
    // (pre: prew is this lane's word of record f, loaded earlier by the caller)
    const int w = pre ? prew : L.tiles[(size_t)f * LORA_PLAN_WAVE_WORDS + (lane & 15)];
    if (copy && L.copy_tiles && threadIdx.x < LORA_PLAN_WAVE_WORDS)
      L.copy_tiles[(size_t)f * LORA_PLAN_WAVE_WORDS + threadIdx.x] = w;
    const int sid = __builtin_amdgcn_readlane(w, 0);
    tr.cnt = __builtin_amdgcn_readlane(w, 1);
    tr.vrow0 = __builtin_amdgcn_readlane(w, 2);
    const int rk = __builtin_amdgcn_readlane(w, 3);
    tr.rank = rk > 0 && rk < g.R ? rk : g.R;
#pragma unroll
    for (int r = 0; r < TM; ++r) {
      tr.tok[r] = __builtin_amdgcn_readlane(w, 4 + r);
      tr.aid[r] = sid;
    }
  } else {
    int r0, cnt, sid = -1;
    if constexpr (MODE == kSegs) {
      if (!find_tile<TM>(L, f, r0, cnt, sid)) return false;
      r0 = __builtin_amdgcn_readfirstlane(r0);
      cnt = __builtin_amdgcn_readfirstlane(cnt);
      sid = __builtin_amdgcn_readfirstlane(sid);
    } else {
      r0 = f * TM;
      if (r0 >= L.num_rows) return false;
      cnt = min(TM, L.num_rows - r0);
    }
    // r0 + cnt <= num_rows by construction (find_tile clamps segments to the
    // row count; rows mode stops at it); the clamp keeps the load in bounds
    // whatever the metadata holds.
    const int ri = max(0, min(r0 + min(lane, max(cnt, 1) - 1), L.num_rows - 1));
    const int tv = L.tok[ri];
    const int av = MODE == kRows ? L.ids[ri] : sid;
    tr.cnt = cnt;
    tr.vrow0 = r0;
#pragma unroll
    for (int r = 0; r < TM; ++r) {
      tr.tok[r] = __builtin_amdgcn_readlane(tv, r);
      tr.aid[r] = MODE == kRows ? __builtin_amdgcn_readlane(av, r) : sid;
    }
  }
  uint32_t valid = 0;
#pragma unroll
  for (int r = 0; r < TM; ++r) {
    const bool ok = r < tr.cnt && tr.vrow0 >= 0 && tr.vrow0 + r < L.num_rows && tr.tok[r] >= 0 &&
                    tr.tok[r] < g.T && tr.aid[r] >= 0 && tr.aid[r] < g.max_loras;
    valid |= (ok ? 1u : 0u) << r;
    if (!ok) tr.tok[r] = 0;
  }
  tr.valid = valid;
  return true;
}

// Next adapter group of a tile: the adapter of the lowest pending row and the
// mask of pending rows that use it (one group per tile except in rows mode).
template <int TM>
__device__ __forceinline__ uint32_t next_group(uint32_t todo, const int (&aid)[TM], int& a) {
  const int first = __builtin_ctz(todo);
  a = -1;
#pragma unroll
  for (int r = 0; r < TM; ++r)
    if (r == first) a = aid[r];
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < TM; ++r)
    if (((todo >> r) & 1u) && aid[r] == a) m |= 1u << r;
  return m;
}

template <int N> struct Log2 { static constexpr int value = 1 + Log2<N / 2>::value; };
template <> struct Log2<1> { static constexpr int value = 0; };

// Sum V values across the 64 lanes of a wavefront.  Each butterfly step halves
// the number of values a lane carries (it keeps one half, sends the other), so
// V values cost V - 1 + (6 - log2 V) shuffles instead of 6 V.  On return lane l
// holds the complete sum of value index l >> (6 - log2 V).
template <int V>
__device__ __forceinline__ float wave_sum_many(float (&val)[V], int lane) {
  constexpr int P = Log2<V>::value;
  static_assert((1 << P) == V && P <= 6, "V must be a power of two <= 64");
#pragma unroll
  for (int step = 0; step < P; ++step) {
    const int half = V >> (step + 1);
    const int mask = 32 >> step;
    const bool upper = (lane & mask) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float lo = val[i], hi = val[i + half];
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      val[i] = keep + __shfl_xor(send, mask, 64);
    }
  }
  float r = val[0];
#pragma unroll
  for (int mask = 32 >> P; mask >= 1; mask >>= 1) r += __shfl_xor(r, mask, 64);
  return r;
}

// ------------------------------------------------------------ shrink (VALU)
//
// grid.x = tiles * S * (R / RC), blockDim = 64 * W with W = min(16, K / 512
// rounded up).  Workgroup (tile, slice s, rank chunk c) computes
// v[row][s][c*RC .. c*RC+RC) for the tile's rows.  Wave w covers the 512-wide
// K chunks w, w + W, ... (8 elements per lane, one 16-byte load per row and
// adapter row), so for K <= 8192 each wave issues all of its loads at once.
// Loads are unconditional (out-of-range lanes read a clamped address and are
// zeroed), which keeps the memory counters exact and the loads in flight.
template <typename E, int TM, int RC, int MODE>
__global__ __launch_bounds__(1024) void shrink_wave_kernel(const E* __restrict__ x,
                                                           const E* __restrict__ A,
                                                           float* __restrict__ v, RowList L,
                                                           Geo g, PlanArg<MODE> pa) {
  constexpr int V = RC * TM;
  constexpr int P = Log2<V>::value;
  __shared__ float red[16][V];
  const int W = blockDim.x >> 6;
  const int nrc = g.R / RC;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_tile = g.S * nrc;
  const int f = bid / per_tile;
  const int rem = bid - f * per_tile;
  const int s = rem / nrc;
  const int c = rem - s * nrc;
  TileRows<TM> tr;
  if (!tile_rows<TM, MODE>(L, g, f, pa, tr, s == 0 && c == 0)) return;
  uint32_t todo = tr.valid;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int SR = g.S * g.R;
  const int nchunk = (g.K + 511) / 512;

  // rows m of the tile that use adapter a
  auto group = [&](uint32_t m, int a) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    const E* Ab = A + ((size_t)(a * g.S + s) * g.R + (size_t)c * RC) * g.K;
    for (int q = wave; q < nchunk; q += W) {
      const int k0 = q * 512 + lane * 8;
      const bool kin = k0 < g.K;
      const int kc = kin ? k0 : 0;
      const uint32_t kmask = kin ? 0xffffffffu : 0u;
      typename El<E>::Raw ar[RC], xr[TM];
#pragma unroll
      for (int rr = 0; rr < RC; ++rr) ar[rr] = El<E>::raw8(Ab + (size_t)rr * g.K + kc);
#pragma unroll
      for (int r = 0; r < TM; ++r) xr[r] = El<E>::raw8(x + (size_t)tr.tok[r] * g.K + kc);
      float af[RC][8];
#pragma unroll
      for (int rr = 0; rr < RC; ++rr) {
        El<E>::mask(ar[rr], kmask);  // lanes past K contribute zero
        El<E>::unpack(ar[rr], af[rr]);
      }
#pragma unroll
      for (int r = 0; r < TM; ++r) {
        float xf[8];
        El<E>::unpack(xr[r], xf);
#pragma unroll
        for (int rr = 0; rr < RC; ++rr) {
          float d = acc[rr * TM + r];
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(af[rr][e], xf[e], d);
          acc[rr * TM + r] = d;
        }
      }
    }
    const float sum = wave_sum_many<V>(acc, lane);
    if ((lane & ((64 >> P) - 1)) == 0) red[wave][lane >> (6 - P)] = sum;
    __syncthreads();
    if (threadIdx.x < V) {
      const int idx = threadIdx.x;
      const int rr = idx / TM, r = idx - rr * TM;
      if ((m >> r) & 1u) {
        float tot = 0.f;
        for (int w = 0; w < W; ++w) tot += red[w][idx];
        v[(size_t)(tr.vrow0 + r) * SR + s * g.R + c * RC + rr] = tot;
      }
    }
  };
  if constexpr (MODE == kRows) {
    while (todo) {
      int a;
      const uint32_t m = next_group<TM>(todo, tr.aid, a);
      todo &= ~m;
      group(m, a);
      __syncthreads();  // red is rewritten by the next group
    }
  } else if (todo) {
    group(todo, tr.aid[0]);  // one adapter per tile
  }
}

// ------------------------------------------------------------ expand (VALU)
//
// grid.x = tiles * column chunks (kExpandCols columns of one slice each).
// Thread j owns output column col0 + j.  Per adapter group the tile's B block
// (KB ranks per pass) and the group's v rows are staged in LDS: every thread
// first issues all of its global loads (contiguous 16-byte vectors), then
// writes LDS, so the copy costs one memory round trip.  B rows are padded by
// 16 bytes in LDS, which makes the row-per-thread reads conflict-free.  KB is
// the pool's rank rounded up to 16 or 64, so no thread loads vectors that are
// never used.  v is the sum of the shrink's kparts partials (row i of partial
// p at p * v_rows + i), added in order 0, 1, ...; KP >= kparts partials are
// loaded, those past kparts as zeros, so all loads are issued at once.
template <typename E, int TM, int KB, int KP, int MODE>
__global__ __launch_bounds__(256) void expand_wave_kernel(const float* __restrict__ v,
                                                          const E* __restrict__ B,
                                                          E* __restrict__ y, RowList L, Geo g,
                                                          Chunks ch, int kparts, int v_rows,
                                                          PlanArg<MODE> pa) {
  constexpr int NC = kExpandCols;      // 256 columns per workgroup
  constexpr int VEC = El<E>::kVec;     // elements per 16-byte vector
  constexpr int LDB = KB + VEC;        // LDS row stride: 16 bytes of padding
  constexpr int MAXV = NC * KB / VEC / 256;  // B vectors per thread per pass
  // v vectors per thread staged in one go: all of R for R <= KB (KB = 16) or
  // R <= 256 (KB = 64; R <= 64 when partials are summed, which only pools of
  // R <= 64 have); larger R goes through a plain loop
  constexpr int NVV = (TM * (KB == 64 ? (KP > 1 ? 64 : 256) : KB) / 4 + 255) / 256;
  static_assert(KB % VEC == 0 && MAXV >= 1, "rank block must hold whole vectors");
  extern __shared__ __align__(16) unsigned char lds_raw[];
  // Bs: NC staged rows plus one dump row that absorbs stores of idle lanes (so
  // no store, and hence no load feeding it, sits under a branch); vs: TM rows
  // of v plus a 16-byte dump slot
  E* Bs = reinterpret_cast<E*>(lds_raw);                                       // [NC + 1][LDB]
  float* vs = reinterpret_cast<float*>(lds_raw + sizeof(E) * (NC + 1) * LDB);  // [TM * R + 4]

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int f = bid / ch.total;
  const int cidx = bid - f * ch.total;
  int s = 0;
#pragma unroll
  for (int i = 1; i < LORA_MAX_SLICES; ++i)
    if (i < g.S && cidx >= ch.start[i]) s = i;
  const int col0 = (cidx - ch.start[s]) * NC;
  const int ncv = min(NC, g.out[s] - col0);
  TileRows<TM> tr;
  if (!tile_rows<TM, MODE>(L, g, f, pa, tr)) return;
  uint32_t todo = tr.valid;
  const int tid = threadIdx.x;
  const int R = g.R;
  const int SR = g.S * R;
  const int r0 = tr.vrow0;
  const int np = KP == 1 ? 1 : kparts;  // partials of v (one unless KP > 1)
  // y of every valid row is read up front so its latency overlaps the B / v
  // staging; each row is written exactly once, by the group that owns it
  const int colc = tid < ncv ? tid : 0;
  E* yb = y + g.off[s] + col0 + colc;
  E yv[TM];
#pragma unroll
  for (int r = 0; r < TM; ++r) yv[r] = yb[(size_t)tr.tok[r] * g.O];

  // rows m of the tile that use adapter a
  auto group = [&](uint32_t m, int a) {
    float acc[TM];
#pragma unroll
    for (int r = 0; r < TM; ++r) acc[r] = 0.f;
    const E* Bg = B + ((size_t)a * g.O + g.off[s] + col0) * R;
    for (int kb = 0; kb < R; kb += KB) {
      const int kw = min(KB, R - kb);   // multiple of 8
      const int vpr = kw / VEC;         // vectors per staged row
      const int nvec = ncv * vpr;
      u32x4 braw[MAXV];
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int idx = tid + 256 * j;
        const bool ok = idx < nvec;
        const int row = ok ? idx / vpr : 0;
        const int q = ok ? idx - row * vpr : 0;
        braw[j] = ld16(Bg + (size_t)row * R + kb + q * VEC);
      }
      // v rows of this group (zeros for rows outside it), on the first pass
      f32x4 vraw[NVV];
      const int nv4 = TM * R / 4;
      if (kb == 0) {
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
          const int i = tid + 256 * j;
          const int r = i < nv4 ? (i * 4) / R : 0;
          const bool mem = i < nv4 && ((m >> r) & 1u);
          const int k = mem ? i * 4 - r * R : 0;
          const size_t off = (size_t)(r0 + (mem ? r : 0)) * SR + s * R + k;
          u32x4 raw[KP];
#pragma unroll
          for (int p = 0; p < KP; ++p)
            raw[p] = ld16(v + off + (size_t)(p < np ? p : 0) * v_rows * SR) &
                     all_or_none(mem && p < np);
          f32x4 sum = __builtin_bit_cast(f32x4, raw[0]);
#pragma unroll
          for (int p = 1; p < KP; ++p) sum += __builtin_bit_cast(f32x4, raw[p]);
          vraw[j] = sum;
        }
      }
      __syncthreads();                  // previous readers of Bs / vs are done
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int idx = tid + 256 * j;
        const bool ok = idx < nvec;
        const int row = ok ? idx / vpr : NC;
        const int q = ok ? idx - row * vpr : 0;
        *reinterpret_cast<u32x4*>(Bs + row * LDB + q * VEC) = braw[j];
      }
      if (kb == 0) {
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
          const int i = tid + 256 * j;
          *reinterpret_cast<f32x4*>(vs + (i < nv4 ? i * 4 : nv4 * 4)) = vraw[j];
        }
        for (int i = tid + 256 * NVV; i < nv4; i += 256) {  // large R: rare, plain loop
          const int r = (i * 4) / R;
          const bool mem = (m >> r) & 1u;
          const int k = i * 4 - r * R;
          f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int p = 0; mem && p < np; ++p)
            sum += *reinterpret_cast<const f32x4*>(v + ((size_t)p * v_rows + r0 + r) * SR +
                                                   s * R + k);
          *reinterpret_cast<f32x4*>(vs + i * 4) = sum;
        }
      }
      __syncthreads();
      if (tid < ncv) {
        for (int k = 0; k < kw; k += 8) {
          float b[8];
          El<E>::load8(Bs + tid * LDB + k, b);
#pragma unroll
          for (int r = 0; r < TM; ++r) {
            const float* vr = vs + r * R + kb + k;
            float d = acc[r];
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(b[e], vr[e], d);
            acc[r] = d;
          }
        }
      }
    }
    if (tid < ncv) {
#pragma unroll
      for (int r = 0; r < TM; ++r) {
        if ((m >> r) & 1u) yb[(size_t)tr.tok[r] * g.O] = El<E>::put(El<E>::get(yv[r]) + acc[r]);
      }
    }
  };
  if constexpr (MODE == kRows) {
    while (todo) {
      int a;
      const uint32_t m = next_group<TM>(todo, tr.aid, a);
      todo &= ~m;
      group(m, a);
      __syncthreads();  // Bs / vs are rewritten by the next group
    }
  } else if (todo) {
    group(todo, tr.aid[0]);  // one adapter per tile
  }
}

// One 64-wide K step of the decode-tile shrink, loaded as whole 128-byte
// lines: lane l holds 8 elements at k = 8 (l / 8) of token row l % 8 (xv) and
// of ranks 16 t + 8 j + l % 8 (av[t][j]); msk zeroes a lane past K.  An MFMA
// sums over its 32 k in any order, so the step is two MFMAs over the halves
// S0 = {16 g .. 16 g + 8} and S1 = {16 g + 8 .. 16 g + 16} (g = l / 16, the
// operand's k group): the S1 half of rows 0..7 (and the S0 half of ranks
// 8..15) sits 8 lanes away and a DPP rotate within each row of 16 lanes brings
// it over.  MFMA rows 8..15 are never used.
template <int NT>
__device__ __forceinline__ void tile_step_mfma(const u32x4& xv, const u32x4 (&av)[NT][2],
                                               uint32_t msk, uint32_t lo8, f32x4 (&d)[NT]) {
  const u32x4 xm = xv & msk;
  const bf16x8 x0 = __builtin_bit_cast(bf16x8, xm);
  const bf16x8 x1 = __builtin_bit_cast(bf16x8, rot8_rows16(xm));
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const u32x4 a0 = av[t][0] & msk, a1 = av[t][1] & msk;
    const u32x4 r0 = rot8_rows16(a0), r1 = rot8_rows16(a1);
    const u32x4 b0 = pick(lo8, a0, r1);  // ranks at S0
    const u32x4 b1 = pick(lo8, r0, a1);  // ranks at S1
    d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, __builtin_bit_cast(bf16x8, b0), d[t], 0, 0,
                                                   0);
    d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, __builtin_bit_cast(bf16x8, b1), d[t], 0, 0,
                                                   0);
  }
}

// ------------------------------------------ decode in one launch (bf16, MFMA)
//
// For small decode plans (records passed by value, bf16, R <= 32): a
// workgroup computes its tile's v = x A_a^T itself and applies it to
// kOnepassCols output columns of one slice, so no workgroup depends on
// another and one launch covers both stages.  Each column chunk of a tile
// re-reads the tile's x rows and the adapter's A rows (from L2 after the
// first); for a decode batch those are a few hundred KB, against the cost of a
// second launch and a grid-wide dependency.
//
// grid = tiles * column chunks, 512 threads (8 waves).
//   shrink: D[m][n] = sum_k x[tok[m]][k] A[a][s][n][k] as v_mfma_f32_16x16x32_bf16
//           tiles (rows m = tokens, 8 of 16 used; columns n = ranks, NT tiles
//           of 16), loads of whole 128-byte lines (tile_step_mfma), the
//           64-wide K steps dealt round-robin over the waves, CB / 2 steps per
//           wave loaded at once (CB = the wave's share of K in 32-wide chunks,
//           up to 16 / NT); the waves' partial tiles are summed in a fixed
//           order in LDS.
// Every workgroup pulls the adapter's A rows and the tile's x rows through one
// compute unit, whose few outstanding misses bound the rate, so the form only
// pays where a second launch costs more: plans of at most kArgTilesS tiles.
//   expand: thread j owns column col0 + j: its B row (R bf16) comes straight
//           from HBM (consecutive threads read consecutive rows), v from LDS
//           (broadcast reads), and y of each valid row is read before the
//           shrink and written once at the end.
constexpr int kOnepassCols = 512;
constexpr int kOnepassWaves = kOnepassCols / 64;

template <int NT, int CB, int MODE>
__global__ __launch_bounds__(kOnepassCols) void decode_onepass_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    uint16_t* __restrict__ y, RowList L, Geo g, Chunks ch, PlanArg<MODE> pa) {
  constexpr int TM = kWaveTileRows;
  constexpr int RM = 16 * NT;          // ranks covered by the MFMA tiles (>= R)
  static_assert(CB % 2 == 0 && CB / 2 * (1 + 2 * NT) <= 24,
                "a batch keeps at most 24 loads per lane in flight");
  static_assert(TM <= 16, "tile rows fit one MFMA tile");
  __shared__ float red[kOnepassWaves][16][RM + 1];
  __shared__ float vs[TM][RM];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int f = bid / ch.total;
  const int cidx = bid - f * ch.total;
  int s = 0;
#pragma unroll
  for (int i = 1; i < LORA_MAX_SLICES; ++i)
    if (i < g.S && cidx >= ch.start[i]) s = i;
  const int col0 = (cidx - ch.start[s]) * kOnepassCols;
  const int ncv = min(kOnepassCols, g.out[s] - col0);
  TileRows<TM> tr;
  if (!tile_rows<TM, MODE>(L, g, f, pa, tr) || tr.valid == 0) return;
  const int a = tr.aid[0];  // one adapter per tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int R = g.R;

  // shrink: whole 128-byte lines per load, two MFMAs per 64-wide K step
  // (tile_step_mfma); rows past the tile repeat row 0 and ranks past R repeat
  // rank R - 1 (their outputs are never used)
  constexpr int SB = CB / 2;  // K steps of 64 per wave per batch
  const int m = lane & 15;
  const int r8 = lane & 7, kx = (lane >> 3) * 8;
  // (a lane with kx >= K only ever loads masked steps; kxa keeps its address
  // inside the row, which holds K >= 8 elements)
  const int kxa = min(kx, g.K - 8);
  int tk = tr.tok[0];
#pragma unroll
  for (int r = 1; r < TM; ++r)
    if (r8 == r) tk = tr.tok[r];
  const uint16_t* xp = x + (size_t)tk * g.K + kxa;
  const uint16_t* ap[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      ap[t][j] = A + ((size_t)(a * g.S + s) * R + min(16 * t + 8 * j + r8, R - 1)) * g.K + kxa;
  const uint32_t lo8 = all_or_none(m < 8);
  f32x4 d[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) d[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (g.K + 63) / 64;
  u32x4 xv[SB], av[SB][NT][2];
  uint32_t msk[SB];
  // every load of a batch is issued before the first MFMA waits on one, so a
  // batch costs one memory round trip
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int k = (c0 + u * kOnepassWaves) * 64;
      const bool ok = k + kx < g.K;
      const int kc = ok ? k : 0;
      msk[u] = all_or_none(ok);
      xv[u] = ld16(xp + kc);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) av[u][t][j] = ld16(ap[t][j] + kc);
    }
  };
  auto mma_batch = [&] {
#pragma unroll
    for (int u = 0; u < SB; ++u) tile_step_mfma<NT>(xv[u], av[u], msk[u], lo8, d);
  };
  constexpr int kStride = kOnepassWaves * SB;
  load_batch(wave);

  // y of the tile's rows and this thread's B row (needed last, issued after
  // the first batch so that waiting on the batch does not wait on them)
  const int colc = tid < ncv ? tid : 0;
  uint16_t* yb = y + g.off[s] + col0 + colc;
  uint16_t yv[TM];
#pragma unroll
  for (int r = 0; r < TM; ++r) yv[r] = yb[(size_t)tr.tok[r] * g.O];
  const uint16_t* Bg = B + ((size_t)a * g.O + g.off[s] + col0 + colc) * R;
  u32x4 braw[2 * NT];
#pragma unroll
  for (int q = 0; q < 2 * NT; ++q) braw[q] = ld16(Bg + min(8 * q, R - 8)) & all_or_none(8 * q < R);
  __builtin_amdgcn_sched_barrier(0);
  mma_batch();
  for (int c0 = wave + kStride; c0 < nst; c0 += kStride) {
    load_batch(c0);
    __builtin_amdgcn_sched_barrier(0);
    mma_batch();
  }
  // lane l holds D[4 (l / 16) + j][l % 16] of each rank tile
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave][4 * (lane >> 4) + j][16 * t + m] = d[t][j];
  __syncthreads();
  if (tid < TM * RM) {
    const int r = tid / RM, n = tid - r * RM;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kOnepassWaves; ++w) acc += red[w][r][n];
    vs[r][n] = n < R ? acc : 0.f;
  }
  __syncthreads();

  // expand
  if (tid < ncv) {
    float b[RM];
#pragma unroll
    for (int q = 0; q < 2 * NT; ++q) {
      float t8[8];
      El<uint16_t>::unpack({braw[q]}, t8);
#pragma unroll
      for (int e = 0; e < 8; ++e) b[8 * q + e] = t8[e];
    }
#pragma unroll
    for (int r = 0; r < TM; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < RM; ++k) acc = fmaf(b[k], vs[r][k], acc);
      if ((tr.valid >> r) & 1u)
        yb[(size_t)tr.tok[r] * g.O] = El<uint16_t>::put(El<uint16_t>::get(yv[r]) + acc);
    }
  }
}

// ------------------------------- shrink (MFMA, wavefront tiles, bf16, R <= 64)
//
// grid = tiles * S * kparts, 256 threads (4 waves).  Workgroup (tile, slice s,
// part p) writes partial p of v for the tile's rows: the sum over the part's
// contiguous range of 64-wide K steps of
//   D[m][n] = sum_k x[tok[m]][k] * A_pool[a][s][n][k]
// as v_mfma_f32_16x16x32_bf16 tiles (rows m = the tile's tokens, columns n =
// ranks, NT tiles of 16).  Every rank of the slice comes out of one pass over
// x, where the VALU shrink reads x once per 4-rank chunk.
//
// Loads cover whole 128-byte lines: per K step, lane l loads 8 elements at
// k = 8 (l / 8) of row l % 8 (one instruction for the 8 token rows of x, two
// per 16 ranks of A).  An MFMA sums over its 32 k in any order, so each step
// is two MFMAs over the halves S0 = {16 g .. 16 g + 8} and S1 = {16 g + 8 ..
// 16 g + 16} (g = l / 16, the operand's k group); a DPP rotate by 8 lanes
// within each row of 16 moves the S1 half of rows 0..7 (and of ranks 8..15)
// to the lanes the MFMA reads it from.  MFMA rows 8..15 are never used.
//
// The part's steps are dealt round-robin over the waves; a wave issues the
// loads of CB / 2 steps before the first MFMA of the batch waits on them.  The
// waves' partial tiles are summed in a fixed order in LDS, so the result does
// not depend on timing.  Splitting K over workgroups spreads the x and A
// loads over more compute units.
// (the body takes its workgroup index bid among nwg workgroups and its LDS,
// tile_shrink_lds<NT>() 16-byte aligned floats, so that a combined launch can
// run it beside the 64-row shrink)
template <int NT> constexpr int tile_shrink_lds() {
  return kTileShrinkWaves * kWaveTileRows * (16 * NT + 1);
}

template <int NT, int CB, int MODE>
__device__ __forceinline__ void shrink_tile_mfma_body(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ A,
                                                      float* __restrict__ v, const RowList& L,
                                                      const Geo& g, int kparts, int v_rows,
                                                      const PlanArg<MODE>& pa, int bid, int nwg,
                                                      float* lds, bool pre = false,
                                                      int prew = 0) {
  constexpr int TM = kWaveTileRows, NW = kTileShrinkWaves, RM = 16 * NT, SB = CB / 2;
  static_assert(TM == 8, "x rows fill lanes l % 8");
  static_assert(SB >= 1 && SB * (1 + 2 * NT) <= 18, "a batch keeps at most 18 loads per lane in flight");
  float (*red)[TM][RM + 1] = reinterpret_cast<float (*)[TM][RM + 1]>(lds);
  const int per_tile = g.S * kparts;
  const int f0 = bid / per_tile;
  const int rem = bid - f0 * per_tile;
  const int s = rem / kparts;
  const int part = rem - s * kparts;
  // one record per workgroup, except for a device-built plan (kListWalk):
  // records f0, f0 + G, ... (G = the grid's records) until the first one
  // without rows (its records come first, then empty ones to its capacity)
  constexpr bool kWalk = MODE == kListWalk;
  const int G = kWalk ? nwg / per_tile : 1;
  if (kWalk && f0 >= G) return;  // workgroups past whole groups of per_tile take no records
  for (int f = f0;; f += G) {
  if (kWalk && f != f0) lds_barrier();  // red of the previous record is read
  TileRows<TM> tr;
  if (!tile_rows<TM, MODE>(L, g, f, pa, tr, s == 0 && part == 0, pre && f == f0, prew) ||
      tr.cnt <= 0)
    return;
  if (tr.valid == 0) {
    if (kWalk) continue;
    return;
  }
  const int a = tr.aid[0];  // one adapter per tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int R = g.R;
  const int nst = (g.K + 63) / 64;
  const int per = (nst + kparts - 1) / kparts;
  const int s_lo = min(nst, part * per), s_hi = min(nst, s_lo + per);

  // load roles: row l % 8 (token, or rank 8 j + l % 8 of a rank tile), k offset
  // 8 (l / 8) of the step (kept inside the row for K < 64: lanes past K only
  // ever load masked steps)
  const int r8 = lane & 7, kx = (lane >> 3) * 8;
  const int kxa = min(kx, g.K - 8);
  int tk = tr.tok[0];
#pragma unroll
  for (int r = 1; r < TM; ++r)
    if (r8 == r) tk = tr.tok[r];
  const uint16_t* xp = x + (size_t)tk * g.K + kxa;
  const uint16_t* ap[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j)  // ranks past the adapter's re-read its last row (cache-hot)
      ap[t][j] = A + ((size_t)(a * g.S + s) * R + min(16 * t + 8 * j + r8, tr.rank - 1)) * g.K + kxa;
  const uint32_t lo8 = all_or_none((lane & 15) < 8);  // operand rows / ranks 0..7 of a tile
  f32x4 d[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) d[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = s_lo + wave; c0 < s_hi; c0 += NW * SB) {
    u32x4 xv[SB], av[SB][NT][2];
    uint32_t msk[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int st = c0 + u * NW;
      const bool ok = st < s_hi && st * 64 + kx < g.K;
      const int kc = ok ? st * 64 : 0;
      msk[u] = all_or_none(ok);
      xv[u] = ld16(xp + kc);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) av[u][t][j] = ld16(ap[t][j] + kc);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < SB; ++u) tile_step_mfma<NT>(xv[u], av[u], msk[u], lo8, d);
  }
  // lane l holds D[4 (l / 16) + j][l % 16] of each rank tile; lanes 0 .. 4 TM - 1
  // hold the tile's rows
  if (lane < 4 * TM) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][4 * (lane >> 4) + j][16 * t + (lane & 15)] = d[t][j];
  }
  __syncthreads();
  const int SR = g.S * R;
  for (int i = tid; i < TM * RM; i += 64 * NW) {
    const int r = i / RM, n = i - r * RM;
    if (n < R && ((tr.valid >> r) & 1u)) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += red[w][r][n];
      v[((size_t)part * v_rows + tr.vrow0 + r) * SR + s * R + n] = n < tr.rank ? acc : 0.f;
    }
  }
  if (!kWalk) return;
  }
}

template <int NT, int CB, int MODE>
__global__ __launch_bounds__(64 * kTileShrinkWaves) void shrink_tile_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ A, float* __restrict__ v,
    RowList L, Geo g, int kparts, int v_rows, PlanArg<MODE> pa) {
  __shared__ __align__(16) float red[tile_shrink_lds<NT>()];
  shrink_tile_mfma_body<NT, CB, MODE>(x, A, v, L, g, kparts, v_rows, pa,
                                      xcd_remap(blockIdx.x, gridDim.x), (int)gridDim.x, red);
}

// ------------------------------- expand (MFMA, wavefront tiles, bf16, R <= 64)
//
// grid = tiles * column chunks (kTileExpandCols columns of one slice each),
// 256 threads (4 waves).  For a tile of at most 8 rows, D = Btile * v^T as
// v_mfma_f32_16x16x32_bf16 tiles: rows = output columns, columns = the tile's
// tokens (8 of 16 used), K = ranks in chunks of 32; two MFMAs per tile and
// chunk take the hi and lo bf16 halves of the fp32 v.  Wave w covers the
// pairs of 16-column tiles w, w + 4, ... of the chunk.  Inside a pair, MFMA
// row n of the first tile reads B column 8 (n / 4) + n % 4 and of the second
// the same + 4, so lane (g, m) ends with columns 8 g .. 8 g + 8 of token m and
// reads and writes them as one 16-byte access.  The B rows (32 contiguous
// bytes of ranks per column and chunk) and y of all of the wave's pairs are
// loaded before v is needed; v (the sum of the shrink's kparts partials in
// order 0, 1, ..., split into hi + lo) is staged once in LDS.  y leaves
// through raw buffer stores; lanes without a row store to a dropped offset.
constexpr int kTileExpandWaves = 4;
constexpr int kTileExpandPairs = 4;  // pairs of 16-column tiles per wave
constexpr int kTileExpandCols = 32 * kTileExpandPairs * kTileExpandWaves;

// (the body takes its workgroup index bid among nwg workgroups and its LDS,
// tile_expand_lds<NKC>() 16-byte aligned elements: the hi rows, then the lo
// rows, so that a combined launch can run it beside the 64-row expand)
template <int NKC> constexpr int tile_expand_ldv() { return 32 * NKC + 8; }
template <int NKC> constexpr int tile_expand_lds() {
  return 2 * kWaveTileRows * tile_expand_ldv<NKC>();
}

template <int NKC, int KP, int MODE>
__device__ __forceinline__ void expand_tile_mfma_body(const float* __restrict__ v,
                                                      const uint16_t* __restrict__ B,
                                                      uint16_t* __restrict__ y, const RowList& L,
                                                      const Geo& g, const Chunks& ch, int kparts,
                                                      int v_rows, const PlanArg<MODE>& pa, int bid,
                                                      int nwg, uint16_t* lds, bool pre = false,
                                                      int prew = 0) {
  constexpr int TM = kWaveTileRows, PPW = kTileExpandPairs, NW = kTileExpandWaves;
  constexpr int LDV = tile_expand_ldv<NKC>();  // LDS row of v in bf16 (ranks covered + padding)
  static_assert(TM <= 16 && TM * 64 / 4 <= 64 * NW, "one v vector per thread");
  static_assert((TM * LDV * 2) % 16 == 0, "the lo rows start 16-byte aligned");
  uint16_t* vh = lds;
  uint16_t* vl = lds + TM * LDV;
  const int f0 = bid / ch.total;
  const int cidx = bid - f0 * ch.total;
  int s = 0;
#pragma unroll
  for (int i = 1; i < LORA_MAX_SLICES; ++i)
    if (i < g.S && cidx >= ch.start[i]) s = i;
  const int col0 = (cidx - ch.start[s]) * kTileExpandCols;
  const int out_s = g.out[s];
  // one record per workgroup, except for a device-built plan (kListWalk):
  // records f0, f0 + G, ... (G = the grid's records) until the first one
  // without rows (its records come first, then empty ones to its capacity)
  constexpr bool kWalk = MODE == kListWalk;
  const int G = kWalk ? nwg / ch.total : 1;
  if (kWalk && f0 >= G) return;  // workgroups past whole groups of ch.total take no records
  for (int f = f0;; f += G) {
  if (kWalk && f != f0) lds_barrier();  // vh / vl of the previous record are read
  TileRows<TM> tr;
  if (!tile_rows<TM, MODE>(L, g, f, pa, tr, false, pre && f == f0, prew) || tr.cnt <= 0)
    return;
  if (tr.valid == 0) {
    if (kWalk) continue;
    return;
  }
  const int a = tr.aid[0];  // one adapter per tile
  // (in a walk the thread index passes through an empty asm statement, so the
  // lane-dependent offsets below are recomputed per record rather than held
  // in registers across the loop, which would not fit four workgroups per CU)
  int tid = threadIdx.x;
  if constexpr (kWalk) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int i16 = lane & 15, g4 = lane >> 4;
  const int R = g.R;
  const int np = KP == 1 ? 1 : kparts;
  const __amdgpu_buffer_rsrc_t yb = make_rsrc(y, (uint32_t)((size_t)g.T * g.O * sizeof(uint16_t)));

  // this lane's token (MFMA column i16) and its y row
  int my_tok = tr.tok[0];
#pragma unroll
  for (int r = 1; r < TM; ++r)
    if (i16 == r) my_tok = tr.tok[r];
  const bool tok_ok = i16 < TM && ((tr.valid >> i16) & 1u);
  const size_t yrow = (size_t)my_tok * g.O + g.off[s];

  // B rows and y of the wave's pairs: they do not depend on v, so they go first
  const uint16_t* Ba = B + ((size_t)a * g.O + g.off[s]) * R;
  u32x4 bt[PPW][2][NKC], yr[PPW];
#pragma unroll
  for (int q = 0; q < PPW; ++q) {
    const int pc = col0 + 32 * (wave + NW * q);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = pc + 8 * (i16 >> 2) + 4 * h + (i16 & 3);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int k = 32 * kc + 8 * g4;
        const bool ok = c < out_s && k < tr.rank;  // ranks past the adapter's are zero
        bt[q][h][kc] = ld16(Ba + (size_t)(ok ? c : 0) * R + (ok ? k : 0)) & all_or_none(ok);
      }
    }
    const int yc = pc + 8 * g4;
    yr[q] = ld16(y + yrow + (yc < out_s ? yc : 0));
  }

  // v of the tile's rows: the sum of the partials, split into hi + lo bf16
  // (rows without a valid token are zero)
  const int SR = g.S * R;
  if (tid < TM * R / 4) {
    const int r = (tid * 4) / R, k = tid * 4 - r * R;
    const bool ok = (tr.valid >> r) & 1u;
    const size_t off = ((size_t)tr.vrow0 + (ok ? r : 0)) * SR + s * R + k;
    u32x4 raw[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p)
      raw[p] = ld16(v + off + (size_t)(p < np ? p : 0) * v_rows * SR) & all_or_none(ok && p < np);
    float e[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KP; ++p) {  // fixed order: partial 0, 1, ...
      e[0] += __uint_as_float(raw[p].x);
      e[1] += __uint_as_float(raw[p].y);
      e[2] += __uint_as_float(raw[p].z);
      e[3] += __uint_as_float(raw[p].w);
    }
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hb[i] = f32_to_bf16_bits(e[i]);
      lb[i] = f32_to_bf16_bits(e[i] - __uint_as_float(hb[i] << 16));
    }
    *reinterpret_cast<u32x2*>(&vh[r * LDV + k]) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
    *reinterpret_cast<u32x2*>(&vl[r * LDV + k]) = u32x2{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)};
  }
  __syncthreads();
  // MFMA B operand: lane (g, m) holds ranks 32 kc + 8 g .. +8 of token row m
  // (zero past the tile's rows and past R)
  bf16x8 vhi[NKC], vlo[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const int k = 32 * kc + 8 * g4;
    const bool ok = i16 < TM && k < R;
    const int o = (ok ? i16 : 0) * LDV + (ok ? k : 0);
    const uint32_t msk = all_or_none(ok);
    vhi[kc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&vh[o]) & msk);
    vlo[kc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&vl[o]) & msk);
  }
#pragma unroll
  for (int q = 0; q < PPW; ++q) {
    f32x4 d0 = f32x4{0.f, 0.f, 0.f, 0.f}, d1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, bt[q][0][kc]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, bt[q][1][kc]);
      d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, vhi[kc], d0, 0, 0, 0);
      d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, vlo[kc], d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, vhi[kc], d1, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, vlo[kc], d1, 0, 0, 0);
    }
    // lane (g, m): d0[j] is column 8 g + j and d1[j] column 8 g + 4 + j of token m
    const float add[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
    const uint32_t wi[4] = {yr[q].x, yr[q].y, yr[q].z, yr[q].w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(wi[i] << 16) + add[2 * i];
      const float hi = __uint_as_float(wi[i] & 0xffff0000u) + add[2 * i + 1];
      o[i] = pack_bf16x2(lo, hi);
    }
    const int yc = col0 + 32 * (wave + NW * q) + 8 * g4;
    const uint32_t off = (tok_ok && yc < out_s)
                             ? (uint32_t)((yrow + (size_t)yc) * sizeof(uint16_t))
                             : kDropOffset;
    st16_buf(u32x4{o[0], o[1], o[2], o[3]}, yb, off);
  }
  if (!kWalk) return;
  }
}

template <int NKC, int KP, int MODE>
__global__ __launch_bounds__(64 * kTileExpandWaves) void expand_tile_mfma_kernel(
    const float* __restrict__ v, const uint16_t* __restrict__ B, uint16_t* __restrict__ y,
    RowList L, Geo g, Chunks ch, int kparts, int v_rows, PlanArg<MODE> pa) {
  __shared__ __align__(16) uint16_t lds[tile_expand_lds<NKC>()];
  expand_tile_mfma_body<NKC, KP, MODE>(v, B, y, L, g, ch, kparts, v_rows, pa,
                                       xcd_remap(blockIdx.x, gridDim.x), (int)gridDim.x, lds);
}

// Tile lookup of the MFMA kernels (segments or tile-list mode): first row r0
// of the row list, row count and adapter slot, the same in every lane.  The
// tile-list record is (slot, rows, first row, tok0); tok0 >= 0 says the tile's
// tokens are tok0, tok0 + 1, ... (row r0 + i reads token tok0 + i) and need
// not be read from the list; segments mode gives tok0 = -1.
template <int TMR, int MODE>
__device__ __forceinline__ bool mfma_tile(const RowList& L, int f, int& r0, int& cnt, int& sid,
                                          int& tok0, int& rk, bool copy = false) {
  tok0 = -1;
  rk = 0;
  if constexpr (MODE == kList) {
    if (f >= L.num_tiles) return false;
    const int w = L.tiles[(size_t)f * LORA_PLAN_MFMA_WORDS + (threadIdx.x & 3)];
    if (copy && L.copy_tiles && threadIdx.x < LORA_PLAN_MFMA_WORDS)
      L.copy_tiles[(size_t)f * LORA_PLAN_MFMA_WORDS + threadIdx.x] = w;
    sid = __builtin_amdgcn_readlane(w, 0);
    const int w1 = __builtin_amdgcn_readlane(w, 1);
    cnt = w1 & 0xffff;
    rk = (int)((uint32_t)w1 >> 16);
    r0 = __builtin_amdgcn_readlane(w, 2);
    tok0 = __builtin_amdgcn_readlane(w, 3);
  } else {
    if (!find_tile_wave<TMR>(L, f, r0, cnt, sid)) return false;
  }
  cnt = min(cnt, TMR);
  return true;
}

// ------------------------------------------------------------ shrink (MFMA)
//
// bf16 only.  grid.x = tiles * S * ksplit, grid.y = ceil(R / 64).  A workgroup
// computes the 64 rows of its tile against ranks 64 * blockIdx.y .. +64 over the
// K range of its split (a contiguous run of 64-wide K steps) and writes partial
// `part` of v:  v[(part * v_rows + row) * S * R + s * R + rank].
// Per K step the x tile [64 rows][64 k] and the adapter tile [64 ranks][64 k]
// move HBM -> registers -> LDS with coalesced 16-byte loads (8 lanes per
// 128-byte row piece); loads run two steps ahead and LDS is double-buffered,
// with one barrier per step.  Wave (wm, wr) multiplies rows 32 wm .. +32 by
// ranks 32 wr .. +32 as 2 x 2 MFMA tiles of 16 x 16, two k-chunks of 32 per
// step; fragments are 16-byte LDS reads (rows padded to 144 bytes).
// (the body takes its workgroup index bid, its rank block rblk and its LDS,
// kRegShrinkLds 16-byte aligned elements: x tiles, then adapter tiles)
constexpr int kRegShrinkRow = 64 + 8;  // LDS row: 64 k plus padding
constexpr int kRegShrinkLds = 2 * 2 * 64 * kRegShrinkRow;

template <int MODE>
__device__ __forceinline__ void shrink_mfma_body(const uint16_t* __restrict__ x,
                                                 const uint16_t* __restrict__ A,
                                                 float* __restrict__ v, const RowList& L,
                                                 const Geo& g, int ksplit, int v_rows, int bid,
                                                 int rblk, uint16_t* lds) {
  constexpr int TM = kMfmaTileRows, NR = 64, KS = 64, LDS_ROW = kRegShrinkRow;
  static_assert(TM == 64, "staging covers 64 rows");
  uint16_t (*xs)[TM * LDS_ROW] = reinterpret_cast<uint16_t (*)[TM * LDS_ROW]>(lds);
  uint16_t (*as)[NR * LDS_ROW] = reinterpret_cast<uint16_t (*)[NR * LDS_ROW]>(lds + 2 * TM * LDS_ROW);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int wm = wave & 1, wr = wave >> 1;
  const int i16 = lane & 15, grp = lane >> 4;
  const int per_tile = g.S * ksplit;
  const int f = bid / per_tile;
  const int rem = bid - f * per_tile;
  const int s = rem / ksplit;
  const int part = rem - s * ksplit;
  int r0, cnt, sid, tok0;
  const bool copy = s == 0 && part == 0 && rblk == 0;
  int rk_rec;
  if (!mfma_tile<TM, MODE>(L, f, r0, cnt, sid, tok0, rk_rec, copy)) return;
  if (sid < 0 || sid >= g.max_loras || cnt < 1 || r0 < 0 || r0 + cnt > L.num_rows) return;
  const int rr = rk_rec > 0 && rk_rec < g.R ? rk_rec : g.R;  // the adapter's ranks
  const int rank0 = rblk * NR;
  // K steps of this split
  const int nsteps = (g.K + KS - 1) / KS;
  const int per = (nsteps + ksplit - 1) / ksplit;
  const int st0 = min(nsteps, part * per), st1 = min(nsteps, st0 + per);

  // staging: thread t carries 16 bytes at k = 8 (t % 8) of rows / ranks t / 8
  // and t / 8 + 32
  const int c8 = tid & 7, srow = tid >> 3;
  const uint16_t* xp[2];
  const uint16_t* ap[2];
  uint32_t xm[2], am[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = srow + 32 * j;
    const int tk = tok0 >= 0 ? tok0 + min(r, cnt - 1) : L.tok[r0 + min(r, cnt - 1)];
    if (copy && L.copy_tok && tok0 < 0 && c8 == 0 && r < cnt) L.copy_tok[r0 + r] = tk;
    const bool ok = r < cnt && tk >= 0 && tk < g.T;
    xp[j] = x + (size_t)(ok ? tk : 0) * g.K;
    xm[j] = all_or_none(ok);
    const int rk = rank0 + r;
    const bool rok = rk < rr;  // ranks past the adapter's are zero: not loaded
    ap[j] = A + ((size_t)(sid * g.S + s) * g.R + (rok ? rk : 0)) * g.K;
    am[j] = all_or_none(rok);
  }
  // loads of K step `st` (a step at or past the K range reads clamped
  // addresses and is zeroed)
  auto gload = [&](int st, u32x4(&r)[4]) {
    const int kk = st * KS + 8 * c8;
    const bool in = kk < g.K;
    const int kc = in ? kk : 0;
    const uint32_t km = all_or_none(in);
#pragma unroll
    for (int j = 0; j < 2; ++j) r[j] = ld16_nt(xp[j] + kc) & (km & xm[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) r[2 + j] = ld16(ap[j] + kc) & (km & am[j]);
  };
  auto lstore = [&](int b, const u32x4(&r)[4]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<u32x4*>(&xs[b][(srow + 32 * j) * LDS_ROW + 8 * c8]) = r[j];
      *reinterpret_cast<u32x4*>(&as[b][(srow + 32 * j) * LDS_ROW + 8 * c8]) = r[2 + j];
    }
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int b) {
#pragma unroll
    for (int kc = 0; kc < KS; kc += 32) {
      bf16x8 xa[2], ab[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        xa[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                &xs[b][(32 * wm + 16 * mt + i16) * LDS_ROW + kc + 8 * grp]));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        ab[nt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                &as[b][(32 * wr + 16 * nt + i16) * LDS_ROW + kc + 8 * grp]));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt], ab[nt], acc[mt][nt], 0, 0, 0);
    }
  };
  u32x4 ra[4], rb[4];
  gload(st0, ra);
  gload(st0 + 1, rb);
  for (int st = st0; st < st1; st += 2) {
    lstore(0, ra);
    gload(st + 2, ra);
    __syncthreads();
    mma(0);
    if (st + 1 >= st1) break;
    lstore(1, rb);
    gload(st + 3, rb);
    __syncthreads();
    mma(1);
  }
  // D layout: lane (grp, i16) holds rows 4 grp + j (j < 4) of rank column i16
  const int SR = g.S * g.R;
  float* vp = v + ((size_t)part * v_rows + r0) * SR + s * g.R;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int rk = rank0 + 32 * wr + 16 * nt + i16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 32 * wm + 16 * mt + 4 * grp + j;
        if (row < cnt && rk < g.R) vp[(size_t)row * SR + rk] = rk < rr ? acc[mt][nt][j] : 0.f;
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void shrink_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ A,
                                                          float* __restrict__ v, RowList L,
                                                          Geo g, int ksplit, int v_rows) {
  __shared__ __align__(16) uint16_t lds[kRegShrinkLds];
  shrink_mfma_body<MODE>(x, A, v, L, g, ksplit, v_rows, xcd_remap(blockIdx.x, gridDim.x),
                         blockIdx.y, lds);
}

// ------------------------------------------------- shrink (MFMA, LDS by DMA)
//
// The same work as shrink_mfma_kernel (bf16; grid.x = tiles * S * ksplit,
// grid.y = ceil(R / 64); a workgroup computes 64 rows x 64 ranks over the K
// steps of its split) for K a multiple of 64, with the tiles moved by gfx950's
// direct global -> LDS loads (global_load_lds_dwordx4): no registers hold the
// data in flight, so a ring of three stages keeps the next two K steps in
// flight at every step, where the register-staged kernel holds one to two.
//
// A stage is the x tile [64 rows][64 k] and the adapter tile [64 ranks][64 k],
// 8 KB each, rows of 128 bytes without padding (a DMA instruction writes 64
// lanes x 16 bytes contiguously).  Wave w loads rows 16 w .. 16 w + 16 of
// both with two instructions each; lane l of an instruction covers row
// 8 b + l / 8 and 16-byte slot l % 8, which holds the row's k chunk
// (l % 8) ^ swz(row).  The MFMA operand reads (16 lanes, 16 consecutive rows,
// one k chunk) then fall into 16 different banks groups.
//
// Rows past the tile's rows and ranks past the adapter's are loaded from a
// clamped address: each feeds only its own D row or column, which is never
// stored (rows) or stored as zero (ranks), so no mask is needed; a K tail
// would mix into every sum, hence K % 64 == 0.  Steps past the split's last
// one re-read it (cache hits) so every wave issues four loads per step.  The
// loads count on vmcnt: a step's data is in LDS once at most one later step's
// four loads are outstanding, and the barrier after that wait (which also
// waits for the wave's own LDS reads) publishes every wave's part and retires
// the previous step's reads of the stage reloaded next.
__device__ __forceinline__ int dma_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// A launch of at most one workgroup per compute unit takes four stages
// instead, loads three steps ahead: a lone workgroup's loads in flight set
// its compute unit's rate (a 3 967-token prefill shrink, 195 workgroups:
// 14.3 -> 12.5 us; the 4096-token rank-64 decode shrink, 248: 12.2 -> 10.7
// us), while where units hold two workgroups three stages keep enough in
// flight (the 8 772-token prefill shrink, 435 workgroups: 20.8 -> 21.8 us
// with four; gate_up, 618: 27.3 -> 30.3 us).
// (the body takes its workgroup index bid, its rank block rblk and the
// stages, 16-byte aligned LDS arrays of kDmaStage elements: st_0, st_1, st_2
// for three, NST consecutive ones from st_0 above that, so that a combined
// launch can run it beside the 8-row tile shrink)
constexpr int kDmaStage = 2 * 64 * 64;  // one stage: the x tile, then the adapter tile
// s_waitcnt operand: at most n vector memory operations and no LDS one
// outstanding (vmcnt in bits 3:0 and 15:14, expcnt 7 = no wait)
constexpr int vm_wait_lgkm0(int n) { return ((n >> 4) & 3) << 14 | 0x70 | (n & 15); }

template <int MODE, int NST = 3>
__device__ __forceinline__ void shrink_mfma_dma_body(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ A,
                                                     float* __restrict__ v, const RowList& L,
                                                     const Geo& g, int ksplit, int v_rows, int bid,
                                                     int rblk, uint16_t* st_0, uint16_t* st_1,
                                                     uint16_t* st_2) {
  constexpr int TM = kMfmaTileRows, NR = 64, KS = 64, TILE = 64 * KS;
  static_assert(TM == 64 && 2 * TILE == kDmaStage, "64 rows per tile");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int wm = wave & 1, wr = wave >> 1;
  const int i16 = lane & 15, grp = lane >> 4;
  const int per_tile = g.S * ksplit;
  const int f = bid / per_tile;
  const int rem = bid - f * per_tile;
  const int s = rem / ksplit;
  const int part = rem - s * ksplit;
  int r0, cnt, sid, tok0;
  const bool copy = s == 0 && part == 0 && rblk == 0;
  int rk_rec;
  if (!mfma_tile<TM, MODE>(L, f, r0, cnt, sid, tok0, rk_rec, copy)) return;
  if (sid < 0 || sid >= g.max_loras || cnt < 1 || r0 < 0 || r0 + cnt > L.num_rows) return;
  const int rr = rk_rec > 0 && rk_rec < g.R ? rk_rec : g.R;  // the adapter's ranks
  const int rank0 = rblk * NR;
  const int nsteps = g.K / KS;
  const int per = (nsteps + ksplit - 1) / ksplit;
  const int st0 = min(nsteps, part * per), st1 = min(nsteps, st0 + per);

  // DMA sources: rows 8 b + l / 8 of block b = 2 wave + j, k chunk (l % 8) ^ swz
  const uint16_t* xsrc[2];
  const uint16_t* asrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * (2 * wave + j) + (lane >> 3);
    const int c = (lane & 7) ^ dma_swz(row);
    const int rc = min(row, cnt - 1);
    const int tk = tok0 >= 0 ? tok0 + rc : L.tok[r0 + rc];
    if (copy && L.copy_tok && tok0 < 0 && (lane & 7) == 0 && row < cnt) L.copy_tok[r0 + row] = tk;
    xsrc[j] = x + (size_t)(tk >= 0 && tk < g.T ? tk : 0) * g.K + 8 * c;
    const int rk = rank0 + row;
    asrc[j] = A + ((size_t)(sid * g.S + s) * g.R + (rk < rr ? rk : 0)) * g.K + 8 * c;
  }
  auto issue = [&](int st, uint16_t* sd) {
    const int kk = min(st, st1 - 1) * KS;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_global_load_lds(xsrc[j] + kk, sd + (2 * wave + j) * 512, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(asrc[j] + kk, sd + TILE + (2 * wave + j) * 512, 16, 0, 0);
    }
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const uint16_t* xt) {
    const uint16_t* at = xt + TILE;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8 xa[2], ab[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = 32 * wm + 16 * mt + i16;
        const int slot = (4 * kc + grp) ^ dma_swz(row);
        xa[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&xt[row * KS + 8 * slot]));
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = 32 * wr + 16 * nt + i16;
        const int slot = (4 * kc + grp) ^ dma_swz(row);
        ab[nt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&at[row * KS + 8 * slot]));
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt], ab[nt], acc[mt][nt], 0, 0, 0);
    }
  };
  // one step: wait for its own four loads (the next step's four may stay
  // outstanding), barrier, refill the stage the previous step read, compute
  // (the empty asm statements keep the compiler from moving LDS accesses
  // across the barrier, which it does not treat as a memory operation)
  auto step = [&](int st, const uint16_t* cur, uint16_t* nxt) {
    __builtin_amdgcn_s_waitcnt(kWaitVm4Lgkm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(st + 2, nxt);
    mma(cur);
  };
  if constexpr (NST == 3) {
    if (st0 < st1) {  // a split past the last K step leaves its partial at zero
      issue(st0, st_0);
      issue(st0 + 1, st_1);
      for (int st = st0; st < st1; st += 6) {
        step(st, st_0, st_2);
        if (st + 1 >= st1) break;
        step(st + 1, st_1, st_0);
        if (st + 2 >= st1) break;
        step(st + 2, st_2, st_1);
        if (st + 3 >= st1) break;
        step(st + 3, st_0, st_2);
        if (st + 4 >= st1) break;
        step(st + 4, st_1, st_0);
        if (st + 5 >= st1) break;
        step(st + 5, st_2, st_1);
      }
      // every load has landed before the workgroup ends
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
  } else {
    // the same with NST stages: wait until only the NST - 2 later steps' loads
    // are outstanding, barrier, refill the stage step st - 1 read
    static_assert(NST >= 4 && NST <= 6, "stages");
    if (st0 < st1) {
      for (int i = 0; i < NST - 1; ++i) issue(st0 + i, st_0 + i * kDmaStage);
      int cur = 0;  // stage of step st
      for (int st = st0; st < st1; ++st) {
        __builtin_amdgcn_s_waitcnt(vm_wait_lgkm0(4 * (NST - 2)));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(st + NST - 1, st_0 + (cur == 0 ? NST - 1 : cur - 1) * kDmaStage);
        mma(st_0 + cur * kDmaStage);
        cur = cur == NST - 1 ? 0 : cur + 1;
      }
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
  }
  // D layout: lane (grp, i16) holds rows 4 grp + j (j < 4) of rank column i16
  const int SR = g.S * g.R;
  float* vp = v + ((size_t)part * v_rows + r0) * SR + s * g.R;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int rk = rank0 + 32 * wr + 16 * nt + i16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 32 * wm + 16 * mt + 4 * grp + j;
        if (row < cnt && rk < g.R) vp[(size_t)row * SR + rk] = rk < rr ? acc[mt][nt][j] : 0.f;
      }
    }
  }
}

template <int MODE, int NST>
__global__ __launch_bounds__(256, NST == 3 ? 3 : 2) void shrink_mfma_dma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ A, float* __restrict__ v,
    RowList L, Geo g, int ksplit, int v_rows) {
  __shared__ __align__(16) uint16_t st[NST * kDmaStage];
  shrink_mfma_dma_body<MODE, NST>(x, A, v, L, g, ksplit, v_rows,
                                  xcd_remap(blockIdx.x, gridDim.x), blockIdx.y, st,
                                  st + kDmaStage, st + 2 * kDmaStage);
}

// ------------------------------------------------------------ expand (MFMA)
//
// bf16 only.  grid.x = tiles * column chunks of 128 (one slice each).  The
// workgroup's y tile [64 tokens][128 columns] and, per pass of 64 ranks, the B
// tile [128 columns][64 ranks] (contiguous in the pool) and the v tile
// [64 rows][64 ranks] are staged in LDS with coalesced 16-byte loads, all of a
// pass issued before any LDS store.  v is the sum of the shrink's ksplit
// partials, split into hi = rne_bf16(v) and lo = rne_bf16(v - hi), which keeps
// about 16 mantissa bits of the fp32 intermediate.  Wave w computes
// D = Btile * v^T for tokens 16 w .. +16: eight 16 x 16 tiles, two MFMAs (hi,
// lo) per tile and 32-rank chunk.  Inside a pair of tiles, MFMA row n of tile
// 2q maps to column 32 q + 8 (n / 4) + n % 4 and of tile 2q+1 to the same + 4,
// so lane (g, m) ends with columns 32 q + 8 g .. +8 of token m and updates
// them in LDS with one 16-byte read and write; the tile then leaves with
// coalesced 16-byte stores (16 lanes per 256-byte row piece).
template <int MODE>
__global__ __launch_bounds__(256) void expand_mfma_kernel(const float* __restrict__ v,
                                                          const uint16_t* __restrict__ B,
                                                          uint16_t* __restrict__ y, RowList L,
                                                          Geo g, Chunks ch, int ksplit,
                                                          int v_rows) {
  constexpr int TM = kMfmaTileRows, NC = kExpandMfmaCols, KB = 64;
  constexpr int LDK = KB + 8, LDY = NC + 8;
  static_assert(TM == 64 && NC == 128, "staging covers 64 tokens x 128 columns");
  __shared__ __align__(16) uint16_t bs[NC * LDK];
  __shared__ __align__(16) uint16_t vh[TM * LDK];
  __shared__ __align__(16) uint16_t vl[TM * LDK];
  __shared__ __align__(16) uint16_t ys[TM * LDY];
  __shared__ int s_tok[TM];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int m16 = lane & 15, grp = lane >> 4;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int f = bid / ch.total;
  const int cidx = bid - f * ch.total;
  int s = 0;
#pragma unroll
  for (int i = 1; i < LORA_MAX_SLICES; ++i)
    if (i < g.S && cidx >= ch.start[i]) s = i;
  const int col0 = (cidx - ch.start[s]) * NC;
  const int out_s = g.out[s];
  int r0, cnt, sid, tok0;
  int rk_rec;
  if (!mfma_tile<TM, MODE>(L, f, r0, cnt, sid, tok0, rk_rec)) return;
  if (sid < 0 || sid >= g.max_loras || cnt < 1 || r0 < 0 || r0 + cnt > L.num_rows) return;
  const int R = g.R;
  const int SR = g.S * R;
  if (tid < TM) {
    const int tk = tok0 >= 0 ? tok0 + min(tid, cnt - 1) : L.tok[r0 + min(tid, cnt - 1)];
    s_tok[tid] = (tid < cnt && tk >= 0 && tk < g.T) ? tk : -1;
  }
  __syncthreads();
  // y / v staging: row (t / 16) + 16 j; y columns col0 + 8 (t % 16) .. +8,
  // v ranks 4 (t % 16) .. +4 of the pass
  const int q16 = tid & 15, srow = tid >> 4;
  const int ycol = col0 + 8 * q16;
  const bool ycol_ok = ycol < out_s;
  u32x4 yr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tk = s_tok[srow + 16 * j];
    yr[j] = ld16(y + (size_t)(tk >= 0 ? tk : 0) * g.O + g.off[s] + (ycol_ok ? ycol : 0));
  }
  f32x4 acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* Bt = B + ((size_t)sid * g.O + g.off[s] + col0) * R;
  // B staging: column (t / 8) + 32 j, ranks 8 (t % 8) .. +8 of the pass
  const int b8 = tid & 7, bcol = tid >> 3;
  for (int kb0 = 0; kb0 < R; kb0 += KB) {
    const int kw = min(KB, R - kb0);  // multiple of 8
    u32x4 vr[4][kMaxKsplitWide];
    const bool vk_ok = 4 * q16 < kw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = srow + 16 * j;
      const bool ok = vk_ok && s_tok[row] >= 0;
      const uint32_t m = all_or_none(ok);
#pragma unroll
      for (int p = 0; p < kMaxKsplitWide; ++p) {
        const bool pin = p < ksplit;
        const size_t off = ((size_t)(pin ? p : 0) * v_rows + r0 + (ok ? row : 0)) * SR + s * R +
                           kb0 + (ok ? 4 * q16 : 0);
        vr[j][p] = ld16(v + off) & (m & all_or_none(pin));
      }
    }
    u32x4 br[4];
    const bool bk_ok = 8 * b8 < kw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = bcol + 32 * j;
      const bool ok = bk_ok && col0 + c < out_s;
      br[j] = ld16(Bt + (size_t)(ok ? c : 0) * R + kb0 + (ok ? 8 * b8 : 0)) & all_or_none(ok);
    }
    if (kb0 > 0) __syncthreads();  // MFMA readers of the previous pass are done
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4*>(&bs[(bcol + 32 * j) * LDK + 8 * b8]) = br[j];
      float e[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < kMaxKsplitWide; ++p) {  // fixed order: partial 0, 1, ...
        e[0] += __uint_as_float(vr[j][p].x);
        e[1] += __uint_as_float(vr[j][p].y);
        e[2] += __uint_as_float(vr[j][p].z);
        e[3] += __uint_as_float(vr[j][p].w);
      }
      uint32_t h[4], l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = f32_to_bf16_bits(e[i]);
        l[i] = f32_to_bf16_bits(e[i] - __uint_as_float(h[i] << 16));
      }
      const int vo = (srow + 16 * j) * LDK + 4 * q16;
      *reinterpret_cast<u32x2*>(&vh[vo]) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *reinterpret_cast<u32x2*>(&vl[vo]) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
      if (kb0 == 0) *reinterpret_cast<u32x4*>(&ys[(srow + 16 * j) * LDY + 8 * q16]) = yr[j];
    }
    __syncthreads();
    for (int kk = 0; kk < kw; kk += 32) {
      const int vo = (16 * wave + m16) * LDK + kk + 8 * grp;
      const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&vh[vo]));
      const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&vl[vo]));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int q = nt >> 1, hi = nt & 1;
        const int crow = 32 * q + 8 * (m16 >> 2) + 4 * hi + (m16 & 3);
        const bf16x8 ba = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&bs[crow * LDK + kk + 8 * grp]));
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ba, bh, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ba, bl, acc[nt], 0, 0, 0);
      }
    }
  }
  // y update in LDS: lane (grp, m16) owns token row 16 wave + m16, columns
  // 32 q + 8 grp .. +8 of pair q
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint16_t* yp = &ys[(16 * wave + m16) * LDY + 32 * q + 8 * grp];
    const u32x4 w = *reinterpret_cast<const u32x4*>(yp);
    const f32x4 d0 = acc[2 * q], d1 = acc[2 * q + 1];
    const float add[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
    const uint32_t wi[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(wi[i] << 16) + add[2 * i];
      const float hi = __uint_as_float(wi[i] & 0xffff0000u) + add[2 * i + 1];
      o[i] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(yp) = u32x4{o[0], o[1], o[2], o[3]};
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = srow + 16 * j;
    const int tk = s_tok[row];
    if (tk >= 0 && ycol_ok)
      *reinterpret_cast<u32x4*>(y + (size_t)tk * g.O + g.off[s] + ycol) =
          *reinterpret_cast<const u32x4*>(&ys[row * LDY + 8 * q16]);
  }
}

// ------------------------------------------------------------ expand (MFMA, R <= 64)
//
// bf16, pools of rank R <= 64.  A workgroup covers a group of up to `cpw`
// consecutive column chunks of 128 columns of one slice of its tile
// (gr.start[s] is the first group of slice s).  Wave w owns tokens 16 w .. +16
// of the tile and computes D = v * Btile^T with v as the MFMA's first operand
// (D rows = tokens) and the B tile as its second (D columns = output
// columns): in MFMA tile nt (of 8 per chunk), D column j reads B column
// 8 j + nt.  Lane (g, j) then holds, over the 8 tiles, columns 8 j .. 8 j + 8
// of tokens 4 g .. 4 g + 4, so for each of its four tokens it reads and writes
// 16 contiguous bytes of y, and the 16 lanes of one g cover 256 contiguous
// bytes of one token's row: every y load and store instruction moves whole
// 128-byte lines, with the streaming (non-temporal) cache policy.
// v (the sum of the shrink's partials in fixed order, split into hi + lo bf16,
// two MFMAs per tile and 32-rank chunk) stays in registers for the whole
// group: lane (g, j) holds ranks 32 kc + 8 g .. +8 of token row 16 w + j.
// The B tile [128 columns][R] goes through LDS once per chunk (coalesced
// 16-byte loads, 8 lanes per 128-byte row); column c is stored at LDS row
// (c % 8) * 16 + c / 8, so the 16 lanes reading columns 8 j + nt hit 16
// consecutive padded rows and no two of them share a bank.  The next chunk's
// B and y are loaded while the current one is computed; y leaves through raw
// buffer stores (y must span less than 2 GiB): lanes without a row store to a
// dropped offset, so no store sits under a branch.
// (the body takes its workgroup index bid and its LDS, the B tile of
// kExpandRowsLds 16-byte aligned elements and the tile's tokens, so that a
// combined launch can run it beside the 8-row tile expand)
constexpr int kExpandRowsLdk = 64 + 8;  // LDS row of the B tile: 64 ranks plus padding
constexpr int kExpandRowsLds = kExpandMfmaCols * kExpandRowsLdk;

template <int MODE, int KP>
__device__ __forceinline__ void expand_mfma_rows_body(const float* __restrict__ v,
                                                      const uint16_t* __restrict__ B,
                                                      uint16_t* __restrict__ y, const RowList& L,
                                                      const Geo& g, const Chunks& ch,
                                                      const Chunks& gr, int ksplit, int v_rows,
                                                      int cpw, int bid, uint16_t* bs, int* s_tok) {
  constexpr int TM = kMfmaTileRows, NC = kExpandMfmaCols, KB = 64;
  constexpr int LDK = kExpandRowsLdk;
  // KP partials of v are loaded (those past ksplit as zeros); splits of more
  // than kMaxKsplitWide happen only for pools of rank <= 32: one 32-rank chunk
  constexpr int NKC = KP > kMaxKsplitWide ? 1 : 2;
  static_assert(KP == kMaxKsplitWide || KP == kMaxKsplit, "four or eight partials");
  static_assert(TM == 64 && NC == 128 && LDK == KB + 8, "64 tokens x 128 columns per chunk");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int j16 = lane & 15, grp = lane >> 4;
  const int f = bid / gr.total;
  const int gidx = bid - f * gr.total;
  int s = 0;
#pragma unroll
  for (int i = 1; i < LORA_MAX_SLICES; ++i)
    if (i < g.S && gidx >= gr.start[i]) s = i;
  const int c_begin = ch.start[s] + (gidx - gr.start[s]) * cpw;
  const int c_end = min(ch.start[s + 1], c_begin + cpw);
  const int out_s = g.out[s];
  int r0, cnt, sid, tok0;
  int rk_rec;
  if (!mfma_tile<TM, MODE>(L, f, r0, cnt, sid, tok0, rk_rec)) return;
  if (sid < 0 || sid >= g.max_loras || cnt < 1 || r0 < 0 || r0 + cnt > L.num_rows) return;
  const int R = g.R;  // <= 64, a multiple of 8
  const int rr = rk_rec > 0 && rk_rec < R ? rk_rec : R;  // the adapter's ranks
  const int SR = g.S * R;
  const __amdgpu_buffer_rsrc_t yb = make_rsrc(y, (uint32_t)((size_t)g.T * g.O * sizeof(uint16_t)));
  if (tid < TM) {
    const int tk = tok0 >= 0 ? tok0 + min(tid, cnt - 1) : L.tok[r0 + min(tid, cnt - 1)];
    s_tok[tid] = (tid < cnt && tk >= 0 && tk < g.T) ? tk : -1;
  }
  // v operands: token row 16 wave + j16, ranks 32 kc + 8 grp .. +8 (kc < 2);
  // the partials are summed in order 0, 1, ... (missing ones load as zeros).
  // Their loads are issued first and summed only after the first chunk's y
  // and B loads are issued, so the y round trip overlaps the v one (loads
  // complete in order: waiting for v leaves the later ones in flight)
  const int row = 16 * wave + j16;
  const bool row_ok = row < cnt;
  u32x4 vr[NKC][KP][2];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const int k0 = 32 * kc + 8 * grp;
    const bool ok = row_ok && k0 < rr;
    const uint32_t m = all_or_none(ok);
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const bool pin = p < ksplit;
      const size_t off =
          ((size_t)(pin ? p : 0) * v_rows + r0 + (ok ? row : 0)) * SR + s * R + (ok ? k0 : 0);
      const uint32_t mm = m & all_or_none(pin);
      vr[kc][p][0] = ld16(v + off) & mm;
      vr[kc][p][1] = ld16(v + off + 4) & mm;
    }
  }
  __syncthreads();  // s_tok
  // this lane's four tokens (rows 16 wave + 4 grp + r): the byte offset of
  // each one's y row in this slice (token 0's for a missing row, which only
  // feeds loads), and bit r of tok_ok set for a real token; y spans less
  // than 2 GiB, so 32-bit offsets suffice
  uint32_t yo[4];
  uint32_t tok_ok = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tk = s_tok[16 * wave + 4 * grp + r];
    tok_ok |= (tk >= 0 ? 1u : 0u) << r;
    yo[r] = (uint32_t)(((size_t)(tk >= 0 ? tk : 0) * g.O + g.off[s]) * sizeof(uint16_t));
  }
  // staging lanes: B column (t / 8) + 32 q with ranks 8 (t % 8) .. +8; ranks
  // past the adapter's are zero: not loaded
  const int b8 = tid & 7, bcol = tid >> 3;
  const bool bk_ok = 8 * b8 < rr;
  // loads of chunk c: B (zeroed where written to LDS) and this lane's y
  auto load_chunk = [&](int c, u32x4(&br)[4], u32x4(&yr)[4]) {
    const int col0 = (c - ch.start[s]) * NC;
    // the chunk's B block: NC columns of R ranks (at most 16 KB)
    const __amdgpu_buffer_rsrc_t bt = make_rsrc(
        const_cast<uint16_t*>(B) + ((size_t)sid * g.O + g.off[s] + col0) * R,
        (uint32_t)(NC * R * sizeof(uint16_t)));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = bcol + 32 * q;
      const bool ok = bk_ok && col0 + cc < out_s;
      br[q] = ld16_buf(bt, ok ? (uint32_t)((cc * R + 8 * b8) * sizeof(uint16_t)) : 0u);
    }
    const int col = col0 + 8 * j16;
    const uint32_t cb = (uint32_t)(col < out_s ? col : 0) * (uint32_t)sizeof(uint16_t);
#pragma unroll
    for (int r = 0; r < 4; ++r) yr[r] = ld16_buf_nt(yb, yo[r] + cb);
  };
  // a group holds at least one chunk (group gi < ceil(chunks / cpw)), so the
  // first chunk's loads are not held back behind a loop-entry test
  __builtin_assume(c_begin < c_end);
  u32x4 br[4], yn[4];
  load_chunk(c_begin, br, yn);
  __builtin_amdgcn_sched_barrier(0);  // the chunk's loads stay ahead of the v sum
  bf16x8 vh[NKC], vl[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    float e[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KP; ++p) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        e[4 * h + 0] += __uint_as_float(vr[kc][p][h].x);
        e[4 * h + 1] += __uint_as_float(vr[kc][p][h].y);
        e[4 * h + 2] += __uint_as_float(vr[kc][p][h].z);
        e[4 * h + 3] += __uint_as_float(vr[kc][p][h].w);
      }
    }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h0 = f32_to_bf16_bits(e[2 * i]), h1 = f32_to_bf16_bits(e[2 * i + 1]);
      const uint32_t l0 = f32_to_bf16_bits(e[2 * i] - __uint_as_float(h0 << 16));
      const uint32_t l1 = f32_to_bf16_bits(e[2 * i + 1] - __uint_as_float(h1 << 16));
      hw[i] = h0 | (h1 << 16);
      lw[i] = l0 | (l1 << 16);
    }
    vh[kc] = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
    vl[kc] = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
  }
  for (int c = c_begin; c < c_end; ++c) {
    const int col0 = (c - ch.start[s]) * NC;
    u32x4 yc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) yc[r] = yn[r];
    if (c > c_begin) __syncthreads();  // MFMA readers of the previous chunk's bs are done
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = bcol + 32 * q;
      const uint32_t m = all_or_none(bk_ok && col0 + cc < out_s);
      *reinterpret_cast<u32x4*>(&bs[((cc & 7) * 16 + (cc >> 3)) * LDK + 8 * b8]) = br[q] & m;
    }
    // the next chunk's loads overlap this one (the last chunk reloads itself:
    // unconditional loads keep the memory counters exact)
    load_chunk(min(c + 1, c_end - 1), br, yn);
    __syncthreads();
    f32x4 acc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      if (32 * kc < rr) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          // B column 8 j16 + nt sits at LDS row nt * 16 + j16
          const bf16x8 bb = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(&bs[(nt * 16 + j16) * LDK + 32 * kc + 8 * grp]));
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh[kc], bb, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vl[kc], bb, acc[nt], 0, 0, 0);
        }
      }
    }
    // y update in registers: lane (grp, j16) owns columns col0 + 8 j16 .. +8 of
    // its four tokens; acc[nt][r] is column col0 + 8 j16 + nt of token r
    const int col = col0 + 8 * j16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t wi[4] = {yc[r].x, yc[r].y, yc[r].z, yc[r].w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(wi[i] << 16) + acc[2 * i][r];
        const float hi = __uint_as_float(wi[i] & 0xffff0000u) + acc[2 * i + 1][r];
        o[i] = pack_bf16x2(lo, hi);
      }
      const uint32_t off = (((tok_ok >> r) & 1u) && col < out_s)
                               ? yo[r] + (uint32_t)col * (uint32_t)sizeof(uint16_t)
                               : kDropOffset;
      st16_buf_nt(u32x4{o[0], o[1], o[2], o[3]}, yb, off);
    }
  }
}

template <int MODE, int KP>
__global__ __launch_bounds__(256, 4) void expand_mfma_rows_kernel(
    const float* __restrict__ v, const uint16_t* __restrict__ B, uint16_t* __restrict__ y,
    RowList L, Geo g, Chunks ch, Chunks gr, int ksplit, int v_rows, int cpw) {
  __shared__ __align__(16) uint16_t bs[kExpandRowsLds];
  __shared__ int s_tok[kMfmaTileRows];
  expand_mfma_rows_body<MODE, KP>(v, B, y, L, g, ch, gr, ksplit, v_rows, cpw,
                                  xcd_remap(blockIdx.x, gridDim.x), bs, s_tok);
}

// ------------------------------------------ one launch per stage (device plans)
//
// A device-built plan knows its record counts only on the GPU, so the host
// launches its 64-row and its 8-row tiles at their capacities.  Launched apart,
// every stage costs two launches even where one kind has no records (a
// prefill batch has no 8-row tiles, a small decode batch no 64-row ones), and
// the second waits for the first to drain.  These kernels run both in one
// grid, in every workgroup one after the other: hardware workgroup ids below
// nmp (nm rounded up to a multiple of the XCD count, so the ids below nm
// spread over every XCD) first take their 64-row tile, then every workgroup
// walks the 8-row records.  The walk's first record is loaded at the start,
// so in a batch without 8-row tiles the check costs no round trip at the end.
// Both bodies share one LDS array, with a barrier for LDS only between them
// (the 64-row tile's last stores stay in flight).  The 64-row workgroups are
// dealt to the XCDs in chunks of kComboXcdChunk consecutive ids
// (xcd_remap_chunks): the records past the real ones are empty, and one
// contiguous range per XCD would leave them all to the last XCDs.  Measured
// from device ids (both calls of the mixed MLP, 8 prefill sequences + 256
// decode rows): 499 -> 434 us with chunks of 8 to 32; the prefill batch,
// fused QKV and 64-row decode unchanged.
constexpr int kComboXcdChunk = 16;
template <int MODE>
__device__ __forceinline__ void walk_first_word(const RowList& Lw, int bid, int nwg, int per,
                                                int& w, bool& pre) {
  const int G = nwg / per;
  const int f0 = bid / per;
  pre = f0 < G && f0 < Lw.num_tiles;
  w = 0;
  if (pre) w = Lw.tiles[(size_t)f0 * LORA_PLAN_WAVE_WORDS + (threadIdx.x & 15)];
}

template <int NT, int CB, bool DMA>
__global__ __launch_bounds__(256, 3) void shrink_combo_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ A, float* __restrict__ v,
    RowList Lm, RowList Lw, Geo g, int ksplit, int kparts, int v_rows, int nm, int nmp,
    int xchunk) {
  constexpr int kLds = DMA ? 3 * kDmaStage : kRegShrinkLds;  // uint16 elements
  static_assert(tile_shrink_lds<NT>() * 4 <= kLds * 2, "the tile shrink's LDS fits");
  static_assert(64 * kTileShrinkWaves == 256, "both bodies run 256 threads");
  __shared__ __align__(16) uint16_t lds[kLds];
  const int b = blockIdx.x, nwg = (int)gridDim.x;
  const int bw = xcd_remap(b, nwg);
  int w0;
  bool pre;
  walk_first_word<kListWalk>(Lw, bw, nwg, g.S * kparts, w0, pre);
  if (b < nmp) {
    const int bid = xcd_remap_chunks(b, nmp, xchunk);
    if (bid < nm) {
      if constexpr (DMA)
        shrink_mfma_dma_body<kList>(x, A, v, Lm, g, ksplit, v_rows, bid, 0, lds, lds + kDmaStage,
                                    lds + 2 * kDmaStage);
      else
        shrink_mfma_body<kList>(x, A, v, Lm, g, ksplit, v_rows, bid, 0, lds);
    }
    lds_barrier();  // the 64-row tile's LDS accesses are done
  }
  shrink_tile_mfma_body<NT, CB, kListWalk>(x, A, v, Lw, g, kparts, v_rows, PlanArg<kListWalk>{},
                                           bw, nwg, reinterpret_cast<float*>(lds), pre, w0);
}

// The 8-row walk sums kparts partials of v (KPW loads, those past kparts as
// zeros), the 64-row part ksplit (KPR loads).
template <int NKC, int KPR, int KPW>
__global__ __launch_bounds__(256, 4) void expand_combo_kernel(
    const float* __restrict__ v, const uint16_t* __restrict__ B, uint16_t* __restrict__ y,
    RowList Lm, RowList Lw, Geo g, Chunks chm, Chunks gr, Chunks chw, int ksplit, int kparts,
    int v_rows, int cpw, int nm, int nmp, int xchunk) {
  static_assert(tile_expand_lds<NKC>() <= kExpandRowsLds, "the tile expand's LDS fits");
  static_assert(64 * kTileExpandWaves == 256, "both bodies run 256 threads");
  __shared__ __align__(16) uint16_t lds[kExpandRowsLds];
  __shared__ int s_tok[kMfmaTileRows];
  const int b = blockIdx.x, nwg = (int)gridDim.x;
  const int bw = xcd_remap(b, nwg);
  int w0;
  bool pre;
  walk_first_word<kListWalk>(Lw, bw, nwg, chw.total, w0, pre);
  if (b < nmp) {
    const int bid = xcd_remap_chunks(b, nmp, xchunk);
    if (bid < nm)
      expand_mfma_rows_body<kList, KPR>(v, B, y, Lm, g, chm, gr, ksplit, v_rows, cpw, bid, lds,
                                        s_tok);
    lds_barrier();  // the 64-row tile's LDS accesses are done
  }
  expand_tile_mfma_body<NKC, KPW, kListWalk>(v, B, y, Lw, g, chw, kparts, v_rows,
                                             PlanArg<kListWalk>{}, bw, nwg, lds, pre, w0);
}

// ------------------------------------------------------------ pool load
//
// One slice of one adapter into its slot: A rows copied and zero-padded to R;
// B scaled in fp32, rounded once to the pool dtype, zero-padded to R columns.
template <typename E>
__global__ __launch_bounds__(256) void pool_load_kernel(const E* __restrict__ Asrc,
                                                        const E* __restrict__ Bsrc,
                                                        E* __restrict__ Adst, E* __restrict__ Bdst,
                                                        int r, int R, int K, int out_s,
                                                        float scale) {
  const size_t na = (size_t)R * K, nb = (size_t)out_s * R;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < na + nb;
       i += (size_t)gridDim.x * 256) {
    if (i < na) {
      const size_t k = i / K, j = i - k * K;
      Adst[i] = (int)k < r ? Asrc[k * K + j] : El<E>::put(0.f);
    } else {
      const size_t b = i - na;
      const size_t jr = b / R, k = b - jr * R;
      Bdst[b] = (int)k < r ? El<E>::put(El<E>::get(Bsrc[jr * r + k]) * scale) : El<E>::put(0.f);
    }
  }
}

// ================================================================ launchers

static int32_t hip_check(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LORA_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return LORA_OK;
}

static Chunks make_chunks(const Geo& g, int nc) {
  Chunks c;
  int acc = 0;
  for (int s = 0; s < LORA_MAX_SLICES + 1; ++s) c.start[s] = 0;
  for (int s = 0; s < g.S; ++s) {
    c.start[s] = acc;
    acc += (g.out[s] + nc - 1) / nc;
  }
  for (int s = g.S; s <= LORA_MAX_SLICES; ++s) c.start[s] = acc;
  c.total = acc;
  return c;
}

static unsigned grid_of(int64_t n) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(n, (int64_t)1 << 31));
}

// Records one launch of the 8-row tile kernels covers with its grid: every
// record, except for a device-built plan (kListWalk), whose record count is a
// capacity and mostly empty records for a prefill batch: there the grid holds
// at most about kTileWalkWgs workgroups, each walking its records with that
// stride (one workgroup per record would launch thousands that read one
// record and exit).  768 is one resident round of the tile kernels (three
// 256-thread workgroups per compute unit, 256 compute units): a batch without
// 8-row tiles then costs one round of workgroups that each read one record.
constexpr int64_t kTileWalkWgs = 768;
template <int MODE> static int64_t walk_records(int64_t tiles, int64_t per_record) {
  if (MODE != kListWalk) return tiles;
  return std::max<int64_t>(
      1, std::min<int64_t>(tiles, kTileWalkWgs / std::max<int64_t>(1, per_record)));
}

// Upper bound on the tiles of `tm` rows in a device row list (segments or rows
// mode); surplus workgroups exit after the lookup.
static int64_t count_tiles(const RowList& L, int tm) {
  if (L.ids) return ((int64_t)L.num_rows + tm - 1) / tm;
  int64_t n = ((int64_t)L.num_rows + tm - 1) / tm + L.num_segs;
  if (L.seg_max < INT32_MAX)  // every covered segment is at most seg_max rows long
    n = std::min<int64_t>(n, (int64_t)L.num_segs * (((int64_t)L.seg_max + tm - 1) / tm));
  return n;
}

template <typename E, int MODE>
static int32_t launch_shrink_wave(const Geo& g, const void* x, const void* A, float* v,
                                  const RowList& L, int64_t tiles, hipStream_t st,
                                  const PlanArg<MODE>& pa = PlanArg<MODE>{}) {
  if (tiles <= 0) return LORA_OK;
  const int waves = std::min(16, (g.K + 511) / 512);
  const int64_t grid = tiles * g.S * (g.R / 4);
  if (grid > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large for one shrink launch");
  hipLaunchKernelGGL((shrink_wave_kernel<E, kWaveTileRows, 4, MODE>), dim3(grid_of(grid)),
                     dim3(64 * waves), 0, st, (const E*)x, (const E*)A, v, L, g, pa);
  return hip_check("shrink_wave launch");
}

template <typename E, int KB, int KP, int MODE>
static int32_t launch_expand_wave_kb(const Geo& g, const float* v, const void* B, void* y,
                                     const RowList& L, int64_t tiles, int kparts, int v_rows,
                                     hipStream_t st, const PlanArg<MODE>& pa) {
  const Chunks ch = make_chunks(g, kExpandCols);
  const int64_t grid = tiles * ch.total;
  if (grid > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large for one expand launch");
  const size_t lds = sizeof(E) * (kExpandCols + 1) * (KB + 16 / sizeof(E)) +
                     sizeof(float) * (kWaveTileRows * g.R + 4);
  if (lds > 160 * 1024) return fail(LORA_E_SHAPE, "max_lora_rank too large for the expand kernel");
  hipLaunchKernelGGL((expand_wave_kernel<E, kWaveTileRows, KB, KP, MODE>), dim3(grid_of(grid)),
                     dim3(256), lds, st, v, (const E*)B, (E*)y, L, g, ch, kparts, v_rows, pa);
  return hip_check("expand_wave launch");
}

template <typename E, int KP, int MODE>
static int32_t launch_expand_wave_kp(const Geo& g, const float* v, const void* B, void* y,
                                     const RowList& L, int64_t tiles, int kparts, int v_rows,
                                     hipStream_t st, const PlanArg<MODE>& pa) {
  return g.R <= 16
             ? launch_expand_wave_kb<E, 16, KP, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa)
             : launch_expand_wave_kb<E, 64, KP, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa);
}

// kparts: partials of v to sum (1 for the VALU shrink; only bf16 plans use more)
template <typename E, int MODE>
static int32_t launch_expand_wave(const Geo& g, const float* v, const void* B, void* y,
                                  const RowList& L, int64_t tiles, hipStream_t st,
                                  const PlanArg<MODE>& pa = PlanArg<MODE>{}, int kparts = 1,
                                  int v_rows = 0) {
  if (tiles <= 0) return LORA_OK;
  if (kparts < 1 || kparts > kMaxKsplitWave) return fail(LORA_E_ARG, "bad K split %d", kparts);
  if constexpr (sizeof(E) == 2 && (MODE == kList || MODE == kArg || MODE == kArgL)) {
    if (kparts > tile_kparts_max(g.R)) return fail(LORA_E_ARG, "bad K split %d", kparts);
    if (kparts > 4)
      return launch_expand_wave_kb<E, 16, 8, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa);
    if (kparts > 2)
      return launch_expand_wave_kp<E, 4, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa);
    if (kparts > 1)
      return launch_expand_wave_kp<E, 2, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa);
  } else {
    if (kparts > 1) return fail(LORA_E_ARG, "one partial of v expected");
  }
  return launch_expand_wave_kp<E, 1, MODE>(g, v, B, y, L, tiles, 1, v_rows, st, pa);
}

// MFMA expand of wavefront tiles (bf16, R <= 64, y under 2 GiB), kparts
// partials of v.
template <int NKC, int KP, int MODE>
static int32_t launch_expand_tile_k(const Geo& g, const float* v, const void* B, void* y,
                                    const RowList& L, int64_t tiles, int kparts, int v_rows,
                                    hipStream_t st, const PlanArg<MODE>& pa) {
  const Chunks ch = make_chunks(g, kTileExpandCols);
  if (tiles * ch.total > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large for one expand launch");
  const int64_t grid = walk_records<MODE>(tiles, ch.total) * ch.total;
  hipLaunchKernelGGL((expand_tile_mfma_kernel<NKC, KP, MODE>), dim3(grid_of(grid)),
                     dim3(64 * kTileExpandWaves), 0, st, v, (const uint16_t*)B, (uint16_t*)y, L,
                     g, ch, kparts, v_rows, pa);
  return hip_check("expand_tile_mfma launch");
}

template <int NKC, int MODE>
static int32_t launch_expand_tile_nkc(const Geo& g, const float* v, const void* B, void* y,
                                      const RowList& L, int64_t tiles, int kparts, int v_rows,
                                      hipStream_t st, const PlanArg<MODE>& pa) {
  // (eight partials occur only for pools of rank <= 16, one 32-rank chunk; a
  // walk over two 32-rank chunks takes at most kMaxWalkKpartsWide: with more
  // its loop runs out of scalar registers)
  if constexpr (MODE != kListWalk || NKC == 1) {
    if (kparts > 4)
      return launch_expand_tile_k<NKC, 8, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa);
  }
  if constexpr (MODE == kListWalk && NKC == 2) {
    if (kparts > kMaxWalkKpartsWide) return fail(LORA_E_ARG, "bad K split %d", kparts);
  } else {
    if (kparts > 2)
      return launch_expand_tile_k<NKC, 4, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa);
  }
  if (kparts > 1)
    return launch_expand_tile_k<NKC, 2, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa);
  return launch_expand_tile_k<NKC, 1, MODE>(g, v, B, y, L, tiles, 1, v_rows, st, pa);
}

template <int MODE>
static int32_t launch_expand_tile(const Geo& g, const float* v, const void* B, void* y,
                                  const RowList& L, int64_t tiles, int kparts, int v_rows,
                                  hipStream_t st, const PlanArg<MODE>& pa = PlanArg<MODE>{}) {
  if (tiles <= 0) return LORA_OK;
  if (kparts < 1 || kparts > tile_kparts_max(g.R)) return fail(LORA_E_ARG, "bad K split %d", kparts);
  if (g.R > 64 || (int64_t)g.T * g.O * 2 >= (int64_t)kDropOffset)
    return fail(LORA_E_SHAPE, "the MFMA tile expand needs R <= 64 and y under 2 GiB");
  return g.R <= 32
             ? launch_expand_tile_nkc<1, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa)
             : launch_expand_tile_nkc<2, MODE>(g, v, B, y, L, tiles, kparts, v_rows, st, pa);
}

// MFMA shrink of wavefront tiles (bf16, R <= 64), kparts partials of v.
template <int NT, int MODE>
static int32_t launch_shrink_tile_nt(const Geo& g, const void* x, const void* A, float* v,
                                     const RowList& L, int64_t tiles, int kparts, int v_rows,
                                     hipStream_t st, const PlanArg<MODE>& pa) {
  constexpr int CB = tile_shrink_cb(16 * NT);
  if (tiles * g.S * kparts > INT32_MAX)
    return fail(LORA_E_SHAPE, "batch too large for one shrink launch");
  const int64_t grid = walk_records<MODE>(tiles, (int64_t)g.S * kparts) * g.S * kparts;
  hipLaunchKernelGGL((shrink_tile_mfma_kernel<NT, CB, MODE>), dim3(grid_of(grid)),
                     dim3(64 * kTileShrinkWaves), 0, st, (const uint16_t*)x, (const uint16_t*)A,
                     v, L, g, kparts, v_rows, pa);
  return hip_check("shrink_tile_mfma launch");
}

template <int MODE>
static int32_t launch_shrink_tile(const Geo& g, const void* x, const void* A, float* v,
                                  const RowList& L, int64_t tiles, int kparts, int v_rows,
                                  hipStream_t st, const PlanArg<MODE>& pa = PlanArg<MODE>{}) {
  if (tiles <= 0) return LORA_OK;
  if (kparts < 1 || kparts > tile_kparts_max(g.R)) return fail(LORA_E_ARG, "bad K split %d", kparts);
  static_assert(kMaxKsplitWave == 8, "launchers cover up to 8 partials");
  switch (tile_shrink_rank_tiles(g.R)) {
    case 1: return launch_shrink_tile_nt<1, MODE>(g, x, A, v, L, tiles, kparts, v_rows, st, pa);
    case 2: return launch_shrink_tile_nt<2, MODE>(g, x, A, v, L, tiles, kparts, v_rows, st, pa);
    default: return launch_shrink_tile_nt<4, MODE>(g, x, A, v, L, tiles, kparts, v_rows, st, pa);
  }
}

template <int NT, int CB, int MODE>
static int32_t launch_onepass_cb(const Geo& g, const void* x, const void* A, const void* B,
                                 void* y, const RowList& L, int tiles, hipStream_t st,
                                 const PlanArg<MODE>& pa) {
  const Chunks ch = make_chunks(g, kOnepassCols);
  const int64_t grid = (int64_t)tiles * ch.total;
  if (grid > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large for one launch");
  hipLaunchKernelGGL((decode_onepass_kernel<NT, CB, MODE>), dim3(grid_of(grid)),
                     dim3(kOnepassCols), 0, st, (const uint16_t*)x, (const uint16_t*)A,
                     (const uint16_t*)B, (uint16_t*)y, L, g, ch, pa);
  return hip_check("decode_onepass launch");
}

// CB: 32-wide K chunks per wave per batch, the wave's share of K rounded up to
// 4, at most 16 (R <= 16) or 8 (R <= 32)
template <int MODE>
static int32_t launch_onepass(const Geo& g, const void* x, const void* A, const void* B, void* y,
                              const RowList& L, int tiles, hipStream_t st, const PlanArg<MODE>& pa) {
  const int share = ((g.K + 31) / 32 + kOnepassWaves - 1) / kOnepassWaves;
  const int cb = std::min((share + 3) / 4 * 4, g.R <= 16 ? 16 : 8);
  if (g.R <= 16) {
    switch (cb) {
      case 4: return launch_onepass_cb<1, 4, MODE>(g, x, A, B, y, L, tiles, st, pa);
      case 8: return launch_onepass_cb<1, 8, MODE>(g, x, A, B, y, L, tiles, st, pa);
      case 12: return launch_onepass_cb<1, 12, MODE>(g, x, A, B, y, L, tiles, st, pa);
      default: return launch_onepass_cb<1, 16, MODE>(g, x, A, B, y, L, tiles, st, pa);
    }
  }
  return cb == 4 ? launch_onepass_cb<2, 4, MODE>(g, x, A, B, y, L, tiles, st, pa)
                 : launch_onepass_cb<2, 8, MODE>(g, x, A, B, y, L, tiles, st, pa);
}

template <int MODE>
static int32_t launch_shrink_mfma(const Geo& g, const void* x, const void* A, float* v,
                                  const RowList& L, int64_t tiles, int ksplit, int v_rows,
                                  hipStream_t st) {
  if (tiles <= 0) return LORA_OK;
  if (ksplit < 1 || ksplit > (g.R > 32 ? kMaxKsplitWide : kMaxKsplit))
    return fail(LORA_E_ARG, "bad K split %d", ksplit);
  if (tiles * g.S * ksplit > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large for one launch");
  const unsigned gy = (unsigned)((g.R + 63) / 64);
  // the DMA-staged form needs whole K steps; measured faster up to K = 4096
  // (in = 4096 prefill 24.0 -> 23.0 us, gate_up 40.3 -> 31.1 us, a 4096-token
  // decode 13.0 -> 11.2 us) and slower at K = 14336 (down 62.1 -> 66.3 us),
  // so wider K keeps the register-staged kernel
  if (g.K % 64 == 0 && g.K <= kDmaShrinkMaxK) {
    // four stages when no compute unit gets a second workgroup
    // (LORA_DMA_STAGES=3 or 4 overrides, for tuning)
    bool four = tiles * g.S * ksplit * gy <= kComputeUnits;
    if (const char* e = std::getenv("LORA_DMA_STAGES")) four = e[0] == '4';
    if (four)
      hipLaunchKernelGGL((shrink_mfma_dma_kernel<MODE, 4>),
                         dim3(grid_of(tiles * g.S * ksplit), gy), dim3(256), 0, st,
                         (const uint16_t*)x, (const uint16_t*)A, v, L, g, ksplit, v_rows);
    else
      hipLaunchKernelGGL((shrink_mfma_dma_kernel<MODE, 3>),
                         dim3(grid_of(tiles * g.S * ksplit), gy), dim3(256), 0, st,
                         (const uint16_t*)x, (const uint16_t*)A, v, L, g, ksplit, v_rows);
    return hip_check("shrink_mfma_dma launch");
  }
  hipLaunchKernelGGL(shrink_mfma_kernel<MODE>, dim3(grid_of(tiles * g.S * ksplit), gy), dim3(256),
                     0, st, (const uint16_t*)x, (const uint16_t*)A, v, L, g, ksplit, v_rows);
  return hip_check("shrink_mfma launch");
}

// Column groups of up to cpw chunks of one slice: group gi belongs to slice s
// when start[s] <= gi < start[s + 1].
static Chunks make_groups(const Geo& g, int cpw) {
  Chunks c;
  int acc = 0;
  for (int s = 0; s < LORA_MAX_SLICES + 1; ++s) c.start[s] = 0;
  for (int s = 0; s < g.S; ++s) {
    c.start[s] = acc;
    const int chunks = (g.out[s] + kExpandMfmaCols - 1) / kExpandMfmaCols;
    acc += (chunks + cpw - 1) / cpw;
  }
  for (int s = g.S; s <= LORA_MAX_SLICES; ++s) c.start[s] = acc;
  c.total = acc;
  return c;
}

// Column chunks per workgroup of the 64-row expand (R <= 64) for `tiles`
// records whose v has `ksplit` partials: the count, 1 to 8, that leaves the
// least on the busiest compute unit (the most chunks on a tie), ceil(wgs /
// 256) workgroups of
//   v partials (64 rows x R x 4 bytes each) + cpw x (the chunk's y read and
//   written, 64 x 128 elements each way, and its B block, 128 x R)
//   + 192 KB, the fixed cost of a workgroup (its prologue's round trips),
// a workgroup alone on its compute unit counted 1.25 times (it pulls more
// slowly than several together).  Fitted to measurements of every count
// (expand, us): the 8 772-token prefill takes 7 (38.3 against 38.8 at 5,
// 40.0 at 8); a 3 967-token prefill 5 (19.9; 20.6 at 3, 22.6 at 4); the
// 4096-row decodes 8 (rank 16: 16.7, 16.2 at 4, 17.7 at 2; rank 64: 17.4,
// 18.2 at 4, 21.8 at 2); gate_up 8 (191; 194 at 7, 198 at 5); down 8 (36.1;
// 37.7 at 5, 39.7 at 4).
static int expand_cpw(const Geo& g, int64_t tiles, int ksplit) {
  const int64_t eb = elem_bytes(g.dtype);
  const int64_t vbytes = (int64_t)kMfmaTileRows * g.R * 4 * ksplit;
  const int64_t cbytes = (int64_t)kMfmaTileRows * kExpandMfmaCols * eb * 2 +
                         (int64_t)kExpandMfmaCols * g.R * eb;
  constexpr int64_t kFixed = 192 * 1024;
  int best = 1;
  int64_t best_cost = -1;
  for (int cpw = 1; cpw <= 8; ++cpw) {
    const int64_t wgs = tiles * make_groups(g, cpw).total;
    const int64_t per_cu = (wgs + kComputeUnits - 1) / kComputeUnits;
    int64_t cost = per_cu * (vbytes + cpw * cbytes + kFixed);
    if (wgs <= kComputeUnits) cost = cost * 5 / 4;
    if (best_cost < 0 || cost <= best_cost) {  // a tie goes to fewer workgroups
      best_cost = cost;
      best = cpw;
    }
  }
  if (const char* e = std::getenv("LORA_EXPAND_MFMA_CPW")) {  // tuning / test override
    const long o = std::strtol(e, nullptr, 10);
    if (o >= 1 && o <= 8) best = (int)o;
  }
  return best;
}

template <int MODE>
static int32_t launch_expand_mfma(const Geo& g, const float* v, const void* B, void* y,
                                  const RowList& L, int64_t tiles, int ksplit, int v_rows,
                                  hipStream_t st) {
  if (tiles <= 0) return LORA_OK;
  if (ksplit < 1 || ksplit > (g.R > 32 ? kMaxKsplitWide : kMaxKsplit))
    return fail(LORA_E_ARG, "bad K split %d", ksplit);
  const Chunks ch = make_chunks(g, kExpandMfmaCols);
  if (tiles * ch.total > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large for one launch");
  if (g.R <= 64 && (int64_t)g.T * g.O * 2 < (int64_t)kDropOffset) {
    const int cpw = expand_cpw(g, tiles, ksplit);
    const Chunks gr = make_groups(g, cpw);
    if (ksplit > kMaxKsplitWide)  // R <= 32 (checked above)
      hipLaunchKernelGGL((expand_mfma_rows_kernel<MODE, kMaxKsplit>), dim3(grid_of(tiles * gr.total)),
                         dim3(256), 0, st, v, (const uint16_t*)B, (uint16_t*)y, L, g, ch, gr,
                         ksplit, v_rows, cpw);
    else
      hipLaunchKernelGGL((expand_mfma_rows_kernel<MODE, kMaxKsplitWide>),
                         dim3(grid_of(tiles * gr.total)), dim3(256), 0, st, v, (const uint16_t*)B,
                         (uint16_t*)y, L, g, ch, gr, ksplit, v_rows, cpw);
    return hip_check("expand_mfma_rows launch");
  }
  hipLaunchKernelGGL(expand_mfma_kernel<MODE>, dim3(grid_of(tiles * ch.total)), dim3(256), 0, st,
                     v, (const uint16_t*)B, (uint16_t*)y, L, g, ch, ksplit, v_rows);
  return hip_check("expand_mfma launch");
}

int32_t run_shrink(const Geo& g, const void* x, const void* A, float* v, RowList L,
                   hipStream_t st) {
  if (L.num_rows <= 0) return LORA_OK;
  const bool bf = g.dtype == LORA_BF16;
  if (L.ids) {  // BGMV rows
    const int64_t tiles = count_tiles(L, kWaveTileRows);
    return bf ? launch_shrink_wave<uint16_t, kRows>(g, x, A, v, L, tiles, st)
              : launch_shrink_wave<float, kRows>(g, x, A, v, L, tiles, st);
  }
  if (L.num_segs <= 0) return LORA_OK;
  const int thr = bf ? sgmv_mfma_min_rows() : INT32_MAX;
  RowList Lm = L, Lw = L;
  Lm.seg_min = thr;
  Lm.seg_max = INT32_MAX;
  Lw.seg_min = 0;
  Lw.seg_max = thr - 1;
  if (thr != INT32_MAX) {
    if (int32_t e = launch_shrink_mfma<kSegs>(g, x, A, v, Lm, count_tiles(Lm, kMfmaTileRows), 1,
                                              L.num_rows, st))
      return e;
  }
  const int64_t tw = count_tiles(Lw, kWaveTileRows);
  return bf ? launch_shrink_wave<uint16_t, kSegs>(g, x, A, v, Lw, tw, st)
            : launch_shrink_wave<float, kSegs>(g, x, A, v, Lw, tw, st);
}

int32_t run_expand(const Geo& g, const float* v, const void* B, void* y, RowList L,
                   hipStream_t st) {
  if (L.num_rows <= 0) return LORA_OK;
  const bool bf = g.dtype == LORA_BF16;
  if (L.ids) {
    const int64_t tiles = count_tiles(L, kWaveTileRows);
    return bf ? launch_expand_wave<uint16_t, kRows>(g, v, B, y, L, tiles, st)
              : launch_expand_wave<float, kRows>(g, v, B, y, L, tiles, st);
  }
  if (L.num_segs <= 0) return LORA_OK;
  const int thr = bf ? sgmv_mfma_min_rows() : INT32_MAX;
  RowList Lm = L, Lw = L;
  Lm.seg_min = thr;
  Lm.seg_max = INT32_MAX;
  Lw.seg_min = 0;
  Lw.seg_max = thr - 1;
  if (thr != INT32_MAX) {
    if (int32_t e = launch_expand_mfma<kSegs>(g, v, B, y, Lm, count_tiles(Lm, kMfmaTileRows), 1,
                                              L.num_rows, st))
      return e;
  }
  const int64_t tw = count_tiles(Lw, kWaveTileRows);
  return bf ? launch_expand_wave<uint16_t, kSegs>(g, v, B, y, Lw, tw, st)
            : launch_expand_wave<float, kSegs>(g, v, B, y, Lw, tw, st);
}

// Row lists of a plan's wavefront and MFMA tiles.  for_shrink: the lists read
// the image and copy it to p.copy_* (when set); else they read the copy.
static void plan_lists(const TilePlan& p, RowList& Lw, RowList& Lm, bool for_shrink = true) {
  const bool use_copy = !for_shrink && p.copy_perm && p.copy_wave && p.copy_mfma;
  const int32_t* perm = use_copy ? p.copy_perm : p.perm;
  Lw = RowList{perm, nullptr, nullptr, nullptr, nullptr, use_copy ? p.copy_wave : p.wave, 0,
               p.num_rows, p.wave_tiles, 0, INT32_MAX, nullptr, nullptr};
  Lm = RowList{perm, nullptr, nullptr, nullptr, nullptr, use_copy ? p.copy_mfma : p.mfma, 0,
               p.num_rows, p.mfma_tiles, 0, INT32_MAX, nullptr, nullptr};
  if (for_shrink) {
    Lw.copy_tiles = p.copy_wave;
    Lm.copy_tiles = p.copy_mfma;
    Lm.copy_tok = p.copy_perm;
  }
}

// Small plans (wavefront tiles only, at most kArgTilesL records, slots below
// 2^28) with host records go by value, in the smaller capacity that fits.
static bool small_plan(const TilePlan& p, const Geo& g) {
  return p.wave_host != nullptr && p.mfma_tiles == 0 && p.wave_tiles <= kArgTilesL &&
         g.max_loras <= (1 << 28);
}

template <int MODE> static PlanArg<MODE> pack_arg(const TilePlan& p) {
  PlanArg<MODE> a;
  for (int i = 0; i < arg_tiles<MODE>() * kArgWords; ++i) a.w[i] = -1;
  for (int f = 0; f < p.wave_tiles; ++f) {
    const int32_t* rec = p.wave_host + (size_t)f * LORA_PLAN_WAVE_WORDS;
    int32_t* o = a.w + f * kArgWords;
    o[0] = (int32_t)(((uint32_t)rec[1] << 28) | ((uint32_t)rec[0] & 0x0fffffffu));
    o[1] = rec[2];
    for (int r = 0; r < kArgWords - 2; ++r) o[2 + r] = rec[4 + r];
  }
  return a;
}

// Wavefront tiles of bf16 pools with R <= 64 take the MFMA shrink
// (LORA_TILE_MFMA_SHRINK=0 turns it off), which writes the plan's ksplit_wave
// partials of v; the VALU shrink writes one.
static bool tile_mfma_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("LORA_TILE_MFMA_SHRINK");
    return !(e && e[0] == '0');
  }();
  return on;
}
static bool use_tile_mfma(const Geo& g) {
  return g.dtype == LORA_BF16 && g.R <= 64 && tile_mfma_enabled();
}
static int wave_kparts(const Geo& g, const TilePlan& p) {
  return use_tile_mfma(g) ? p.ksplit_wave : 1;
}
// ... and the MFMA expand when y spans less than 2 GiB (raw buffer stores;
// LORA_TILE_MFMA_EXPAND=0 turns it off)
static bool use_tile_mfma_expand(const Geo& g) {
  static const bool on = [] {
    const char* e = std::getenv("LORA_TILE_MFMA_EXPAND");
    return !(e && e[0] == '0');
  }();
  return on && use_tile_mfma(g) && (int64_t)g.T * g.O * 2 < (int64_t)kDropOffset;
}

// kListWalk reaches only the MFMA tile kernels; the VALU kernels read the
// same records one per workgroup (kList)
template <int MODE> constexpr int valu_mode() { return MODE == kListWalk ? kList : MODE; }

template <int MODE>
static int32_t launch_plan_wave_expand(const Geo& g, const float* v, const void* B, void* y,
                                       const RowList& Lw, const TilePlan& p, hipStream_t st,
                                       const PlanArg<MODE>& pa = PlanArg<MODE>{}) {
  if (use_tile_mfma_expand(g))
    return launch_expand_tile<MODE>(g, v, B, y, Lw, p.wave_tiles, wave_kparts(g, p), p.num_rows,
                                    st, pa);
  constexpr int VM = valu_mode<MODE>();
  const PlanArg<VM> pv{};
  const PlanArg<VM>& pav = [&]() -> const PlanArg<VM>& {
    if constexpr (VM == MODE) return pa; else return pv;
  }();
  return g.dtype == LORA_BF16
             ? launch_expand_wave<uint16_t, VM>(g, v, B, y, Lw, p.wave_tiles, st, pav,
                                                wave_kparts(g, p), p.num_rows)
             : launch_expand_wave<float, VM>(g, v, B, y, Lw, p.wave_tiles, st, pav);
}

template <int MODE>
static int32_t launch_plan_wave_shrink(const Geo& g, const void* x, const void* A, float* v,
                                       const RowList& Lw, const TilePlan& p, hipStream_t st,
                                       const PlanArg<MODE>& pa = PlanArg<MODE>{}) {
  if (use_tile_mfma(g))
    return launch_shrink_tile<MODE>(g, x, A, v, Lw, p.wave_tiles, p.ksplit_wave, p.num_rows, st,
                                    pa);
  constexpr int VM = valu_mode<MODE>();
  const PlanArg<VM> pv{};
  const PlanArg<VM>& pav = [&]() -> const PlanArg<VM>& {
    if constexpr (VM == MODE) return pa; else return pv;
  }();
  return g.dtype == LORA_BF16
             ? launch_shrink_wave<uint16_t, VM>(g, x, A, v, Lw, p.wave_tiles, st, pav)
             : launch_shrink_wave<float, VM>(g, x, A, v, Lw, p.wave_tiles, st, pav);
}

// One launch per stage for a device-built plan (p.walk) whose 8-row tiles take
// the MFMA tile kernels: both tile kinds in one grid (shrink_combo_kernel,
// expand_combo_kernel).  LORA_COMBINED_LAUNCH=0 turns it off (read on every
// call, so a test can compare both forms in one process).
static bool combo_enabled() {
  const char* e = std::getenv("LORA_COMBINED_LAUNCH");
  return !(e && e[0] == '0');
}
static bool combo_shrink_ok(const Geo& g, const TilePlan& p) {
  return combo_enabled() && p.walk && p.mfma_tiles > 0 && p.wave_tiles > 0 && use_tile_mfma(g);
}
// ... the expand's 64-row part needs y under 2 GiB (raw buffer stores), as
// the 8-row part does
static bool combo_expand_ok(const Geo& g, const TilePlan& p) {
  return combo_shrink_ok(g, p) && use_tile_mfma_expand(g);
}

static int64_t round_xcd(int64_t n) { return (n + kNumXcd - 1) / kNumXcd * kNumXcd; }

template <int NT, bool DMA>
static int32_t launch_shrink_combo_k(const Geo& g, const void* x, const void* A, float* v,
                                     const RowList& Lm, const RowList& Lw, const TilePlan& p,
                                     hipStream_t st) {
  constexpr int CB = tile_shrink_cb(16 * NT);
  const int64_t nm = (int64_t)p.mfma_tiles * g.S * p.ksplit;
  const int64_t per = (int64_t)g.S * p.ksplit_wave;
  const int64_t nw = walk_records<kListWalk>(p.wave_tiles, per) * per;
  const int64_t nmp = round_xcd(nm);
  if (nmp > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large for one shrink launch");
  // every workgroup walks the 8-row records after its 64-row tile (if any)
  hipLaunchKernelGGL((shrink_combo_kernel<NT, CB, DMA>), dim3((unsigned)std::max(nmp, nw)),
                     dim3(256), 0, st, (const uint16_t*)x, (const uint16_t*)A, v, Lm, Lw, g,
                     p.ksplit, p.ksplit_wave, p.num_rows, (int)nm, (int)nmp, kComboXcdChunk);
  return hip_check("shrink_combo launch");
}

template <int NT>
static int32_t launch_shrink_combo_nt(const Geo& g, const void* x, const void* A, float* v,
                                      const RowList& Lm, const RowList& Lw, const TilePlan& p,
                                      hipStream_t st) {
  // the 64-row part takes the DMA-staged body where launch_shrink_mfma would
  return g.K % 64 == 0 && g.K <= kDmaShrinkMaxK
             ? launch_shrink_combo_k<NT, true>(g, x, A, v, Lm, Lw, p, st)
             : launch_shrink_combo_k<NT, false>(g, x, A, v, Lm, Lw, p, st);
}

static int32_t launch_shrink_combo(const Geo& g, const void* x, const void* A, float* v,
                                   const RowList& Lm, const RowList& Lw, const TilePlan& p,
                                   hipStream_t st) {
  if (p.ksplit < 1 || p.ksplit > (g.R > 32 ? kMaxKsplitWide : kMaxKsplit))
    return fail(LORA_E_ARG, "bad K split %d", p.ksplit);
  if (p.ksplit_wave < 1 || p.ksplit_wave > tile_kparts_max(g.R))
    return fail(LORA_E_ARG, "bad K split %d", p.ksplit_wave);
  switch (tile_shrink_rank_tiles(g.R)) {
    case 1: return launch_shrink_combo_nt<1>(g, x, A, v, Lm, Lw, p, st);
    case 2: return launch_shrink_combo_nt<2>(g, x, A, v, Lm, Lw, p, st);
    default: return launch_shrink_combo_nt<4>(g, x, A, v, Lm, Lw, p, st);
  }
}

template <int NKC, int KPR, int KPW>
static int32_t launch_expand_combo_k(const Geo& g, const float* v, const void* B, void* y,
                                     const RowList& Lm, const RowList& Lw, const TilePlan& p,
                                     hipStream_t st) {
  // the 64-row part as launch_expand_mfma lays it out
  const Chunks chm = make_chunks(g, kExpandMfmaCols);
  const int cpw = expand_cpw(g, p.mfma_tiles, p.ksplit);
  const Chunks gr = make_groups(g, cpw);
  const Chunks chw = make_chunks(g, kTileExpandCols);
  const int64_t nm = (int64_t)p.mfma_tiles * gr.total;
  const int64_t nw = walk_records<kListWalk>(p.wave_tiles, chw.total) * chw.total;
  const int64_t nmp = round_xcd(nm);
  if (nmp > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large for one expand launch");
  // every workgroup walks the 8-row records after its 64-row tile (if any)
  hipLaunchKernelGGL((expand_combo_kernel<NKC, KPR, KPW>), dim3((unsigned)std::max(nmp, nw)),
                     dim3(256), 0, st, v, (const uint16_t*)B, (uint16_t*)y, Lm, Lw, g, chm, gr,
                     chw, p.ksplit, p.ksplit_wave, p.num_rows, cpw, (int)nm, (int)nmp,
                     kComboXcdChunk);
  return hip_check("expand_combo launch");
}

template <int NKC, int KPR>
static int32_t launch_expand_combo_kpw(const Geo& g, const float* v, const void* B, void* y,
                                       const RowList& Lm, const RowList& Lw, const TilePlan& p,
                                       hipStream_t st) {
  // the walk's partials as launch_expand_tile_nkc takes them (eight only with
  // one 32-rank chunk)
  if constexpr (NKC == 1) {
    if (p.ksplit_wave > 4)
      return launch_expand_combo_k<NKC, KPR, 8>(g, v, B, y, Lm, Lw, p, st);
  }
  if constexpr (NKC == 2) {
    if (p.ksplit_wave > kMaxWalkKpartsWide)
      return fail(LORA_E_ARG, "bad K split %d", p.ksplit_wave);
  } else {
    if (p.ksplit_wave > 2) return launch_expand_combo_k<NKC, KPR, 4>(g, v, B, y, Lm, Lw, p, st);
  }
  if (p.ksplit_wave > 1) return launch_expand_combo_k<NKC, KPR, 2>(g, v, B, y, Lm, Lw, p, st);
  return launch_expand_combo_k<NKC, KPR, 1>(g, v, B, y, Lm, Lw, p, st);
}

static int32_t launch_expand_combo(const Geo& g, const float* v, const void* B, void* y,
                                   const RowList& Lm, const RowList& Lw, const TilePlan& p,
                                   hipStream_t st) {
  if (p.ksplit < 1 || p.ksplit > (g.R > 32 ? kMaxKsplitWide : kMaxKsplit))
    return fail(LORA_E_ARG, "bad K split %d", p.ksplit);
  if (p.ksplit_wave < 1 || p.ksplit_wave > tile_kparts_max(g.R))
    return fail(LORA_E_ARG, "bad K split %d", p.ksplit_wave);
  if (g.R > 32) return launch_expand_combo_kpw<2, kMaxKsplitWide>(g, v, B, y, Lm, Lw, p, st);
  return p.ksplit > kMaxKsplitWide
             ? launch_expand_combo_kpw<1, kMaxKsplit>(g, v, B, y, Lm, Lw, p, st)
             : launch_expand_combo_kpw<1, kMaxKsplitWide>(g, v, B, y, Lm, Lw, p, st);
}

int32_t run_plan_shrink(const Geo& g, const void* x, const void* A, float* v, const TilePlan& p,
                        hipStream_t st) {
  const bool bf = g.dtype == LORA_BF16;
  if (p.mfma_tiles > 0 && !bf) return fail(LORA_E_DTYPE, "MFMA tiles need a bf16 pool");
  RowList Lw, Lm;
  plan_lists(p, Lw, Lm);
  if (small_plan(p, g)) {
    if (p.wave_tiles <= kArgTilesS)
      return launch_plan_wave_shrink<kArg>(g, x, A, v, Lw, p, st, pack_arg<kArg>(p));
    return launch_plan_wave_shrink<kArgL>(g, x, A, v, Lw, p, st, pack_arg<kArgL>(p));
  }
  if (combo_shrink_ok(g, p)) return launch_shrink_combo(g, x, A, v, Lm, Lw, p, st);
  if (int32_t e = launch_shrink_mfma<kList>(g, x, A, v, Lm, p.mfma_tiles, p.ksplit, p.num_rows,
                                            st))
    return e;
  return p.walk ? launch_plan_wave_shrink<kListWalk>(g, x, A, v, Lw, p, st)
                : launch_plan_wave_shrink<kList>(g, x, A, v, Lw, p, st);
}

int32_t run_plan_expand(const Geo& g, const float* v, const void* B, void* y, const TilePlan& p,
                        hipStream_t st) {
  const bool bf = g.dtype == LORA_BF16;
  if (p.mfma_tiles > 0 && !bf) return fail(LORA_E_DTYPE, "MFMA tiles need a bf16 pool");
  RowList Lw, Lm;
  plan_lists(p, Lw, Lm, /*for_shrink=*/false);
  if (small_plan(p, g)) {
    if (p.wave_tiles <= kArgTilesS)
      return launch_plan_wave_expand<kArg>(g, v, B, y, Lw, p, st, pack_arg<kArg>(p));
    return launch_plan_wave_expand<kArgL>(g, v, B, y, Lw, p, st, pack_arg<kArgL>(p));
  }
  if (combo_expand_ok(g, p)) return launch_expand_combo(g, v, B, y, Lm, Lw, p, st);
  if (int32_t e = launch_expand_mfma<kList>(g, v, B, y, Lm, p.mfma_tiles, p.ksplit, p.num_rows,
                                            st))
    return e;
  return p.walk ? launch_plan_wave_expand<kListWalk>(g, v, B, y, Lw, p, st)
                : launch_plan_wave_expand<kList>(g, v, B, y, Lw, p, st);
}

// One launch for both stages (decode_onepass_kernel) when the plan goes by
// value in the small tier (at most kArgTilesS tiles, compact records), the
// pool is bf16, R <= 32 and T < 65536; LORA_ONEPASS_DECODE=0 turns it off.
static bool onepass_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("LORA_ONEPASS_DECODE");
    return !(e && e[0] == '0');
  }();
  return on;
}

bool plan_is_onepass(const Geo& g, const TilePlan& p) {
  return onepass_enabled() && g.dtype == LORA_BF16 && small_plan(p, g) && p.wave_tiles > 0 &&
         p.wave_tiles <= kArgTilesS && g.R <= 32 && g.T < 65536;
}

// The compact by-value records of the one-launch decode kernel (tokens below
// 65536, so 0xffff marks a row past the tile).
static PlanArg<kArgC> pack_arg_compact(const TilePlan& p) {
  PlanArg<kArgC> a;
  for (int i = 0; i < kArgTilesS * kArgCWords; ++i) a.w[i] = 0xffffffffu;
  for (int f = 0; f < p.wave_tiles && f < kArgTilesS; ++f) {
    const int32_t* rec = p.wave_host + (size_t)f * LORA_PLAN_WAVE_WORDS;
    uint32_t* o = a.w + f * kArgCWords;
    o[0] = ((uint32_t)rec[1] << 28) | ((uint32_t)rec[0] & 0x0fffffffu);
    for (int r = 0; r < kWaveTileRows; ++r) {
      const uint32_t t = rec[4 + r] >= 0 ? (uint32_t)rec[4 + r] & 0xffffu : 0xffffu;
      o[1 + r / 2] = (o[1 + r / 2] & ~(0xffffu << (16 * (r & 1)))) | (t << (16 * (r & 1)));
    }
  }
  return a;
}

bool device_plan_is_onepass(const Geo& g, int32_t cap) {
  return onepass_enabled() && g.dtype == LORA_BF16 && g.R <= 32 && cap > 0 &&
         cap <= kDeviceOnepassCap;
}

int32_t run_plan_onepass_list(const Geo& g, const void* x, const void* A, const void* B, void* y,
                              const TilePlan& p, hipStream_t st) {
  RowList Lw, Lm;
  plan_lists(p, Lw, Lm);
  return launch_onepass<kList>(g, x, A, B, y, Lw, p.wave_tiles, st, PlanArg<kList>{});
}

int32_t run_plan_apply(const Geo& g, const void* x, const void* A, const void* B, void* y,
                       const TilePlan& p, float* v, hipStream_t st) {
  if (!plan_is_onepass(g, p)) {
    if (int32_t e = run_plan_shrink(g, x, A, v, p, st)) return e;
    return run_plan_expand(g, v, B, y, p, st);
  }
  RowList Lw, Lm;
  plan_lists(p, Lw, Lm);
  return launch_onepass<kArgC>(g, x, A, B, y, Lw, p.wave_tiles, st, pack_arg_compact(p));
}

int32_t run_pool_load(const Geo& g, void* A_slot_slice, void* B_slot_slice, const void* Asrc,
                      const void* Bsrc, int r, int out_s, float scale, hipStream_t st) {
  const size_t n = (size_t)g.R * g.K + (size_t)out_s * g.R;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
  if (g.dtype == LORA_BF16) {
    hipLaunchKernelGGL(pool_load_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st,
                       (const uint16_t*)Asrc, (const uint16_t*)Bsrc, (uint16_t*)A_slot_slice,
                       (uint16_t*)B_slot_slice, r, g.R, g.K, out_s, scale);
  } else {
    hipLaunchKernelGGL(pool_load_kernel<float>, dim3(blocks), dim3(256), 0, st,
                       (const float*)Asrc, (const float*)Bsrc, (float*)A_slot_slice,
                       (float*)B_slot_slice, r, g.R, g.K, out_s, scale);
  }
  return hip_check("pool_load launch");
}

}  // namespace lora
