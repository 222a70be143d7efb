// Device-side metadata builder: the arrays of lora_build_meta ([TGI] step 4:
// the rows of a batch sorted by adapter id, SGMV rows into segments of one
// adapter, BGMV rows into a per-row list) computed on the GPU from device ids,
// so a batch needs no host round trip and the whole delta path can be
// captured in a graph.  One workgroup:
//   1. a histogram of the SGMV and BGMV rows per adapter (LDS atomics: counts
//      do not depend on their order);
//   2. exclusive scans of both histograms and of the non-empty SGMV bins give
//      every adapter its first position and its segment;
//   3. the rows' keys are staged in LDS by blocks, and the rows are placed in
//      token order, 64 at a time: lanes with the same (adapter, set) key take
//      consecutive positions in lane order, so the sort is stable and the
//      result is the host builder's, bit for bit.  One wavefront places a
//      block, or, for pools of at most kParMaxLoras slots and large blocks,
//      all 16 each place a contiguous sixteenth from their own positions;
//   4. optionally (lora_apply_device), the tile records of a device-built
//      plan in the host plan's format, up to fixed capacities.  A plan's
//      build writes its v-row -> token map in step 3 in place of the arrays
//      above, and no segments or padding: its kernels read only the plan.
// Arrays are padded so the grouped entry points can take upper-bound sizes:
// segments past num_segs have length 0, BGMV rows past num_bgmv_rows have
// id -1 (skipped by the kernels), and sgmv_perm past num_sgmv_rows is 0.
#include <hip/hip_runtime.h>

#include <climits>

#include "lora_internal.h"
#include "lora_kernels.h"

namespace lora {

constexpr int kMetaThreads = 1024;
// Pools of at most this many slots place rows with all 16 wavefronts (each
// with its own per-key counters in LDS: 16 x 2 x kParMaxLoras words).
constexpr int kParMaxLoras = 256;
// ... for blocks of more rows than this (smaller blocks: the three extra
// barriers cost more than the single wavefront's chain).
constexpr int kParMinRows = 1024;
constexpr int kMetaWaves = kMetaThreads / 64;
// Rows per thread whose ids are loaded at once by the histogram loop, and by
// the per-wavefront histogram (one memory round trip for batches of up to
// 16 x 64 x 16 rows).
constexpr int kHistBatch = 8;
constexpr int kWaveHistBatch = 16;

using i32x4 = int32_t __attribute__((ext_vector_type(4)));
static_assert(LORA_PLAN_WAVE_WORDS == 16 && LORA_PLAN_MFMA_WORDS == 4,
              "records are written as 16-byte words");

// The lanes of this wavefront whose key equals this lane's, for keys in
// [0, 2^kbits): the AND, over the key's bits, of the ballot of lanes that agree
// with this lane on that bit.  Lanes with a negative key are in no mask.  Its
// cost does not depend on how many distinct keys the wavefront holds.
__device__ __forceinline__ uint64_t same_key_lanes(int key, int kbits) {
  uint64_t m = __ballot(key >= 0);
  for (int b = 0; b < kbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Inclusive prefix sums over the lanes of each row of 16 (row_incl_scan) and
// over the whole wavefront (wave_incl_scan), with DPP moves: shifts by 1, 2, 4
// and 8 lanes within each row (lanes with no source add 0), then lane 15 of
// rows 0 and 2 added to rows 1 and 3, and lane 31 to rows 2 and 3.
__device__ __forceinline__ int row_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x = row_incl_scan(x);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Sum of per-wavefront values s[w * stride] over the wavefronts before `wave`
// (excl) and over all of them (tot): lane w < kMetaWaves holds wavefront w's
// value and a scan over the first row of lanes adds them up, so no wavefront
// walks the others'.  `wave` is uniform.
__device__ __forceinline__ void wave_prefix(const int32_t* s, int stride, int wave, int lane,
                                            int& excl, int& tot) {
  static_assert(kMetaWaves == 16, "one value per lane of the first row");
  int x = lane < kMetaWaves ? s[lane * stride] : 0;
  x = row_incl_scan(x);
  tot = __builtin_amdgcn_readlane(x, kMetaWaves - 1);
  excl = wave > 0 ? __builtin_amdgcn_readlane(x, wave > 0 ? wave - 1 : 0) : 0;
}

// Set bits of m below this lane (popc(m & lanes below) with mbcnt).
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// bins[key] += 1 for every active lane with key >= 0.  Sorted batches give
// whole wavefronts of one key, whose atomics on one LDS word would serialize:
// then the first lane adds the count once.
__device__ __forceinline__ void count_keys(int32_t* bins, int key) {
  const uint64_t active = __ballot(true);
  const int k0 = __builtin_amdgcn_readlane(key, __builtin_ctzll(active));
  if (k0 >= 0 && __ballot(key == k0) == active) {
    if ((int)(threadIdx.x & 63) == __builtin_ctzll(active)) atomicAdd(&bins[k0], __popcll(active));
  } else if (key >= 0) {
    atomicAdd(&bins[key], 1);
  }
}

__global__ __launch_bounds__(kMetaThreads) void build_meta_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ prefill, int32_t T,
    int32_t max_loras, int32_t all_sgmv, lora_meta m, int32_t* __restrict__ counts,
    int32_t kcap, DevicePlanOut plan) {
  // [max_loras] SGMV bins, [max_loras] BGMV bins, then the keys of a block of
  // kcap rows (int16: 2 id + set, or -1)
  extern __shared__ int32_t lds[];
  __shared__ int32_t s_bad;
  __shared__ int32_t s_wsum[kMetaThreads / 64][3];
  int32_t* cs = lds;
  int32_t* cb = lds + max_loras;
  // with a plan (lora_apply_device) only the plan is written: its v-row ->
  // token map and records; the grouped entry points' arrays (m), which its
  // kernels never read, are left alone
  const bool meta_out = plan.tiles == nullptr;  // uniform
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int nw = kMetaThreads / 64;
  const bool one_block = T <= kcap;
  const bool par_slots = max_loras <= kParMaxLoras;  // uniform
  const int nkeys = 2 * max_loras;
  int32_t* wcnt = lds + 2 * max_loras + kcap / 2 + (plan.tiles ? 2 * (max_loras + 1) : 0);
  // a batch of one block placed by all wavefronts counts each wavefront's
  // keys in the histogram pass already, over the rows that wavefront places
  const bool wave_hist = one_block && par_slots && T > kParMinRows;  // uniform
  for (int a = tid; a < max_loras; a += kMetaThreads) {
    cs[a] = 0;
    cb[a] = 0;
  }
  if (wave_hist)
    for (int k = tid; k < nw * nkeys; k += kMetaThreads) wcnt[k] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // 1. histogram; a batch that fits one block of keys also stages its keys
  //    here, so placement does not read the ids again.  Each thread loads the
  //    ids and flags of kHistBatch rows before it counts any of them, so the
  //    loop waits on memory once per batch, not once per row.
  int16_t* keys = reinterpret_cast<int16_t*>(lds + 2 * max_loras);
  // every lane loads (rows past T repeat row T - 1 and count as rows without
  // adapter), so no branch waits on a load; without flags the loads of pf
  // read the ids' bytes and pmask drops them
  const uint8_t* pf = prefill != nullptr ? prefill : reinterpret_cast<const uint8_t*>(ids);
  const uint32_t pmask = prefill != nullptr ? 0xffu : 0u;
  if (wave_hist) {
    // wavefront w: rows [lo, hi), the contiguous share placement gives it,
    // counted by key (2 id + set) into its own counters
    const int sb = ((T + nw - 1) / nw + 63) / 64 * 64;
    const int lo = min(T, wave * sb), hi = min(T, lo + sb);
    int32_t* my = wcnt + wave * nkeys;
    for (int i0 = lo; i0 < hi; i0 += 64 * kWaveHistBatch) {  // uniform
      int av[kWaveHistBatch];
      uint32_t pv[kWaveHistBatch];
#pragma unroll
      for (int u = 0; u < kWaveHistBatch; ++u) {
        const int tc = min(i0 + 64 * u + lane, hi - 1);
        av[u] = ids[tc];
        pv[u] = pf[tc];
      }
#pragma unroll
      for (int u = 0; u < kWaveHistBatch; ++u) {
        if (i0 + 64 * u >= hi) break;  // uniform
        const int t = i0 + 64 * u + lane;
        const int a = t < hi ? av[u] : -1;
        const bool ok = a >= 0 && a < max_loras;
        const bool sg = ok && (all_sgmv || (pv[u] & pmask) != 0);
        const int key = ok ? 2 * a + (sg ? 1 : 0) : -1;
        if (t < hi) keys[t] = (int16_t)key;
        if (a < -1 || a >= max_loras) atomicAdd(&s_bad, 1);
        count_keys(my, key);
      }
    }
  }
  for (int t0 = 0; t0 < T && !wave_hist; t0 += kMetaThreads * kHistBatch) {
    int av[kHistBatch];
    uint32_t pv[kHistBatch];
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) {
      const int tc = min(t0 + u * kMetaThreads + tid, T - 1);
      av[u] = ids[tc];
      pv[u] = pf[tc];
    }
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) {
      if (t0 + u * kMetaThreads >= T) break;  // uniform
      const int t = t0 + u * kMetaThreads + tid;
      const int a = t < T ? av[u] : -1;
      const bool ok = a >= 0 && a < max_loras;
      const bool sg = ok && (all_sgmv || (pv[u] & pmask) != 0);
      if (one_block && t < T) keys[t] = (int16_t)(ok ? 2 * a + (sg ? 1 : 0) : -1);
      if (a < -1 || a >= max_loras) atomicAdd(&s_bad, 1);
      // cs and cb are adjacent: bin max_loras + a is cb[a]
      count_keys(cs, ok ? (sg ? a : max_loras + a) : -1);
    }
  }
  __syncthreads();

  // 2. exclusive scans over the bins; thread tid owns bins [a0, a1) (the
  // per-wavefront counts, if any, summed into them first)
  const int per = (max_loras + kMetaThreads - 1) / kMetaThreads;
  const int a0 = min(max_loras, tid * per), a1 = min(max_loras, a0 + per);
  if (wave_hist) {
    for (int a = a0; a < a1; ++a) {
      int sgc = 0, bgc = 0;
#pragma unroll
      for (int w = 0; w < kMetaWaves; ++w) {
        sgc += wcnt[w * nkeys + 2 * a + 1];
        bgc += wcnt[w * nkeys + 2 * a];
      }
      cs[a] = sgc;
      cb[a] = bgc;
    }
  }
  int v[3] = {0, 0, 0};  // SGMV rows, BGMV rows, SGMV segments
  for (int a = a0; a < a1; ++a) {
    v[0] += cs[a];
    v[1] += cb[a];
    v[2] += cs[a] > 0;
  }
  int inc[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) inc[i] = wave_incl_scan(v[i]);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < 3; ++i) s_wsum[wave][i] = inc[i];
  }
  __syncthreads();
  int base[3], tot[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) wave_prefix(&s_wsum[0][i], 3, wave, lane, base[i], tot[i]);
  int es = base[0] + inc[0] - v[0], eb = base[1] + inc[1] - v[1], eg = base[2] + inc[2] - v[2];
  for (int a = a0; a < a1; ++a) {
    const int c = cs[a], d = cb[a];
    if (c > 0 && meta_out) {
      m.seg_starts[eg] = es;
      m.seg_lens[eg] = c;
      m.seg_ids[eg] = a;
      ++eg;
    }
    cs[a] = es;  // the bins become the next free position of each adapter
    es += c;
    cb[a] = eb;
    eb += d;
  }
  const int ns = tot[0], nb = tot[1], nseg = tot[2];
  if (tid == 0) {
    counts[0] = ns;
    counts[1] = nseg;
    counts[2] = nb;
  }
  if (meta_out) {
    for (int i = nseg + tid; i < max_loras; i += kMetaThreads) {
      m.seg_starts[i] = ns;
      m.seg_lens[i] = 0;
      m.seg_ids[i] = 0;
    }
    for (int i = ns + tid; i < T; i += kMetaThreads) m.sgmv_perm[i] = 0;
    for (int i = nb + tid; i < T; i += kMetaThreads) {
      m.bgmv_tok[i] = 0;
      m.bgmv_ids[i] = -1;
    }
  }
  __syncthreads();
  if (tid == 0) counts[3] = s_bad;

  // 3. stable placement, by blocks of kcap rows: every thread stages the
  // block's keys in LDS, then the rows are placed 64 at a time.  A chunk
  // gathers the next free position of each lane's key, ranks equal keys by
  // lane order with ballots (registers only), and the first lane of each key
  // writes the key's new next free position.  With at most kParMaxLoras slots
  // and blocks of more than kParMinRows rows, each wavefront takes a
  // contiguous sixteenth of the block: it counts its
  // keys into its own counters, a prefix over the wavefronts per key turns the
  // counts into each wavefront's first positions, and the wavefronts place
  // their rows at once (rows keep token order, so the sort stays stable).
  // Otherwise one wavefront places the whole block.
  const int kbits = 32 - __clz(2 * max_loras - 1);  // bits of the largest key
  for (int b0 = 0; b0 < T; b0 += kcap) {
    const int nbk = min(kcap, T - b0);
    __syncthreads();  // the previous block's keys are placed
    for (int i0 = 0; i0 < nbk && !one_block; i0 += kMetaThreads * kHistBatch) {
      int av[kHistBatch];
      uint32_t pv[kHistBatch];
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {  // unconditional loads, as in the histogram
        const int tc = b0 + min(i0 + u * kMetaThreads + tid, nbk - 1);
        av[u] = ids[tc];
        pv[u] = pf[tc];
      }
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        const int i = i0 + u * kMetaThreads + tid;
        const int a = av[u];
        const bool ok = a >= 0 && a < max_loras;
        const bool sg = all_sgmv || (pv[u] & pmask) != 0;
        if (i < nbk) keys[i] = (int16_t)(ok ? 2 * a + (sg ? 1 : 0) : -1);
      }
    }
    const bool par = par_slots && nbk > kParMinRows;  // uniform
    int32_t* my = wcnt + wave * nkeys;  // this wavefront's counters (par)
    int lo = 0, hi = 0;                  // the rows this wavefront places
    if (par) {
      const int sb = ((nbk + nw - 1) / nw + 63) / 64 * 64;
      lo = min(nbk, wave * sb);
      hi = min(nbk, lo + sb);
      if (!wave_hist) {  // (else counted by the histogram pass)
        for (int k = lane; k < nkeys; k += 64) my[k] = 0;
        __syncthreads();  // keys staged, counters cleared
        for (int i = lo + lane; i < hi; i += 64) count_keys(my, keys[i]);
        __syncthreads();
      }
      for (int k = tid; k < nkeys; k += kMetaThreads) {
        int32_t* pos = (k & 1) ? &cs[k >> 1] : &cb[k >> 1];
        int base = *pos;
        int c[kMetaWaves];  // all counts read before the first is replaced
#pragma unroll
        for (int w = 0; w < kMetaWaves; ++w) c[w] = wcnt[w * nkeys + k];
#pragma unroll
        for (int w = 0; w < kMetaWaves; ++w) {
          wcnt[w * nkeys + k] = base;
          base += c[w];
        }
        *pos = base;
      }
    } else {
      hi = wave == 0 ? nbk : 0;
    }
    __syncthreads();
    // equal keys take consecutive positions in lane order; the lowest lane of
    // each key moves the key's next free position.  A chunk whose rows all
    // have one key (sorted batches) skips the per-bit ballots, and while
    // consecutive such chunks share their key its next position stays in a
    // register (ckey, cpos: uniform), so only the first of them reads it
    int ckey = -1, cpos = 0;
    for (int c = lo; c < hi; c += 64) {
      const int i = c + lane;
      const int key = i < hi ? keys[i] : -1;
      const uint64_t valid = __ballot(key >= 0);
      if (valid == 0) continue;  // uniform: no row of this chunk has an adapter
      const int k0 = __builtin_amdgcn_readlane(key, __builtin_ctzll(valid));
      const bool uni = __ballot(key == k0) == valid;  // uniform
      int32_t* pos;
      int p0, rank, cnt;
      bool first;
      if (uni) {
        pos = par ? &my[k0] : (k0 & 1) ? &cs[k0 >> 1] : &cb[k0 >> 1];
        p0 = k0 == ckey ? cpos : *pos;
        rank = lanes_below(valid);
        cnt = __popcll(valid);
        first = (int)lane == __builtin_ctzll(valid);
        ckey = k0;
        cpos = p0 + cnt;
      } else {
        ckey = -1;  // positions move through LDS only
        pos = par ? &my[key] : (key & 1) ? &cs[key >> 1] : &cb[key >> 1];
        p0 = key >= 0 ? *pos : 0;
        const uint64_t mk = same_key_lanes(key, kbits);
        rank = lanes_below(mk);
        cnt = __popcll(mk);
        first = key >= 0 && rank == 0;
      }
      const int p = p0 + rank;
      if (key >= 0 && p < T) {
        const int t = b0 + i;
        if (!meta_out) {
          // the device plan's v-row -> token map: SGMV rows, then BGMV rows
          const int vr = (key & 1) ? p : ns + p;
          if (vr < T) plan.perm[vr] = t;
        } else if (key & 1) {
          m.sgmv_perm[p] = t;
        } else {
          m.bgmv_tok[p] = t;
          m.bgmv_ids[p] = key >> 1;
        }
      }
      if (first) *pos = p0 + cnt;
    }
  }
  if (plan.tiles == nullptr) return;

  // 4. a device-built plan (lora_apply_device), records as the host plan's:
  // 8-row tiles (slot, rows, first v row, 0, tokens, -1 past the last row) and
  // 64-row MFMA tiles (slot, rows, first v row, first token when the tile's
  // tokens are consecutive, else -1); v rows are the SGMV rows, then the BGMV
  // rows.  After placement each bin holds its slot's end position, and slots
  // are laid out back to back, so a slot's rows run from the previous slot's
  // end to its own.  A slot's SGMV rows take MFMA tiles when there are at
  // least mfma_min of them, its BGMV rows when there are at least bgmv_min of
  // them and such runs hold at least bgmv_total rows of the batch (a block
  // sum decides that first).  Exclusive scans of both tile counts per slot give
  // each slot's first records, and one thread per record finds its slot by
  // binary search.  Records from the last tile up to the capacity get 0 rows
  // (the kernels skip them), so launches can take the capacities as grids.
  __syncthreads();  // placement (wavefront 0) is complete
  int32_t* toff = lds + 2 * max_loras + kcap / 2;  // [max_loras + 1], after the keys
  int32_t* moff = toff + max_loras + 1;            // [max_loras + 1]
  int lr = 0;  // BGMV rows in runs of at least bgmv_min rows
  for (int a = a0; a < a1; ++a) {
    const int bc = cb[a] - (a > 0 ? cb[a - 1] : 0);
    lr += bc >= plan.bgmv_min ? bc : 0;
  }
  lr = __builtin_amdgcn_readlane(wave_incl_scan(lr), 63);
  if (lane == 0) s_wsum[wave][2] = lr;
  __syncthreads();
  int lr_before, lrt;
  wave_prefix(&s_wsum[0][2], 3, wave, lane, lr_before, lrt);
  const int bmin = lrt >= plan.bgmv_total ? plan.bgmv_min : INT_MAX;  // uniform
  auto tiles_of = [&](int sc, int bc, int& w8, int& w64) {
    const bool ms = sc >= plan.mfma_min, mb = bc >= bmin;
    w8 = (ms ? 0 : (sc + 7) / 8) + (mb ? 0 : (bc + 7) / 8);
    w64 = (ms ? (sc + LORA_PLAN_MFMA_ROWS - 1) / LORA_PLAN_MFMA_ROWS : 0) +
          (mb ? (bc + LORA_PLAN_MFMA_ROWS - 1) / LORA_PLAN_MFMA_ROWS : 0);
  };
  int nt = 0, nmf = 0;
  for (int a = a0; a < a1; ++a) {
    const int sc = cs[a] - (a > 0 ? cs[a - 1] : 0), bc = cb[a] - (a > 0 ? cb[a - 1] : 0);
    int w8, w64;
    tiles_of(sc, bc, w8, w64);
    nt += w8;
    nmf += w64;
  }
  const int inct = wave_incl_scan(nt), incm = wave_incl_scan(nmf);
  if (lane == 63) {
    s_wsum[wave][0] = inct;
    s_wsum[wave][1] = incm;
  }
  __syncthreads();
  int tb, ttot, mb, mtot;
  wave_prefix(&s_wsum[0][0], 3, wave, lane, tb, ttot);
  wave_prefix(&s_wsum[0][1], 3, wave, lane, mb, mtot);
  tb += inct - nt;
  mb += incm - nmf;
  for (int a = a0; a < a1; ++a) {
    const int sc = cs[a] - (a > 0 ? cs[a - 1] : 0), bc = cb[a] - (a > 0 ? cb[a - 1] : 0);
    int w8, w64;
    tiles_of(sc, bc, w8, w64);
    toff[a] = tb;
    moff[a] = mb;
    tb += w8;
    mb += w64;
  }
  if (tid == 0) {
    toff[max_loras] = ttot;
    moff[max_loras] = mtot;
  }
  __syncthreads();
  // the last slot whose first record is at or before f owns record f (empty
  // slots before it have smaller indices)
  // rank a record carries: 0 = the pool's R, else the slot's rank rounded up
  // to 8 (slot_ranks as lora_apply_ranked's; the kernels clamp any value)
  auto rank_of = [&](int slot) {
    if (plan.slot_ranks == nullptr) return 0;
    const int r = plan.slot_ranks[slot];
    const int r8 = (r + 7) / 8 * 8;
    return r > 0 && r8 < plan.R ? r8 : 0;
  };
  auto owner = [&](const int32_t* off, int f) {
    int lo = 0, hi = max_loras - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= f) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  // 8-row records: the real ones (16-byte stores), then the rest of the
  // capacity (0 rows, tokens -1) as consecutive 16-byte words
  const int nreal = min(ttot, plan.cap);
  for (int f = tid; f < nreal; f += kMetaThreads) {
    int slot = 0, rows = 0, vrow = 0;
    {
      slot = owner(toff, f);
      const int s0 = slot > 0 ? cs[slot - 1] : 0, b0 = slot > 0 ? cb[slot - 1] : 0;
      const int sc = cs[slot] - s0;
      // 8-row tiles: the SGMV rows' (unless on MFMA tiles), then the BGMV rows'
      const int lt = f - toff[slot], tsg = sc >= plan.mfma_min ? 0 : (sc + 7) / 8;
      if (lt < tsg) {
        vrow = s0 + LORA_PLAN_WAVE_ROWS * lt;
        rows = min(LORA_PLAN_WAVE_ROWS, cs[slot] - vrow);
      } else {
        const int first = b0 + LORA_PLAN_WAVE_ROWS * (lt - tsg);
        rows = min(LORA_PLAN_WAVE_ROWS, cb[slot] - first);
        vrow = ns + first;
      }
    }
    // the tokens (the v-row map from vrow on) are loaded unconditionally (a
    // real record has rows >= 1; lanes past it repeat its last row), so no
    // branch waits on a load
    const int last = max(rows, 1) - 1;
    const int32_t* src = plan.perm + (rows > 0 ? vrow : 0);  // (rows 0 not expected)
    int tk[LORA_PLAN_WAVE_ROWS];
#pragma unroll
    for (int i = 0; i < LORA_PLAN_WAVE_ROWS; ++i) tk[i] = src[min(i, last)];
#pragma unroll
    for (int i = 0; i < LORA_PLAN_WAVE_ROWS; ++i) tk[i] = i < rows ? tk[i] : -1;
    i32x4* r4 = reinterpret_cast<i32x4*>(plan.tiles + (size_t)f * LORA_PLAN_WAVE_WORDS);
    r4[0] = i32x4{slot, rows, vrow, rows > 0 ? rank_of(slot) : 0};
    r4[1] = i32x4{tk[0], tk[1], tk[2], tk[3]};
    r4[2] = i32x4{tk[4], tk[5], tk[6], tk[7]};
    r4[3] = i32x4{-1, -1, -1, -1};
  }
  {
    i32x4* r4 = reinterpret_cast<i32x4*>(plan.tiles);
    const int64_t q1 = (int64_t)plan.cap * (LORA_PLAN_WAVE_WORDS / 4);
    for (int64_t q = (int64_t)nreal * (LORA_PLAN_WAVE_WORDS / 4) + tid; q < q1; q += kMetaThreads)
      r4[q] = (q & 3) == 0 ? i32x4{0, 0, 0, 0} : i32x4{-1, -1, -1, -1};
  }
  for (int f = tid; f < plan.mcap; f += kMetaThreads) {
    int slot = 0, rows = 0, vrow = 0, tok0 = -1;
    if (f < mtot) {
      // 64-row tiles: the SGMV rows' (if on MFMA tiles), then the BGMV rows'
      slot = owner(moff, f);
      const int s0 = slot > 0 ? cs[slot - 1] : 0, b0 = slot > 0 ? cb[slot - 1] : 0;
      const int sc = cs[slot] - s0;
      const int lt = f - moff[slot];
      const int msg = sc >= plan.mfma_min ? (sc + LORA_PLAN_MFMA_ROWS - 1) / LORA_PLAN_MFMA_ROWS : 0;
      if (lt < msg) {
        const int first = s0 + LORA_PLAN_MFMA_ROWS * lt;
        rows = min(LORA_PLAN_MFMA_ROWS, cs[slot] - first);
        vrow = first;
      } else {
        const int first = b0 + LORA_PLAN_MFMA_ROWS * (lt - msg);
        rows = min(LORA_PLAN_MFMA_ROWS, cb[slot] - first);
        vrow = ns + first;
      }
      const int32_t* src = plan.perm + vrow;
      // a slot's rows of one set are in increasing token order (the sort is
      // stable), so they are consecutive exactly when last - first = rows - 1
      const int t0 = src[0];
      tok0 = src[rows - 1] - t0 == rows - 1 ? t0 : -1;
    }
    reinterpret_cast<i32x4*>(plan.mtiles)[f] =
        i32x4{slot, rows > 0 ? rows | (rank_of(slot) << 16) : 0, vrow, tok0};
  }
}

int32_t run_build_meta_device(const int32_t* ids, const uint8_t* prefill, int32_t T,
                              int32_t max_loras, bool all_sgmv, const lora_meta& m,
                              int32_t* counts, hipStream_t st, const DevicePlanOut* plan) {
  // LDS: the bins, the keys of a block of rows, then (with a plan) each
  // slot's first record of both kinds; up to 128 KB in all
  const int64_t bins = (int64_t)2 * max_loras * sizeof(int32_t);
  const int64_t toff = plan ? (int64_t)2 * (max_loras + 1) * sizeof(int32_t) : 0;
  const int64_t wcnt = max_loras <= kParMaxLoras
                           ? (int64_t)(kMetaThreads / 64) * 2 * max_loras * sizeof(int32_t)
                           : 0;
  int64_t kcap = ((int64_t)128 * 1024 - bins - toff - wcnt) / (int64_t)sizeof(int16_t) / 64 * 64;
  kcap = std::max<int64_t>(64, std::min<int64_t>(kcap, ((int64_t)T + 63) / 64 * 64));
  hipLaunchKernelGGL(build_meta_kernel, dim3(1), dim3(kMetaThreads),
                     (size_t)(bins + kcap * (int64_t)sizeof(int16_t) + toff + wcnt), st, ids,
                     prefill,
                     T, max_loras, all_sgmv ? 1 : 0, m, counts, (int32_t)kcap,
                     plan ? *plan : DevicePlanOut{nullptr, 0, nullptr, 0, 0, 0, 0, nullptr, nullptr, 0});
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LORA_E_HIP, "build_meta launch: %s", hipGetErrorString(e));
  return LORA_OK;
}

}  // namespace lora
