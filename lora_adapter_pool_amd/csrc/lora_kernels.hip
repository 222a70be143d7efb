// gfx950 (MI355X) kernels of the multi-LoRA delta path.
//
// Two stages per row list ([TGI] step 4 of the TGI multi-LoRA article: shrink
// x -> r, then expand r -> out, grouped by adapter):
//   shrink: v[i][s][k]   = sum_j A_pool[a][s][k][j] * x[t][j]          (fp32 acc)
//   expand: y[t][off_s+j] = rne(y[t][off_s+j] + sum_k B_pool[a][off_s+j][k] * v[i][s][k])
//
// Row lists are either SGMV segments (rows perm[seg_start .. +len), one adapter
// per segment) or BGMV rows (tok[i], ids[i] per row).  Work is cut into tiles of
// consecutive rows; a BGMV tile may hold several adapters and processes each
// distinct adapter once (rows come sorted by adapter, so usually one).
//
// Kernels:
//   shrink_wave   VALU, 4 waves split K, 8 contiguous elements per lane
//                 (16-byte loads), rank chunks across workgroups; the K
//                 reduction is a wavefront transpose-reduce plus a fixed-order
//                 sum of the four waves' partials in LDS (deterministic).
//   expand_wave   VALU, one output column per thread; the B block of the tile
//                 is copied from HBM into LDS with contiguous 16-byte loads and
//                 read back row-per-thread (padded rows, no bank conflicts);
//                 v rows are LDS broadcasts.
//   shrink_mfma   bf16 MFMA 16x16x32 for long SGMV segments: x rows are the
//                 A operand, adapter A rows the B operand, fp32 accumulators;
//                 two waves split K, partials summed in fixed order.
//   expand_mfma   bf16 MFMA 16x16x32 computing (B_pool tile) x v^T so that each
//                 lane ends with 8 consecutive output columns of one token
//                 (16-byte y read-modify-write); fp32 v enters as a hi + lo
//                 bf16 pair (two MFMAs), keeping ~16 mantissa bits of v.
//
// Workgroup ids are remapped so that consecutive tiles (which share adapter
// weights and, across rank chunks, x rows) land on the same XCD's L2: the
// hardware deals workgroups round-robin over the 8 XCDs.
//
// Every token index and adapter slot read from device metadata is bounds-checked
// against T and max_loras; rows that fail are skipped, never dereferenced.
#include <hip/hip_runtime.h>

#include "lora_internal.h"
#include "lora_kernels.h"

namespace lora {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                   // nearest, ties to even
  return u >> 16;
}

template <typename E> struct El;

template <> struct El<float> {
  static __device__ __forceinline__ void load8(const float* p, float (&o)[8]) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
    o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y);
    o[2] = __uint_as_float(a.z); o[3] = __uint_as_float(a.w);
    o[4] = __uint_as_float(b.x); o[5] = __uint_as_float(b.y);
    o[6] = __uint_as_float(b.z); o[7] = __uint_as_float(b.w);
  }
  static __device__ __forceinline__ float get(float v) { return v; }
  static __device__ __forceinline__ float put(float v) { return v; }
};

template <> struct El<uint16_t> {
  static __device__ __forceinline__ void load8(const uint16_t* p, float (&o)[8]) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    o[0] = __uint_as_float(a.x << 16); o[1] = __uint_as_float(a.x & 0xffff0000u);
    o[2] = __uint_as_float(a.y << 16); o[3] = __uint_as_float(a.y & 0xffff0000u);
    o[4] = __uint_as_float(a.z << 16); o[5] = __uint_as_float(a.z & 0xffff0000u);
    o[6] = __uint_as_float(a.w << 16); o[7] = __uint_as_float(a.w & 0xffff0000u);
  }
  static __device__ __forceinline__ float get(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  static __device__ __forceinline__ uint16_t put(float v) {
    return static_cast<uint16_t>(f32_to_bf16_bits(v));
  }
};

// Workgroups are dealt round-robin over the XCDs; give each XCD a contiguous
// range of logical ids (a bijection on [0, n)).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n / kNumXcd, r = n % kNumXcd;
  const int x = bid % kNumXcd, k = bid / kNumXcd;
  return x * q + min(x, r) + k;
}

// Locate tile `f` of a row list.  BGMV: fixed row ranges of TM rows.  SGMV:
// tiles of TM rows inside each segment whose (clamped) length lies in
// [seg_min, seg_max], in segment order.  Returns false past the last tile.
template <int TM>
__device__ __forceinline__ bool find_tile(const RowList& L, int f, int& r0, int& cnt, int& sid) {
  if (L.ids) {
    r0 = f * TM;
    if (r0 >= L.num_rows) return false;
    cnt = min(TM, L.num_rows - r0);
    sid = -1;
    return true;
  }
  for (int gi = 0; gi < L.num_segs; ++gi) {
    const int st = L.seg_starts[gi];
    int ln = L.seg_lens[gi];
    if (st < 0 || st >= L.num_rows || ln <= 0) continue;
    ln = min(ln, L.num_rows - st);
    if (ln < L.seg_min || ln > L.seg_max) continue;
    const int nt = (ln + TM - 1) / TM;
    if (f < nt) {
      r0 = st + f * TM;
      cnt = min(TM, ln - f * TM);
      sid = L.seg_ids[gi];
      return true;
    }
    f -= nt;
  }
  return false;
}

// Token and adapter slot of each tile row; bit r of the result marks row r valid.
template <int TM>
__device__ __forceinline__ uint32_t load_tile_rows(const RowList& L, const Geo& g, int r0, int cnt,
                                                   int sid, int (&tok)[TM], int (&aid)[TM]) {
  uint32_t valid = 0;
#pragma unroll
  for (int r = 0; r < TM; ++r) {
    int t = -1, a = -1;
    if (r < cnt) {
      t = L.tok[r0 + r];
      a = L.ids ? L.ids[r0 + r] : sid;
    }
    const bool ok = t >= 0 && t < g.T && a >= 0 && a < g.max_loras;
    tok[r] = ok ? t : 0;
    aid[r] = ok ? a : -1;
    valid |= (ok ? 1u : 0u) << r;
  }
  return valid;
}

// Next adapter group of a tile: the adapter of the lowest pending row and the
// mask of pending rows that use it.
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
// grid.x = tiles * S * (R / RC).  Workgroup (tile, slice s, rank chunk c)
// computes v[row][s][c*RC .. c*RC+RC) for the tile's rows.  Wave w covers the
// K chunks w, w+4, ... of 512 elements (8 per lane).
template <typename E, int TM, int RC>
__global__ __launch_bounds__(256) void shrink_wave_kernel(const E* __restrict__ x,
                                                          const E* __restrict__ A,
                                                          float* __restrict__ v, RowList L,
                                                          Geo g) {
  constexpr int V = RC * TM;
  constexpr int P = Log2<V>::value;
  __shared__ float red[4][V];
  const int nrc = g.R / RC;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_tile = g.S * nrc;
  const int f = bid / per_tile;
  const int rem = bid - f * per_tile;
  const int s = rem / nrc;
  const int c = rem - s * nrc;
  int r0, cnt, sid;
  if (!find_tile<TM>(L, f, r0, cnt, sid)) return;
  int tok[TM], aid[TM];
  uint32_t todo = load_tile_rows<TM>(L, g, r0, cnt, sid, tok, aid);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int SR = g.S * g.R;

  while (todo) {
    int a;
    const uint32_t m = next_group<TM>(todo, aid, a);
    todo &= ~m;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    const E* Ab = A + ((size_t)(a * g.S + s) * g.R + (size_t)c * RC) * g.K;
    for (int k0 = wave * 512 + lane * 8; k0 < g.K; k0 += 4 * 512) {
      float av[RC][8];
#pragma unroll
      for (int rr = 0; rr < RC; ++rr) El<E>::load8(Ab + (size_t)rr * g.K + k0, av[rr]);
#pragma unroll
      for (int r = 0; r < TM; ++r) {
        if (!((m >> r) & 1u)) continue;
        float xv[8];
        El<E>::load8(x + (size_t)tok[r] * g.K + k0, xv);
#pragma unroll
        for (int rr = 0; rr < RC; ++rr) {
          float d = acc[rr * TM + r];
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(av[rr][e], xv[e], d);
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
        const float tot = ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
        v[(size_t)(r0 + r) * SR + s * g.R + c * RC + rr] = tot;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ expand (VALU)
//
// grid.x = tiles * column chunks (kExpandCols columns of one slice each).
// Thread j owns output column col0 + j; the tile's B block is staged in LDS
// 64 ranks at a time, v rows are staged once.
template <typename E, int TM>
__global__ __launch_bounds__(256) void expand_wave_kernel(const float* __restrict__ v,
                                                          const E* __restrict__ B,
                                                          E* __restrict__ y, RowList L, Geo g,
                                                          Chunks ch) {
  constexpr int NC = kExpandCols;      // 256 columns per workgroup
  constexpr int KB = 64;               // ranks staged per pass
  constexpr int PAD = 16 / sizeof(E);  // row padding: 16 bytes
  constexpr int LDB = KB + PAD;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  E* Bs = reinterpret_cast<E*>(lds_raw);                                   // [NC][LDB]
  float* vs = reinterpret_cast<float*>(lds_raw + sizeof(E) * NC * LDB);    // [TM][R]

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int f = bid / ch.total;
  const int cidx = bid - f * ch.total;
  int s = 0;
#pragma unroll
  for (int i = 1; i < LORA_MAX_SLICES; ++i)
    if (i < g.S && cidx >= ch.start[i]) s = i;
  const int col0 = (cidx - ch.start[s]) * NC;
  const int ncv = min(NC, g.out[s] - col0);
  int r0, cnt, sid;
  if (!find_tile<TM>(L, f, r0, cnt, sid)) return;
  int tok[TM], aid[TM];
  uint32_t todo = load_tile_rows<TM>(L, g, r0, cnt, sid, tok, aid);
  const int tid = threadIdx.x;
  const int R = g.R;
  const int SR = g.S * R;

  while (todo) {
    int a;
    const uint32_t m = next_group<TM>(todo, aid, a);
    todo &= ~m;
    // v rows of this group (zeros for rows outside it)
    for (int i = tid; i < TM * R; i += 256) {
      const int r = i / R, k = i - r * R;
      vs[i] = ((m >> r) & 1u) ? v[(size_t)(r0 + r) * SR + s * R + k] : 0.f;
    }
    float acc[TM];
#pragma unroll
    for (int r = 0; r < TM; ++r) acc[r] = 0.f;
    const E* Bg = B + ((size_t)a * g.O + g.off[s] + col0) * R;
    for (int kb = 0; kb < R; kb += KB) {
      const int kw = min(KB, R - kb);   // multiple of 8
      const int vpr = kw / 8;           // 8-element vectors per staged row
      __syncthreads();                  // previous readers of Bs are done
      for (int i = tid; i < ncv * vpr; i += 256) {
        const int row = i / vpr, q = i - row * vpr;
        const E* src = Bg + (size_t)row * R + kb + q * 8;
        E* dst = Bs + row * LDB + q * 8;
        if constexpr (sizeof(E) == 2) {
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
        } else {
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
          *reinterpret_cast<u32x4*>(dst + 4) = *reinterpret_cast<const u32x4*>(src + 4);
        }
      }
      __syncthreads();
      if (tid < ncv) {
        for (int k = 0; k < kw; k += 8) {
          float b[8];
          El<E>::load8(Bs + tid * LDB + k, b);
#pragma unroll
          for (int r = 0; r < TM; ++r) {
            if (!((m >> r) & 1u)) continue;
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
        if (!((m >> r) & 1u)) continue;
        E* yp = y + (size_t)tok[r] * g.O + g.off[s] + col0 + tid;
        *yp = El<E>::put(El<E>::get(*yp) + acc[r]);
      }
    }
    __syncthreads();  // vs is rewritten by the next group
  }
}

// ------------------------------------------------------------ shrink (MFMA)
//
// bf16 only.  grid.x = tiles(32 rows) * S, grid.y = rank blocks of 64.
// Wave (wm, wk): rows 16*wm .. +16 of the tile, K steps of 128 with index
// congruent to wk mod 2.  Per step each lane loads 4 x 16 bytes of its x row
// and of each of NT adapter rows; MFMA p covers k in [k0 + 32p, k0 + 32p + 32),
// lane group g = lane / 16 holding k0 + 32p + 8g .. +8 of both operands.
template <int NT>
__global__ __launch_bounds__(256) void shrink_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ A,
                                                          float* __restrict__ v, RowList L,
                                                          Geo g) {
  constexpr int TMR = 32;
  __shared__ f32x4 part[2][NT][64];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int f = bid / g.S;
  const int s = bid - f * g.S;
  const int rank0 = blockIdx.y * 64;
  int r0, cnt, sid;
  if (!find_tile<TMR>(L, f, r0, cnt, sid)) return;
  if (sid < 0 || sid >= g.max_loras) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wk = wave >> 1;
  const int i16 = lane & 15, grp = lane >> 4;
  const int row = 16 * wm + i16;  // operand row of this lane
  int t = -1;
  if (row < cnt) t = L.tok[r0 + row];
  const bool xrow_ok = t >= 0 && t < g.T;
  const uint16_t* xr = x + (size_t)(xrow_ok ? t : 0) * g.K;
  const uint16_t* Ab = A + ((size_t)(sid * g.S + s) * g.R + rank0 + i16) * g.K;

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = wk * 128; k0 < g.K; k0 += 256) {
    u32x4 xf[4];
    u32x4 af[NT][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int kp = k0 + 32 * p + 8 * grp;
      const bool in = kp < g.K;
      xf[p] = (in && xrow_ok) ? *reinterpret_cast<const u32x4*>(xr + kp) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int n = 0; n < NT; ++n)
        af[n][p] = in ? *reinterpret_cast<const u32x4*>(Ab + (size_t)(16 * n) * g.K + kp)
                      : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bf16x8 xa = __builtin_bit_cast(bf16x8, xf[p]);
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, af[n][p]),
                                                         acc[n], 0, 0, 0);
    }
  }
  if (wk == 1) {
#pragma unroll
    for (int n = 0; n < NT; ++n) part[wm][n][lane] = acc[n];
  }
  __syncthreads();
  if (wk == 0) {
    const int SR = g.S * g.R;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const f32x4 o = part[wm][n][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int orow = 16 * wm + 4 * grp + j;  // D row of this lane
        if (orow < cnt) {
          const int tt = L.tok[r0 + orow];
          if (tt >= 0 && tt < g.T)
            v[(size_t)(r0 + orow) * SR + s * g.R + rank0 + 16 * n + i16] = acc[n][j] + o[j];
        }
      }
    }
  }
}

// ------------------------------------------------------------ expand (MFMA)
//
// bf16 only.  grid.x = tiles(32 rows) * column chunks of 128 (one slice each).
// Wave (wt, wc): tokens 16*wt .. +16, columns 64*wc .. +64 of the chunk, as two
// pairs of 16-column MFMA tiles.  The MFMA computes D = Bt * v^T (rows = output
// columns, columns = tokens).  Inside a pair, MFMA row n of tile 2q maps to
// column 32q + 8(n/4) + n%4 and of tile 2q+1 to the same + 4, so lane (g, m)
// ends with columns 32q + 8g .. +8 of token m: one 16-byte y access.
__global__ __launch_bounds__(256) void expand_mfma_kernel(const float* __restrict__ v,
                                                          const uint16_t* __restrict__ B,
                                                          uint16_t* __restrict__ y, RowList L,
                                                          Geo g, Chunks ch) {
  constexpr int TMR = 32;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int f = bid / ch.total;
  const int cidx = bid - f * ch.total;
  int s = 0;
#pragma unroll
  for (int i = 1; i < LORA_MAX_SLICES; ++i)
    if (i < g.S && cidx >= ch.start[i]) s = i;
  const int col0 = (cidx - ch.start[s]) * kExpandMfmaCols;
  int r0, cnt, sid;
  if (!find_tile<TMR>(L, f, r0, cnt, sid)) return;
  if (sid < 0 || sid >= g.max_loras) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wt = wave & 1, wc = wave >> 1;
  const int m16 = lane & 15, grp = lane >> 4;
  const int R = g.R;
  const int SR = g.S * R;
  const int out_s = g.out[s];

  // B-operand token of this lane (column m16 of the MFMA)
  const int trow = 16 * wt + m16;
  int t = -1;
  if (trow < cnt) t = L.tok[r0 + trow];
  const bool tok_ok = t >= 0 && t < g.T;
  const float* vr = v + (size_t)(r0 + (trow < cnt ? trow : 0)) * SR + s * R;

  // A-operand rows: output columns of this lane for each of the 4 tiles
  const int cbase = col0 + 64 * wc;
  const uint16_t* Bb = B + ((size_t)sid * g.O + g.off[s]) * R;
  int ccol[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int q = nt >> 1, hi = nt & 1;
    ccol[nt] = cbase + 32 * q + 8 * (m16 >> 2) + 4 * hi + (m16 & 3);
  }

  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < R; kb += 32) {
    const int kk = kb + 8 * grp;
    const bool kin = kk < R;
    // v (fp32) -> hi + lo bf16
    u32x4 vh = {0, 0, 0, 0}, vl = {0, 0, 0, 0};
    if (kin && tok_ok) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(vr + kk);
      const f32x4 b = *reinterpret_cast<const f32x4*>(vr + kk + 4);
      const float e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t h[8], l[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        h[i] = f32_to_bf16_bits(e[i]);
        l[i] = f32_to_bf16_bits(e[i] - __uint_as_float(h[i] << 16));
      }
      vh = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      vl = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
    }
    const bf16x8 bh = __builtin_bit_cast(bf16x8, vh);
    const bf16x8 bl = __builtin_bit_cast(bf16x8, vl);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      u32x4 bw = {0, 0, 0, 0};
      if (kin && ccol[nt] < out_s) bw = *reinterpret_cast<const u32x4*>(Bb + (size_t)ccol[nt] * R + kk);
      const bf16x8 ba = __builtin_bit_cast(bf16x8, bw);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ba, bh, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ba, bl, acc[nt], 0, 0, 0);
    }
  }
  if (!tok_ok) return;
  uint16_t* yr = y + (size_t)t * g.O + g.off[s];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = cbase + 32 * q + 8 * grp;
    if (c >= out_s) continue;
    u32x4 yw = *reinterpret_cast<const u32x4*>(yr + c);
    const f32x4 d0 = acc[2 * q], d1 = acc[2 * q + 1];
    const float add[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
    uint32_t w[4] = {yw.x, yw.y, yw.z, yw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16) + add[2 * i];
      const float hi = __uint_as_float(w[i] & 0xffff0000u) + add[2 * i + 1];
      w[i] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
    }
    *reinterpret_cast<u32x4*>(yr + c) = u32x4{w[0], w[1], w[2], w[3]};
  }
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

// Number of tiles of `tm` rows for a row list; exact when the host knows the
// segment lengths, otherwise an upper bound (surplus workgroups exit at once).
static int64_t count_tiles(const RowList& L, int tm, const int32_t* host_seg_starts,
                           const int32_t* host_seg_lens) {
  if (L.ids) return (L.num_rows + tm - 1) / tm;
  if (!host_seg_lens) return (int64_t)(L.num_rows + tm - 1) / tm + L.num_segs;
  int64_t n = 0;
  for (int i = 0; i < L.num_segs; ++i) {
    const int st = host_seg_starts[i];
    int ln = host_seg_lens[i];
    if (st < 0 || st >= L.num_rows || ln <= 0) continue;
    ln = std::min(ln, L.num_rows - st);
    if (ln < L.seg_min || ln > L.seg_max) continue;
    n += (ln + tm - 1) / tm;
  }
  return n;
}

static int sgmv_mfma_min_rows() {
  static int v = [] {
    const char* e = std::getenv("LORA_SGMV_MFMA_MIN_ROWS");
    int x = e ? std::atoi(e) : kSgmvMfmaMinRows;
    return x < 1 ? 1 : x;
  }();
  return v;
}

static bool mfma_eligible(const Geo& g) { return g.dtype == LORA_BF16 && g.R % 16 == 0; }

template <typename E>
static int32_t launch_shrink_wave(const Geo& g, const void* x, const void* A, float* v,
                                  const RowList& L, int64_t tiles, hipStream_t st) {
  if (tiles <= 0) return LORA_OK;
  if (g.R % 8 == 0 && g.R >= 64) {
    const int64_t grid = tiles * g.S * (g.R / 8);
    if (grid > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large");
    hipLaunchKernelGGL((shrink_wave_kernel<E, kWaveTileRows, 8>), dim3((unsigned)grid), dim3(256),
                       0, st, (const E*)x, (const E*)A, v, L, g);
  } else {
    const int64_t grid = tiles * g.S * (g.R / 4);
    if (grid > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large");
    hipLaunchKernelGGL((shrink_wave_kernel<E, kWaveTileRows, 4>), dim3((unsigned)grid), dim3(256),
                       0, st, (const E*)x, (const E*)A, v, L, g);
  }
  return hip_check("shrink_wave launch");
}

template <typename E>
static int32_t launch_expand_wave(const Geo& g, const float* v, const void* B, void* y,
                                  const RowList& L, int64_t tiles, hipStream_t st) {
  if (tiles <= 0) return LORA_OK;
  const Chunks ch = make_chunks(g, kExpandCols);
  const int64_t grid = tiles * ch.total;
  if (grid > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large");
  const size_t lds = sizeof(E) * kExpandCols * (64 + 16 / sizeof(E)) +
                     sizeof(float) * kWaveTileRows * g.R;
  if (lds > 160 * 1024) return fail(LORA_E_SHAPE, "max_lora_rank too large for the expand kernel");
  hipLaunchKernelGGL((expand_wave_kernel<E, kWaveTileRows>), dim3((unsigned)grid), dim3(256), lds,
                     st, v, (const E*)B, (E*)y, L, g, ch);
  return hip_check("expand_wave launch");
}

static int32_t launch_shrink_mfma(const Geo& g, const void* x, const void* A, float* v,
                                  const RowList& L, int64_t tiles, hipStream_t st) {
  if (tiles <= 0) return LORA_OK;
  const int64_t gx = tiles * g.S;
  if (gx > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large");
  const int full = g.R / 64, rest = (g.R % 64) / 16;
  if (full > 0) {
    hipLaunchKernelGGL((shrink_mfma_kernel<4>), dim3((unsigned)gx, full), dim3(256), 0, st,
                       (const uint16_t*)x, (const uint16_t*)A, v, L, g);
    if (int32_t e = hip_check("shrink_mfma launch")) return e;
  }
  if (rest > 0) {
    // remaining ranks: shift A and v by the full blocks via blockIdx.y offset
    Geo g2 = g;
    const int off = full * 64;
    // A rows and v columns start at rank `off`; kernels index rank0 = blockIdx.y*64 = 0
    const uint16_t* A2 = (const uint16_t*)A + (size_t)off * g.K;
    float* v2 = v + off;
    switch (rest) {
      case 1: hipLaunchKernelGGL((shrink_mfma_kernel<1>), dim3((unsigned)gx, 1), dim3(256), 0, st,
                                 (const uint16_t*)x, A2, v2, L, g2); break;
      case 2: hipLaunchKernelGGL((shrink_mfma_kernel<2>), dim3((unsigned)gx, 1), dim3(256), 0, st,
                                 (const uint16_t*)x, A2, v2, L, g2); break;
      default: hipLaunchKernelGGL((shrink_mfma_kernel<3>), dim3((unsigned)gx, 1), dim3(256), 0, st,
                                  (const uint16_t*)x, A2, v2, L, g2); break;
    }
    if (int32_t e = hip_check("shrink_mfma launch")) return e;
  }
  return LORA_OK;
}

static int32_t launch_expand_mfma(const Geo& g, const float* v, const void* B, void* y,
                                  const RowList& L, int64_t tiles, hipStream_t st) {
  if (tiles <= 0) return LORA_OK;
  const Chunks ch = make_chunks(g, kExpandMfmaCols);
  const int64_t grid = tiles * ch.total;
  if (grid > INT32_MAX) return fail(LORA_E_SHAPE, "batch too large");
  hipLaunchKernelGGL(expand_mfma_kernel, dim3((unsigned)grid), dim3(256), 0, st, v,
                     (const uint16_t*)B, (uint16_t*)y, L, g, ch);
  return hip_check("expand_mfma launch");
}

int32_t run_shrink(const Geo& g, const void* x, const void* A, float* v, RowList L,
                   const int32_t* host_seg_starts, const int32_t* host_seg_lens, hipStream_t st) {
  if (L.num_rows <= 0) return LORA_OK;
  if (L.ids) {  // BGMV
    L.seg_min = 0;
    L.seg_max = INT32_MAX;
    const int64_t tiles = count_tiles(L, kWaveTileRows, nullptr, nullptr);
    return g.dtype == LORA_BF16 ? launch_shrink_wave<uint16_t>(g, x, A, v, L, tiles, st)
                                : launch_shrink_wave<float>(g, x, A, v, L, tiles, st);
  }
  if (L.num_segs <= 0) return LORA_OK;
  const int thr = mfma_eligible(g) ? sgmv_mfma_min_rows() : INT32_MAX;
  RowList Lm = L, Lw = L;
  Lm.seg_min = thr;
  Lm.seg_max = INT32_MAX;
  Lw.seg_min = 0;
  Lw.seg_max = thr - 1;
  if (thr != INT32_MAX) {
    const int64_t tm = count_tiles(Lm, 32, host_seg_starts, host_seg_lens);
    if (int32_t e = launch_shrink_mfma(g, x, A, v, Lm, tm, st)) return e;
  }
  const int64_t tw = count_tiles(Lw, kWaveTileRows, host_seg_starts, host_seg_lens);
  return g.dtype == LORA_BF16 ? launch_shrink_wave<uint16_t>(g, x, A, v, Lw, tw, st)
                              : launch_shrink_wave<float>(g, x, A, v, Lw, tw, st);
}

int32_t run_expand(const Geo& g, const float* v, const void* B, void* y, RowList L,
                   const int32_t* host_seg_starts, const int32_t* host_seg_lens, hipStream_t st) {
  if (L.num_rows <= 0) return LORA_OK;
  if (L.ids) {
    L.seg_min = 0;
    L.seg_max = INT32_MAX;
    const int64_t tiles = count_tiles(L, kWaveTileRows, nullptr, nullptr);
    return g.dtype == LORA_BF16 ? launch_expand_wave<uint16_t>(g, v, B, y, L, tiles, st)
                                : launch_expand_wave<float>(g, v, B, y, L, tiles, st);
  }
  if (L.num_segs <= 0) return LORA_OK;
  const int thr = mfma_eligible(g) ? sgmv_mfma_min_rows() : INT32_MAX;
  RowList Lm = L, Lw = L;
  Lm.seg_min = thr;
  Lm.seg_max = INT32_MAX;
  Lw.seg_min = 0;
  Lw.seg_max = thr - 1;
  if (thr != INT32_MAX) {
    const int64_t tm = count_tiles(Lm, 32, host_seg_starts, host_seg_lens);
    if (int32_t e = launch_expand_mfma(g, v, B, y, Lm, tm, st)) return e;
  }
  const int64_t tw = count_tiles(Lw, kWaveTileRows, host_seg_starts, host_seg_lens);
  return g.dtype == LORA_BF16 ? launch_expand_wave<uint16_t>(g, v, B, y, Lw, tw, st)
                              : launch_expand_wave<float>(g, v, B, y, Lw, tw, st);
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
