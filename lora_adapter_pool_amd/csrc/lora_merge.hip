// Merged-weight mode: one adapter folded into a copy of the base weight,
//   W_out[o][k] = round(W[o][k] + sum_r B_pool[a][off_s + o][r] * A_pool[a][s][r][k]),
// for one slot a and slice s ([QA] follow-up on merging an adapter into the
// base: a server that runs a single fine-tune merges it and pays nothing per
// request; one that serves many keeps the runtime delta).  B_pool already holds
// the scale, so this is W + s_a B A.  Accumulation in fp32, one final
// rounding to the pool dtype (nearest, ties to even).
//
// bf16 pools: the sum over ranks is a dense contraction [out_s x R] x [R x K],
// so it runs on MFMA (v_mfma_f32_16x16x32_bf16).  The first operand is B_pool
// as stored (rank-contiguous rows); A_pool is rank-major, so a workgroup
// stages its columns of A transposed in LDS.
//   - ranks <= 128 (merge_rows_kernel): a workgroup owns 256 columns and walks
//     several 64-row blocks, reusing the staged A; each lane ends with 16
//     contiguous bytes of W per row, so W goes from HBM to registers and back.
//   - larger ranks (merge_mfma_kernel): a workgroup owns a 128 x 64 tile of W:
//     4 waves x 32 rows, each wave 2 x 4 MFMA tiles per 32 ranks; the products
//     go through LDS so W is read and written 16 bytes a lane, whole 128-byte
//     lines per 8 lanes.
// fp32 pools: a plain VALU kernel, 4 columns a thread.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>

#include "lora_internal.h"
#include "lora_kernels.h"

namespace lora {

namespace {

typedef uint32_t m_u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 m_bf16x8 __attribute__((ext_vector_type(8)));
typedef float m_f32x4 __attribute__((ext_vector_type(4)));
typedef float m_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 m_bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileO = 128;  // W rows per workgroup
constexpr int kTileK = 64;   // W columns per workgroup
constexpr int kLdd = kTileK + 4;  // fp32 words per row of the staged products

__device__ __forceinline__ uint32_t rne_pack(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(m_f32x2{lo, hi}, m_bf16x2));
}

__device__ __forceinline__ m_u32x4 load16(const void* p) {
  return *reinterpret_cast<const m_u32x4*>(p);
}

__device__ __forceinline__ uint32_t mask_of(bool b) { return b ? 0xffffffffu : 0u; }

}  // namespace

// LDS bytes of merge_mfma_kernel for pool rank R.
static size_t merge_lds_bytes(int R) {
  const int nrc = (R + 31) / 32;
  return (size_t)kTileK * (32 * nrc + 8) * sizeof(uint16_t) + (size_t)kTileO * kLdd * sizeof(float);
}

__global__ __launch_bounds__(256) void merge_mfma_kernel(const uint16_t* __restrict__ Ap,
                                                         const uint16_t* __restrict__ Bp,
                                                         const uint16_t* W, uint16_t* Wo, int R,
                                                         int K, int out_s) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int nrc = (R + 31) / 32;   // 32-rank chunks
  const int ldr = 32 * nrc + 8;    // bf16 per staged column of A (rows stay 16-byte aligned)
  uint16_t* At = reinterpret_cast<uint16_t*>(lds);  // [kTileK][ldr]: A transposed
  float* Dt = reinterpret_cast<float*>(lds + (size_t)kTileK * ldr * sizeof(uint16_t));
  const int k0 = blockIdx.x * kTileK, o0 = blockIdx.y * kTileO;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // 0. this thread's 4 chunks of 8 columns of the W tile, loaded first so the
  //    reads are in flight during the staging and the products
  constexpr int kChunks = kTileO * (kTileK / 8) / 256;
  m_u32x4 wreg[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c = tid + 256 * i, row = c >> 3, j = c & 7, o = o0 + row, k = k0 + 8 * j;
    const bool ok = o < out_s && k < K;
    wreg[i] = load16(W + (ok ? (size_t)o * K + k : 0)) & mask_of(ok);
  }

  // 1. A[r][k0 .. k0 + 64) -> At[k][r]; ranks R .. 32 nrc and columns past K are 0
  for (int c = tid; c < 32 * nrc * (kTileK / 8); c += 256) {
    const int r = c >> 3, j = c & 7, k = k0 + 8 * j;
    const bool ok = r < R && k < K;  // K is a multiple of 8: a chunk is whole or absent
    const m_u32x4 a = load16(Ap + (ok ? (size_t)r * K + k : 0)) & mask_of(ok);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      At[(8 * j + i) * ldr + r] = (uint16_t)(a[i >> 1] >> (16 * (i & 1)));
  }
  __syncthreads();

  // 2. products: MFMA A operand = B rows (o, 8 ranks), B operand = A^T (k, 8 ranks);
  //    lane l holds row / column l % 16 and ranks 8 (l / 16) .. + 8 of a 32-rank chunk
  const int m16 = lane & 15, g = lane >> 4;
  m_f32x4 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = m_f32x4{0.f, 0.f, 0.f, 0.f};
  for (int rc = 0; rc < nrc; ++rc) {
    const int r = 32 * rc + 8 * g;
    m_bf16x8 bo[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int o = o0 + 32 * wave + 16 * mt + m16;
      const bool ok = o < out_s && r < R;  // R is a multiple of 8
      bo[mt] = __builtin_bit_cast(
          m_bf16x8, load16(Bp + (ok ? (size_t)o * R + r : 0)) & mask_of(ok));
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const m_bf16x8 at = __builtin_bit_cast(
          m_bf16x8, *reinterpret_cast<const m_u32x4*>(&At[(16 * nt + m16) * ldr + r]));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bo[mt], at, acc[mt][nt], 0, 0, 0);
    }
  }
  // D lane l: rows 4 (l / 16) + j, column l % 16 of each 16 x 16 tile
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        Dt[(32 * wave + 16 * mt + 4 * g + j) * kLdd + 16 * nt + m16] = acc[mt][nt][j];
  __syncthreads();

  // 3. W + products, rounded once; 8 columns a lane, 8 lanes a 128-byte row
#pragma unroll
  for (int ci = 0; ci < kChunks; ++ci) {
    const int c = tid + 256 * ci, row = c >> 3, j = c & 7, o = o0 + row, k = k0 + 8 * j;
    if (o >= out_s || k >= K) continue;
    const size_t at = (size_t)o * K + k;
    const m_u32x4 w = wreg[ci];
    const float* d = &Dt[row * kLdd + 8 * j];
    m_u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16) + d[2 * i];
      const float hi = __uint_as_float(w[i] & 0xffff0000u) + d[2 * i + 1];
      out[i] = rne_pack(lo, hi);
    }
    *reinterpret_cast<m_u32x4*>(Wo + at) = out;
  }
}

// bf16, pool rank R <= 128 (NRC = ceil(R / 32) chunks of 32 ranks).  A
// workgroup owns kMrCols columns of W and walks nblk consecutive blocks of
// kMrRows rows: the slot's A for those columns is staged once, transposed, in
// LDS (At[column][rank]) and serves every block, so its reads are spread over
// nblk blocks.  Wave w owns rows 16 w .. +16 of a block and computes
// D = B_rows * At^T with B's rows as the MFMA's first operand (D rows = W
// rows) and At as its second (D columns = W columns).  In MFMA tile nt (8 per
// 128-column half) column j reads W column 8 j + nt, so lane (g, j) holds,
// over the 8 tiles, columns 8 j .. 8 j + 8 of rows 4 g .. 4 g + 4: it reads
// and writes them as 16-byte accesses and W goes from HBM to registers and
// back with no LDS pass.  Column c of a half sits at LDS row (c % 8) * 16 +
// c / 8 of that half, so the 16 lanes reading columns 8 j + nt hit 16
// consecutive padded rows (no two in one bank); the staging writes go lane by
// lane along the ranks (consecutive 2-byte words).  The next block's W and B
// loads are issued before the current block's products are written back.
constexpr int kMrCols = 256;  // W columns per workgroup (two halves of 128)
constexpr int kMrRows = 64;   // W rows per block (4 waves x 16)

template <int NRC>
__global__ __launch_bounds__(256, 2) void merge_rows_kernel(const uint16_t* __restrict__ Ap,
                                                            const uint16_t* __restrict__ Bp,
                                                            const uint16_t* W, uint16_t* Wo,
                                                            int R, int K, int out_s, int nblk) {
  constexpr int RP = 32 * NRC;    // ranks staged (zero past R)
  constexpr int LDR = RP + 8;     // bf16 per staged column (rows stay 16-byte aligned)
  __shared__ __align__(16) uint16_t At[kMrCols * LDR];
  const int k0 = blockIdx.x * kMrCols;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int j16 = lane & 15, g = lane >> 4;
  auto lds_row = [](int c) { return (c >> 7) * 128 + (c & 7) * 16 + ((c & 127) >> 3); };

  // this lane's W pieces of block b: rows 16 wave + 4 g + jj, columns
  // k0 + 128 h + 8 j16 .. +8 (zero past out_s or K; K is a multiple of 8)
  auto load_w = [&](int b, m_u32x4 (&w)[2][4]) {
    const int ob = (blockIdx.y * nblk + b) * kMrRows + 16 * wave + 4 * g;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int o = ob + jj, k = k0 + 128 * h + 8 * j16;
        const bool ok = o < out_s && k < K;
        w[h][jj] = load16(W + (ok ? (size_t)o * K + k : 0)) & mask_of(ok);
      }
  };
  // MFMA first operand: B row 16 wave + j16 of block b, ranks 32 rc + 8 g .. +8
  auto load_b = [&](int b, m_u32x4 (&br)[NRC]) {
    const int o = (blockIdx.y * nblk + b) * kMrRows + 16 * wave + j16;
#pragma unroll
    for (int rc = 0; rc < NRC; ++rc) {
      const int r = 32 * rc + 8 * g;
      const bool ok = o < out_s && r < R;  // R is a multiple of 8
      br[rc] = load16(Bp + (ok ? (size_t)o * R + r : 0)) & mask_of(ok);
    }
  };
  // block 0's loads are in flight during the staging of A; B before W, so
  // the products, which wait for B, leave the W loads outstanding
  m_u32x4 wc[2][4], bc[NRC];
  load_b(0, bc);
  load_w(0, wc);

  // stage A[r][k0 .. k0 + 256) -> At[lds_row(k)][r]; lanes go along the ranks
  for (int c = tid; c < RP * (kMrCols / 8); c += 256) {
    const int r = c % RP, j = c / RP, k = k0 + 8 * j;
    const bool ok = r < R && k < K;
    const m_u32x4 a = load16(Ap + (ok ? (size_t)r * K + k : 0)) & mask_of(ok);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      At[lds_row(8 * j + i) * LDR + r] = (uint16_t)(a[i >> 1] >> (16 * (i & 1)));
  }
  __syncthreads();

  for (int b = 0; b < nblk; ++b) {
    if ((blockIdx.y * nblk + b) * kMrRows >= out_s) break;  // uniform
    m_f32x4 acc[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[h][nt] = m_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rc = 0; rc < NRC; ++rc) {
      const m_bf16x8 bo = __builtin_bit_cast(m_bf16x8, bc[rc]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          // W column 128 h + 8 j16 + nt sits at LDS row 128 h + nt * 16 + j16
          const m_bf16x8 at = __builtin_bit_cast(
              m_bf16x8,
              *reinterpret_cast<const m_u32x4*>(&At[(128 * h + nt * 16 + j16) * LDR + 32 * rc + 8 * g]));
          acc[h][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bo, at, acc[h][nt], 0, 0, 0);
        }
    }
    // lane (g, j16): acc[h][nt][jj] is row 4 g + jj, column 128 h + 8 j16 + nt
    const int ob = (blockIdx.y * nblk + b) * kMrRows + 16 * wave + 4 * g;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int o = ob + jj, k = k0 + 128 * h + 8 * j16;
        m_u32x4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(wc[h][jj][i] << 16) + acc[h][2 * i][jj];
          const float hi = __uint_as_float(wc[h][jj][i] & 0xffff0000u) + acc[h][2 * i + 1][jj];
          out[i] = rne_pack(lo, hi);
        }
        if (o < out_s && k < K) *reinterpret_cast<m_u32x4*>(Wo + (size_t)o * K + k) = out;
      }
    if (b + 1 < nblk) {  // the next block's loads, B first
      load_b(b + 1, bc);
      load_w(b + 1, wc);
    }
  }
}

__global__ __launch_bounds__(256) void merge_f32_kernel(const float* __restrict__ Ap,
                                                        const float* __restrict__ Bp,
                                                        const float* W, float* Wo, int R, int K,
                                                        int out_s) {
  const int k = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (k >= K) return;  // K is a multiple of 8: k + 4 <= K
  for (int o = blockIdx.y; o < out_s; o += gridDim.y) {
    const size_t at = (size_t)o * K + k;
    const m_f32x4 w = *reinterpret_cast<const m_f32x4*>(W + at);
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < R; ++r) {
      const float b = Bp[(size_t)o * R + r];
      const m_f32x4 a = *reinterpret_cast<const m_f32x4*>(Ap + (size_t)r * K + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = fmaf(b, a[i], s[i]);
    }
    *reinterpret_cast<m_f32x4*>(Wo + at) = m_f32x4{w[0] + s[0], w[1] + s[1], w[2] + s[2], w[3] + s[3]};
  }
}

int32_t run_merge(const Geo& g, const void* A_slot_slice, const void* B_slot_slice,
                  const void* W, void* W_out, int out_s, hipStream_t st) {
  if (g.dtype == LORA_BF16 && g.R <= 128) {
    // row blocks per workgroup: enough that about 512 workgroups (two per
    // compute unit) share the weight, at most 8
    const int ncb = (g.K + kMrCols - 1) / kMrCols, nrb = (out_s + kMrRows - 1) / kMrRows;
    int nblk = (int)std::max<int64_t>(1, std::min<int64_t>(8, (int64_t)nrb * ncb / 512));
    if (const char* e = std::getenv("LORA_MERGE_NBLK")) {  // tuning override
      const long o = std::strtol(e, nullptr, 10);
      if (o >= 1 && o <= 64) nblk = (int)o;
    }
    const dim3 grid(ncb, (nrb + nblk - 1) / nblk);
    const uint16_t* A16 = (const uint16_t*)A_slot_slice;
    const uint16_t* B16 = (const uint16_t*)B_slot_slice;
    switch ((g.R + 31) / 32) {
      case 1:
        hipLaunchKernelGGL(merge_rows_kernel<1>, grid, dim3(256), 0, st, A16, B16,
                           (const uint16_t*)W, (uint16_t*)W_out, g.R, g.K, out_s, nblk);
        break;
      case 2:
        hipLaunchKernelGGL(merge_rows_kernel<2>, grid, dim3(256), 0, st, A16, B16,
                           (const uint16_t*)W, (uint16_t*)W_out, g.R, g.K, out_s, nblk);
        break;
      case 3:
        hipLaunchKernelGGL(merge_rows_kernel<3>, grid, dim3(256), 0, st, A16, B16,
                           (const uint16_t*)W, (uint16_t*)W_out, g.R, g.K, out_s, nblk);
        break;
      default:
        hipLaunchKernelGGL(merge_rows_kernel<4>, grid, dim3(256), 0, st, A16, B16,
                           (const uint16_t*)W, (uint16_t*)W_out, g.R, g.K, out_s, nblk);
        break;
    }
  } else if (g.dtype == LORA_BF16) {
    const dim3 grid((g.K + kTileK - 1) / kTileK, (out_s + kTileO - 1) / kTileO);
    hipLaunchKernelGGL(merge_mfma_kernel, grid, dim3(256), merge_lds_bytes(g.R), st,
                       (const uint16_t*)A_slot_slice, (const uint16_t*)B_slot_slice,
                       (const uint16_t*)W, (uint16_t*)W_out, g.R, g.K, out_s);
  } else {
    const dim3 grid((g.K / 4 + 255) / 256, (unsigned)(out_s < 65535 ? out_s : 65535));
    hipLaunchKernelGGL(merge_f32_kernel, grid, dim3(256), 0, st, (const float*)A_slot_slice,
                       (const float*)B_slot_slice, (const float*)W, (float*)W_out, g.R, g.K,
                       out_s);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LORA_E_HIP, "merge launch: %s", hipGetErrorString(e));
  return LORA_OK;
}

}  // namespace lora

extern "C" int32_t lora_merge_weights(const lora_pool_desc* desc, const void* A_pool,
                                      const void* B_pool, int32_t slot, int32_t slice,
                                      const void* W, void* W_out, void* stream) {
  using namespace lora;
  clear_error();
  Geo g;
  if (int32_t e = check_desc(desc, &g)) return e;
  if (!A_pool || !B_pool || !W || !W_out)
    return fail(LORA_E_ARG, "A_pool, B_pool, W and W_out must not be NULL");
  if (slot < 0 || slot >= g.max_loras)
    return fail(LORA_E_ID, "slot %d is outside [0, %d)", slot, g.max_loras);
  if (slice < 0 || slice >= g.S) return fail(LORA_E_ID, "slice %d is outside [0, %d)", slice, g.S);
  if (g.R > LORA_MERGE_MAX_RANK)
    return fail(LORA_E_RANK, "merge supports max_lora_rank <= %d, got %d", LORA_MERGE_MAX_RANK,
                g.R);
  if (!aligned16(A_pool) || !aligned16(B_pool) || !aligned16(W) || !aligned16(W_out))
    return fail(LORA_E_ALIGN, "A_pool, B_pool, W and W_out must be 16-byte aligned");
  const int64_t eb = elem_bytes(g.dtype);
  const int out_s = g.out[slice];
  const int64_t wbytes = (int64_t)out_s * g.K * eb;
  const char* w = (const char*)W;
  const char* wo = (const char*)W_out;
  if (w != wo && w < wo + wbytes && wo < w + wbytes)
    return fail(LORA_E_ARG, "W and W_out overlap without being the same buffer");
  const char* Ad = (const char*)A_pool + ((int64_t)slot * g.S + slice) * g.R * (int64_t)g.K * eb;
  const char* Bd = (const char*)B_pool + ((int64_t)slot * g.O + g.off[slice]) * (int64_t)g.R * eb;
  return run_merge(g, Ad, Bd, W, W_out, out_s, (hipStream_t)stream);
}
