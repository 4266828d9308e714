// gemm_tile.hpp -- the LDS-pipelined MFMA tile kernel for gfx950.
//
// One workgroup (256 threads = 4 waves of 64) computes a BM x BN tile of C.
// Per k-step of 64:
//   global -> registers   128-bit loads, coalesced along the operand's
//                         contiguous index;
//   registers -> LDS      into the stage not being read, with an XOR swizzle
//                         of 16-byte chunks so that MFMA operand reads and the
//                         stores hit distinct banks;
//   LDS -> MFMA           each wave owns a (BM/2) x (BN/2) sub-tile made of
//                         32x32 blocks and issues v_mfma_f32_32x32x16_{f16,bf16}
//                         with fp32 accumulators.
// Two LDS stages plus one register stage form a three-deep software pipeline:
// while the waves multiply stage s, the loads for the next-but-one k-step are
// in flight and the next k-step is being written into stage s^1.  One
// workgroup barrier per k-step.
//
// After the k loop the epilogue (bias add, then ReLU or GELU) runs on the
// fp32 accumulators and each lane writes four consecutive outputs of one row
// with one vector store: the kernel never writes an intermediate tensor.
// (Tile-level fusion of load -> GEMM -> activation -> store: TileFusion
// "基础GEMM示例"; epilogue on the fragment before write-back: csdn
// "从零开始学习 TileLang" ch.10 sec. 10.8; block rasterisation for L2 reuse:
// atlascloud.ai "Writing high-performance kernels in TileLang", section
// "Écrivons un GEMM".)
//
// Both operands reach LDS in one layout: rows along M (for A) or N (for B),
// 64 k values per row, k contiguous.  An operand whose k index is contiguous
// in memory (A row-major, B column-major) is copied 16 bytes at a time.  An
// operand whose M/N index is contiguous (A column-major, B row-major) is
// loaded as 8-wide rows along M/N for several k, transposed in registers,
// and written k-contiguous.
//
// The MFMA is issued with B's fragment as the first operand and A's as the
// second, so the 32x32 result block arrives transposed: lane l holds
// C[m = l % 32][n = 8q + 4(l / 32) + e] for q, e in 0..3, i.e. four
// consecutive columns of one row -- the shape of one vector store.
#pragma once

#include "kernels.hpp"

namespace ge {
namespace tile {

constexpr int kBK = 64;             // k extent of one stage
constexpr int kRowBytes = kBK * 2;  // one LDS row: 64 16-bit elements
constexpr int kThreads = 256;

// 16-byte chunk c of LDS row r is stored at chunk position c ^ swz(r).
// Operand reads: the 16 lanes of a quarter-wave read 16 consecutive rows at
// one logical chunk; swz maps them to 8 distinct positions for rows r..r+7
// and, as rows r and r+1 sit 128 B apart, to 16 distinct 16-byte bank
// groups over 16 rows.  Transposed writes: 8 lanes write rows 8t + j
// (t = 0..7) and get positions c ^ j ^ t, again distinct.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <int R, bool KMAJ>
struct Loader;

// k-contiguous operand: row r of the tile is X[(r0 + r) * ld + k].
template <int R>
struct Loader<R, true> {
  static constexpr int CH = R * kBK / 8 / kThreads;  // 16-byte chunks per thread
  const char* g;
  int64_t chunk_row_step;  // bytes between this thread's consecutive chunks (32 rows)
  u32x4 r[CH];

  __device__ __forceinline__ Loader(const void* X, int r0, int ld, int tid) {
    g = (const char*)X + ((int64_t)(r0 + (tid >> 3)) * ld + (tid & 7) * 8) * 2;
    chunk_row_step = (int64_t)32 * ld * 2;
  }
  __device__ __forceinline__ void load(int kt) {
    const char* p = g + (int64_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < CH; ++i) r[i] = *(const u32x4*)(p + i * chunk_row_step);
  }
  __device__ __forceinline__ void store(char* s, int tid) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = i * 32 + (tid >> 3);
      *(u32x4*)(s + row * kRowBytes + (((tid & 7) ^ swz(row)) << 4)) = r[i];
    }
  }
};

// M/N-contiguous operand: row r of the tile (an M or N index) at k is
// X[k * ld + r0 + r].  Each thread loads KB k-rows of 8 consecutive M/N
// values and writes, for each of the 8, its KB k-values contiguously.
template <int R>
struct Loader<R, false> {
  static constexpr int KB = R / 32;  // k values per thread: 8, 4 or 2
  static constexpr int NG = R / 8;   // 8-wide groups along M/N
  static_assert(KB >= 2 && KB <= 8, "tile extent");
  const char* g;
  int64_t kstep;  // bytes between consecutive k rows
  int ng, kg;
  u32x4 r[KB];

  __device__ __forceinline__ Loader(const void* X, int r0, int ld, int tid) {
    ng = tid % NG;
    kg = tid / NG;
    kstep = (int64_t)ld * 2;
    g = (const char*)X + ((int64_t)kg * KB * ld + r0 + ng * 8) * 2;
  }
  __device__ __forceinline__ void load(int kt) {
    const char* p = g + (int64_t)kt * kBK * kstep;
#pragma unroll
    for (int i = 0; i < KB; ++i) r[i] = *(const u32x4*)(p + i * kstep);
  }
  // 16-bit element j (0..7) of a 128-bit register
  static __device__ __forceinline__ uint32_t half_of(const u32x4& v, int j) {
    const uint32_t w = v[j >> 1];
    return (j & 1) ? (w >> 16) : (w & 0xffffu);
  }
  __device__ __forceinline__ void store(char* s, int) const {
    const int k0 = kg * KB;
    const int c = k0 >> 3;
    const int inner = (k0 & 7) * 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = ng * 8 + j;
      char* dst = s + row * kRowBytes + ((c ^ swz(row)) << 4) + inner;
      uint32_t w[KB / 2];
#pragma unroll
      for (int e = 0; e < KB / 2; ++e) w[e] = half_of(r[2 * e], j) | (half_of(r[2 * e + 1], j) << 16);
      if constexpr (KB == 8) *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
      else if constexpr (KB == 4) *(u32x2*)dst = u32x2{w[0], w[1]};
      else *(uint32_t*)dst = w[0];
    }
  }
};

// Tile id -> (tile_m, tile_n).  Workgroups are handed to the 8 XCDs round
// robin (id % 8), so ids are first renumbered to make each XCD's share a
// contiguous run; that run is then laid out in panels of `panel` tile-rows,
// column by column, so the tiles one XCD runs together share A rows and B
// columns in its L2.
__device__ __forceinline__ void raster(int bid, int tiles_m, int tiles_n, int panel, int& tm, int& tn) {
  const int G = tiles_m * tiles_n;
  int lw = bid;
  if ((G & 7) == 0) lw = (bid & 7) * (G >> 3) + (bid >> 3);
  const int per_panel = panel * tiles_n;
  const int p = lw / per_panel;
  const int r = lw - p * per_panel;
  const int rows = min(panel, tiles_m - p * panel);
  tm = p * panel + r % rows;
  tn = r / rows;
}

template <int BM, int BN, typename TIn, typename TOut, int EPI>
__device__ __forceinline__ void write_tile(const f32x16 (&acc)[BM / 64][BN / 64], const TIn* __restrict__ bias,
                                          TOut* __restrict__ C, int N, int m_w, int n_w, int lane) {
  constexpr int TM = BM / 64, TN = BN / 64;
  const int m_l = lane & 31;
  const int n_l = 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    f32x4 b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (epi_has_bias<EPI>()) b[q] = load_bias4<TIn>(bias + n_w + j * 32 + 8 * q + n_l);
      else b[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      TOut* row = C + (int64_t)(m_w + i * 32 + m_l) * N + n_w + j * 32 + n_l;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        store4<TOut>(row + 8 * q, epilogue<EPI>(acc[i][j][4 * q + 0], b[q].x),
                     epilogue<EPI>(acc[i][j][4 * q + 1], b[q].y), epilogue<EPI>(acc[i][j][4 * q + 2], b[q].z),
                     epilogue<EPI>(acc[i][j][4 * q + 3], b[q].w));
      }
    }
  }
}

template <int BM, int BN, typename TIn, typename TOut, bool A_KMAJ, bool B_KMAJ>
__global__ __launch_bounds__(kThreads) void gemm_tile_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                             const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                             int M, int N, int K, int epi, int tiles_m, int tiles_n,
                                                             int panel) {
  constexpr int WM = BM / 2, WN = BN / 2;  // wave sub-tile
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  constexpr int STAGE = A_BYTES + B_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  raster(blockIdx.x, tiles_m, tiles_n, panel, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  Loader<BM, A_KMAJ> la(A, m0, A_KMAJ ? K : M, tid);
  Loader<BN, B_KMAJ> lb(B, n0, B_KMAJ ? K : N, tid);

  // Per-lane LDS read offsets.  Fragment i of a wave's operand covers rows
  // w0 + 32 i + (lane % 32), logical chunk 2 kk + lane / 32 for k-substep kk.
  const int f_lane = (lane & 7) ^ ((lane & 31) >> 3);
  int sw[4][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int p = 0; p < 2; ++p) sw[kk][p] = (((2 * kk + (lane >> 5)) ^ f_lane ^ (4 * p)) << 4);
  const int a_row = (wm * WM + (lane & 31)) * kRowBytes;
  const int b_row = (wn * WN + (lane & 31)) * kRowBytes;
  const int a_par = (wm * WM / 32) & 1;
  const int b_par = (wn * WN / 32) & 1;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int KT = K / kBK;
  la.load(0);
  lb.load(0);
  la.store(smem, tid);
  lb.store(smem + A_BYTES, tid);
  if (KT > 1) {
    la.load(1);
    lb.load(1);
  }
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const char* sa = smem + (kt & 1) * STAGE;
    const char* sb = sa + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *(const u32x4*)(sa + a_row + i * 32 * kRowBytes + sw[kk][(a_par + i) & 1]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = *(const u32x4*)(sb + b_row + j * 32 * kRowBytes + sw[kk][(b_par + j) & 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32<TIn>(bf[j], af[i], acc[i][j]);
    }
    if (kt + 1 < KT) {
      char* na = smem + ((kt + 1) & 1) * STAGE;
      la.store(na, tid);
      lb.store(na + A_BYTES, tid);
      if (kt + 2 < KT) {
        la.load(kt + 2);
        lb.load(kt + 2);
      }
    }
    __syncthreads();
  }

  const int m_w = m0 + wm * WM, n_w = n0 + wn * WN;
  switch (epi) {
    case GEMM_EPI_NONE: write_tile<BM, BN, TIn, TOut, GEMM_EPI_NONE>(acc, bias, C, N, m_w, n_w, lane); break;
    case GEMM_EPI_RELU: write_tile<BM, BN, TIn, TOut, GEMM_EPI_RELU>(acc, bias, C, N, m_w, n_w, lane); break;
    case GEMM_EPI_BIAS_RELU: write_tile<BM, BN, TIn, TOut, GEMM_EPI_BIAS_RELU>(acc, bias, C, N, m_w, n_w, lane); break;
    case GEMM_EPI_BIAS_GELU: write_tile<BM, BN, TIn, TOut, GEMM_EPI_BIAS_GELU>(acc, bias, C, N, m_w, n_w, lane); break;
    default: write_tile<BM, BN, TIn, TOut, GEMM_EPI_BIAS>(acc, bias, C, N, m_w, n_w, lane); break;
  }
}

// Host launch of one instantiation.
template <int BM, int BN, typename TIn, typename TOut, bool A_KMAJ, bool B_KMAJ>
hipError_t launch(const LaunchArgs& a) {
  const int tiles_m = a.M / BM, tiles_n = a.N / BN;
  const int panel = tiles_m < 4 ? tiles_m : 4;
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, TIn, TOut, A_KMAJ, B_KMAJ>), dim3(tiles_m * tiles_n), dim3(kThreads), 0,
                     a.stream, (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K, a.epi,
                     tiles_m, tiles_n, panel);
  return hipGetLastError();
}

template <int BM, int BN, typename TIn, typename TOut>
LaunchFn pick_layout(int la, int lb) {
  const bool ak = la == GEMM_EPI_ROW_MAJOR, bk = lb == GEMM_EPI_COL_MAJOR;
  if (ak && bk) return &launch<BM, BN, TIn, TOut, true, true>;
  if (ak && !bk) return &launch<BM, BN, TIn, TOut, true, false>;
  if (!ak && bk) return &launch<BM, BN, TIn, TOut, false, true>;
  return &launch<BM, BN, TIn, TOut, false, false>;
}

}  // namespace tile

}  // namespace ge
