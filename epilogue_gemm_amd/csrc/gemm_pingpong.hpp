// gemm_pingpong.hpp -- 256x256 MFMA tile kernel with two wave groups that
// take turns: while one group runs a k-step's MFMAs back to back from
// registers, the other reads its fragments from LDS (and group 0 copies
// the next tile global -> LDS).  Operands must be k-contiguous (A row-major,
// B column-major) and K a multiple of 128.
//
// In the two-stage kernel (gemm_tile.hpp) every wave interleaves its MFMAs
// with its own LDS reads and global->LDS copies, and all waves meet at the
// same barrier, so a stall in the memory path stops every MFMA pipe at
// once.  Here the 8 waves form two groups of 4, one wave of each group per
// SIMD: group g owns output rows 128 g .. 128 g + 127 of the tile and each
// of its waves a 128 x 64 block (4 x 2 MFMA blocks of 32 x 32).  Time is
// cut into phases separated by workgroup barriers:
//
//   phase 2t      group 0: the 32 MFMAs of k-step t       group 1: read k-step t's fragments
//   phase 2t + 1  group 0: copy tile t+2 into the stage    group 1: the 32 MFMAs of k-step t
//                          of tile t, read k-step t+1's
//                          fragments
//
// so on every SIMD one wave multiplies while the other moves data.  A wave
// holds a whole k-step's fragments (16 of A, 8 of B: 96 VGPRs) next to its
// 128 accumulators.  A tile's copies have about two phases to land.
//
// LDS layout, swizzle, direct copies and epilogue are those of
// gemm_tile.hpp.  (Software pipelining of the k loop: atlascloud.ai
// "Writing high-performance kernels in TileLang", section "Écrivons un
// GEMM"; epilogue on the accumulator fragment: csdn "从零开始学习
// TileLang" ch.10 sec. 10.8.)
#pragma once

#include "gemm_tile.hpp"

namespace ge {
namespace pingpong {

using tile::DirectLoader;
using tile::kRowBytes;

constexpr int kBM = 256, kBN = 256;
constexpr int kOp = kBM * kRowBytes;  // one operand of one stage: 32 KiB

template <typename TIn, typename TOut, int EPI>
__global__ __launch_bounds__(512) void gemm_pingpong_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                            const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                            int M, int N, int K, int tiles_m, int tiles_n,
                                                            int panel) {
  constexpr int WM = 128, WN = 64;   // one wave's block
  constexpr int TM = 4, TN = 2;      // 32 x 32 MFMA blocks in it
  constexpr int NI = DirectLoader<kBM, 4>::NI;  // copies per operand per group-0 wave per k-step

  __shared__ __attribute__((aligned(1024))) char sA0[kOp];
  __shared__ __attribute__((aligned(1024))) char sA1[kOp];
  __shared__ __attribute__((aligned(1024))) char sB0[kOp];
  __shared__ __attribute__((aligned(1024))) char sB1[kOp];
  struct Stage {
    char* a;
    char* b;
  };
  const Stage stage0{sA0, sB0}, stage1{sA1, sB1};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, w4 = wave & 3;

  int tm, tn;
  tile::raster(blockIdx.x, tiles_m, tiles_n, panel, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int KT = K / tile::kBK;  // even (checked on the host)

  // group 0's four waves copy both operands
  const DirectLoader<kBM, 4> da(A, m0, M, K, lane, w4);
  const DirectLoader<kBN, 4> db(B, n0, N, K, lane, w4);

  // Fragment f of k-substep kk: rows w0 + 32 f + lane % 32, logical chunk
  // 2 kk + lane / 32; the swizzle of those rows is f_lane ^ 4 ((w0/32 + f) & 1),
  // and w0 / 32 is even for A (w0 = 128 g) and for B (w0 = 64 w).
  const int a_row = (grp * WM + (lane & 31)) * kRowBytes;
  const int b_row = (w4 * WN + (lane & 31)) * kRowBytes;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // a whole k-step's fragments
  u32x4 fa[4][TM], fb[4][TN];

  // The swizzled offsets are recomputed from the lane index at every read
  // phase (the empty asm hides that the index does not change), so they
  // occupy registers only while the reads are issued: next to the
  // accumulators and a k-step of fragments there is no room to keep them.
  auto read_all = [&](const Stage& st) __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    const int f_l = ((l & 7) ^ ((l & 31) >> 3) ^ (l >> 5)) << 4;
    const int ra = a_row + f_l, rb = b_row + f_l;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // (2 kk + lane / 32) ^ f_lane ^ 4 p, times 16: lane / 32 is already in f_l
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[kk][i] = *(const u32x4*)(st.a + (ra ^ ((2 * kk ^ 4 * (i & 1)) << 4)) + i * 32 * kRowBytes);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[kk][j] = *(const u32x4*)(st.b + (rb ^ ((2 * kk ^ 4 * (j & 1)) << 4)) + j * 32 * kRowBytes);
    }
  };
  auto multiply = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32<TIn>(fb[kk][j], fa[kk][i], acc[i][j]);
  };
  auto copy = [&](const Stage& st, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      da.issue(st.a, kt, i);
      db.issue(st.b, kt, i);
    }
  };
  // Workgroup barrier fenced on both sides: no instruction is scheduled
  // across it, and (memory clobber) no memory access is moved across it.
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // Both groups run the same sequence -- read k-step t's fragments, then
  // multiply them -- group 1 one phase behind group 0; only the copies,
  // their waits and the barriers at the two ends depend on the group, so
  // the data registers follow one path.  Barriers, numbered per wave:
  // group 0 ends R(t) at 2 + 2t and X(t) at 3 + 2t, group 1 ends R(t) at
  // 3 + 2t and X(t) at 4 + 2t (its barrier 2 closes its idle first phase).
  // Hence group 0's X(t) meets group 1's R(t) and group 0's R(t+1) meets
  // group 1's X(t).
  //
  // Group 0 does the copies, at the start of its R(t): tile t+1 goes into
  // the stage of tile t-1, whose last reader (group 1's R(t-1)) ended at
  // the barrier before.  It waits for them at the end of X(t), before the
  // barrier after which both groups may read tile t+1.  MORE: there is a
  // tile t+1; LAST: group 1 has no barrier after its last multiply.
  auto step = [&](const Stage& cur, const Stage& nxt, int t, auto MORE_, auto LAST_)
                  __attribute__((always_inline)) {
    constexpr bool MORE = decltype(MORE_)::value != 0;
    constexpr bool LAST = decltype(LAST_)::value != 0;
    // R(t)
    if constexpr (MORE)
      if (grp == 0) copy(nxt, t + 1);
    __builtin_amdgcn_sched_barrier(0);
    read_all(cur);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads are in registers
    barrier();
    // X(t)
    multiply();
    // group 0: this wave's copies of tile t+1.  Group 1 has nothing in
    // flight, but waits too so that the compiler, which does not know which
    // group copied, sees every copy waited for on every path (else it
    // waits before the next reads, stalling group 0 on copies it just issued)
    __builtin_amdgcn_sched_barrier(0);  // the wait stays behind the MFMAs
    if constexpr (MORE) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if constexpr (LAST) {
      if (grp == 0) barrier();
    } else {
      barrier();
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // prologue: group 0 copies tile 0 and waits for it
  if (grp == 0) {
    copy(stage0, 0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  barrier();
  if (grp == 1) barrier();

  // K is a multiple of 128, so tile t sits in stage t % 2 and the last
  // tile in stage 1.
  step(stage0, stage1, 0, I1{}, I0{});
  for (int t = 1; t < KT - 1; t += 2) {
    step(stage1, stage0, t, I1{}, I0{});
    step(stage0, stage1, t + 1, I1{}, I0{});
  }
  step(stage1, stage0, KT - 1, I0{}, I1{});

  // Group 0 reaches this point while group 1 still multiplies its last
  // k-step; no wave reads the operand stages any more, so each wave takes a
  // private staging area there: wave w uses half w / 4 of array w % 4.
  char* const stage_w = (w4 == 0 ? sA0 : w4 == 1 ? sA1 : w4 == 2 ? sB0 : sB1) + grp * (kOp / 2);
  static_assert(32 * WN * sizeof(TOut) <= (size_t)kOp / 2, "staging area");
  tile::write_tile<WM, WN, TIn, TOut, EPI>(acc, bias, C, N, m0 + grp * WM, n0 + w4 * WN, lane, stage_w);
}

template <typename TIn, typename TOut, int EPI>
hipError_t launch(const LaunchArgs& a) {
  const int tiles_m = a.M / kBM, tiles_n = a.N / kBN;
  const int panel = tiles_m < 4 ? tiles_m : 4;
  hipLaunchKernelGGL((gemm_pingpong_kernel<TIn, TOut, EPI>), dim3(tiles_m * tiles_n), dim3(512), 0, a.stream,
                     (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K, tiles_m,
                     tiles_n, panel);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
LaunchFn pick(int la, int lb, int epi) {
  if (la != GEMM_EPI_ROW_MAJOR || lb != GEMM_EPI_COL_MAJOR) return nullptr;
  switch (epi) {
    case GEMM_EPI_NONE: return &launch<TIn, TOut, GEMM_EPI_NONE>;
    case GEMM_EPI_RELU: return &launch<TIn, TOut, GEMM_EPI_RELU>;
    case GEMM_EPI_BIAS_RELU: return &launch<TIn, TOut, GEMM_EPI_BIAS_RELU>;
    case GEMM_EPI_BIAS_GELU: return &launch<TIn, TOut, GEMM_EPI_BIAS_GELU>;
    case GEMM_EPI_BIAS: return &launch<TIn, TOut, GEMM_EPI_BIAS>;
    default: return nullptr;
  }
}

}  // namespace pingpong
}  // namespace ge
