// gemm_ring.hpp -- 256x256 MFMA tile kernel fed by a four-slot LDS ring of
// 32-deep k-steps, for operands whose k index is contiguous in memory
// (A row-major, B column-major).
//
// The two-stage kernel (gemm_tile.hpp) can only refill a 64-deep stage once
// every wave has finished reading it, so all of a k-step's global->LDS
// copies are issued in one quarter of the k-step; the texture path then
// backs up and the waves stall behind their own loads.  Here the tile is
// cut into 32-deep k-steps held in a ring of NS = 4 slots: while k-step t
// is multiplied from slot t % 4, slot (t + 1) % 4 holds the next tile,
// slot (t + 2) % 4 is landing, and slot (t + 3) % 4 -- read for the last
// time during k-step t - 1 -- receives tile t + 3.  Its copies are spread
// evenly over all 32 MFMA slots of the k-step, and each tile has about two
// k-steps between the issue of its copies and its first read.
//
// LDS: one row per M (A) or N (B) index, 32 k values = 64 bytes, 16-byte
// chunk c of row r stored at position c ^ ((r >> 2) & 3).  A 16-lane
// group of a fragment read takes one chunk of 16 consecutive rows: rows
// r and r + 4 fall on the same banks (256 bytes apart) and the swizzle
// gives them different positions, so the 16 reads hit 16 distinct 16-byte
// bank groups.  One direct 128-bit buffer load per wave fills 1 KiB = 16
// rows; lane L writes bytes 16 L .. 16 L + 15 of it, i.e. row L / 4 at
// position L % 4, so it fetches logical chunk (L % 4) ^ ((L >> 4) & 3).
//
// One workgroup barrier per k-step, between its two 16-deep substeps:
// after it, every wave's copies of tile t + 1 have landed (so substep 1
// may read its first fragments) and every wave has finished reading tile
// t - 1 (so copies into that slot may start).  Each wave waits only for
// its own copies of tile t + 1; those of t + 2 and half of t + 3 stay in
// flight (vector-memory operations complete in issue order).
//
// The 32x32x16 MFMA, the transposed accumulator layout and the epilogue
// are those of gemm_tile.hpp (write_tile).  Software pipelining across a
// ring of shared-memory stages: atlascloud.ai "Writing high-performance
// kernels in TileLang", section "Écrivons un GEMM" (pipelined k loop);
// epilogue on the accumulator fragment: csdn "从零开始学习 TileLang"
// ch.10 sec. 10.8.
#pragma once

#include "gemm_tile.hpp"

namespace ge {
namespace ring {

using tile::lds_ptr;
using tile::make_rsrc;

constexpr int kNS = 4;                   // ring slots
constexpr int kBK = 32;                  // k extent of one slot
constexpr int kRowBytes = kBK * 2;       // 64
constexpr int kBM = 256, kBN = 256;      // workgroup tile
constexpr int kOpBytes = kBM * kRowBytes;  // one operand in one slot: 16 KiB

template <int I>
using IC = std::integral_constant<int, I>;

// Direct global -> LDS copies of one k-contiguous operand: instruction i of
// wave w (of NW) fills tile rows (NW i + w) * 16 .. +15 of a slot.  The
// swizzle position depends on the lane only, so one per-lane offset serves
// every instruction and k-step.
template <int NW>
struct Copier {
  static constexpr int NI = kBM / (16 * NW);  // instructions per wave per k-step
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff;
  uint32_t step_i;  // bytes between the row blocks of consecutive instructions
  int wave;

  __device__ __forceinline__ Copier(const void* X, int r0, int rows_total, int ld, int lane, int wave_) {
    const char* base = (const char*)X + (int64_t)r0 * ld * 2;
    rsrc = make_rsrc(base, (uint32_t)((int64_t)(rows_total - r0) * ld * 2));
    wave = wave_;
    const int row = wave * 16 + (lane >> 2);
    voff = (uint32_t)(row * ld * 2 + (((lane & 3) ^ ((lane >> 4) & 3)) << 4));
    step_i = (uint32_t)(NW * 16 * ld * 2);
  }
  // instruction i of tile kt into the operand area `dst` of a slot
  __device__ __forceinline__ void issue(char* dst, int kt, int i) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + (NW * i + wave) * 1024), 16, voff,
                                             (uint32_t)i * step_i + (uint32_t)kt * kRowBytes, 0, 0);
  }
};

// vmcnt(VM) lgkmcnt(0), then the workgroup barrier
template <int VM>
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM) & ~(15 << 8));
  __builtin_amdgcn_s_barrier();
}

template <int NW, typename TIn, typename TOut, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_ring_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                             const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                             int M, int N, int K, int tiles_m, int tiles_n,
                                                             int panel) {
  // NW waves in a 2 x (NW / 2) grid, each owning a WM x WN sub-tile
  constexpr int WM = kBM / 2, WN = kBN / (NW / 2);
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int NMF = TM * TN;                // MFMAs per substep
  constexpr int NDR = TM + TN;                // fragment reads per substep
  constexpr int NI = Copier<NW>::NI;
  constexpr int NDL = 2 * NI;                 // copies per wave per k-step
  constexpr int NDH = NDL / 2;                // ... per substep
  static_assert(NMF >= NDR && NMF >= NDH, "slot schedule");

  // one array per operand and slot, so that every LDS access names its
  // slot statically and reads are never ordered behind copies into
  // another slot
  __shared__ __attribute__((aligned(1024))) char sA0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sA2[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sA3[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB2[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB3[kOpBytes];
  struct Slot {
    char* a;
    char* b;
  };
  auto slot_of = [&](auto S) -> Slot {
    constexpr int s = decltype(S)::value % kNS;
    if constexpr (s == 0) return Slot{sA0, sB0};
    else if constexpr (s == 1) return Slot{sA1, sB1};
    else if constexpr (s == 2) return Slot{sA2, sB2};
    else return Slot{sA3, sB3};
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);

  int tm, tn;
  tile::raster(blockIdx.x, tiles_m, tiles_n, panel, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  const Copier<NW> ca(A, m0, M, K, lane, wave);
  const Copier<NW> cb(B, n0, N, K, lane, wave);

  // Fragment i of a wave's operand: rows w0 + 32 i + lane % 32, logical
  // chunk 2 kk + lane / 32 for substep kk; the swizzle of those rows is
  // ((lane >> 2) & 3) whatever w0 and i.
  const int sw0 = (((lane >> 5) ^ ((lane >> 2) & 3)) << 4);
  const int sw1 = (((2 + (lane >> 5)) ^ ((lane >> 2) & 3)) << 4);
  const int a_row = (wm * WM + (lane & 31)) * kRowBytes;
  const int b_row = (wn * WN + (lane & 31)) * kRowBytes;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // fragments of substep 0 (fa0, fb0) and substep 1 (fa1, fb1)
  u32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  auto read_frag = [&](const Slot& s, int sw, int f, u32x4(&xa)[TM], u32x4(&xb)[TN]) __attribute__((always_inline)) {
    if (f < TM) xa[f] = *(const u32x4*)(s.a + a_row + f * 32 * kRowBytes + sw);
    else xb[f - TM] = *(const u32x4*)(s.b + b_row + (f - TM) * 32 * kRowBytes + sw);
  };
  auto copy = [&](const Slot& s, int kt, int d) __attribute__((always_inline)) {
    if (d < NI) ca.issue(s.a, kt, d);
    else cb.issue(s.b, kt, d - NI);
  };

  // k-step t, its tile in slot S.  LOAD: issue the copies of tile t + 3
  // into slot S + 3.  VMID: the vmcnt of the mid barrier (-1: no barrier,
  // the last k-step).  NEXT: read substep 0 of tile t + 1 from slot S + 1.
  auto kstep = [&](auto S, auto LOAD_, auto VMID_, auto NEXT_, int t) __attribute__((always_inline)) {
    constexpr bool LOAD = decltype(LOAD_)::value != 0;
    constexpr int VMID = decltype(VMID_)::value;
    constexpr bool NEXT = decltype(NEXT_)::value != 0;
    const Slot cur = slot_of(S);
    const Slot nxt = slot_of(IC<decltype(S)::value + 1>{});
    const Slot dst = slot_of(IC<decltype(S)::value + kNS - 1>{});
    // substep 0: multiply k 0..15, read k 16..31 of this tile
#pragma unroll
    for (int s = 0; s < NMF; ++s) {
      acc[s / TN][s % TN] = mfma32<TIn>(fb0[s % TN], fa0[s / TN], acc[s / TN][s % TN]);
      if (s < NDR) read_frag(cur, sw1, s, fa1, fb1);
      if constexpr (LOAD) {
#pragma unroll
        for (int d = 0; d < NDH; ++d)
          if (d * NMF / NDH == s) copy(dst, t + kNS - 1, d);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (VMID >= 0) ring_barrier<VMID>();
    __builtin_amdgcn_sched_barrier(0);
    // substep 1: multiply k 16..31, read k 0..15 of the next tile
#pragma unroll
    for (int s = 0; s < NMF; ++s) {
      acc[s / TN][s % TN] = mfma32<TIn>(fb1[s % TN], fa1[s / TN], acc[s / TN][s % TN]);
      if constexpr (NEXT)
        if (s < NDR) read_frag(nxt, sw0, s, fa0, fb0);
      if constexpr (LOAD) {
#pragma unroll
        for (int d = 0; d < NDH; ++d)
          if (d * NMF / NDH == s) copy(dst, t + kNS - 1, NDH + d);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // K is a multiple of 4 k-steps, so tile t sits in slot t % 4 and the
  // loop runs whole turns of the ring; the last turn is peeled.
  const int KT = K / kBK;

  // prologue: tiles 0, 1, 2 in flight; wait for tile 0
  static_for<kNS - 1>([&](auto U) {
    const Slot s = slot_of(U);
#pragma unroll
    for (int d = 0; d < NDL; ++d) copy(s, decltype(U)::value, d);
  });
  ring_barrier<(kNS - 2) * NDL>();
#pragma unroll
  for (int f = 0; f < NDR; ++f) read_frag(slot_of(IC<0>{}), sw0, f, fa0, fb0);

  // steady state: the mid barrier waits for tile t + 1; tile t + 2 and the
  // first half of tile t + 3 may stay in flight
  constexpr int V_STEADY = (kNS - 2) * NDL - NDH;
  int t = 0;
  for (; t + 2 * kNS <= KT; t += kNS) {
    static_for<kNS>([&](auto S) { kstep(S, IC<1>{}, IC<V_STEADY>{}, IC<1>{}, t + decltype(S)::value); });
  }
  // last turn: only its first k-step copies (the last tile); then nothing
  // remains in flight after the third
  kstep(IC<0>{}, IC<1>{}, IC<V_STEADY>{}, IC<1>{}, t);
  kstep(IC<1>{}, IC<0>{}, IC<NDL>{}, IC<1>{}, t + 1);
  kstep(IC<2>{}, IC<0>{}, IC<0>{}, IC<1>{}, t + 2);
  kstep(IC<3>{}, IC<0>{}, IC<-1>{}, IC<0>{}, t + 3);

  // Every wave is done with the ring: reuse slot arrays as the per-wave
  // staging areas of the epilogue (one 16 KiB array each).
  __syncthreads();
  static_assert(NW <= 8 && 32 * WN * sizeof(TOut) <= (size_t)kOpBytes, "staging area");
  char* const stage_w = wave == 0   ? sA0
                        : wave == 1 ? sA1
                        : wave == 2 ? sA2
                        : wave == 3 ? sA3
                        : wave == 4 ? sB0
                        : wave == 5 ? sB1
                        : wave == 6 ? sB2
                                    : sB3;
  tile::write_tile<WM, WN, TIn, TOut, EPI>(acc, bias, C, N, m0 + wm * WM, n0 + wn * WN, lane, stage_w);
}

template <int NW, typename TIn, typename TOut, int EPI>
hipError_t launch(const LaunchArgs& a) {
  const int tiles_m = a.M / kBM, tiles_n = a.N / kBN;
  const int panel = tiles_m < 4 ? tiles_m : 4;
  hipLaunchKernelGGL((gemm_ring_kernel<NW, TIn, TOut, EPI>), dim3(tiles_m * tiles_n), dim3(NW * 64), 0, a.stream,
                     (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K, tiles_m,
                     tiles_n, panel);
  return hipGetLastError();
}

// Only A row-major with B column-major (both k-contiguous) is served.
template <int NW, typename TIn, typename TOut>
LaunchFn pick(int la, int lb, int epi) {
  if (la != GEMM_EPI_ROW_MAJOR || lb != GEMM_EPI_COL_MAJOR) return nullptr;
  switch (epi) {
    case GEMM_EPI_NONE: return &launch<NW, TIn, TOut, GEMM_EPI_NONE>;
    case GEMM_EPI_RELU: return &launch<NW, TIn, TOut, GEMM_EPI_RELU>;
    case GEMM_EPI_BIAS_RELU: return &launch<NW, TIn, TOut, GEMM_EPI_BIAS_RELU>;
    case GEMM_EPI_BIAS_GELU: return &launch<NW, TIn, TOut, GEMM_EPI_BIAS_GELU>;
    case GEMM_EPI_BIAS: return &launch<NW, TIn, TOut, GEMM_EPI_BIAS>;
    default: return nullptr;
  }
}

}  // namespace ring
}  // namespace ge
