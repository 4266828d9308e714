// gemm_ring.hpp -- the small-tile GEMM with a deep LDS ring: 64 x 64 tiles of
// C for problems too small to give 256 CUs big tiles (1024^3: 256 tiles of
// 64 x 64, one per CU), where the two-stage pipeline of gemm_tile.hpp is
// bound by load latency: a 64-deep k-step of a 64 x 64 tile is 4 MFMAs per
// wave, about 60 ns, while a copy that misses L2 takes a microsecond or
// more, so every k-step would wait for its copies.  Here K is walked in
// chunks of 64 through a ring of P LDS slots: while chunk c is multiplied,
// chunks c+1 .. c+P-1 are in flight (with P = 8, 112 KiB per CU), and the
// latency is paid about once instead of once per k-step.
//
// Per slot: A's 64 rows x 64 k (8 KiB, k contiguous, 16-byte chunks of a row
// at position c ^ swz(row)) and B's 64 columns x 64 k (8 KiB): for a
// column-major B (k contiguous) the same layout as A; for a row-major B (n
// contiguous) 64 k-rows of 64 n, chunk c of k-row k at position
// c ^ 2 (k & 3).  Both are filled by direct buffer_load ... lds copies, each
// wave instruction one KiB of 8 rows (DirectLoader for the k-contiguous
// operands, the same scheme along k-rows for the row-major B).
//
// Four waves in a 2 x 2 grid, each owning a 32 x 32 block of the tile and
// all of K: v_mfma_f32_32x32x16 with B's fragment as the first operand (so
// the result arrives transposed, as write_tile expects: lane l holds
// C[l % 32][8 q + 4 (l / 32) + e]).  A's fragment (row 32 wm + l % 32,
// k-chunk 2 q + l / 32) is one 16-byte read under swz (measured free of
// bank conflicts).  A row-major B's fragment -- eight consecutive k of one
// column n per lane -- comes from two transposing reads ds_read_b64_tr_b16:
// in each 16-lane group, lane s = 4 i + a gives the address of columns
// nb + 4 a .. + 3 of k-row kb + i, and lane j = 4 a + b receives column
// nb + j at k-rows kb .. kb + 3; under the c ^ 2 (k & 3) layout the 16 lanes
// of a read touch 8 distinct 16-byte bank groups, each as two 8-byte halves.
//
// Synchronisation is the ring's: chunk c sits in slot c % P (the chunk
// count is a multiple of P, or odd with P = 2, where the one chunk past the
// last whole turn has a code path of its own; so every slot index is a
// compile-time constant;
// one __shared__ object per slot, so the compiler can tell a read of one
// slot from a copy in flight into another); one barrier per chunk, after each
// wave's s_waitcnt on its own copies of that chunk, makes the slot complete
// and proves every wave is past the previous chunk, whose slot then receives
// chunk c + P - 1.  K not a multiple of 64: the k axis is shifted by
// kpad = 64 - K % 64 so that chunk 0 is the partial one and its positions
// k < 0 load as zeros.  The last tile row and column
// are shifted back to end at M and N (they recompute part of a neighbour
// with the same k order, so with identical values); a problem with fewer
// than 64 rows or columns takes one tile there, masked past the end.  With
// A column-major the last tile row is not shifted (its first row would not
// fall on a 16-byte chunk when M % 8 != 0) but masked past M; likewise the
// last tile column when N % 8 != 0 or C's rows are not 16-byte aligned
// (RAG), whose edge outputs the epilogue then handles element by element.  (Pipelined tile copies and block rasterisation:
// atlascloud.ai "Writing high-performance kernels in TileLang", section
// "Écrivons un GEMM"; epilogue on the accumulator fragment: csdn
// "从零开始学习 TileLang" ch.10 sec. 10.8; small problems that leave the
// GPU's cores idle: same tutorial, ch.17 sec. 17.3.)
#pragma once

#include "gemm_tile.hpp"

namespace ge {
namespace ring {

using tile::DirectLoader;
using tile::kBK;
using tile::kRowBytes;
using tile::lds_ptr;
using tile::swz;

constexpr int kTile = 64;                   // BM = BN
constexpr int kNW = 4;                      // waves
constexpr int kOpBytes = kTile * kRowBytes;  // 8 KiB: one operand's share of a slot

// One __shared__ object per slot, A's 8 KiB then B's.  (The compiler keeps
// apart the LDS objects that direct copies in flight are writing, so that a
// read of another object need not wait for them, only for a limited number
// of objects -- with one object per operand and slot, the 14 of seven
// chunks in flight exceeded it and every ring turn began with a wait for all
// copies; seven objects stay within it.)
template <int J>
__device__ __forceinline__ char* slot_obj() {
  __shared__ __attribute__((aligned(1024))) char s[2 * kOpBytes];
  return s;
}
template <int P, int... J>
__device__ __forceinline__ void slots(char* (&sa)[P], char* (&sb)[P], std::integer_sequence<int, J...>) {
  ((sa[J] = slot_obj<J>()), ...);
  ((sb[J] = slot_obj<J>() + kOpBytes), ...);
}

// Chunk in the oldest slot complete: each wave has at most PENDING of its
// own copies outstanding, then all waves meet (the empty asm statements keep
// the compiler from moving LDS accesses across the barrier).
template <int PENDING>
__device__ __forceinline__ void arrive() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(PENDING) & ~(15 << 8));  // vmcnt(PENDING) lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Row-major B (K x N, n contiguous) into a slot: 64 k-rows of the tile's 64
// columns, 128 bytes each.  (A column-major A, M x K with m contiguous, is
// loaded the same way with m for n: 64 k-rows of the tile's 64 rows.)  Instruction t (of 8, wave w issues t = w and
// w + 4) fills k-rows 8 t .. 8 t + 7: lane L takes k-row 8 t + L / 8 and
// lands at chunk position L % 8, so it loads n-chunk (L % 8) ^ 2 ((L / 8) & 3)
// of that k-row (8 t is a multiple of 4, so the swizzle depends on L only).
struct RowBLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff;      // lane's offset within an instruction's 8 k-rows
  uint32_t row_bytes;  // ldb * 2
  int wave, lane;

  __device__ __forceinline__ RowBLoader(const void* B, int n0, int N, int K, int ldb, int kpad, int lane_,
                                        int wave_) {
    // base at k = -kpad, column n0; the range ends with the last k-row
    const char* base = (const char*)B + (int64_t)n0 * 2 - (int64_t)kpad * ldb * 2;
    rsrc = tile::make_rsrc(base, (uint32_t)((int64_t)(K + kpad) * ldb * 2 - (int64_t)n0 * 2));
    row_bytes = (uint32_t)ldb * 2u;
    lane = lane_;
    wave = wave_;
    const int chunk = (lane & 7) ^ (2 * ((lane >> 3) & 3));
    voff = (uint32_t)(lane >> 3) * row_bytes + (uint32_t)(chunk << 4);
    // columns past N load nothing (N < 64, or the unshifted last tile row
    // of a column-major A: a chunk that starts before N is loaded whole,
    // its tail from the padding of a leading dimension that is a multiple
    // of 8, and feeds only outputs that are not stored)
    if (n0 + 8 * chunk >= N) voff = 0xFFFFFFF0u;
  }
  // instruction i (0, 1) of chunk kt
  __device__ __forceinline__ void issue(char* dst, int kt, int i) const {
    const int t = wave + kNW * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + t * 1024), 16, voff,
                                             (uint32_t)(kt * kBK + 8 * t) * row_bytes, 0, 0);
  }
  // chunk 0 when the k axis is shifted: k-rows below kpad load as zeros
  __device__ __forceinline__ void issue_first(char* dst, int i, int kpad) const {
    const int t = wave + kNW * i;
    const int row = 8 * t + (lane >> 3);
    const uint32_t v = row < kpad ? 0xFFFFFFF0u : voff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + t * 1024), 16, v, (uint32_t)(8 * t) * row_bytes, 0,
                                             0);
  }
};

template <typename TIn, typename TOut, int EPI, bool BROW, int P, bool ACOL, bool RAG>
__global__ __launch_bounds__(kNW * 64) void gemm_ring_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                             const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                             int M, int N, int K, int tiles_m, int tiles_n, int panel,
                                                             int lda, int ldb, int ldc,
                                                             const float* __restrict__ scale,
                                                             const TOut* __restrict__ res,
                                                             const float* __restrict__ out_scale) {
  static_assert(P >= 2 && P <= 9, "ring slots");
  constexpr int OPS = 4;  // copies per wave per chunk: two for A, two for B
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  tile::raster(blockIdx.x, tiles_m, tiles_n, panel, tm, tn);
  // A problem smaller than the tile (M or N below 64) is covered by one
  // tile row or column at 0, its rows or columns past the end loading
  // nothing and storing nothing (MASK below); a column-major A keeps its
  // last tile row in place, masked past M.
  const int m0 = ACOL ? tm * kTile : max(0, min(tm * kTile, M - kTile));
  const int n0 = RAG ? tn * kTile : max(0, min(tn * kTile, N - kTile));
  const int kpad = (-K) & (kBK - 1);
  const int nchunks = (K + kpad) / kBK;

  char* sa[P];
  char* sb[P];
  slots<P>(sa, sb, std::make_integer_sequence<int, P>{});

  const DirectLoader<kTile, kNW> da(A, m0, M, lda, kpad, tid, wave);
  const RowBLoader ra(A, m0, M, K, lda, kpad, lane, wave);  // A column-major
  // (only one of the two B movers is used)
  const DirectLoader<kTile, kNW> db(B, n0, N, ldb, kpad, tid, wave);
  const RowBLoader rb(B, n0, N, K, ldb, kpad, lane, wave);

  auto issue = [&](int j, int c) __attribute__((always_inline)) {
    if (c == 0 && kpad != 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (ACOL) ra.issue_first(sa[j], i, kpad);
        else da.issue_first(sa[j], i, lane, kpad);
        if constexpr (BROW) rb.issue_first(sb[j], i, kpad);
        else db.issue_first(sb[j], i, lane, kpad);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (ACOL) ra.issue(sa[j], c, i);
        else da.issue(sa[j], c, i);
        if constexpr (BROW) rb.issue(sb[j], c, i);
        else db.issue(sb[j], c, i);
      }
    }
  };

  // Fragment offsets.  A (and a column-major B): row 32 w + l % 32, chunk
  // 2 q + l / 32 at position (2 q + l / 32) ^ swz(row); swz(row) =
  // f ^ 4 ((w32 ... )), computed per q here (four reads per chunk).
  const int r32 = lane & 31, h = lane >> 5;
  int a_off[4], b_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ra = 32 * wm + r32, rbn = 32 * wn + r32;
    a_off[q] = ra * kRowBytes + (((2 * q + h) ^ swz(ra)) << 4);
    b_off[q] = rbn * kRowBytes + (((2 * q + h) ^ swz(rbn)) << 4);
  }
  // Row-major B: k-row 16 q + 8 h + i (+ 4 for the second read), columns
  // 32 wn + 16 g + 4 a .. + 3, i.e. n-chunk 4 wn + 2 g + a / 2 at position
  // chunk ^ 2 i, bytes 8 (a % 2) within it.
  const int s16 = lane & 15, ti = s16 >> 2, ta = s16 & 3, tg = (lane >> 4) & 1;
  const int tr_off = (8 * h + ti) * kRowBytes + (((4 * wn + 2 * tg + (ta >> 1)) ^ (2 * ti)) << 4) + 8 * (ta & 1);
  // column-major A: the same with the wave's rows 32 wm .. for its columns
  const int tr_off_a = (8 * h + ti) * kRowBytes + (((4 * wm + 2 * tg + (ta >> 1)) ^ (2 * ti)) << 4) + 8 * (ta & 1);

  f32x16 acc = f32x16{};
  // eight consecutive k of one row (column) per lane from a k-row layout:
  // two transposing reads, k-rows 16 q + 8 h + i and + 4
  auto read_tr = [&](const char* p0) __attribute__((always_inline)) {
    typedef short s4v __attribute__((vector_size(8)));
    typedef __attribute__((address_space(3))) s4v lds_s4v;
    const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(lds_ptr)p0);
    const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(lds_ptr)(p0 + 4 * kRowBytes));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };
  auto compute = [&](int j) __attribute__((always_inline)) {
    u32x4 a[4], b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (ACOL) a[q] = read_tr(sa[j] + 16 * q * kRowBytes + tr_off_a);
      else a[q] = *(const u32x4*)(sa[j] + a_off[q]);
      if constexpr (BROW) {
        b[q] = read_tr(sb[j] + 16 * q * kRowBytes + tr_off);
      } else {
        b[q] = *(const u32x4*)(sb[j] + b_off[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = mfma32<TIn>(b[q], a[q], acc);
  };

  // Chunk c lives in slot c % P (the chunk count is a multiple of P, or any
  // count for P = 2; checked on the host): one code path into the loop, so
  // that the compiler sees the same copies in flight on entry and around
  // the back edge and can tell every slot's copies apart.  Chunks 0 .. P-2
  // first.
  static_for<P - 1>([&](auto jc) __attribute__((always_inline)) {
    constexpr int jj = decltype(jc)::value;
    issue(jj, jj);
  });
  int c0 = 0;
  // whole turns of the ring
  for (; c0 + P < nchunks; c0 += P) {
    static_for<P>([&](auto jc) __attribute__((always_inline)) {
      constexpr int jj = decltype(jc)::value;
      arrive<OPS * (P - 2)>();
      issue((jj + P - 1) % P, c0 + jj + P - 1);
      compute(jj);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  // Two slots and an odd chunk count (K <= 64 among them): the loop has
  // issued the last chunk, into slot 0, and nothing follows it.  Either
  // way one chunk is in flight in slot 0 here.
  bool odd = false;
  if constexpr (P == 2) odd = (nchunks & 1) != 0;
  if (odd) {
    arrive<0>();
    compute(0);
  } else {
    // last P chunks: only the first still has a chunk to issue
    static_for<P>([&](auto jc) __attribute__((always_inline)) {
      constexpr int jj = decltype(jc)::value;
      if constexpr (jj == 0) {
        arrive<OPS * (P - 2)>();
        issue(P - 1, c0 + P - 1);
      } else {
        arrive<OPS * (P - 1 - jj)>();
      }
      compute(jj);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // Every wave is done with the ring: stage the epilogue in it (4 KiB per
  // wave at most: 32 rows x 32 fp32 outputs).
  __syncthreads();
  char* stage_w;
  if constexpr (P >= 4) stage_w = wave == 0 ? sa[0] : wave == 1 ? sa[1] : wave == 2 ? sa[2] : sa[3];
  else stage_w = (wave & 1 ? sa[1] : sa[0]) + (wave >> 1) * (kOpBytes / 2);
  static_assert(32 * 32 * sizeof(TOut) <= (size_t)kOpBytes / 2, "staging area");
  const f32x16 accs[1][1] = {{acc}};
  const int mw = m0 + 32 * wm, nw = n0 + 32 * wn;
  if constexpr (RAG)
    tile::write_tile<32, 32, TIn, TOut, EPI, true, true, true>(accs, bias, C, ldc, mw, nw, lane, stage_w, scale, res,
                                                               out_scale, M, N);
  else if (M < kTile || N < kTile || (ACOL && M % kTile != 0))
    tile::write_tile<32, 32, TIn, TOut, EPI, true, true>(accs, bias, C, ldc, mw, nw, lane, stage_w, scale, res,
                                                         out_scale, M, N);
  else if (scale != nullptr || res != nullptr || out_scale != nullptr)
    tile::write_tile<32, 32, TIn, TOut, EPI, true>(accs, bias, C, ldc, mw, nw, lane, stage_w, scale, res, out_scale);
  else
    tile::write_tile<32, 32, TIn, TOut, EPI, false>(accs, bias, C, ldc, mw, nw, lane, stage_w, nullptr, nullptr,
                                                    nullptr);
}

template <typename TIn, typename TOut, int EPI, bool BROW, int P, bool ACOL>
hipError_t launch(const LaunchArgs& a) {
  const int tiles_m = (a.M + kTile - 1) / kTile, tiles_n = (a.N + kTile - 1) / kTile;
  const int panel = tiles_m < 4 ? tiles_m : 4;
  // N or ldc off the 16-byte output chunks (or, row-major B, N off its
  // 8-column chunks): the masked instance (not built for eight slots, which
  // the plan does not offer for these problems: see ring_ragged)
  if constexpr (P != 8) {
    if (ring_ragged(a.N, a.ldc, (int)sizeof(TOut), BROW)) {
      hipLaunchKernelGGL((gemm_ring_kernel<TIn, TOut, EPI, BROW, P, ACOL, true>), dim3(tiles_m * tiles_n),
                         dim3(kNW * 64), 0, a.stream, (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias,
                         (TOut*)a.C, a.M, a.N, a.K, tiles_m, tiles_n, panel, a.lda, a.ldb, a.ldc, a.scale,
                         (const TOut*)a.residual, a.out_scale);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_ring_kernel<TIn, TOut, EPI, BROW, P, ACOL, false>), dim3(tiles_m * tiles_n), dim3(kNW * 64),
                     0, a.stream, (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K,
                     tiles_m, tiles_n, panel, a.lda, a.ldb, a.ldc, a.scale, (const TOut*)a.residual, a.out_scale);
  return hipGetLastError();
}

template <typename TIn, typename TOut, bool BROW, int P, bool ACOL>
LaunchFn pick_epi(int epi) {
  switch (epi) {
    case GEMM_EPI_NONE: return &launch<TIn, TOut, GEMM_EPI_NONE, BROW, P, ACOL>;
    case GEMM_EPI_RELU: return &launch<TIn, TOut, GEMM_EPI_RELU, BROW, P, ACOL>;
    case GEMM_EPI_BIAS_RELU: return &launch<TIn, TOut, GEMM_EPI_BIAS_RELU, BROW, P, ACOL>;
    case GEMM_EPI_BIAS_GELU: return &launch<TIn, TOut, GEMM_EPI_BIAS_GELU, BROW, P, ACOL>;
    case GEMM_EPI_BIAS: return &launch<TIn, TOut, GEMM_EPI_BIAS, BROW, P, ACOL>;
    case GEMM_EPI_SILU: return &launch<TIn, TOut, GEMM_EPI_SILU, BROW, P, ACOL>;
    case GEMM_EPI_BIAS_SILU: return &launch<TIn, TOut, GEMM_EPI_BIAS_SILU, BROW, P, ACOL>;
    default: return nullptr;
  }
}

// A and B in either layout
template <typename TIn, typename TOut, int P>
LaunchFn pick(int la, int lb, int epi) {
  const bool brow = lb == GEMM_EPI_ROW_MAJOR;
  if (la == GEMM_EPI_ROW_MAJOR)
    return brow ? pick_epi<TIn, TOut, true, P, false>(epi) : pick_epi<TIn, TOut, false, P, false>(epi);
  return brow ? pick_epi<TIn, TOut, true, P, true>(epi) : pick_epi<TIn, TOut, false, P, true>(epi);
}

}  // namespace ring
}  // namespace ge
