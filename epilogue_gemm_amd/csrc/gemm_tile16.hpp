// gemm_tile16.hpp -- the 256x256 tile kernel of gemm_tile.hpp built on
// v_mfma_f32_16x16x32_{f16,bf16} with four waves, for A row-major and B
// either column-major (k contiguous) or row-major (n contiguous, BROW).
//
// Why 16x16x32.  A 32x32x16 MFMA reads and rewrites 16 fp32 accumulators per
// lane for 32 768 FLOP; a 16x16x32 one reads and rewrites 4 for 16 384 FLOP,
// so per FLOP it moves half the accumulator bytes through the register file
// (the operands cost the same per FLOP).  The large squares run at the
// chip's power limit, where the clock follows the energy spent per FLOP.
// With four waves (one per SIMD, 128x128 each) the fragments of both
// operands are double-buffered in the 256 architectural registers next to
// the 256 accumulator registers, and each LDS byte read feeds 128 MACs.
//
// The LDS layout (but for the swizzle), the direct global->LDS copies (with
// the K-tail shift), the raster and the two-stage pipeline are those of
// gemm_tile.hpp;
// a 64-deep k-step is two substeps of k = 32:
//   substep 0   multiply k 0..31 of tile kt, read k 32..63 of it;
//   barrier     after this wave's copies of tile kt + 1 have landed: every
//               wave is done reading tile kt's stage, tile kt + 1 is whole;
//   substep 1   multiply k 32..63, read k 0..31 of tile kt + 1, and copy
//               tile kt + 2 into the stage tile kt leaves, one copy every
//               four MFMAs.
// Fragment f (A or B) of substep kk: rows w0 + 16 f + lane % 16, logical
// 16-byte chunk 4 kk + lane / 16, at chunk position (4 kk + lane / 16) ^
// (row & 7) (swz16 in gemm_tile.hpp: measured free of bank conflicts).  With B's fragment as the first
// operand the 16x16 result arrives transposed: lane l holds
// C[m = l % 16][n = 4 (l / 16) + e], e = 0..3 -- four consecutive columns of
// one row.
//
// Row-major B (BROW).  A stage holds 64 k-rows of 256 n (512 bytes each);
// 16-byte chunk c of k-row r sits at position c ^ 2 tau(r), tau(r) = (r & 3)
// + 4 ((r >> 3) & 1), filled by direct copies of two k-rows per wave
// instruction (RowB256 below).  B's fragment -- eight consecutive k of one
// column per lane -- comes from two transposing reads ds_read_b64_tr_b16 of
// four k-rows each: in each 16-lane group, lane 4 i + a gives the address
// of columns nb + 4 a .. + 3 of k-row kb + i, and lane j receives column
// nb + j at k-rows kb .. kb + 3.  With group g reading k-rows 8 g .. 8 g + 7
// of the substep, the 32 lanes of a read's half see tau = i + 4 (g & 1),
// eight distinct values, and fetch 32 distinct 8-byte words modulo 256
// bytes: one pass, no bank conflict.  The position of fragment f is
// 2 (f ^ tau) + (a >> 1): a per-lane base XOR 32 f bytes, eight offsets
// kept in registers; the substep and the second read are immediates.
// (Tile-level fusion of load -> GEMM -> epilogue -> store:
// TileFusion "基础GEMM示例"; epilogue on the accumulator fragment: csdn
// "从零开始学习 TileLang" ch.10 sec. 10.8; pipelining and rasterisation:
// atlascloud.ai "Writing high-performance kernels in TileLang", section
// "Écrivons un GEMM".)
#pragma once

#include "gemm_tile.hpp"

namespace ge {
namespace tile16 {

using tile::DirectLoader;
using tile::kBK;
using tile::kRowBytes;
using tile::lds_ptr;

// Direct copies of a row-major B tile, 64 k-rows of 256 columns, into the
// layout above: wave instruction i (0..7) of a k-step moves k-rows 2 t and
// 2 t + 1, t = wave + 4 i, to bytes 1024 t .. + 1023 of the stage; lane l
// takes k-row 2 t + l / 32, position l % 32, so it loads chunk
// (l % 32) ^ 2 tau, and tau = 2 (wave & 1) + l / 32 + 4 (i & 1).  The
// buffer starts at k = -kpad (the K-tail shift of DirectLoader) and ends
// with the last k-row; its range must fit 32-bit offsets (host check).
struct RowB256 {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[2];  // instructions with i even, odd
  uint32_t row_bytes;
  int wave;

  __device__ __forceinline__ RowB256(const void* B, int n0, int K, int ldb, int kpad, int lane, int wave_) {
    const char* base = (const char*)B + (int64_t)n0 * 2 - (int64_t)kpad * ldb * 2;
    rsrc = tile::make_rsrc(base, (uint32_t)((int64_t)(K + kpad) * ldb * 2 - (int64_t)n0 * 2));
    row_bytes = (uint32_t)ldb * 2u;
    wave = wave_;
    const int h = lane >> 5, pos = lane & 31;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int tau = 2 * (wave & 1) + h + 4 * v;
      voff[v] = (uint32_t)h * row_bytes + (uint32_t)((pos ^ (2 * tau)) << 4);
    }
  }
  __device__ __forceinline__ void issue(char* dst, int kt, int i) const {
    const int t = wave + 4 * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + t * 1024), 16, voff[i & 1],
                                             (uint32_t)(kt * kBK + 2 * t) * row_bytes, 0, 0);
  }
  // k-step 0 of a shifted k axis: k-rows below kpad load as zeros
  __device__ __forceinline__ void issue_first(char* dst, int i, int lane, int kpad) const {
    const int t = wave + 4 * i;
    const uint32_t v = 2 * t + (lane >> 5) < kpad ? 0xFFFFFFF0u : voff[i & 1];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + t * 1024), 16, v, (uint32_t)(2 * t) * row_bytes,
                                             0, 0);
  }
};

template <typename TIn>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (__is_same(TIn, f16))
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
}

// Epilogue of one wave's WM x WN sub-tile from 16x16 blocks, as
// tile::write_tile: bias, optional column scale, activation, optional
// residual and output scale on the accumulators, conversion, then each
// 16-row band through a private LDS staging area (16-byte chunks swizzled by
// row) and out with 16-byte stores along rows.
// RAGC: columns from n_lim on are not stored (the unshifted last tile
// column of a problem whose N or ldc is off the 16-byte output chunks);
// groups of four columns and 16-byte chunks that reach past n_lim, or lie
// on a row that is not 16-byte aligned, are read and stored element by
// element.
// Four consecutive outputs of the output format as stored (raw bits), and
// their fp32 values.
template <typename T>
struct Raw4 {
  using type = u32x2;  // 16-bit formats
};
template <>
struct Raw4<float> {
  using type = f32x4;
};
template <>
struct Raw4<fp8e4m3> {
  using type = uint32_t;
};
template <typename T>
__device__ __forceinline__ f32x4 raw4_to_f32(typename Raw4<T>::type w) {
  if constexpr (sizeof(T) == 1) {
    return f32x4{__builtin_amdgcn_cvt_f32_fp8((int)w, 0), __builtin_amdgcn_cvt_f32_fp8((int)w, 1),
                 __builtin_amdgcn_cvt_f32_fp8((int)w, 2), __builtin_amdgcn_cvt_f32_fp8((int)w, 3)};
  } else if constexpr (sizeof(T) == 4) {
    return w;
  } else {
    return f32x4{to_f32(__builtin_bit_cast(T, (uint16_t)(w.x & 0xffffu))),
                 to_f32(__builtin_bit_cast(T, (uint16_t)(w.x >> 16))),
                 to_f32(__builtin_bit_cast(T, (uint16_t)(w.y & 0xffffu))),
                 to_f32(__builtin_bit_cast(T, (uint16_t)(w.y >> 16)))};
  }
}

template <int WM, int WN, typename TIn, typename TOut, int EPI, bool EXTRAS, bool RAGC = false>
__device__ __forceinline__ void write_tile16(const f32x4 (&acc)[WM / 16][WN / 16], const TIn* __restrict__ bias,
                                            TOut* __restrict__ C, int ldc, int m_w, int n_w, int lane, char* stage,
                                            const float* __restrict__ scale, const TOut* __restrict__ res,
                                            const float* __restrict__ out_scale, int n_lim = 0) {
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int OSZ = (int)sizeof(TOut);
  constexpr int CPR = WN * OSZ / 16;              // 16-byte chunks per staged row
  constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;  // swizzle mask
  constexpr int RPI = 64 / CPR;                   // rows per store instruction
  const int m_l = lane & 15, g = lane >> 4;
  const bool has_os = EXTRAS && out_scale != nullptr;
  const float os = has_os ? *out_scale : 1.0f;

  // bias of this lane's four columns in each 16-column block, in fp32
  // once (every row block reuses them)
  f32x4 bq[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if constexpr (epi_has_bias<EPI>()) {
      const int col = n_w + j * 16 + 4 * g;
      if (!RAGC || col + 4 <= n_lim) {
        const u32x2 w = *(const u32x2*)(bias + col);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bq[j][e] = to_f32(__builtin_bit_cast(TIn, (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu))));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) bq[j][e] = col + e < n_lim ? to_f32(bias[col + e]) : 0.0f;
      }
    } else {
      bq[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  // The extras on aligned columns: the column scale once, and each band's
  // residual (raw bits) loaded while the band before it is worked on, so
  // that no band waits on its own loads.
  constexpr bool PIPE = EXTRAS && !RAGC;
  using RawT = typename Raw4<TOut>::type;
  f32x4 scq[PIPE ? TN : 1];
  RawT rq[2][PIPE ? TN : 1];
  if constexpr (PIPE) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n_w + j * 16 + 4 * g;
      scq[j] = scale ? *(const f32x4*)(scale + col) : f32x4{1.0f, 1.0f, 1.0f, 1.0f};
      if (res) rq[0][j] = *(const RawT*)(res + (int64_t)(m_w + m_l) * ldc + col);
    }
  }

  static_for<TM>([&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    if constexpr (PIPE && i + 1 < TM) {
      if (res) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          rq[(i + 1) & 1][j] = *(const RawT*)(res + (int64_t)(m_w + (i + 1) * 16 + m_l) * ldc + n_w + j * 16 + 4 * g);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n_w + j * 16 + 4 * g;
      f32x4 sc = f32x4{1.0f, 1.0f, 1.0f, 1.0f}, r = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (EXTRAS) {
        if constexpr (RAGC) {
          // whole groups of four on 4-element aligned rows as vectors, the
          // others element by element
          const bool whole = col + 4 <= n_lim;
          const int64_t at = (int64_t)(m_w + i * 16 + m_l) * ldc + col;
          const bool rvec = whole && (at & 3) == 0;
          if (scale && whole) sc = *(const f32x4*)(scale + col);
          if (res && rvec) r = load4<TOut>(res + at);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < n_lim) {
              if (scale && !whole) sc[e] = scale[col + e];
              if (res && !rvec) r[e] = out_to_f32(res[at + e]);
            }
        } else {
          sc = scq[j];
          if (res) r = raw4_to_f32<TOut>(rq[i & 1][j]);
        }
      }
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = epilogue_ex<EPI>(acc[i][j][e], bq[j][e], EXTRAS && scale != nullptr, sc[e], EXTRAS && res != nullptr,
                                r[e], has_os, os);
      // columns j*16 + 4g .. +3 of row m_l
      if constexpr (OSZ == 1) {
        *(uint32_t*)(stage + m_l * WN + ((j ^ (m_l & SWM)) << 4) + 4 * g) = pack4_e4m3(v[0], v[1], v[2], v[3]);
      } else if constexpr (OSZ == 4) {
        const int c = 4 * j + g;
        *(f32x4*)(stage + m_l * (WN * 4) + ((c ^ (m_l & SWM)) << 4)) = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        const int c = 2 * j + (g >> 1);
        const u32x2 w = u32x2{pack2_out<TOut>(v[0], v[1]), pack2_out<TOut>(v[2], v[3])};
        *(u32x2*)(stage + m_l * (WN * 2) + ((c ^ (m_l & SWM)) << 4) + 8 * (g & 1)) = w;
      }
    }
    // read back along rows: lane -> (row r, chunk c), store 16 bytes
#pragma unroll
    for (int t = 0; t < 16 / RPI; ++t) {
      const int r = t * RPI + lane / CPR, c = lane % CPR;
      const u32x4 d = *(const u32x4*)(stage + r * (WN * OSZ) + ((c ^ (r & SWM)) << 4));
      if constexpr (RAGC) {
        constexpr int EPC = 16 / OSZ;  // outputs per chunk
        const int col0 = n_w + c * EPC;
        if (col0 < n_lim) {
          const int64_t at = (int64_t)(m_w + i * 16 + r) * ldc + col0;
          TOut* dst = C + at;
          if (col0 + EPC <= n_lim && at % EPC == 0) {
            *(u32x4*)dst = d;
          } else {
#pragma unroll
            for (int e = 0; e < EPC; ++e)
              if (col0 + e < n_lim) {
                if constexpr (OSZ == 2) ((uint16_t*)dst)[e] = (uint16_t)(d[e >> 1] >> (16 * (e & 1)));
                else if constexpr (OSZ == 4) ((uint32_t*)dst)[e] = d[e];
                else ((uint8_t*)dst)[e] = (uint8_t)(d[e >> 2] >> (8 * (e & 3)));
              }
          }
        }
      } else {
        *(u32x4*)((char*)(C + (int64_t)(m_w + i * 16 + r) * ldc + n_w) + c * 16) = d;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// RAG (B column-major only): N or ldc off the 16-byte output chunks -- the
// last tile column is not shifted back but masked past N (B's rows past N
// load as zeros) and the epilogue handles its edge element by element.
template <typename TIn, typename TOut, int EPI, bool BROW, bool RAG>
__global__ __launch_bounds__(256) void gemm_tile16_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                          const TIn* __restrict__ bias, TOut* __restrict__ C, int M,
                                                          int N, int K, int tiles_m, int tiles_n, int panel, int lda,
                                                          int ldb, int ldc, const float* __restrict__ scale,
                                                          const TOut* __restrict__ res,
                                                          const float* __restrict__ out_scale) {
  constexpr int NW = 4, BM = 256, BN = 256;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  __shared__ __attribute__((aligned(1024))) char sA0[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA1[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB0[B_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB1[B_BYTES];
  struct Stage {
    char* a;
    char* b;
  };
  const Stage stage0{sA0, sB0}, stage1{sA1, sB1};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / 2, wn = wave % 2;

  int tm, tn;
  tile::raster(blockIdx.x, tiles_m, tiles_n, panel, tm, tn);
  // the last tile row or column is shifted back to end at M or N (it
  // rewrites part of its neighbour with identical values); RAG keeps the
  // last tile column in place
  static_assert(!(RAG && BROW), "row-major B: N % 8 = 0");
  const int m0 = min(tm * BM, M - BM), n0 = RAG ? tn * BN : min(tn * BN, N - BN);
  const int kpad = (-K) & (kBK - 1);

  const DirectLoader<BM, NW, true> da(A, m0, M, lda, kpad, tid, wave);
  // (only one of the two B movers is used)
  const DirectLoader<BN, NW, true> db(B, n0, N, ldb, kpad, tid, wave);
  const RowB256 rb(B, n0, K, ldb, kpad, lane, wave);

  // Fragment rows w0 + 16 f + lane % 16 (w0 a multiple of 64) have the
  // swizzle swz16(lane % 16), so one per-lane offset per operand and substep
  // covers every fragment; the rest (16 f rows, the stage) is an immediate.
  const int sl = tile::swz16(lane & 15);
  const int a_row = (wm * WM + (lane & 15)) * kRowBytes;
  const int b_row = (wn * WN + (lane & 15)) * kRowBytes;
  int aoff[2], boff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    aoff[kk] = a_row + (((4 * kk + (lane >> 4)) ^ sl) << 4);
    boff[kk] = b_row + (((4 * kk + (lane >> 4)) ^ sl) << 4);
  }
  // row-major B: fragment f at k-row 8 g + i (+ 32 kk, + 4 for the second
  // read), bytes 256 wn + 32 (f ^ tau) + 8 a
  int btr[TN];
  if constexpr (BROW) {
    const int g = lane >> 4, ti = (lane >> 2) & 3, ta = lane & 3;
    const int tau = ti + 4 * (g & 1);
#pragma unroll
    for (int f = 0; f < TN; ++f) btr[f] = (8 * g + ti) * 512 + 256 * wn + 32 * (f ^ tau) + 8 * ta;
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // fragments of one substep, double buffered
  u32x4 fa[2][TM], fb[2][TN];
  // read f of a substep: B's fragments first (the first row of MFMAs needs
  // all of them), then A's in the order the rows use them
  auto read_frag = [&](const Stage& st, int kk, int f, u32x4 (&xa)[TM], u32x4 (&xb)[TN]) __attribute__((always_inline)) {
    if (f < TN) {
      if constexpr (BROW) {
        typedef short s4v __attribute__((vector_size(8)));
        typedef __attribute__((address_space(3))) s4v lds_s4v;
        char* p0 = st.b + btr[f] + kk * 32 * 512;
        const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(lds_ptr)p0);
        const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(lds_ptr)(p0 + 4 * 512));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        xb[f] = u32x4{l2.x, l2.y, h2.x, h2.y};
      } else {
        xb[f] = *(const u32x4*)(st.b + boff[kk] + f * 16 * kRowBytes);
      }
    } else {
      xa[f - TN] = *(const u32x4*)(st.a + aoff[kk] + (f - TN) * 16 * kRowBytes);
    }
  };

  constexpr int NMF = TM * TN;  // 64 MFMAs per substep
  constexpr int NDR = TM + TN;  // 16 fragment reads per substep
  constexpr int NDA = DirectLoader<BM, NW, true>::NI;
  constexpr int NDL = NDA + DirectLoader<BN, NW, true>::NI;  // 16 copies per k-step

  // One substep: NMF slots of one MFMA and its share of the memory work,
  // expanded at compile time (a rolled loop would index the accumulators
  // dynamically); nothing moves across a slot boundary.
  //   fragment read f of the next substep: slot f * NMF / NDR;
  //   copies of tile kt + 2 (substep 1 only): spread over the slots.
  auto substep = [&](auto sub_c, const u32x4 (&xa)[TM], const u32x4 (&xb)[TN], const Stage& rd, int rd_kk,
                     bool do_read, u32x4 (&na)[TM], u32x4 (&nb)[TN], const Stage& dl_dst, bool do_direct, int kt)
                     __attribute__((always_inline)) {
    constexpr int sub = decltype(sub_c)::value;
    static_for<NMF>([&](auto slot_c) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      constexpr int i = slot / TN, j = slot % TN;
      acc[i][j] = mfma16<TIn>(xb[j], xa[i], acc[i][j]);
      if constexpr (slot % (NMF / NDR) == 0)
        if (do_read) read_frag(rd, rd_kk, slot / (NMF / NDR), na, nb);
      if constexpr (sub == 1) {
        if (do_direct) {
          static_for<NDL>([&](auto d_c) __attribute__((always_inline)) {
            constexpr int d = decltype(d_c)::value;
            if constexpr (d * NMF / NDL == slot) {
              if constexpr (d < NDA) da.issue(dl_dst.a, kt + 2, d);
              else if constexpr (BROW) rb.issue(dl_dst.b, kt + 2, d - NDA);
              else db.issue(dl_dst.b, kt + 2, d - NDA);
            }
          });
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // k-step kt with tile kt in `cur` and `nxt` receiving kt + 1
  auto kstep = [&](const Stage& cur, const Stage& nxt, int kt, bool more1, bool more2) __attribute__((always_inline)) {
    substep(std::integral_constant<int, 0>{}, fa[0], fb[0], cur, 1, true, fa[1], fb[1], cur, false, kt);
    // this wave's copies of tile kt + 1 are its only outstanding ones
    tile::kloop_barrier<0>();
    __builtin_amdgcn_sched_barrier(0);
    substep(std::integral_constant<int, 1>{}, fa[1], fb[1], nxt, 0, more1, fa[0], fb[0], cur, more2, kt);
  };

  // Tile t lives in stage (t + KT) % 2, so that the last two tiles are
  // always in stages 0 and 1 and the k loop ends with two peeled k-steps.
  // KT >= 2, i.e. K > 64 (checked on the host).
  const int KT = (K + kpad) / kBK;
  auto prologue = [&](const Stage& s_first, const Stage& s_second) __attribute__((always_inline)) {
    if (kpad == 0) {
#pragma unroll
      for (int d = 0; d < NDL; ++d) {
        if (d < NDA) da.issue(s_first.a, 0, d);
        else if constexpr (BROW) rb.issue(s_first.b, 0, d - NDA);
        else db.issue(s_first.b, 0, d - NDA);
      }
    } else {
#pragma unroll
      for (int d = 0; d < NDL; ++d) {
        if (d < NDA) da.issue_first(s_first.a, d, lane, kpad);
        else if constexpr (BROW) rb.issue_first(s_first.b, d - NDA, lane, kpad);
        else db.issue_first(s_first.b, d - NDA, lane, kpad);
      }
    }
#pragma unroll
    for (int d = 0; d < NDL; ++d) {
      if (d < NDA) da.issue(s_second.a, 1, d);
      else if constexpr (BROW) rb.issue(s_second.b, 1, d - NDA);
      else db.issue(s_second.b, 1, d - NDA);
    }
    // tile 0 complete; tile 1's copies may stay in flight
    tile::kloop_barrier<NDL>();
#pragma unroll
    for (int f = 0; f < NDR; ++f) read_frag(s_first, 0, f, fa[0], fb[0]);
  };

  int kt = 0;
  if (KT & 1) {
    prologue(stage1, stage0);
    kstep(stage1, stage0, 0, true, true);
    kt = 1;
  } else {
    prologue(stage0, stage1);
  }
  for (; kt + 4 <= KT; kt += 2) {
    kstep(stage0, stage1, kt, true, true);
    kstep(stage1, stage0, kt + 1, true, true);
  }
  kstep(stage0, stage1, kt, true, false);
  kstep(stage1, stage0, kt + 1, false, false);

  // Every wave is done with the operand stages: reuse them as the staging
  // areas of the epilogue, one array per wave.
  __syncthreads();
  static_assert(16 * WN * sizeof(TOut) <= (size_t)A_BYTES, "staging area");
  char* const stage_w = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sB0 : sB1;
  if (scale != nullptr || res != nullptr || out_scale != nullptr)
    write_tile16<WM, WN, TIn, TOut, EPI, true, RAG>(acc, bias, C, ldc, m0 + wm * WM, n0 + wn * WN, lane, stage_w,
                                                    scale, res, out_scale, N);
  else
    write_tile16<WM, WN, TIn, TOut, EPI, false, RAG>(acc, bias, C, ldc, m0 + wm * WM, n0 + wn * WN, lane, stage_w,
                                                     nullptr, nullptr, nullptr, N);
}

template <typename TIn, typename TOut, int EPI, bool BROW>
hipError_t launch(const LaunchArgs& a) {
  const int tiles_m = (a.M + 255) / 256, tiles_n = (a.N + 255) / 256;
  const int panel = tiles_m < 4 ? tiles_m : 4;
  if constexpr (!BROW) {
    constexpr int EPC = 16 / (int)sizeof(TOut);
    if (a.N % EPC != 0 || a.ldc % EPC != 0) {
      hipLaunchKernelGGL((gemm_tile16_kernel<TIn, TOut, EPI, BROW, true>), dim3(tiles_m * tiles_n), dim3(256), 0,
                         a.stream, (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K,
                         tiles_m, tiles_n, panel, a.lda, a.ldb, a.ldc, a.scale, (const TOut*)a.residual,
                         a.out_scale);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_tile16_kernel<TIn, TOut, EPI, BROW, false>), dim3(tiles_m * tiles_n), dim3(256), 0,
                     a.stream, (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K,
                     tiles_m, tiles_n, panel, a.lda, a.ldb, a.ldc, a.scale, (const TOut*)a.residual, a.out_scale);
  return hipGetLastError();
}

template <typename TIn, typename TOut, bool BROW>
LaunchFn pick_epi(int epi) {
  switch (epi) {
    case GEMM_EPI_NONE: return &launch<TIn, TOut, GEMM_EPI_NONE, BROW>;
    case GEMM_EPI_RELU: return &launch<TIn, TOut, GEMM_EPI_RELU, BROW>;
    case GEMM_EPI_BIAS_RELU: return &launch<TIn, TOut, GEMM_EPI_BIAS_RELU, BROW>;
    case GEMM_EPI_BIAS_GELU: return &launch<TIn, TOut, GEMM_EPI_BIAS_GELU, BROW>;
    case GEMM_EPI_BIAS: return &launch<TIn, TOut, GEMM_EPI_BIAS, BROW>;
    case GEMM_EPI_SILU: return &launch<TIn, TOut, GEMM_EPI_SILU, BROW>;
    case GEMM_EPI_BIAS_SILU: return &launch<TIn, TOut, GEMM_EPI_BIAS_SILU, BROW>;
    default: return nullptr;
  }
}

// A row-major with B column-major (both k-contiguous), or with B
// row-major when BROW.
template <typename TIn, typename TOut, bool BROW>
LaunchFn pick(int la, int lb, int epi) {
  if (la != GEMM_EPI_ROW_MAJOR || lb != (BROW ? GEMM_EPI_ROW_MAJOR : GEMM_EPI_COL_MAJOR)) return nullptr;
  return pick_epi<TIn, TOut, BROW>(epi);
}

}  // namespace tile16
}  // namespace ge
