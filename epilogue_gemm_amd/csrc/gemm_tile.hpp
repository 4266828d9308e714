// gemm_tile.hpp -- the LDS-pipelined MFMA tile kernel for gfx950.
//
// One workgroup (4 or 8 waves of 64) computes a BM x BN tile of C, looping
// over k in steps of 64.  Both operands are staged in LDS in one layout:
// rows along M (for A) or N (for B), 64 k values per row, k contiguous, the
// 16-byte chunks of each row XOR-swizzled.  The waves form a 2 x (NW / 2)
// grid, each owning a (BM / 2) x (2 BN / NW) sub-tile made of 32x32 blocks,
// and feed v_mfma_f32_32x32x16_{f16,bf16} from LDS, accumulating in fp32.
// (gemm_tile16.hpp builds the 256 x 256, four-wave tile for k-contiguous
// operands on 16x16x32 MFMAs from the same loaders, raster and pipeline.)
//
// Getting a k-step into LDS:
//   * an operand whose k index is contiguous in memory (A row-major, B
//     column-major) is copied global -> LDS by 128-bit buffer loads that
//     write LDS directly (no VGPR round trip, no LDS store instruction);
//     each wave instruction fills 1 KiB = 8 rows, and each lane fetches the
//     global chunk that belongs at its LDS position under the swizzle;
//   * an operand whose M/N index is contiguous (A column-major, B row-major)
//     is loaded 8 M/N-values wide for several k into registers, transposed
//     in registers and written k-contiguous.
//
// Pipeline: two LDS stages, statically distinct (the loop is unrolled by
// two) so the compiler can tell a read of one stage from an in-flight
// direct load into the other.  In k-step kt (tile kt in stage s):
//   substeps 0..2  multiply, read the next substep's fragments, and for a
//                  register-staged operand write tile kt+1 into stage s^1
//                  and refill its registers with tile kt+2;
//   barrier        after waiting for this wave's direct loads of tile kt+1;
//   substep 3      multiply, read substep 0 of stage s^1, and issue the
//                  direct loads of tile kt+2 into stage s, which every wave
//                  finished reading before the barrier.
// Every MFMA slot carries an explicit share of the memory instructions;
// slots are fenced so the issue order is the one written here.
//
// After the k loop the epilogue (bias add, then ReLU or GELU) runs on the
// fp32 accumulators and each lane writes four consecutive outputs of one row
// with one vector store: the kernel never writes an intermediate tensor.
// (Tile-level fusion of load -> GEMM -> activation -> store: TileFusion
// "基础GEMM示例"; epilogue on the fragment before write-back: csdn
// "从零开始学习 TileLang" ch.10 sec. 10.8; software pipelining and block
// rasterisation for L2 reuse: atlascloud.ai "Writing high-performance kernels
// in TileLang", section "Écrivons un GEMM".)
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

// 16-byte chunk c of LDS row r is stored at chunk position c ^ swz(r).
// Operand reads: the 16 lanes of a quarter-wave read 16 consecutive rows at
// one logical chunk; swz maps them to 8 distinct positions for rows r..r+7
// and, as rows r and r+1 sit 128 B apart, to 16 distinct 16-byte bank
// groups over 16 rows.  Transposed writes: 8 lanes write rows 8t + j
// (t = 0..7) and get positions c ^ j ^ t, again distinct.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// The swizzle of the 16x16x32 kernel (gemm_tile16.hpp), chosen by
// measurement: its fragment reads (16 consecutive rows per quarter-wave, the
// four quarters at chunks c .. c + 3) were timed on the chip in a
// ds_read_b128 probe, counting SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE
// per instruction: c ^ (row & 7) takes 4 LDS cycles per read with no
// conflict cycles, while c ^ swz(row), and c ^ (bits 1 and 2 of the row
// moved to bits 0 and 2), take 8 (a 2-way conflict) and the unswizzled
// layout 16.  (The 32x32x16 reads under swz() measured conflict-free too.)
__device__ __forceinline__ int swz16(int row) { return row & 7; }

// Buffer resource over [base, base + bytes): 128-bit raw buffer loads then
// take one per-lane 32-bit offset plus one wave-uniform offset, so the loop
// carries no 64-bit addresses.  Offsets at or past `bytes` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// k-contiguous operand, global -> LDS directly.  Row r of the tile is
// X[(r0 + r) * ld + k].  When K is not a multiple of the 64-deep k-step,
// the k axis is shifted by kpad = 64 - K % 64 so that the partial step is
// the first one: k-step t covers k in [64 t - kpad, 64 t - kpad + 64), and
// the chunks of step 0 with k < 0 are loaded as zeros (issue_first).
// Instruction i of wave w (of NW) fills tile rows
// (NW i + w) * 8 .. +7; lane L writes LDS bytes 16 L .. 16 L + 15 of that
// KiB, i.e. row (NW i + w) * 8 + L / 8 at chunk position L % 8, so it loads
// logical chunk (L % 8) ^ swz(row).  swz depends on the row only through
// L / 8 and (NW i + w) % 8, which takes NV = 8 / NW values as i varies, so NV
// per-lane offsets cover every instruction; the rest is wave-uniform.
template <int R, int NW, bool M16 = false>
struct DirectLoader {
  __device__ static __forceinline__ int sw(int row) { return M16 ? swz16(row) : swz(row); }
  static constexpr int NI = R / (8 * NW);  // wave instructions per wave per k-step
  static constexpr int NV = 8 / NW;
  static_assert(NV >= 1 && NV <= 2, "4 or 8 waves");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[2];  // fixed extent: an NW-dependent one left host kernel stubs undefined
  uint32_t rows64;  // bytes of 64 rows
  int wave;

  __device__ __forceinline__ DirectLoader(const void* X, int r0, int rows_total, int ld, int kpad, int tid,
                                          int wave_) {
    const char* base = (const char*)X + (int64_t)r0 * ld * 2 - (int64_t)kpad * 2;
    rsrc = make_rsrc(base, (uint32_t)((int64_t)(rows_total - r0) * ld * 2 + (int64_t)kpad * 2));
    wave = wave_;
    const int lane = tid & 63;
    const int rl = lane >> 3, pc = lane & 7;
#pragma unroll
    for (int p = 0; p < NV; ++p) {
      const int row = (NW * p + wave) * 8 + rl;
      voff[p] = (uint32_t)(row * ld * 2 + ((pc ^ sw(row)) << 4));
      // a tile taller than what is left of the operand (a 64-row tile of a
      // problem with fewer rows): rows past the end load nothing
      if (r0 + row >= rows_total) voff[p] = 0xFFFFFFF0u;
    }
    rows64 = (uint32_t)(64 * ld * 2);
  }
  // Issue instruction i of k-step kt into the operand region `dst` of a stage.
  __device__ __forceinline__ void issue(char* dst, int kt, int i) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + (NW * i + wave) * 1024), 16, voff[i % NV],
                                             (i / NV) * rows64 + kt * kRowBytes, 0, 0);
  }
  // Instruction i of k-step 0 when the axis is shifted by kpad (a multiple
  // of 8): a lane whose logical chunk lies at k < 0 takes a per-lane offset
  // past the end of the buffer, which the buffer's range check turns into
  // zeros without a memory access.  (Rows of instruction i are rows of
  // instruction i % NV plus a multiple of 64, so they share the swizzle.)
  __device__ __forceinline__ void issue_first(char* dst, int i, int lane, int kpad) const {
    const int row = (NW * (i % NV) + wave) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ sw(row);
    const uint32_t v = chunk * 8 < kpad ? 0xFFFFFFF0u : voff[i % NV];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + (NW * i + wave) * 1024), 16, v,
                                             (i / NV) * rows64, 0, 0);
  }
};

// M/N-contiguous operand through registers: row r of the tile (an M or N
// index) at k is X[k * ld + r0 + r].  Each thread loads KB k-rows of 8
// consecutive M/N values and writes, for each of the 8, its KB k-values
// contiguously.  The k axis is shifted by kpad as for DirectLoader; rows of
// step 0 with k < 0 load as zeros (load_first).
template <int R, int NT>
struct RegLoader {
  static constexpr int KB = R * 8 / NT;  // k values per thread: 8, 4 or 2
  static constexpr int NG = R / 8;   // 8-wide groups along M/N
  static_assert(KB >= 2 && KB <= 8, "tile extent");
  static constexpr int LOADS = KB;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff;
  uint32_t kstep;  // bytes between consecutive k rows
  int ng, kg;
  u32x4 r[KB];

  __device__ __forceinline__ RegLoader(const void* X, int r0, int k_total, int ld, int kpad, int tid) {
    ng = tid % NG;
    kg = tid / NG;
    kstep = (uint32_t)(ld * 2);
    const char* base = (const char*)X + (int64_t)r0 * 2 - (int64_t)kpad * ld * 2;
    rsrc = make_rsrc(base, (uint32_t)((int64_t)(k_total + kpad) * ld * 2 - (int64_t)r0 * 2));
    voff = (uint32_t)(kg * KB * ld * 2 + ng * 16);
  }
  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int i = 0; i < KB; ++i) r[i] = load16(rsrc, voff, (uint32_t)(kt * kBK + i) * kstep);
  }
  // k-step 0 with the axis shifted by kpad: rows at k < 0 read as zeros
  // (per-lane offset past the end of the buffer: no memory access)
  __device__ __forceinline__ void load_first(int kpad) {
#pragma unroll
    for (int i = 0; i < KB; ++i) r[i] = load16(rsrc, kg * KB + i < kpad ? 0xFFFFFFF0u : voff, (uint32_t)i * kstep);
  }
  // 16-bit element j (0..7) of a 128-bit register
  static __device__ __forceinline__ uint32_t half_of(const u32x4& v, int j) {
    const uint32_t w = v[j >> 1];
    return (j & 1) ? (w >> 16) : (w & 0xffffu);
  }
  __device__ __forceinline__ void store(char* s) const {
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

// Epilogue of one wave's WM x WN sub-tile: bias, activation and conversion
// on the accumulators, then one coalesced store of each output.
//
// The MFMA layout gives lane l four consecutive columns of one row per
// register quad, which as a store would touch 32 rows per instruction.  So
// each 32-row band of the sub-tile is first written to a private LDS
// staging area in row-major order (16-byte chunks XOR-swizzled by row to
// spread the banks), then read back 16 bytes per lane along rows and stored:
// one wave instruction covers whole row segments of the band.  Bands are
// processed one after another so that few values are live at a time.
//
// MASK: the sub-tile may reach past row m_lim or column n_lim of C (a tile
// larger than the problem); outputs there are neither computed from real
// operands nor stored, and the bias, scale and residual past them are not
// read.  (16-byte output chunks lie wholly on one side: n_lim is a multiple
// of 8, of 16 for 1-byte outputs.)
// RAGC (with MASK): n_lim any, and ldc any: groups of four columns and
// 16-byte output chunks that reach past n_lim, or rows of C whose chunks
// are not 16-byte aligned, are read and stored element by element.
template <int WM, int WN, typename TIn, typename TOut, int EPI, bool EXTRAS, bool MASK = false, bool RAGC = false>
__device__ __forceinline__ void write_tile(const f32x16 (&acc)[WM / 32][WN / 32], const TIn* __restrict__ bias,
                                          TOut* __restrict__ C, int ldc, int m_w, int n_w, int lane, char* stage,
                                          const float* __restrict__ scale, const TOut* __restrict__ res,
                                          const float* __restrict__ out_scale, int m_lim = 0, int n_lim = 0) {
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int OSZ = (int)sizeof(TOut);
  constexpr int CPR = WN * OSZ / 16;           // 16-byte chunks per staged row
  constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;  // swizzle mask
  constexpr int RPI = 64 / CPR;                // rows per store instruction
  const int m_l = lane & 31, h = lane >> 5;
  const bool has_os = EXTRAS && out_scale != nullptr;
  const float os = has_os ? *out_scale : 1.0f;

  // bias of this lane's 16 columns in each 32-column block, kept packed
  u32x2 bq[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (epi_has_bias<EPI>()) {
        const int col = n_w + j * 32 + 8 * q + 4 * h;
        if (!MASK || (RAGC ? col + 4 <= n_lim : col < n_lim)) {
          bq[j][q] = *(const u32x2*)(bias + col);
        } else {
          bq[j][q] = u32x2{0u, 0u};
          if constexpr (RAGC) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < n_lim) bq[j][q][e >> 1] |= (uint32_t)bits16(bias[col + e]) << (16 * (e & 1));
          }
        }
      } else {
        bq[j][q] = u32x2{0u, 0u};
      }
    }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // optional column scale and residual of these four outputs
        const int col = n_w + j * 32 + 8 * q + 4 * h;
        f32x4 sc = f32x4{1.0f, 1.0f, 1.0f, 1.0f}, r = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (EXTRAS) {
          const int row = m_w + i * 32 + m_l;
          if constexpr (RAGC) {
            // whole groups of four on 4-element aligned rows as vectors,
            // the others element by element
            if (row < m_lim && col < n_lim) {
              const bool whole = col + 4 <= n_lim;
              const int64_t at = (int64_t)row * ldc + col;
              const bool rvec = whole && (at & 3) == 0;  // the residual's four on one aligned vector
              if (scale && whole) sc = *(const f32x4*)(scale + col);
              if (res && rvec) r = load4<TOut>(res + at);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < n_lim) {
                  if (scale && !whole) sc[e] = scale[col + e];
                  if (res && !rvec) r[e] = out_to_f32(res[at + e]);
                }
            }
          } else {
            const bool in = !MASK || (col < n_lim && row < m_lim);
            if (scale && in) sc = *(const f32x4*)(scale + col);
            if (res && in) r = load4<TOut>(res + (int64_t)row * ldc + col);
          }
        }
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float b = 0.0f;
          if constexpr (epi_has_bias<EPI>()) {
            const uint32_t w = bq[j][q][e >> 1];
            b = to_f32(__builtin_bit_cast(TIn, (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu))));
          }
          v[e] = epilogue_ex<EPI>(acc[i][j][4 * q + e], b, EXTRAS && scale != nullptr, sc[e], EXTRAS && res != nullptr,
                                  r[e], has_os, os);
        }
        // columns j*32 + 8q + 4h .. +3 of row m_l
        if constexpr (OSZ == 1) {
          const int c = 2 * j + (q >> 1);
          *(uint32_t*)(stage + m_l * WN + ((c ^ (m_l & SWM)) << 4) + 8 * (q & 1) + 4 * h) =
              pack4_e4m3(v[0], v[1], v[2], v[3]);
        } else if constexpr (OSZ == 4) {
          const int c = 8 * j + 2 * q + h;
          *(f32x4*)(stage + m_l * (WN * 4) + ((c ^ (m_l & SWM)) << 4)) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          const int c = 4 * j + q;
          const u32x2 w = u32x2{pack2_out<TOut>(v[0], v[1]), pack2_out<TOut>(v[2], v[3])};
          *(u32x2*)(stage + m_l * (WN * 2) + ((c ^ (m_l & SWM)) << 4) + 8 * h) = w;
        }
      }
    }
    // read back along rows: lane -> (row r, chunk c), store 16 bytes
#pragma unroll
    for (int t = 0; t < 32 / RPI; ++t) {
      const int r = t * RPI + lane / CPR, c = lane % CPR;
      const u32x4 d = *(const u32x4*)(stage + r * (WN * OSZ) + ((c ^ (r & SWM)) << 4));
      if constexpr (RAGC) {
        constexpr int EPC = 16 / OSZ;  // outputs per chunk
        const int row = m_w + i * 32 + r, col0 = n_w + c * EPC;
        if (row < m_lim && col0 < n_lim) {
          const int64_t at = (int64_t)row * ldc + col0;
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
      } else if (!MASK || (m_w + i * 32 + r < m_lim && n_w + c * (16 / OSZ) < n_lim)) {
        *(u32x4*)((char*)(C + (int64_t)(m_w + i * 32 + r) * ldc + n_w) + c * 16) = d;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Workgroup barrier for the k loop.  Each wave first waits until at most
// VM of its own vector-memory operations are outstanding (its direct loads
// of the next tile are then in LDS) and its LDS writes are done; unlike
// __syncthreads(), loads issued later may stay in flight.
// The empty asm statements with a memory clobber keep the compiler from
// moving any memory access across the barrier (the barrier builtin itself
// orders no memory for the compiler, and other waves' accesses are what it
// synchronises).
template <int VM>
__device__ __forceinline__ void kloop_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM) & ~(15 << 8));  // vmcnt(VM) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int BN, int NW, typename TIn, typename TOut, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_tile_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                             const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                             int M, int N, int K, int tiles_m, int tiles_n,
                                                             int panel, int lda, int ldb, int ldc,
                                                             const float* __restrict__ scale,
                                                             const TOut* __restrict__ res,
                                                             const float* __restrict__ out_scale) {
  // NW waves in a 2 x (NW / 2) grid, each owning a WM x WN sub-tile
  constexpr int NT = NW * 64;
  constexpr int WM = BM / 2, WN = BN / (NW / 2);
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  // One array per operand and stage, so that every access names its stage
  // statically (and A's stages sit within reach of one 16-bit immediate
  // offset of each other, as do B's).
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
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);

  int tm, tn;
  raster(blockIdx.x, tiles_m, tiles_n, panel, tm, tn);
  // When M or N is not a tile multiple, the last tile row or column is
  // shifted back to end at M or N: it recomputes (and rewrites, with
  // identical values) part of its neighbour, and no access leaves A, B,
  // bias or C.
  const int m0 = min(tm * BM, M - BM), n0 = min(tn * BN, N - BN);
  // K need only be a multiple of 8: the first k-step is then partial, its
  // first kpad k-values zeros (see DirectLoader)
  const int kpad = (-K) & (kBK - 1);

  // Operand movers: direct (k-contiguous) or register-staged (transposed).
  // The unused kind of each operand is never called.
  DirectLoader<BM, NW> da(A, m0, M, lda, kpad, tid, wave);
  DirectLoader<BN, NW> db(B, n0, N, ldb, kpad, tid, wave);
  RegLoader<BM, NT> ra(A, m0, K, lda, kpad, tid);
  RegLoader<BN, NT> rb(B, n0, K, ldb, kpad, tid);

  // Per-lane LDS read offsets.  Fragment i of a wave's operand covers rows
  // w0 + 32 i + (lane % 32), logical chunk 2 kk + lane / 32 for k-substep kk;
  // swz() of those rows is f_lane ^ 4 ((w0 / 32 + i) & 1).
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

  // fragments of one k-substep, double buffered
  u32x4 fa[2][TM], fb[2][TN];
  auto read_frag = [&](const Stage& st, int kk, int f, u32x4 (&xa)[TM], u32x4 (&xb)[TN])
                       __attribute__((always_inline)) {
    if (f < TM) xa[f] = *(const u32x4*)(st.a + a_row + f * 32 * kRowBytes + sw[kk][(a_par + f) & 1]);
    else xb[f - TM] = *(const u32x4*)(st.b + b_row + (f - TM) * 32 * kRowBytes + sw[kk][(b_par + f - TM) & 1]);
  };

  constexpr int NMF = TM * TN;  // MFMAs per substep
  constexpr int NDR = TM + TN;  // LDS fragment reads per substep
  // register loads per k-step (transposed operands)
  constexpr int REG_LOADS = (A_KMAJ ? 0 : RegLoader<BM, NT>::LOADS) + (B_KMAJ ? 0 : RegLoader<BN, NT>::LOADS);
  // direct loads per wave per k-step
  constexpr int NDA = A_KMAJ ? DirectLoader<BM, NW>::NI : 0;
  constexpr int NDL = NDA + (B_KMAJ ? DirectLoader<BN, NW>::NI : 0);

  // One substep: NMF slots, each one MFMA followed by the memory work placed
  // in that slot, in program order; nothing moves across a slot boundary.
  //   fragment reads for the next substep: slots 0 .. NDR-1 (spread when
  //     NMF < NDR);
  //   a register-staged operand (substep 0 for A, substep 0 or 1 for B,
  //     slot 0): write tile kt+1 into `nx`, then reload with tile kt+2;
  //   direct loads of tile kt+2 (substep 3 only): spread over the slots.
  auto substep = [&](int sub, const u32x4 (&xa)[TM], const u32x4 (&xb)[TN], const Stage& rd, int rd_kk, bool do_read,
                     u32x4 (&na)[TM], u32x4 (&nb)[TN], bool do_store, bool do_load, const Stage& nx,
                     const Stage& dl_dst, bool do_direct, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int slot = 0; slot < NMF; ++slot) {
      const int i = slot / TN, j = slot % TN;
      acc[i][j] = mfma32<TIn>(xb[j], xa[i], acc[i][j]);
      if (do_read) {
        if (NMF >= NDR) {
          if (slot < NDR) read_frag(rd, rd_kk, slot, na, nb);
        } else {
#pragma unroll
          for (int f = slot * NDR / NMF; f < (slot + 1) * NDR / NMF; ++f) read_frag(rd, rd_kk, f, na, nb);
        }
      }
      if (sub < 3 && do_store && slot == 0) {
        if (!A_KMAJ && sub == 0) {
          ra.store(nx.a);
          if (do_load) ra.load(kt + 2);
        }
        if (!B_KMAJ && sub == (A_KMAJ ? 0 : 1)) {
          rb.store(nx.b);
          if (do_load) rb.load(kt + 2);
        }
      }
      if constexpr (NDL > 0) if (sub == 3 && do_direct) {
#pragma unroll
        for (int d = 0; d < NDL; ++d) {
          if (d * NMF / NDL == slot) {
            if (d < NDA) da.issue(dl_dst.a, kt + 2, d);
            else db.issue(dl_dst.b, kt + 2, d - NDA);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // k-step kt with tile kt in stage `cur` and stage `nxt` receiving kt + 1.
  auto kstep = [&](const Stage& cur, const Stage& nxt, int kt, bool more1, bool more2) __attribute__((always_inline)) {
    substep(0, fa[0], fb[0], cur, 1, true, fa[1], fb[1], more1, more2, nxt, cur, false, kt);
    substep(1, fa[1], fb[1], cur, 2, true, fa[0], fb[0], more1, more2, nxt, cur, false, kt);
    substep(2, fa[0], fb[0], cur, 3, true, fa[1], fb[1], more1, more2, nxt, cur, false, kt);
    // This wave's direct loads of tile kt + 1 are its oldest outstanding
    // vector-memory operations; the register loads of tile kt + 2 issued in
    // substeps 0..2 may stay in flight.
    if (more2) kloop_barrier<REG_LOADS>();
    else kloop_barrier<0>();
    __builtin_amdgcn_sched_barrier(0);
    substep(3, fa[1], fb[1], nxt, 0, more1, fa[0], fb[0], false, false, nxt, cur, more2, kt);
  };

  // Tile t lives in stage (t + KT) % 2, so that the last two tiles are
  // always in stages 0 and 1 and the k loop ends with two peeled k-steps
  // and no other branches (one straight path keeps the accumulators in
  // place).  KT >= 2, i.e. K > 64 (checked on the host).
  const int KT = (K + kpad) / kBK;
  auto prologue = [&](const Stage& s_first, const Stage& s_second) __attribute__((always_inline)) {
    if (kpad == 0) {
#pragma unroll
      for (int d = 0; d < NDL; ++d) {
        if (d < NDA) da.issue(s_first.a, 0, d);
        else db.issue(s_first.b, 0, d - NDA);
      }
      if constexpr (!A_KMAJ) ra.load(0);
      if constexpr (!B_KMAJ) rb.load(0);
    } else {
#pragma unroll
      for (int d = 0; d < NDL; ++d) {
        if (d < NDA) da.issue_first(s_first.a, d, lane, kpad);
        else db.issue_first(s_first.b, d - NDA, lane, kpad);
      }
      if constexpr (!A_KMAJ) ra.load_first(kpad);
      if constexpr (!B_KMAJ) rb.load_first(kpad);
    }
    if constexpr (!A_KMAJ) ra.store(s_first.a);
    if constexpr (!B_KMAJ) rb.store(s_first.b);
#pragma unroll
    for (int d = 0; d < NDL; ++d) {
      if (d < NDA) da.issue(s_second.a, 1, d);
      else db.issue(s_second.b, 1, d - NDA);
    }
    if constexpr (!A_KMAJ) ra.load(1);
    if constexpr (!B_KMAJ) rb.load(1);
    // tile 0 complete; tile 1's loads may stay in flight
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NDL + REG_LOADS));
    __syncthreads();
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
  // areas of the epilogue, one per wave.
  __syncthreads();
  // (wave w uses part w / 4 of stage array w % 4; BM == BN for every
  // configuration, and a part holds one staged band)
  static_assert(BM == BN && 32 * WN * sizeof(TOut) <= (size_t)A_BYTES / (NW / 4), "staging area");
  char* const stage_w = (wave % 4 == 0 ? sA0 : wave % 4 == 1 ? sA1 : wave % 4 == 2 ? sB0 : sB1) +
                        (wave / 4) * (A_BYTES / (NW / 4));
  // (the optional column scale, residual and output scale get their own
  // copy of the epilogue, so that the plain one carries no tests for them)
  if (scale != nullptr || res != nullptr || out_scale != nullptr)
    write_tile<WM, WN, TIn, TOut, EPI, true>(acc, bias, C, ldc, m0 + wm * WM, n0 + wn * WN, lane, stage_w, scale, res,
                                             out_scale);
  else
    write_tile<WM, WN, TIn, TOut, EPI, false>(acc, bias, C, ldc, m0 + wm * WM, n0 + wn * WN, lane, stage_w, nullptr,
                                              nullptr, nullptr);
}

// Host launch of one instantiation.
template <int BM, int BN, int NW, typename TIn, typename TOut, bool A_KMAJ, bool B_KMAJ, int EPI>
hipError_t launch(const LaunchArgs& a) {
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int panel = tiles_m < 4 ? tiles_m : 4;
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, NW, TIn, TOut, A_KMAJ, B_KMAJ, EPI>), dim3(tiles_m * tiles_n),
                     dim3(NW * 64), 0, a.stream, (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C,
                     a.M, a.N, a.K, tiles_m, tiles_n, panel, a.lda, a.ldb, a.ldc, a.scale, (const TOut*)a.residual,
                     a.out_scale);
  return hipGetLastError();
}

template <int BM, int BN, int NW, typename TIn, typename TOut, bool A_KMAJ, bool B_KMAJ>
LaunchFn pick_epi(int epi) {
  switch (epi) {
    case GEMM_EPI_NONE: return &launch<BM, BN, NW, TIn, TOut, A_KMAJ, B_KMAJ, GEMM_EPI_NONE>;
    case GEMM_EPI_RELU: return &launch<BM, BN, NW, TIn, TOut, A_KMAJ, B_KMAJ, GEMM_EPI_RELU>;
    case GEMM_EPI_BIAS_RELU: return &launch<BM, BN, NW, TIn, TOut, A_KMAJ, B_KMAJ, GEMM_EPI_BIAS_RELU>;
    case GEMM_EPI_BIAS_GELU: return &launch<BM, BN, NW, TIn, TOut, A_KMAJ, B_KMAJ, GEMM_EPI_BIAS_GELU>;
    case GEMM_EPI_BIAS: return &launch<BM, BN, NW, TIn, TOut, A_KMAJ, B_KMAJ, GEMM_EPI_BIAS>;
    case GEMM_EPI_SILU: return &launch<BM, BN, NW, TIn, TOut, A_KMAJ, B_KMAJ, GEMM_EPI_SILU>;
    case GEMM_EPI_BIAS_SILU: return &launch<BM, BN, NW, TIn, TOut, A_KMAJ, B_KMAJ, GEMM_EPI_BIAS_SILU>;
    default: return nullptr;
  }
}

template <int BM, int BN, int NW, typename TIn, typename TOut>
LaunchFn pick_layout(int la, int lb, int epi) {
  const bool ak = la == GEMM_EPI_ROW_MAJOR, bk = lb == GEMM_EPI_COL_MAJOR;
  if (ak && bk) return pick_epi<BM, BN, NW, TIn, TOut, true, true>(epi);
  if (ak && !bk) return pick_epi<BM, BN, NW, TIn, TOut, true, false>(epi);
  if (!ak && bk) return pick_epi<BM, BN, NW, TIn, TOut, false, true>(epi);
  return pick_epi<BM, BN, NW, TIn, TOut, false, false>(epi);
}

}  // namespace tile
}  // namespace ge
