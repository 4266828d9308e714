// kernels.hpp -- host-side view of the three kernel families: their
// configuration tables, the divisibility each one needs, and the launch
// entry each .hip file exports.
#pragma once

#include "common.hpp"

namespace ge {

using LaunchFn = hipError_t (*)(const LaunchArgs&);

struct Problem {
  int64_t M, N, K;
  int in_dt, out_dt, la, lb, epi;
  int64_t lda, ldb, ldc;  // leading dimensions of A, B, C (packed: the contiguous extent)
};

// ---- generic: any shape, layout and alignment -----------------------------
// Extra LaunchArgs fields it needs are the layouts (passed through `Problem`).
LaunchFn generic_launcher(const Problem& p);

// ---- tile: LDS-pipelined MFMA kernel --------------------------------------
struct TileConfig {
  int bm, bn;  // workgroup tile
  int waves;   // waves per workgroup
  const char* name;
  int mfma;    // MFMA block: 32 (32x32x16, any layout) or 16 (16x16x32, A row-major)
  int ring;    // 0: two LDS stages; P > 0: the deep ring of P slots (gemm_ring.hpp, A row-major only)
  bool brow;   // 16x16x32 only: B row-major (transposing LDS reads) instead of column-major
};
int tile_num_configs();
// A ring problem whose N or ldc is off the 16-byte output chunks (or, with
// a row-major B, N off its 8-column chunks): the ring kernels then mask
// their last tile column (two and four slots only).
inline bool ring_ragged(int64_t N, int64_t ldc, int out_bytes, bool brow) {
  const int epc = 16 / out_bytes;
  return N % epc != 0 || ldc % epc != 0 || (brow && N % 8 != 0);
}
const TileConfig& tile_config(int cfg);
bool tile_supports(int cfg, const Problem& p);
int tile_choose(const Problem& p);  // -1 when no config fits
LaunchFn tile_launcher(int cfg, const Problem& p);
// one translation unit per (input, output) format pair
LaunchFn tile_launcher_f16_f16(int cfg, int la, int lb, int epi);
LaunchFn tile_launcher_f16_f32(int cfg, int la, int lb, int epi);
LaunchFn tile_launcher_bf16_bf16(int cfg, int la, int lb, int epi);
LaunchFn tile_launcher_bf16_f32(int cfg, int la, int lb, int epi);
LaunchFn tile_launcher_f16_fp8(int cfg, int la, int lb, int epi);
LaunchFn tile_launcher_bf16_fp8(int cfg, int la, int lb, int epi);
// the ring configurations (5-7), one unit per (input, output) format pair
LaunchFn ring_launcher_f16_f16(int cfg, int la, int lb, int epi);
LaunchFn ring_launcher_f16_f32(int cfg, int la, int lb, int epi);
LaunchFn ring_launcher_f16_fp8(int cfg, int la, int lb, int epi);
LaunchFn ring_launcher_bf16_bf16(int cfg, int la, int lb, int epi);
LaunchFn ring_launcher_bf16_f32(int cfg, int la, int lb, int epi);
LaunchFn ring_launcher_bf16_fp8(int cfg, int la, int lb, int epi);
// the row-major-B 16x16x32 configuration, one unit per input format
LaunchFn tile16_rowb_launcher_f16(int out_dt, int la, int lb, int epi);
LaunchFn tile16_rowb_launcher_bf16(int out_dt, int la, int lb, int epi);

// ---- skinny: weight-streaming kernel for M <= 32 --------------------------
struct SkinnyConfig {
  int waves;   // waves per workgroup
  int stages;  // LDS ring slots: chunks in flight + the one being multiplied
  int kc;      // k-values per chunk
  const char* name;
  bool brow;   // B row-major (K x N, n contiguous) instead of column-major
  int cols;    // output columns per workgroup (32, or 64 with a row-major B)
};
int skinny_num_configs();
const SkinnyConfig& skinny_config(int cfg);
bool skinny_supports(int cfg, const Problem& p);
int skinny_choose(const Problem& p);
// K splits for configuration cfg when a workspace is given: doubled while
// the grid has fewer than 256 workgroups and every split keeps at least
// one chunk per ring slot (1: no split)
int skinny_split(int cfg, const Problem& p);
LaunchFn skinny_launcher(int cfg, const Problem& p);
// one unit per (input, output) format pair (gemm_skinny_<in>_<out>.hip)
LaunchFn skinny_launcher_f16_f16(int cfg, int epi);
LaunchFn skinny_launcher_f16_f32(int cfg, int epi);
LaunchFn skinny_launcher_f16_fp8(int cfg, int epi);
LaunchFn skinny_launcher_bf16_bf16(int cfg, int epi);
LaunchFn skinny_launcher_bf16_f32(int cfg, int epi);
LaunchFn skinny_launcher_bf16_fp8(int cfg, int epi);

// ---- cache eviction for cold-cache timing (flush.hip) ------------------------
// Bytes of the scratch buffer flush_caches reads: twice the 256 MB
// last-level cache.
constexpr size_t kFlushBytes = (size_t)512 << 20;
// Enqueue a kernel on `stream` that reads all kFlushBytes of `scratch`.
hipError_t flush_caches(void* scratch, hipStream_t stream);

// ---- diagnostics (gemm_epi.cpp) ----------------------------------------------
// Record a failed HIP call's code for gemm_epi_last_hip_error (per thread).
void set_last_hip_error(int code);
// The argument checks of gemm_epi_run (GEMM_EPI_OK when a run may proceed).
gemm_epi_status check_run_args(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias, const void* C);

// ---- tuning table (tuning.cpp) ---------------------------------------------
// The measured choice for this exact problem, if one was recorded.
bool tuning_lookup(const Problem& p, int* kernel, int* config);
void tuning_record(const Problem& p, int kernel, int config, float us);

}  // namespace ge
