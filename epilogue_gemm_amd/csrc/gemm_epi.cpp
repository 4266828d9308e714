// gemm_epi.cpp -- host side of the C ABI declared in include/gemm_epi.h:
// argument validation, kernel-family selection, launch on the caller's
// stream.  The plan is a small immutable host object; nothing here
// allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <new>

#include "kernels.hpp"

namespace ge {

// Tile configurations: workgroup tile BM x BN (k-step 64), its waves, each
// owning (BM/2) x (BN/(waves/2)), and the MFMA block.  Larger tiles reuse
// each loaded byte more; smaller ones give small problems enough workgroups
// for 256 CUs; 8 waves put two on each SIMD so one can multiply while the
// other waits; 16x16x32 blocks move half the accumulator bytes per FLOP
// (k-contiguous operands only).
// The ring configurations (64 x 64 tiles, K in 64-deep chunks through 8, 4
// or 2 LDS slots) serve problems whose tiles must be small to fill the CUs,
// where the two-stage pipeline waits on load latency at every k-step.
static const TileConfig kTile[] = {
    {256, 256, 4, "tile_256x256x64", 32, 0},
    {128, 128, 4, "tile_128x128x64", 32, 0},
    {64, 64, 4, "tile_64x64x64", 32, 0},
    {256, 256, 8, "tile_256x256x64_8w", 32, 0},
    {256, 256, 4, "tile_256x256x64_m16", 16, 0},
    {64, 64, 4, "tile_64x64_ring8", 32, 8},
    {64, 64, 4, "tile_64x64_ring4", 32, 4},
    {64, 64, 4, "tile_64x64_ring2", 32, 2},
    {256, 256, 4, "tile_256x256x64_m16_rowb", 16, 0, true},
};

int tile_num_configs() { return (int)(sizeof(kTile) / sizeof(kTile[0])); }
const TileConfig& tile_config(int cfg) { return kTile[cfg]; }

bool tile_supports(int cfg, const Problem& p) {
  if (cfg < 0 || cfg >= tile_num_configs()) return false;
  // M and N need not be tile multiples (the last tile row or column is
  // shifted back to end at M or N), but must hold one tile; rows of every
  // operand and of C must stay 16-byte aligned (N % 8, N % 16 for 1-byte
  // E4M3 output; M % 8 when A is column-major; leading dimensions likewise),
  // and K a multiple of 8 (16-byte chunks) spanning at least two k-steps of
  // 64 (a partial one first, when K % 64 != 0).
  // The 16x16x32 configurations take A row-major and B column-major, or B
  // row-major (its buffer range, K + 64 rows of ldb elements, must fit
  // 32-bit byte offsets).
  // The ring configurations take A and B in either layout; a row-major B's
  // buffer range (K + 64 rows of ldb elements) and a column-major A's (K +
  // 64 columns of lda elements) must fit 32-bit byte offsets.
  const TileConfig& c = kTile[cfg];
  const int n_align = p.out_dt == GEMM_EPI_FP8_E4M3 ? 16 : 8;
  if (c.mfma == 16 &&
      (p.la != GEMM_EPI_ROW_MAJOR || p.lb != (c.brow ? GEMM_EPI_ROW_MAJOR : GEMM_EPI_COL_MAJOR) ||
       (c.brow && (p.K + 64) * p.ldb * 2 >= ((int64_t)1 << 32))))
    return false;
  if (c.ring > 0 && ((p.la == GEMM_EPI_COL_MAJOR && (p.K + 64) * p.lda * 2 >= ((int64_t)1 << 32)) ||
                     (p.lb == GEMM_EPI_ROW_MAJOR && (p.K + 64) * p.ldb * 2 >= ((int64_t)1 << 32))))
    return false;
  // The ring configurations also take M and N below the tile (masked), K
  // <= 64, with A column-major any M (the last tile row masked), and any N
  // and ldc (the last tile column masked, edge outputs element by element);
  // the chunk count must be a multiple of the slot count, save for two
  // slots, which take any.
  const int64_t chunks = (p.K + 63) / 64;
  if (c.ring > 0) {
    const int out_bytes = p.out_dt == GEMM_EPI_F32 ? 4 : p.out_dt == GEMM_EPI_FP8_E4M3 ? 1 : 2;
    if (c.ring == 8 && ring_ragged(p.N, p.ldc, out_bytes, p.lb == GEMM_EPI_ROW_MAJOR)) return false;
    return p.M >= 1 && p.N >= 1 && p.K >= 8 && p.K % 8 == 0 && (chunks % c.ring == 0 || c.ring == 2) &&
           p.lda % 8 == 0 && p.ldb % 8 == 0;
  }
  // The 16x16x32 configuration with a column-major B also takes any N
  // and ldc: its last tile column is then masked, not shifted.
  const bool any_n = c.mfma == 16 && !c.brow;
  return p.M >= c.bm && p.N >= c.bn && (any_n || p.N % n_align == 0) &&
         (p.la == GEMM_EPI_ROW_MAJOR || p.M % 8 == 0) && p.K % 8 == 0 && p.K > 64 && p.lda % 8 == 0 &&
         p.ldb % 8 == 0 && (any_n || p.ldc % n_align == 0);
}

int tile_choose(const Problem& p) {
  // Largest tile that still gives at least one workgroup per CU; else the
  // smallest tile that fits (most parallelism).  With A row-major the 256 x
  // 256 tile runs on 16x16x32 MFMAs with 4 waves (8192^3 bf16 with B
  // column-major: 759 us against 829 us for 8 waves on 32x32x16); a
  // register-staged A keeps the 4-wave 32x32x16 kernel (8 waves measured
  // 12 % slower at 4096^3).
  const bool direct = p.la == GEMM_EPI_ROW_MAJOR && p.lb == GEMM_EPI_COL_MAJOR;
  int fallback = -1;
  for (int c = 0; c < 3; ++c) {
    if (!tile_supports(c, p)) continue;
    const int64_t tiles = ((p.M + kTile[c].bm - 1) / kTile[c].bm) * ((p.N + kTile[c].bn - 1) / kTile[c].bn);
    if (tiles >= 256) {
      fallback = c;
      break;
    }
    fallback = c;
  }
  if (fallback == 0 && direct) return 4;
  // N or ldc off the 16-byte output chunks leaves configurations 0-2; a
  // problem of at least 256 tiles of 256 x 256 still takes the 16x16x32
  // kernel, its last tile column masked
  if (fallback < 0 && direct && ((p.M + 255) / 256) * ((p.N + 255) / 256) >= 256 && tile_supports(4, p)) return 4;
  // both operands n- or k-contiguous along their rows (A row-major, B
  // row-major): the 16x16x32 kernel with transposing reads of B
  if (fallback == 0 && tile_supports(8, p)) return 8;
  // 64 x 64 tiles, or a problem no two-stage tile fits (M or N below 64,
  // K <= 64): a ring whose slot count divides the chunk count -- four slots
  // first (1024^3 fp16 ReLU: 5.0 us warm, 7.3 us on rotated operands,
  // against 5.5 and 7.4 us with eight slots and 7.9 and 11.3 us for the
  // two-stage kernel), then eight, then two
  if (fallback == 2 || fallback < 0)
    for (int c : {6, 5, 7})
      if (tile_supports(c, p)) return c;
  return fallback;
}

LaunchFn tile_launcher(int cfg, const Problem& p) {
  if (kTile[cfg].brow) {
    if (p.in_dt == GEMM_EPI_F16) return tile16_rowb_launcher_f16(p.out_dt, p.la, p.lb, p.epi);
    if (p.in_dt == GEMM_EPI_BF16) return tile16_rowb_launcher_bf16(p.out_dt, p.la, p.lb, p.epi);
    return nullptr;
  }
  const bool f32 = p.out_dt == GEMM_EPI_F32, fp8 = p.out_dt == GEMM_EPI_FP8_E4M3;
  if (kTile[cfg].ring > 0) {
    if (p.in_dt == GEMM_EPI_F16)
      return (fp8 ? ring_launcher_f16_fp8 : f32 ? ring_launcher_f16_f32 : ring_launcher_f16_f16)(cfg, p.la, p.lb,
                                                                                              p.epi);
    if (p.in_dt == GEMM_EPI_BF16)
      return (fp8 ? ring_launcher_bf16_fp8 : f32 ? ring_launcher_bf16_f32 : ring_launcher_bf16_bf16)(cfg, p.la, p.lb,
                                                                                                  p.epi);
    return nullptr;
  }
  if (p.in_dt == GEMM_EPI_F16)
    return (fp8 ? tile_launcher_f16_fp8 : f32 ? tile_launcher_f16_f32 : tile_launcher_f16_f16)(cfg, p.la, p.lb, p.epi);
  if (p.in_dt == GEMM_EPI_BF16)
    return (fp8 ? tile_launcher_bf16_fp8 : f32 ? tile_launcher_bf16_f32 : tile_launcher_bf16_bf16)(cfg, p.la, p.lb,
                                                                                                  p.epi);
  return nullptr;
}

}  // namespace ge

struct gemm_epi_plan_s {
  ge::Problem p;
  int kernel;  // gemm_epi_kernel actually used for aligned pointers
  int config;
  ge::LaunchFn fn;       // chosen family
  ge::LaunchFn generic;  // fallback for unaligned pointers
  const char* name;
  int split;  // K splits of a skinny plan when run with a workspace (1: none)
};

namespace {

thread_local int g_last_hip_error = 0;

}  // namespace

void ge::set_last_hip_error(int code) { g_last_hip_error = code; }

gemm_epi_status ge::check_run_args(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias,
                                   const void* C) {
  // with K = 0 A and B are never read (and may be NULL)
  if (!plan || !C || (plan->p.K > 0 && (!A || !B))) return GEMM_EPI_ERR_INVALID_ARG;
  const bool need_bias = plan->p.epi == GEMM_EPI_BIAS_RELU || plan->p.epi == GEMM_EPI_BIAS_GELU ||
                         plan->p.epi == GEMM_EPI_BIAS || plan->p.epi == GEMM_EPI_BIAS_SILU;
  if (need_bias != (bias != nullptr)) return GEMM_EPI_ERR_INVALID_ARG;
  return GEMM_EPI_OK;
}

namespace {

bool valid_enum_args(gemm_epi_dtype in, gemm_epi_dtype out, gemm_epi_layout la, gemm_epi_layout lb,
                     gemm_epi_epilogue epi) {
  if (in != GEMM_EPI_F16 && in != GEMM_EPI_BF16) return false;
  if (out != in && out != GEMM_EPI_F32 && out != GEMM_EPI_FP8_E4M3) return false;
  if ((la != GEMM_EPI_ROW_MAJOR && la != GEMM_EPI_COL_MAJOR) || (lb != GEMM_EPI_ROW_MAJOR && lb != GEMM_EPI_COL_MAJOR))
    return false;
  return epi >= GEMM_EPI_NONE && epi <= GEMM_EPI_BIAS_SILU;
}

bool uses_bias(int epi) {
  return epi == GEMM_EPI_BIAS_RELU || epi == GEMM_EPI_BIAS_GELU || epi == GEMM_EPI_BIAS || epi == GEMM_EPI_BIAS_SILU;
}

// Resolve (kernel, config) for the plan's problem; returns false if that
// family cannot run it.
bool resolve(gemm_epi_plan_s* pl, int kernel, int config) {
  const ge::Problem& p = pl->p;
  // K = 0 (C = act(bias) with the extras): the generic kernel only -- the
  // fast families stream K in 16-byte chunks
  if (p.K == 0 && kernel != GEMM_EPI_KERNEL_GENERIC) {
    if (kernel != GEMM_EPI_KERNEL_AUTO) return false;
    kernel = GEMM_EPI_KERNEL_GENERIC;
    config = 0;
  }
  if (kernel == GEMM_EPI_KERNEL_AUTO) {
    // a measured choice for this exact problem comes first
    int tk, tc;
    if (ge::tuning_lookup(p, &tk, &tc) && tk != GEMM_EPI_KERNEL_AUTO) {
      gemm_epi_plan_s trial = *pl;
      if (resolve(&trial, tk, tc)) {
        *pl = trial;
        return true;
      }
    }
    int c = ge::skinny_choose(p);
    if (c >= 0) return resolve(pl, GEMM_EPI_KERNEL_SKINNY, c);
    c = ge::tile_choose(p);
    if (c >= 0) return resolve(pl, GEMM_EPI_KERNEL_TILE, c);
    return resolve(pl, GEMM_EPI_KERNEL_GENERIC, 0);
  }
  if (kernel == GEMM_EPI_KERNEL_GENERIC) {
    if (config > 0) return false;
    pl->kernel = kernel;
    pl->config = 0;
    pl->fn = pl->generic;
    pl->name = "generic";
    pl->split = 1;
    return pl->fn != nullptr;
  }
  if (kernel == GEMM_EPI_KERNEL_TILE) {
    if (config < 0) config = ge::tile_choose(p);
    if (!ge::tile_supports(config, p)) return false;
    ge::LaunchFn fn = ge::tile_launcher(config, p);
    if (!fn) return false;
    pl->kernel = kernel;
    pl->config = config;
    pl->fn = fn;
    pl->name = ge::tile_config(config).name;
    pl->split = 1;
    return true;
  }
  if (kernel == GEMM_EPI_KERNEL_SKINNY) {
    if (config < 0) config = ge::skinny_choose(p);
    if (!ge::skinny_supports(config, p)) return false;
    ge::LaunchFn fn = ge::skinny_launcher(config, p);
    if (!fn) return false;
    pl->kernel = kernel;
    pl->config = config;
    pl->fn = fn;
    pl->name = ge::skinny_config(config).name;
    pl->split = ge::skinny_split(config, p);
    return true;
  }
  return false;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace of a split-K skinny run: one fp32 32 x cols partial block per
// (column block, split), then one arrival counter per column block.
size_t workspace_bytes(const gemm_epi_plan_s* pl) {
  if (pl->kernel != GEMM_EPI_KERNEL_SKINNY || pl->split <= 1) return 0;
  const int cols = ge::skinny_config(pl->config).cols;
  const size_t nblocks = (size_t)((pl->p.N + cols - 1) / cols);
  return nblocks * (size_t)pl->split * (128 * (size_t)cols) + ((nblocks * 4 + 255) & ~(size_t)255);
}

gemm_epi_status launch(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias,
                       const gemm_epi_extras* extras, void* C, void* workspace, size_t ws_bytes, void* stream) {
  const gemm_epi_status chk = ge::check_run_args(plan, A, B, bias, C);
  if (chk != GEMM_EPI_OK) return chk;
  const float* scale = extras ? extras->col_scale : nullptr;
  const void* residual = extras ? extras->residual : nullptr;
  const float* out_scale = extras ? extras->out_scale : nullptr;
  if (residual) {
    // no residual for a quantised output; and it must not overlap C (edge
    // tiles write some outputs twice)
    if (plan->p.out_dt == GEMM_EPI_FP8_E4M3) return GEMM_EPI_ERR_INVALID_ARG;
    const uintptr_t bytes =
        (uintptr_t)((plan->p.M - 1) * plan->p.ldc + plan->p.N) * (plan->p.out_dt == GEMM_EPI_F32 ? 4u : 2u);
    const uintptr_t r0 = (uintptr_t)residual, c0 = (uintptr_t)C;
    if (r0 < c0 + bytes && c0 < r0 + bytes) return GEMM_EPI_ERR_INVALID_ARG;
  }
  ge::LaunchArgs a;
  a.A = A;
  a.B = B;
  a.bias = bias;
  a.C = C;
  a.M = (int)plan->p.M;
  a.N = (int)plan->p.N;
  a.K = (int)plan->p.K;
  a.lda = (int)plan->p.lda;
  a.ldb = (int)plan->p.ldb;
  a.ldc = (int)plan->p.ldc;
  a.epi = plan->p.epi;
  a.la = plan->p.la;
  a.lb = plan->p.lb;
  a.stream = (hipStream_t)stream;
  a.workspace = nullptr;
  a.split = 1;
  a.scale = scale;
  a.residual = residual;
  a.out_scale = out_scale;
  const bool aligned = aligned16(A) && aligned16(B) && aligned16(C) && (!bias || aligned16(bias)) &&
                       (!scale || aligned16(scale)) && (!residual || aligned16(residual));
  const size_t need = workspace_bytes(plan);
  if (aligned && need > 0 && workspace && aligned16(workspace) && ws_bytes >= need) {
    a.workspace = workspace;
    a.split = plan->split;
  }
  ge::LaunchFn fn = aligned ? plan->fn : plan->generic;
  const hipError_t e = fn(a);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return GEMM_EPI_ERR_HIP;
  }
  return GEMM_EPI_OK;
}

}  // namespace

extern "C" {

gemm_epi_status gemm_epi_plan(gemm_epi_plan_t* out, int64_t M, int64_t N, int64_t K, gemm_epi_dtype in_dtype,
                              gemm_epi_dtype out_dtype, gemm_epi_layout layout_a, gemm_epi_layout layout_b,
                              gemm_epi_epilogue epilogue) {
  if (!out || M <= 0 || N <= 0 || K < 0) return GEMM_EPI_ERR_INVALID_ARG;
  if (!valid_enum_args(in_dtype, out_dtype, layout_a, layout_b, epilogue)) return GEMM_EPI_ERR_INVALID_ARG;
  const int64_t lim = (int64_t)1 << 31;
  if (M >= lim || N >= lim || K >= lim || M * K >= lim || K * N >= lim || M * N >= lim)
    return GEMM_EPI_ERR_UNSUPPORTED;
  gemm_epi_plan_s* pl = new (std::nothrow) gemm_epi_plan_s();
  if (!pl) return GEMM_EPI_ERR_NO_MEMORY;
  pl->p = ge::Problem{M,
                      N,
                      K,
                      (int)in_dtype,
                      (int)out_dtype,
                      (int)layout_a,
                      (int)layout_b,
                      (int)epilogue,
                      layout_a == GEMM_EPI_ROW_MAJOR ? K : M,
                      layout_b == GEMM_EPI_ROW_MAJOR ? N : K,
                      N};
  pl->generic = ge::generic_launcher(pl->p);
  if (!pl->generic || !resolve(pl, GEMM_EPI_KERNEL_AUTO, -1)) {
    delete pl;
    return GEMM_EPI_ERR_UNSUPPORTED;
  }
  *out = pl;
  return GEMM_EPI_OK;
}

gemm_epi_status gemm_epi_run(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias, void* C,
                             void* stream) {
  return launch(plan, A, B, bias, nullptr, C, nullptr, 0, stream);
}

size_t gemm_epi_workspace_size(gemm_epi_plan_t plan) { return plan ? workspace_bytes(plan) : 0; }

gemm_epi_status gemm_epi_run_ws(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias, void* C,
                                void* workspace, size_t workspace_bytes_given, void* stream) {
  return launch(plan, A, B, bias, nullptr, C, workspace, workspace_bytes_given, stream);
}

gemm_epi_status gemm_epi_run_ex(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias,
                                const gemm_epi_extras* extras, void* C, void* workspace, size_t workspace_bytes_given,
                                void* stream) {
  return launch(plan, A, B, bias, extras, C, workspace, workspace_bytes_given, stream);
}

gemm_epi_status gemm_epi_tune(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias, void* C,
                              int iters, int flags, void* stream, float* best_us) {
  if (!plan || !C || (plan->p.K > 0 && (!A || !B)) || iters <= 0 || (flags & ~GEMM_EPI_TUNE_COLD))
    return GEMM_EPI_ERR_INVALID_ARG;
  if (uses_bias(plan->p.epi) != (bias != nullptr)) return GEMM_EPI_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (bias && !aligned16(bias))) return GEMM_EPI_ERR_INVALID_ARG;
  // candidates: every configuration of the fast families that can run the
  // problem; the generic kernel only when none can
  struct Cand {
    int kernel, config;
  };
  Cand cands[64];
  int nc = 0;
  for (int k : {GEMM_EPI_KERNEL_TILE, GEMM_EPI_KERNEL_SKINNY}) {
    const int n = gemm_epi_num_configs((gemm_epi_kernel)k);
    for (int c = 0; c < n && nc < 64; ++c) {
      gemm_epi_plan_s trial = *plan;
      if (resolve(&trial, k, c)) cands[nc++] = Cand{k, c};
    }
  }
  if (nc == 0) cands[nc++] = Cand{GEMM_EPI_KERNEL_GENERIC, 0};
  const hipStream_t s = (hipStream_t)stream;
  const bool cold = (flags & GEMM_EPI_TUNE_COLD) != 0;
  void* scratch = nullptr;
  if (cold && hipMalloc(&scratch, ge::kFlushBytes) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_EPI_ERR_NO_MEMORY;
  }
  hipEvent_t ev[2] = {nullptr, nullptr};
  hipError_t e = hipEventCreate(&ev[0]);
  if (e == hipSuccess) e = hipEventCreate(&ev[1]);
  int best = -1;
  float best_t = 0.0f;
  for (int i = 0; i < nc && e == hipSuccess; ++i) {
    gemm_epi_plan_s trial = *plan;
    resolve(&trial, cands[i].kernel, cands[i].config);
    ge::LaunchArgs a{};
    a.A = A;
    a.B = B;
    a.bias = bias;
    a.C = C;
    a.M = (int)trial.p.M;
    a.N = (int)trial.p.N;
    a.K = (int)trial.p.K;
    a.lda = (int)trial.p.lda;
    a.ldb = (int)trial.p.ldb;
    a.ldc = (int)trial.p.ldc;
    a.epi = trial.p.epi;
    a.la = trial.p.la;
    a.lb = trial.p.lb;
    a.stream = s;
    a.split = 1;
    for (int w = 0; w < 2 && e == hipSuccess; ++w) e = trial.fn(a);  // warm-up
    float ms = 0.0f;
    if (!cold) {
      if (e == hipSuccess) e = hipEventRecord(ev[0], s);
      for (int r = 0; r < iters && e == hipSuccess; ++r) e = trial.fn(a);
      if (e == hipSuccess) e = hipEventRecord(ev[1], s);
      if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
    } else {
      for (int r = 0; r < iters && e == hipSuccess; ++r) {
        e = ge::flush_caches(scratch, s);
        if (e == hipSuccess) e = hipEventRecord(ev[0], s);
        if (e == hipSuccess) e = trial.fn(a);
        if (e == hipSuccess) e = hipEventRecord(ev[1], s);
        if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
        float one = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&one, ev[0], ev[1]);
        ms += one;
      }
    }
    if (e == hipSuccess && (best < 0 || ms < best_t)) {
      best = i;
      best_t = ms;
    }
  }
  for (hipEvent_t x : ev)
    if (x) (void)hipEventDestroy(x);
  if (scratch) {
    const hipError_t f = hipStreamSynchronize(s);
    if (e == hipSuccess) e = f;
    (void)hipFree(scratch);
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return GEMM_EPI_ERR_HIP;
  }
  const float us = best_t * 1000.0f / (float)iters;
  resolve(plan, cands[best].kernel, cands[best].config);
  ge::tuning_record(plan->p, cands[best].kernel, cands[best].config, us);
  if (best_us) *best_us = us;
  return GEMM_EPI_OK;
}

gemm_epi_status gemm_epi_plan_set_ld(gemm_epi_plan_t plan, int64_t lda, int64_t ldb, int64_t ldc) {
  if (!plan) return GEMM_EPI_ERR_INVALID_ARG;
  const ge::Problem& p = plan->p;
  // extent of a stored row (the contiguous one) and the number of rows
  const int64_t a_cols = p.la == GEMM_EPI_ROW_MAJOR ? p.K : p.M, a_rows = p.la == GEMM_EPI_ROW_MAJOR ? p.M : p.K;
  const int64_t b_cols = p.lb == GEMM_EPI_ROW_MAJOR ? p.N : p.K, b_rows = p.lb == GEMM_EPI_ROW_MAJOR ? p.K : p.N;
  if (lda == 0) lda = a_cols;
  if (ldb == 0) ldb = b_cols;
  if (ldc == 0) ldc = p.N;
  if (lda < a_cols || ldb < b_cols || ldc < p.N) return GEMM_EPI_ERR_INVALID_ARG;
  const int64_t lim = (int64_t)1 << 31;
  if (lda >= lim || ldb >= lim || ldc >= lim || (a_rows - 1) * lda + a_cols >= lim ||
      (b_rows - 1) * ldb + b_cols >= lim || (p.M - 1) * ldc + p.N >= lim)
    return GEMM_EPI_ERR_UNSUPPORTED;
  gemm_epi_plan_s trial = *plan;
  trial.p.lda = lda;
  trial.p.ldb = ldb;
  trial.p.ldc = ldc;
  if (!resolve(&trial, GEMM_EPI_KERNEL_AUTO, -1)) return GEMM_EPI_ERR_UNSUPPORTED;
  *plan = trial;
  return GEMM_EPI_OK;
}

gemm_epi_status gemm_epi_destroy(gemm_epi_plan_t plan) {
  delete plan;
  return GEMM_EPI_OK;
}

const char* gemm_epi_status_string(gemm_epi_status status) {
  switch (status) {
    case GEMM_EPI_OK: return "GEMM_EPI_OK";
    case GEMM_EPI_ERR_INVALID_ARG: return "GEMM_EPI_ERR_INVALID_ARG";
    case GEMM_EPI_ERR_UNSUPPORTED: return "GEMM_EPI_ERR_UNSUPPORTED";
    case GEMM_EPI_ERR_HIP: return "GEMM_EPI_ERR_HIP";
    case GEMM_EPI_ERR_NO_MEMORY: return "GEMM_EPI_ERR_NO_MEMORY";
    default: return "GEMM_EPI_ERR_UNKNOWN";
  }
}

int gemm_epi_last_hip_error(void) { return g_last_hip_error; }

gemm_epi_status gemm_epi_plan_select(gemm_epi_plan_t plan, gemm_epi_kernel kernel, int config) {
  if (!plan) return GEMM_EPI_ERR_INVALID_ARG;
  if (kernel < GEMM_EPI_KERNEL_AUTO || kernel > GEMM_EPI_KERNEL_SKINNY) return GEMM_EPI_ERR_INVALID_ARG;
  const int n = gemm_epi_num_configs(kernel);
  if (config < -1 || (kernel != GEMM_EPI_KERNEL_AUTO && config >= n)) return GEMM_EPI_ERR_INVALID_ARG;
  gemm_epi_plan_s trial = *plan;
  if (!resolve(&trial, kernel, kernel == GEMM_EPI_KERNEL_AUTO ? -1 : config)) return GEMM_EPI_ERR_UNSUPPORTED;
  *plan = trial;
  return GEMM_EPI_OK;
}

int gemm_epi_num_configs(gemm_epi_kernel kernel) {
  switch (kernel) {
    case GEMM_EPI_KERNEL_GENERIC: return 1;
    case GEMM_EPI_KERNEL_TILE: return ge::tile_num_configs();
    case GEMM_EPI_KERNEL_SKINNY: return ge::skinny_num_configs();
    default: return 0;
  }
}

const char* gemm_epi_plan_describe(gemm_epi_plan_t plan, gemm_epi_kernel* kernel, int* config) {
  if (!plan) return nullptr;
  if (kernel) *kernel = (gemm_epi_kernel)plan->kernel;
  if (config) *config = plan->config;
  return plan->name;
}

}  // extern "C"
