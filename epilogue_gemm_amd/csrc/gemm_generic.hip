// gemm_generic.hip -- correctness anchor: one thread per output element,
// fp32 fused multiply-add over k, the fp32 epilogue, one store.  Handles any
// M, N, K, either layout of A and B and any pointer alignment.  Slow by
// design; the plan uses it only where the fast kernels do not apply.
//
// A product of two fp16 (11-bit significands) or two bf16 (8-bit) values is
// exact in fp32, so each fma adds an exact product to the running sum.
#include "kernels.hpp"

namespace ge {
namespace {

// Workgroups of 64 x 4 threads: x along N (a wave reads and writes
// consecutive columns), y along M.  The grid's x extent in work-items is
// then N rounded up to 64 (below 2^31 + 64, inside the 2^32 - 1 a grid
// dimension allows, for every N a plan accepts); rows beyond what the y
// extent covers are looped over.
constexpr int kGenThreadsX = 64;
constexpr int kGenThreadsY = 4;

template <typename TIn, typename TOut, int EPI>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                           const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                           int64_t M, int64_t N, int64_t K, int la, int lb,
                                                           int64_t lda, int64_t ldb, int64_t ldc,
                                                           const float* __restrict__ scale,
                                                           const TOut* __restrict__ res,
                                                           const float* __restrict__ out_scale) {
  const int64_t j = (int64_t)blockIdx.x * kGenThreadsX + threadIdx.x;
  if (j >= N) return;
  const int64_t i_step = (int64_t)gridDim.y * kGenThreadsY;
  for (int64_t i = (int64_t)blockIdx.y * kGenThreadsY + threadIdx.y; i < M; i += i_step) {
    // element strides of a(i, k) and b(k, j) along k
    const TIn* pa = la == GEMM_EPI_ROW_MAJOR ? A + i * lda : A + i;
    const int64_t sa = la == GEMM_EPI_ROW_MAJOR ? 1 : lda;
    const TIn* pb = lb == GEMM_EPI_ROW_MAJOR ? B + j : B + j * ldb;
    const int64_t sb = lb == GEMM_EPI_ROW_MAJOR ? ldb : 1;
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) acc = __builtin_fmaf(to_f32(pa[k * sa]), to_f32(pb[k * sb]), acc);
    float b = 0.0f;
    if constexpr (epi_has_bias<EPI>()) b = to_f32(bias[j]);
    const float s = scale ? scale[j] : 1.0f;
    const float r = res ? out_to_f32(res[i * ldc + j]) : 0.0f;
    const float os = out_scale ? *out_scale : 1.0f;
    C[i * ldc + j] = from_f32<TOut>(epilogue_ex<EPI>(acc, b, scale != nullptr, s, res != nullptr, r, out_scale != nullptr, os));
  }
}

template <typename TIn, typename TOut, int EPI>
hipError_t launch_generic(const LaunchArgs& a) {
  const int64_t gx = ((int64_t)a.N + kGenThreadsX - 1) / kGenThreadsX;
  int64_t gy = ((int64_t)a.M + kGenThreadsY - 1) / kGenThreadsY;
  if (gy > 65535) gy = 65535;
  hipLaunchKernelGGL((gemm_generic_kernel<TIn, TOut, EPI>), dim3((unsigned)gx, (unsigned)gy), dim3(kGenThreadsX, kGenThreadsY), 0, a.stream,
                     (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, (int64_t)a.M, (int64_t)a.N,
                     (int64_t)a.K, a.la, a.lb, (int64_t)a.lda, (int64_t)a.ldb, (int64_t)a.ldc, a.scale,
                     (const TOut*)a.residual, a.out_scale);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
LaunchFn pick_epi(int epi) {
  switch (epi) {
    case GEMM_EPI_NONE: return &launch_generic<TIn, TOut, GEMM_EPI_NONE>;
    case GEMM_EPI_RELU: return &launch_generic<TIn, TOut, GEMM_EPI_RELU>;
    case GEMM_EPI_BIAS_RELU: return &launch_generic<TIn, TOut, GEMM_EPI_BIAS_RELU>;
    case GEMM_EPI_BIAS_GELU: return &launch_generic<TIn, TOut, GEMM_EPI_BIAS_GELU>;
    case GEMM_EPI_BIAS: return &launch_generic<TIn, TOut, GEMM_EPI_BIAS>;
    case GEMM_EPI_SILU: return &launch_generic<TIn, TOut, GEMM_EPI_SILU>;
    case GEMM_EPI_BIAS_SILU: return &launch_generic<TIn, TOut, GEMM_EPI_BIAS_SILU>;
    default: return nullptr;
  }
}

}  // namespace

LaunchFn generic_launcher(const Problem& p) {
  if (p.in_dt == GEMM_EPI_F16) {
    if (p.out_dt == GEMM_EPI_F16) return pick_epi<f16, f16>(p.epi);
    if (p.out_dt == GEMM_EPI_F32) return pick_epi<f16, float>(p.epi);
    if (p.out_dt == GEMM_EPI_FP8_E4M3) return pick_epi<f16, fp8e4m3>(p.epi);
  } else if (p.in_dt == GEMM_EPI_BF16) {
    if (p.out_dt == GEMM_EPI_BF16) return pick_epi<bf16, bf16>(p.epi);
    if (p.out_dt == GEMM_EPI_F32) return pick_epi<bf16, float>(p.epi);
    if (p.out_dt == GEMM_EPI_FP8_E4M3) return pick_epi<bf16, fp8e4m3>(p.epi);
  }
  return nullptr;
}

}  // namespace ge
