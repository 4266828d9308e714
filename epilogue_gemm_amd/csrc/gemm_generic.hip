// gemm_generic.hip -- correctness anchor: fp32 fused multiply-add over k in
// order, the fp32 epilogue, one store per output.  Handles any M, N, K
// (K = 0 included), either layout of A and B, any leading dimensions and
// any pointer alignment; the plan uses it only where the fast kernels do
// not apply.
//
// A product of two fp16 (11-bit significands) or two bf16 (8-bit) values is
// exact in fp32, so each fma adds an exact product to the running sum; every
// output's sum takes k = 0, 1, ..., K - 1 in order, whatever the tiling.
//
// Workgroups of 16 x 16 threads own 64 x 64 outputs, thread (tx, ty) rows
// 4 ty .. 4 ty + 3 and columns 4 tx .. 4 tx + 3.  K advances 16 at a time
// through LDS (fp32, k-major, zeros outside the operands), each operand
// element read from memory once per workgroup with 2-byte loads ordered
// along the operand's contiguous axis; the last k-step stops at K, so no
// extra fma touches a sum (which would turn a -0 into +0).
#include "kernels.hpp"

namespace ge {
namespace {

constexpr int kGT = 64;  // outputs per workgroup along M and N
constexpr int kGK = 16;  // k per LDS step

template <typename TIn, typename TOut, int EPI>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                           const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                           int64_t M, int64_t N, int64_t K, int la, int lb,
                                                           int64_t lda, int64_t ldb, int64_t ldc,
                                                           const float* __restrict__ scale,
                                                           const TOut* __restrict__ res,
                                                           const float* __restrict__ out_scale) {
  __shared__ __attribute__((aligned(16))) float As[kGK][kGT];  // As[k][m]
  __shared__ __attribute__((aligned(16))) float Bs[kGK][kGT];  // Bs[k][n]
  const int tx = threadIdx.x, ty = threadIdx.y, tid = ty * 16 + tx;
  const int64_t n0 = (int64_t)blockIdx.x * kGT;
  const int64_t tiles_m = (M + kGT - 1) / kGT;
  // rows beyond what the grid's y extent covers are looped over
  for (int64_t mt = blockIdx.y; mt < tiles_m; mt += gridDim.y) {
    const int64_t m0 = mt * kGT;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += kGK) {
      // this step's tiles: element e of a thread is tile index tid + 256 e;
      // consecutive threads walk the operand's contiguous axis
      float av[4], bv[4];
      int ar[4], ac[4], br[4], bc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = tid + 256 * e;
        // A: row r of the tile (m), column c (k)
        const int r = la == GEMM_EPI_ROW_MAJOR ? idx / kGK : idx % kGT;
        const int c = la == GEMM_EPI_ROW_MAJOR ? idx % kGK : idx / kGT;
        const int64_t m = m0 + r, k = k0 + c;
        av[e] = 0.0f;
        if (m < M && k < K) av[e] = to_f32(la == GEMM_EPI_ROW_MAJOR ? A[m * lda + k] : A[k * lda + m]);
        ar[e] = r;
        ac[e] = c;
        // B: k-row c2, column r2 (n)
        const int r2 = lb == GEMM_EPI_ROW_MAJOR ? idx % kGT : idx / kGK;
        const int c2 = lb == GEMM_EPI_ROW_MAJOR ? idx / kGT : idx % kGK;
        const int64_t n = n0 + r2, k2 = k0 + c2;
        bv[e] = 0.0f;
        if (n < N && k2 < K) bv[e] = to_f32(lb == GEMM_EPI_ROW_MAJOR ? B[k2 * ldb + n] : B[n * ldb + k2]);
        br[e] = r2;
        bc[e] = c2;
      }
      __syncthreads();  // the previous step's reads are done
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        As[ac[e]][ar[e]] = av[e];
        Bs[bc[e]][br[e]] = bv[e];
      }
      __syncthreads();
      const int kn = (int)(K - k0 < kGK ? K - k0 : kGK);
      for (int kk = 0; kk < kn; ++kk) {
        const f32x4 a = *(const f32x4*)&As[kk][4 * ty];
        const f32x4 b = *(const f32x4*)&Bs[kk][4 * tx];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
      }
    }
    const float os = out_scale ? *out_scale : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 4 * ty + i;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + 4 * tx + j;
        if (n >= N) continue;
        float b = 0.0f;
        if constexpr (epi_has_bias<EPI>()) b = to_f32(bias[n]);
        const float s = scale ? scale[n] : 1.0f;
        const float r = res ? out_to_f32(res[m * ldc + n]) : 0.0f;
        C[m * ldc + n] = from_f32<TOut>(epilogue_ex<EPI>(acc[i][j], b, scale != nullptr, s, res != nullptr, r,
                                                         out_scale != nullptr, os));
      }
    }
  }
}

template <typename TIn, typename TOut, int EPI>
hipError_t launch_generic(const LaunchArgs& a) {
  // x: column tiles (at most 2^31 / 64 of them: 16 work-items each, inside
  // the 2^32 - 1 a grid dimension allows); y: row tiles, looped past 65535
  const int64_t gx = ((int64_t)a.N + kGT - 1) / kGT;
  int64_t gy = ((int64_t)a.M + kGT - 1) / kGT;
  if (gy > 65535) gy = 65535;
  hipLaunchKernelGGL((gemm_generic_kernel<TIn, TOut, EPI>), dim3((unsigned)gx, (unsigned)gy), dim3(16, 16), 0,
                     a.stream, (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, (int64_t)a.M,
                     (int64_t)a.N, (int64_t)a.K, a.la, a.lb, (int64_t)a.lda, (int64_t)a.ldb, (int64_t)a.ldc, a.scale,
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
