// gemm_skinny.hip -- C = act(A.B + bias) for M <= 32 rows with B stored
// N x K (k contiguous): the decode-like, weight-streaming shape.
//
// Every B element is used by at most 32 multiply-adds, so the kernel is
// bound by reading B from HBM once (the pages single out very long or very
// narrow matrices as the shapes where a custom kernel pays: csdn
// "从零开始学习 TileLang" ch.10 sec. 10.7).  Design:
//   - a workgroup owns 32 consecutive output columns n and all of K; its
//     NW waves split K into NW contiguous ranges (no cross-workgroup
//     reduction, so bias and the activation are applied exactly once);
//   - each lane streams 64 contiguous bytes of one B row per 64-k chunk
//     straight into MFMA operand registers (two lanes cover one 128-byte
//     line), with the next chunk's loads in flight while the current one is
//     multiplied; A (at most 32 x K) is read the same way and stays hot in L2;
//   - one v_mfma_f32_32x32x16 per 16 k: B's rows are the first operand, A's
//     rows the second, giving lane l the outputs (m = l % 32,
//     n = 8q + 4(l / 32) + e);
//   - the NW partial 32x32 blocks are summed through LDS in a fixed order,
//     then bias, activation, conversion and one store per output.
//
// The k index inside one 64-chunk is permuted identically for both
// operands (lane half h, step q, element e -> k = 32 h + 8 q + e), which
// leaves the sum unchanged.
#include "kernels.hpp"

namespace ge {
namespace {

constexpr int kChunk = 64;  // k per loop step

template <typename TIn, typename TOut, int NW, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                              const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                              int M, int N, int K) {
  __shared__ float red[NW][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 32;
  const int kw = K / NW;  // this wave's k range: [wave * kw, wave * kw + kw)
  const int h = lane >> 5, r = lane & 31;

  const char* pb = (const char*)(B + (int64_t)(n0 + r) * K + wave * kw + 32 * h);
  const bool a_row = r < M;
  const char* pa = (const char*)(A + (int64_t)(a_row ? r : 0) * K + wave * kw + 32 * h);

  f32x16 acc = f32x16{};
  u32x4 bc[4], ac[4], bn[4], an[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bc[q] = *(const u32x4*)(pb + 16 * q);
    ac[q] = a_row ? *(const u32x4*)(pa + 16 * q) : u32x4{0u, 0u, 0u, 0u};
  }
  const int steps = kw / kChunk;
  for (int s = 0; s < steps; ++s) {
    if (s + 1 < steps) {
      const int off = (s + 1) * kChunk * 2;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bn[q] = *(const u32x4*)(pb + off + 16 * q);
        an[q] = a_row ? *(const u32x4*)(pa + off + 16 * q) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = mfma32<TIn>(bc[q], ac[q], acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bc[q] = bn[q];
      ac[q] = an[q];
    }
  }

#pragma unroll
  for (int v = 0; v < 16; ++v) red[wave][v][lane] = acc[v];
  __syncthreads();

  // output (m, n_local), consecutive threads -> consecutive columns
  for (int o = tid; o < 32 * 32; o += NW * 64) {
    const int nl = o & 31, m = o >> 5;
    if (m >= M) continue;
    const int src_lane = m + 32 * ((nl >> 2) & 1);
    const int v = (nl >> 3) * 4 + (nl & 3);
    float z = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) z += red[w][v][src_lane];
    float b = 0.0f;
    if constexpr (epi_has_bias<EPI>()) b = to_f32(bias[n0 + nl]);
    C[(int64_t)m * N + n0 + nl] = from_f32<TOut>(epilogue<EPI>(z, b));
  }
}

template <typename TIn, typename TOut, int NW, int EPI>
hipError_t launch_skinny(const LaunchArgs& a) {
  hipLaunchKernelGGL((gemm_skinny_kernel<TIn, TOut, NW, EPI>), dim3(a.N / 32), dim3(NW * 64), 0, a.stream,
                     (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K);
  return hipGetLastError();
}

template <typename TIn, typename TOut, int NW>
LaunchFn pick_epi(int epi) {
  switch (epi) {
    case GEMM_EPI_NONE: return &launch_skinny<TIn, TOut, NW, GEMM_EPI_NONE>;
    case GEMM_EPI_RELU: return &launch_skinny<TIn, TOut, NW, GEMM_EPI_RELU>;
    case GEMM_EPI_BIAS_RELU: return &launch_skinny<TIn, TOut, NW, GEMM_EPI_BIAS_RELU>;
    case GEMM_EPI_BIAS_GELU: return &launch_skinny<TIn, TOut, NW, GEMM_EPI_BIAS_GELU>;
    case GEMM_EPI_BIAS: return &launch_skinny<TIn, TOut, NW, GEMM_EPI_BIAS>;
    default: return nullptr;
  }
}

template <int NW>
LaunchFn pick_types(const Problem& p) {
  if (p.in_dt == GEMM_EPI_F16) {
    if (p.out_dt == GEMM_EPI_F16) return pick_epi<f16, f16, NW>(p.epi);
    if (p.out_dt == GEMM_EPI_F32) return pick_epi<f16, float, NW>(p.epi);
  } else if (p.in_dt == GEMM_EPI_BF16) {
    if (p.out_dt == GEMM_EPI_BF16) return pick_epi<bf16, bf16, NW>(p.epi);
    if (p.out_dt == GEMM_EPI_F32) return pick_epi<bf16, float, NW>(p.epi);
  }
  return nullptr;
}

const SkinnyConfig kSkinny[] = {
    {16, "skinny_32n_16waves"},
    {8, "skinny_32n_8waves"},
    {4, "skinny_32n_4waves"},
};

}  // namespace

int skinny_num_configs() { return (int)(sizeof(kSkinny) / sizeof(kSkinny[0])); }
const SkinnyConfig& skinny_config(int cfg) { return kSkinny[cfg]; }

bool skinny_supports(int cfg, const Problem& p) {
  if (cfg < 0 || cfg >= skinny_num_configs()) return false;
  const int nw = kSkinny[cfg].waves;
  return p.M >= 1 && p.M <= 32 && p.la == GEMM_EPI_ROW_MAJOR && p.lb == GEMM_EPI_COL_MAJOR && p.N % 32 == 0 &&
         p.K % (kChunk * nw) == 0;
}

int skinny_choose(const Problem& p) {
  for (int c = 0; c < skinny_num_configs(); ++c)
    if (skinny_supports(c, p)) return c;
  return -1;
}

LaunchFn skinny_launcher(int cfg, const Problem& p) {
  switch (kSkinny[cfg].waves) {
    case 16: return pick_types<16>(p);
    case 8: return pick_types<8>(p);
    case 4: return pick_types<4>(p);
    default: return nullptr;
  }
}

}  // namespace ge
