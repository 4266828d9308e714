// gemm_skinny.hip -- C = act(A.B [+ bias]) for M <= 32 rows with B stored
// N x K (k contiguous): the decode-like, weight-streaming shape.
//
// Every B element is used by at most 32 multiply-adds, so the kernel is
// bound by reading B from HBM once (the pages single out very long or very
// narrow matrices as the shapes where a custom kernel pays: csdn
// "从零开始学习 TileLang" ch.10 sec. 10.7).  What decides the rate is how
// many bytes of B each CU keeps in flight, so the design is about depth:
//
//   - a workgroup owns 32 consecutive output columns n and all of K; its NW
//     waves split K into NW contiguous ranges, so there is no reduction
//     across workgroups and bias and activation are applied exactly once;
//   - each wave streams its 32 x (K / NW) slice of B through a private LDS
//     ring of P stages of 32 rows x 64 k (4 KiB) with 128-bit buffer loads
//     that write LDS directly: 8 consecutive lanes read one full 128-byte
//     row segment, each lane fetching the chunk that belongs at its LDS
//     position under an XOR swizzle, so the loads are fully coalesced and
//     cost no VGPRs.  With P stages the wave has P k-chunks in flight; no
//     workgroup barrier is needed because each wave waits only for its own
//     loads (s_waitcnt vmcnt);
//   - A (at most 32 x K, the same for every workgroup, so it stays in L2)
//     goes straight into MFMA operand registers with the same depth P;
//   - one v_mfma_f32_32x32x16 per 16 k: B's rows are the first operand, A's
//     rows the second, giving lane l the outputs (m = l % 32,
//     n = 8 (v / 4) + 4 (l / 32) + v % 4) of accumulator v;
//   - the NW partial 32x32 blocks are summed through LDS in a fixed order,
//     then bias, activation, conversion and one store per output.
//
// Within each 16-k MFMA step lane half h takes k = 8h .. 8h + 7 of both
// operands, so every product pairs matching k.
#include "kernels.hpp"

namespace ge {
namespace {

constexpr int kChunk = 64;              // k per stage
constexpr int kStageBytes = 32 * 128;   // 32 rows x 64 k x 2 bytes

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Ring slot J of every wave: one __shared__ object per slot, so that the
// compiler can tell a read of one slot from a direct load in flight into
// another.
template <int J, int NW>
__device__ __forceinline__ char* ring_slot() {
  __shared__ __attribute__((aligned(1024))) char slot[NW * kStageBytes];
  return slot;
}

template <int P, int NW, int... J>
__device__ __forceinline__ void ring_slots(char* (&s)[P], int wave, std::integer_sequence<int, J...>) {
  ((s[J] = ring_slot<J, NW>() + wave * kStageBytes), ...);
}

template <typename TIn, typename TOut, int NW, int P, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                              const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                              int M, int N, int K) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 32;
  const int kw = K / NW;  // this wave's k range: [wave * kw, wave * kw + kw)
  const int k0 = wave * kw;
  const int steps = kw / kChunk;  // a multiple of P (checked on the host)

  char* slot[P];
  ring_slots<P, NW>(slot, wave, std::make_integer_sequence<int, P>{});

  // B: rows n0 .. n0 + 31.  Instruction i of a stage fills LDS rows
  // 8i .. 8i + 7; lane L lands at row 8i + L / 8, chunk position L % 8, and
  // chunk c of row r sits at position c ^ (r % 8), so the lane loads
  // logical chunk (L % 8) ^ (L / 8).
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (int64_t)n0 * K, (uint32_t)(32u * (uint32_t)K * 2u));
  const uint32_t row_bytes = (uint32_t)K * 2u;
  const uint32_t vb = (uint32_t)(lane >> 3) * row_bytes + (uint32_t)k0 * 2u +
                      (uint32_t)((((lane & 7) ^ (lane >> 3))) << 4);

  // A: rows past M read as zero (outside the buffer resource).
  const int r = lane & 31, h = lane >> 5;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2u);
  const uint32_t va = (uint32_t)r * row_bytes + (uint32_t)k0 * 2u + (uint32_t)h * 16u;

  // B fragment of MFMA q: row r, logical chunk 2q + h.
  int rd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rd[q] = r * 128 + ((((2 * q + h) ^ (r & 7))) << 4);

  u32x4 a[P][4];
  f32x16 acc = f32x16{};

  auto issue = [&](int j, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(slot[j] + i * 1024), 16, vb,
                                               (uint32_t)i * 8u * row_bytes + (uint32_t)s * 128u, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      a[j][q] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)va, (int)((uint32_t)s * 128u + 32u * q), 0));
  };
  auto compute = [&](int j) __attribute__((always_inline)) {
    u32x4 b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = *(const u32x4*)(slot[j] + rd[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = mfma32<TIn>(b[q], a[j][q], acc);
  };

  // 8 vector-memory operations per stage: 4 direct B loads, 4 A loads
  constexpr int kOps = 8;
#pragma unroll
  for (int j = 0; j < P; ++j) issue(j, j);

  int s0 = 0;
  for (; s0 + P < steps; s0 += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      // stage s0 + j complete; the P - 1 later stages may stay in flight
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kOps * (P - 1)));
      compute(j);
      __builtin_amdgcn_sched_barrier(0);
      issue(j, s0 + j + P);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  static_for<P>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kOps * (P - 1 - j)));
    compute(j);
  });

  // Partial sums of the NW waves through LDS (slot 0 is reused once every
  // wave has finished reading the ring), summed in wave order.
  __syncthreads();
  float* red = (float*)ring_slot<0, NW>();
#pragma unroll
  for (int v = 0; v < 16; ++v) red[(wave * 16 + v) * 64 + lane] = acc[v];
  __syncthreads();

  // output (m, n_local), consecutive threads -> consecutive columns
  for (int o = tid; o < 32 * 32; o += NW * 64) {
    const int nl = o & 31, m = o >> 5;
    if (m >= M) continue;
    const int src_lane = m + 32 * ((nl >> 2) & 1);
    const int v = (nl >> 3) * 4 + (nl & 3);
    float z = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) z += red[(w * 16 + v) * 64 + src_lane];
    float b = 0.0f;
    if constexpr (epi_has_bias<EPI>()) b = to_f32(bias[n0 + nl]);
    C[(int64_t)m * N + n0 + nl] = from_f32<TOut>(epilogue<EPI>(z, b));
  }
}

template <typename TIn, typename TOut, int NW, int P, int EPI>
hipError_t launch_skinny(const LaunchArgs& a) {
  hipLaunchKernelGGL((gemm_skinny_kernel<TIn, TOut, NW, P, EPI>), dim3(a.N / 32), dim3(NW * 64), 0, a.stream,
                     (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K);
  return hipGetLastError();
}

template <typename TIn, typename TOut, int NW, int P>
LaunchFn pick_epi(int epi) {
  switch (epi) {
    case GEMM_EPI_NONE: return &launch_skinny<TIn, TOut, NW, P, GEMM_EPI_NONE>;
    case GEMM_EPI_RELU: return &launch_skinny<TIn, TOut, NW, P, GEMM_EPI_RELU>;
    case GEMM_EPI_BIAS_RELU: return &launch_skinny<TIn, TOut, NW, P, GEMM_EPI_BIAS_RELU>;
    case GEMM_EPI_BIAS_GELU: return &launch_skinny<TIn, TOut, NW, P, GEMM_EPI_BIAS_GELU>;
    case GEMM_EPI_BIAS: return &launch_skinny<TIn, TOut, NW, P, GEMM_EPI_BIAS>;
    default: return nullptr;
  }
}

template <int NW, int P>
LaunchFn pick_types(const Problem& p) {
  if (p.in_dt == GEMM_EPI_F16) {
    if (p.out_dt == GEMM_EPI_F16) return pick_epi<f16, f16, NW, P>(p.epi);
    if (p.out_dt == GEMM_EPI_F32) return pick_epi<f16, float, NW, P>(p.epi);
  } else if (p.in_dt == GEMM_EPI_BF16) {
    if (p.out_dt == GEMM_EPI_BF16) return pick_epi<bf16, bf16, NW, P>(p.epi);
    if (p.out_dt == GEMM_EPI_F32) return pick_epi<bf16, float, NW, P>(p.epi);
  }
  return nullptr;
}

// In order of preference; the plan takes the first one whose k granularity
// (64 * waves * stages) divides K.  Each keeps waves x stages x 4 KiB of B
// in flight per workgroup (one workgroup per CU at N = 8192).
const SkinnyConfig kSkinny[] = {
    {8, 4, "skinny_32n_8w_4s"},   // 128 KiB ring
    {16, 2, "skinny_32n_16w_2s"}, // 128 KiB ring
    {4, 8, "skinny_32n_4w_8s"},   // 128 KiB ring
    {8, 2, "skinny_32n_8w_2s"},   // 64 KiB ring
    {4, 4, "skinny_32n_4w_4s"},
    {4, 2, "skinny_32n_4w_2s"},
    {4, 1, "skinny_32n_4w_1s"},
    {1, 1, "skinny_32n_1w_1s"},   // any K divisible by 64
};

}  // namespace

int skinny_num_configs() { return (int)(sizeof(kSkinny) / sizeof(kSkinny[0])); }
const SkinnyConfig& skinny_config(int cfg) { return kSkinny[cfg]; }

bool skinny_supports(int cfg, const Problem& p) {
  if (cfg < 0 || cfg >= skinny_num_configs()) return false;
  const int64_t gran = (int64_t)kChunk * kSkinny[cfg].waves * kSkinny[cfg].stages;
  // 32 rows of B and all of A must be addressable by one buffer resource
  return p.M >= 1 && p.M <= 32 && p.la == GEMM_EPI_ROW_MAJOR && p.lb == GEMM_EPI_COL_MAJOR && p.N % 32 == 0 &&
         p.K % gran == 0 && 32 * p.K * 2 < ((int64_t)1 << 32);
}

int skinny_choose(const Problem& p) {
  for (int c = 0; c < skinny_num_configs(); ++c)
    if (skinny_supports(c, p)) return c;
  return -1;
}

LaunchFn skinny_launcher(int cfg, const Problem& p) {
  const SkinnyConfig& c = kSkinny[cfg];
  if (c.waves == 8 && c.stages == 4) return pick_types<8, 4>(p);
  if (c.waves == 16 && c.stages == 2) return pick_types<16, 2>(p);
  if (c.waves == 4 && c.stages == 8) return pick_types<4, 8>(p);
  if (c.waves == 8 && c.stages == 2) return pick_types<8, 2>(p);
  if (c.waves == 4 && c.stages == 4) return pick_types<4, 4>(p);
  if (c.waves == 4 && c.stages == 2) return pick_types<4, 2>(p);
  if (c.waves == 4 && c.stages == 1) return pick_types<4, 1>(p);
  if (c.waves == 1 && c.stages == 1) return pick_types<1, 1>(p);
  return nullptr;
}

}  // namespace ge
