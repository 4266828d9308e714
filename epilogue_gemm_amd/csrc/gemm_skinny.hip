// gemm_skinny.hip -- C = act(A.B [+ bias]) for M <= 32 rows with B stored
// N x K (k contiguous): the decode-like, weight-streaming shape.
//
// Every B element is used by at most 32 multiply-adds, so the kernel is
// bound by reading B from HBM once (the pages single out very long or very
// narrow matrices as the shapes where a custom kernel pays: csdn
// "从零开始学习 TileLang" ch.10 sec. 10.7).  The design is about keeping
// HBM busy with long contiguous reads:
//
//   - a workgroup owns 32 consecutive output columns n and all of K, so
//     there is no reduction across workgroups and bias and activation are
//     applied exactly once;
//   - K is walked in chunks of KC values.  A chunk of B is 32 rows x KC
//     k-values, and every row segment of it (2 KC bytes) is contiguous in
//     memory: the NW waves copy it into one LDS ring slot with 128-bit
//     buffer loads that write LDS directly, each wave instruction reading
//     1 KiB of consecutive bytes (one row segment, or two or four shorter
//     ones), each lane fetching the 16-byte chunk that belongs at its LDS
//     position under an XOR swizzle.  Long contiguous segments are what
//     keeps HBM close to its streaming rate; the direct loads cost no VGPRs;
//   - workgroup b starts its walk over the chunks at chunk b (mod the
//     count), so that concurrent workgroups read different k offsets: when
//     all of them read the same offset of their rows at once, the traffic
//     bunches on a subset of the HBM channels and the rate drops by a third;
//   - the ring has P slots: while chunk c is multiplied, chunks c+1 ..
//     c+P-1 are in flight.  One workgroup barrier per chunk, after each
//     wave has waited for its own loads of chunk c (s_waitcnt vmcnt), makes
//     the slot complete; it also proves every wave has finished chunk c-1,
//     whose slot then receives chunk c+P-1;
//   - inside a chunk, wave w multiplies its own KC/NW k-values:
//     v_mfma_f32_32x32x16 with B's rows as the first operand (from LDS) and
//     A's rows as the second (A is at most 32 x K and the same for every
//     workgroup, so it is read from L2 straight into operand registers,
//     issued with the chunk's B loads).  Lane l then holds the outputs
//     (m = l % 32, n = 8 (v / 4) + 4 (l / 32) + v % 4) of accumulator v;
//   - the NW partial 32x32 blocks are summed through LDS in wave order,
//     then bias, activation, conversion and one store per output.
//
// Within each 16-k MFMA step lane half h takes k = 8h .. 8h + 7 of both
// operands, so every product pairs matching k.
#include "kernels.hpp"

namespace ge {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, 0);
}

// Ring slot J: one __shared__ object per slot, so that the compiler can
// tell a read of one slot from a direct load in flight into another.
template <int J, int BYTES>
__device__ __forceinline__ char* ring_slot() {
  __shared__ __attribute__((aligned(1024))) char slot[BYTES];
  return slot;
}

template <int BYTES, int P, int... J, int OFF = 0>
__device__ __forceinline__ void ring_slots(char* (&s)[P], std::integer_sequence<int, J...>,
                                           std::integral_constant<int, OFF> = {}) {
  ((s[J] = ring_slot<OFF + J, BYTES>()), ...);
}

// The chunk in the oldest ring slot is complete for the whole workgroup
// once each wave has at most PENDING of its own memory operations
// outstanding and all waves have met; the barrier also orders every wave's
// reads of the previous slot before the loads that overwrite it.
template <int PENDING>
__device__ __forceinline__ void arrive() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(PENDING));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <typename TIn, typename TOut, int NW, int P, int KC, bool A_LDS, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                              const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                              int M, int N, int K) {
  constexpr int RB = KC * 2;            // bytes of one row segment of a chunk
  constexpr int SLOT = 32 * RB;         // one ring slot: 32 rows of B
  constexpr int MF = KC / 16 / NW;      // MFMAs per wave per chunk
  constexpr int ND = SLOT / 1024 / NW;  // direct-load instructions per wave per chunk
  // vector-memory operations per wave per chunk
  constexpr int OPS = ND + (A_LDS ? ND : MF);
  static_assert(MF >= 1 && ND >= 1 && RB >= 256 && RB <= 1024 && P >= 2, "chunk shape");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 32;
  const int nchunks = K / KC;  // a multiple of P (checked on the host)

  // Workgroup b walks the chunks starting at chunk b (mod the count): at
  // any moment the workgroups read at spread-out k offsets of their rows
  // instead of all at the same one, which keeps the load spread evenly over
  // the HBM channels.  (The k order does not change the sum beyond fp32
  // rounding, and each workgroup's order is fixed.)
  const int rot = (int)(blockIdx.x % (unsigned)nchunks);

  char* slot[P];
  ring_slots<SLOT, P>(slot, std::make_integer_sequence<int, P>{});
  // A's chunk (32 rows x KC, rows past M zero) when it is staged in LDS
  char* slot_a[A_LDS ? P : 1];
  if constexpr (A_LDS) ring_slots<SLOT, P>(slot_a, std::make_integer_sequence<int, P>{}, std::integral_constant<int, P>{});

  // B: rows n0 .. n0 + 31.  Wave instruction t (wave w issues t = w ND + d)
  // fills LDS bytes [1024 t, 1024 t + 1024) of the slot: lane L lands at
  // byte 1024 t + 16 L, i.e. row r = (1024 t + 16 L) / RB at chunk
  // position p; chunk g of row r is stored at position g ^ (r % 16), so the
  // lane fetches global chunk p ^ (r % 16) of its row segment.
  const uint32_t row_bytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (int64_t)n0 * K, 32u * row_bytes);
  // A's chunk, when staged in LDS, uses the same mapping, but with the whole
  // row offset in the per-lane part: the buffer's range check covers only
  // that part, and it is what turns rows past M into zeros.
  uint32_t vb[ND], sb[ND], vas[A_LDS ? ND : 1];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const int t = wave * ND + d;
    const int r = (1024 * t + 16 * lane) / RB;
    const int p = ((1024 * t + 16 * lane) % RB) / 16;
    const int r0 = (1024 * t) / RB;  // first row of the instruction (wave-uniform)
    vb[d] = (uint32_t)(r - r0) * row_bytes + (uint32_t)((p ^ (r & 15)) << 4);
    sb[d] = (uint32_t)r0 * row_bytes;
    if constexpr (A_LDS) vas[d] = (uint32_t)r * row_bytes + (uint32_t)((p ^ (r & 15)) << 4);
  }

  // A: rows past M read as zero (outside the buffer resource).  Wave w's
  // k-values of a chunk are [16 MF w, 16 MF (w + 1)).
  const int r = lane & 31, h = lane >> 5;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * row_bytes);
  const uint32_t va = (uint32_t)r * row_bytes + (uint32_t)(wave * MF * 16 + 8 * h) * 2u;

  // B fragment of MFMA q: row r, global chunk g = 2 (w MF + q) + h.
  int rd[MF];
#pragma unroll
  for (int q = 0; q < MF; ++q) rd[q] = r * RB + (((2 * (wave * MF + q) + h) ^ (r & 15)) << 4);

  u32x4 a[A_LDS ? 1 : P][MF];
  f32x16 acc = f32x16{};

  auto issue = [&](int j, int c) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)((c + rot) % nchunks) * RB;
#pragma unroll
    for (int d = 0; d < ND; ++d)
      load_lds16(rb, slot[j] + (wave * ND + d) * 1024, vb[d], sb[d] + kb);
    if constexpr (A_LDS) {
#pragma unroll
      for (int d = 0; d < ND; ++d) load_lds16(ra, slot_a[j] + (wave * ND + d) * 1024, vas[d], kb);
    } else {
#pragma unroll
      for (int q = 0; q < MF; ++q)
        a[j][q] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)va, (int)(kb + 32u * q), 0));
    }
  };
  auto compute = [&](int j) __attribute__((always_inline)) {
    u32x4 b[MF];
#pragma unroll
    for (int q = 0; q < MF; ++q) b[q] = *(const u32x4*)(slot[j] + rd[q]);
    if constexpr (A_LDS) {
      // A's slot has B's layout: lane (m, h) reads row m at B's positions
      u32x4 x[MF];
#pragma unroll
      for (int q = 0; q < MF; ++q) x[q] = *(const u32x4*)(slot_a[j] + rd[q]);
#pragma unroll
      for (int q = 0; q < MF; ++q) acc = mfma32<TIn>(b[q], x[q], acc);
    } else {
#pragma unroll
      for (int q = 0; q < MF; ++q) acc = mfma32<TIn>(b[q], a[j][q], acc);
    }
  };
  // This thread's bias value (every output it writes is in column
  // n0 + tid % 32), loaded now so that its latency hides behind the stream.
  float bias_v = 0.0f;
  if constexpr (epi_has_bias<EPI>()) bias_v = to_f32(bias[n0 + (tid & 31)]);
  __builtin_amdgcn_sched_barrier(0);

  // chunks 0 .. P-2 in flight
#pragma unroll
  for (int j = 0; j + 1 < P; ++j) issue(j, j);

  int c0 = 0;
  for (; c0 + P < nchunks; c0 += P) {
    static_for<P>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      arrive<OPS * (P - 2)>();
      issue((j + P - 1) % P, c0 + j + P - 1);
      compute(j);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  // last P chunks: only the first still has a chunk to issue
  static_for<P>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j == 0) {
      arrive<OPS * (P - 2)>();
      issue(P - 1, c0 + P - 1);
    } else {
      arrive<OPS * (P - 1 - j)>();
    }
    compute(j);
    __builtin_amdgcn_sched_barrier(0);
  });

  // Partial sums of the NW waves through LDS (slot 0, when large enough, is
  // free once every wave is past the barrier below), summed in wave order.
  __syncthreads();
  float* red;
  if constexpr (SLOT >= NW * 4096) red = (float*)slot[0];
  else red = (float*)ring_slot<2 * P, NW * 4096>();
#pragma unroll
  for (int v = 0; v < 16; ++v) red[(wave * 16 + v) * 64 + lane] = acc[v];
  __syncthreads();

  // output (m, n_local), consecutive threads -> consecutive columns; the
  // column n0 + tid % 32 is the same in every pass
  for (int o = tid; o < 32 * 32; o += NW * 64) {
    const int nl = o & 31, m = o >> 5;
    if (m >= M) continue;
    const int src_lane = m + 32 * ((nl >> 2) & 1);
    const int v = (nl >> 3) * 4 + (nl & 3);
    float z = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) z += red[(w * 16 + v) * 64 + src_lane];
    C[(int64_t)m * N + n0 + nl] = from_f32<TOut>(epilogue<EPI>(z, bias_v));
  }
}

template <typename TIn, typename TOut, int NW, int P, int KC, bool A_LDS, int EPI>
hipError_t launch_skinny(const LaunchArgs& a) {
  hipLaunchKernelGGL((gemm_skinny_kernel<TIn, TOut, NW, P, KC, A_LDS, EPI>), dim3(a.N / 32), dim3(NW * 64), 0, a.stream,
                     (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K);
  return hipGetLastError();
}

template <typename TIn, typename TOut, int NW, int P, int KC, bool A_LDS>
LaunchFn pick_epi(int epi) {
  switch (epi) {
    case GEMM_EPI_NONE: return &launch_skinny<TIn, TOut, NW, P, KC, A_LDS, GEMM_EPI_NONE>;
    case GEMM_EPI_RELU: return &launch_skinny<TIn, TOut, NW, P, KC, A_LDS, GEMM_EPI_RELU>;
    case GEMM_EPI_BIAS_RELU: return &launch_skinny<TIn, TOut, NW, P, KC, A_LDS, GEMM_EPI_BIAS_RELU>;
    case GEMM_EPI_BIAS_GELU: return &launch_skinny<TIn, TOut, NW, P, KC, A_LDS, GEMM_EPI_BIAS_GELU>;
    case GEMM_EPI_BIAS: return &launch_skinny<TIn, TOut, NW, P, KC, A_LDS, GEMM_EPI_BIAS>;
    default: return nullptr;
  }
}

template <int NW, int P, int KC, bool A_LDS>
LaunchFn pick_types(const Problem& p) {
  if (p.in_dt == GEMM_EPI_F16) {
    if (p.out_dt == GEMM_EPI_F16) return pick_epi<f16, f16, NW, P, KC, A_LDS>(p.epi);
    if (p.out_dt == GEMM_EPI_F32) return pick_epi<f16, float, NW, P, KC, A_LDS>(p.epi);
  } else if (p.in_dt == GEMM_EPI_BF16) {
    if (p.out_dt == GEMM_EPI_BF16) return pick_epi<bf16, bf16, NW, P, KC, A_LDS>(p.epi);
    if (p.out_dt == GEMM_EPI_F32) return pick_epi<bf16, float, NW, P, KC, A_LDS>(p.epi);
  }
  return nullptr;
}

// In order of preference; the plan takes the first one whose k granularity
// (KC * P) divides K.  LDS ring = P x 32 rows x 2 KC bytes.
const SkinnyConfig kSkinny[] = {
    {4, 4, 256, 1, "skinny_32n_4w_4x256k_al"},   // B + A rings 64 + 64 KiB, 512-byte row segments
    {8, 4, 256, 1, "skinny_32n_8w_4x256k_al"},   // same ring, more waves
    {4, 8, 128, 1, "skinny_32n_4w_8x128k_al"},   // 64 + 64 KiB, 256-byte row segments, 7 chunks in flight
    {8, 2, 512, 1, "skinny_32n_8w_2x512k_al"},   // 64 + 64 KiB, 1 KiB row segments
    {8, 4, 512, 0, "skinny_32n_8w_4x512k"},      // B ring 128 KiB; A read into registers
    {8, 4, 256, 0, "skinny_32n_8w_4x256k"},      // 64 KiB
    {4, 2, 256, 0, "skinny_32n_4w_2x256k"},      // 32 KiB
    {2, 2, 128, 0, "skinny_32n_2w_2x128k"},      // 16 KiB, 256-byte row segments; any K divisible by 256
};

}  // namespace

int skinny_num_configs() { return (int)(sizeof(kSkinny) / sizeof(kSkinny[0])); }
const SkinnyConfig& skinny_config(int cfg) { return kSkinny[cfg]; }

bool skinny_supports(int cfg, const Problem& p) {
  if (cfg < 0 || cfg >= skinny_num_configs()) return false;
  const int64_t gran = (int64_t)kSkinny[cfg].kc * kSkinny[cfg].stages;
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
  switch (cfg) {
    case 0: return pick_types<4, 4, 256, true>(p);
    case 1: return pick_types<8, 4, 256, true>(p);
    case 2: return pick_types<4, 8, 128, true>(p);
    case 3: return pick_types<8, 2, 512, true>(p);
    case 4: return pick_types<8, 4, 512, false>(p);
    case 5: return pick_types<8, 4, 256, false>(p);
    case 6: return pick_types<4, 2, 256, false>(p);
    case 7: return pick_types<2, 2, 128, false>(p);
    default: return nullptr;
  }
}

}  // namespace ge
