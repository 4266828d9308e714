// gemm_skinny.hpp -- C = act(A.B [+ bias]) for M <= 32 rows with B stored
// N x K (k contiguous): the decode-like, weight-streaming shape.  The
// kernel; its instantiations live in one unit per (input, output) format
// pair (gemm_skinny_<in>_<out>.hip) and the configuration table, the
// support rules and the choice in gemm_skinny.hip.
//
// Every B element is used by at most 32 multiply-adds, so the kernel is
// bound by reading B from HBM once (the pages single out very long or very
// narrow matrices as the shapes where a custom kernel pays: csdn
// "从零开始学习 TileLang" ch.10 sec. 10.7).  The design is about keeping
// HBM busy with long contiguous reads:
//
//   - a workgroup owns 32 consecutive output columns n and all of K, so
//     there is no reduction across workgroups and bias and activation are
//     applied exactly once (when N % 32 != 0 the last workgroup is shifted
//     back to end at N: it also computes some of its neighbour's columns,
//     in another k order, and stores only the columns it owns; with N % 8
//     != 0, N < 32 or unaligned rows of C a second instance masks it past
//     N instead, see RAG);
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
//   - A's chunk (at most 32 rows x KC, the same for every workgroup and
//     so served by L2) is copied the same way into a second ring, with the
//     same slot and swizzle;
//   - the rings have P slots: while chunk c is multiplied, chunks c+1 ..
//     c+P-1 are in flight.  One workgroup barrier per chunk, after each
//     wave has waited for its own loads of chunk c (s_waitcnt vmcnt), makes
//     the slot complete; it also proves every wave has finished chunk c-1,
//     whose slot then receives chunk c+P-1.  Chunk c sits in slot
//     (c + off) % P with off chosen so that the last P chunks fill slots
//     0 .. P-1: any chunk count of at least P runs with every slot index a
//     compile-time constant;
//   - inside a chunk, wave w multiplies its own KC/NW k-values:
//     v_mfma_f32_32x32x16 with B's rows as the first operand and A's rows
//     as the second, both from LDS.  Lane l then holds the outputs
//     (m = l % 32, n = 8 (v / 4) + 4 (l / 32) + v % 4) of accumulator v;
//   - the NW partial 32x32 blocks are summed through LDS in wave order,
//     then bias, activation and conversion, and each thread writes four
//     consecutive outputs of a row with one vector store.
//
// Within each 16-k MFMA step lane half h takes k = 8h .. 8h + 7 of both
// operands, so every product pairs matching k.
//
// B row-major (K x N, n contiguous; BROW): a chunk of B is KC k-rows of the
// workgroup's 32 columns (64 contiguous bytes per row), stored in the slot
// row after row by the same direct loads (16 k-rows per wave instruction).
// The MFMA still wants eight consecutive k of one column n per lane; gfx950's
// transposing LDS read ds_read_b64_tr_b16 delivers them: within each group
// of 16 lanes, lane s = 4 i + a supplies the address of 4 consecutive values
// of a row and lane j = 4 a + b receives value b of the rows supplied by
// lanes a, 4 + a, 8 + a, 12 + a.  With lane s pointing at k-row kb + i,
// columns nb + 4 a .. + 3, lane j gets column nb + j at k-rows kb .. kb + 3;
// a second read at kb + 4 completes the eight.
#pragma once

#include "kernels.hpp"

namespace ge {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane,
// with cache policy AUX: 0 (the default, cached) for A, which every
// workgroup reads, and kStreamB for the weight, which is read once.
template <int AUX = 0>
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, AUX);
}

// The weight's copies carry the nontemporal bit (the cache-policy field's
// NT bit on gfx950): each byte of B is read once per launch.  In a bare
// copy loop of this kernel's access pattern (no compute, 128 MiB) it
// measured 28.3 -> 24.0 us, and 32 x 8192 x 8192 bf16 + bias 25.9 -> 23.9 us.
constexpr int kStreamB = 2;

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
// (The empty asm statements with a memory clobber keep the compiler from
// moving LDS accesses across the barrier, which orders no memory for it.)
template <int PENDING>
__device__ __forceinline__ void arrive() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(PENDING));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// RAG (column-major B only): N % 8 != 0, N < 32 or rows of C not 4-element
// aligned -- the last workgroup masked past N instead of shifted back, and
// outputs past N or on unaligned rows handled element by element.  A launch
// takes the plain form whenever it can, so that its code is as without
// these cases.
template <typename TIn, typename TOut, int NW, int P, int KC, int EPI, bool BROW, int CW, int BPOL, bool RAG>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B,
                                                              const TIn* __restrict__ bias, TOut* __restrict__ C,
                                                              int M, int N, int K, int lda, int ldb, int ldc,
                                                              float* __restrict__ part,
                                                              unsigned* __restrict__ arrivals,
                                                              const float* __restrict__ scale,
                                                              const TOut* __restrict__ res,
                                                              const float* __restrict__ out_scale) {
  // CW output columns per workgroup: 32, or 64 with a row-major B, where
  // waves 0 .. NW/2 - 1 take columns 0 .. 31 and the others 32 .. 63 (each
  // half splits the chunk's k-values among its waves; A's chunk is shared).
  constexpr int NH = CW / 32;             // column halves
  constexpr int NWH = NW / NH;            // waves per half
  constexpr int RB = KC * 2;              // bytes of one row segment of a chunk
  constexpr int SLOT = 32 * RB;           // one A ring slot: 32 rows
  constexpr int SLOTB = CW * RB;          // one B ring slot: CW columns x KC
  constexpr int MF = KC / 16 / NWH;       // MFMAs per wave per chunk
  constexpr int NDA = SLOT / 1024 / NW;   // direct-load instructions per wave per chunk, A
  constexpr int NDB = SLOTB / 1024 / NW;  // and B
  constexpr int ND = NDA;                 // (column-major B: NDB == NDA)
  // vector-memory operations per wave per chunk (B's and A's)
  constexpr int OPS = NDA + NDB;
  static_assert(MF >= 1 && NDA >= 1 && RB >= 256 && RB <= 1024 && P >= 2, "chunk shape");
  static_assert(CW == 32 || (CW == 64 && BROW), "columns per workgroup");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // When N % 32 != 0 the last workgroup's columns are shifted back to end
  // at N, so that no access leaves B, bias or C.  It computes some of its
  // neighbour's columns too, but in another k order (its walk starts at
  // another chunk), so its fp32 sums of them may differ in the last bit:
  // it stores only the columns from n_own on, which no other workgroup
  // writes.  (n0 is a multiple of 8, n_own of 32, so an output quad lies
  // wholly on one side.)  With N % 8 != 0 or N < 32 (column-major B) the
  // last workgroup is not shifted: B's rows past N load as zeros, and
  // outputs, bias, scale and residual past N are neither read nor stored.
  static_assert(!(RAG && BROW), "row-major B: N % 8 = 0 and N >= CW");
  constexpr bool shift = !RAG;
  const int n0 = shift ? min((int)blockIdx.x * CW, N - CW) : (int)blockIdx.x * CW;
  const int n_own = (int)blockIdx.x * CW;
  const int hc = wave / NWH, wi = wave % NWH;  // column half, wave within it
  // Split K (part != NULL): workgroup (b, s) of the gridDim.y splits takes
  // chunks [s n, (s + 1) n) of column block b, n = K / KC / splits.
  const int nsplit = (int)gridDim.y, split = (int)blockIdx.y;
  // K not a multiple of KC: the k axis is shifted by kpad = KC - K % KC so
  // that the partial chunk is chunk 0, which covers k in [-kpad, KC - kpad);
  // its positions k < 0 are loaded as zeros (issue).
  const int kpad = (-K) & (KC - 1);
  const int nchunks = (K + kpad) / KC / nsplit;  // at least P (checked on the host)
  const int cbase = split * nchunks;

  // Workgroup b walks the chunks starting at chunk b (mod the count): at
  // any moment the workgroups read at spread-out k offsets of their rows
  // instead of all at the same one, which keeps the load spread evenly over
  // the HBM channels.  (The k order does not change the sum beyond fp32
  // rounding, and each workgroup's order is fixed.)
  const int rot = (int)(blockIdx.x % (unsigned)nchunks);

  char* slot[P];
  ring_slots<SLOTB, P>(slot, std::make_integer_sequence<int, P>{});
  // A's chunk: 32 rows x KC, rows past M zero
  char* slot_a[P];
  ring_slots<SLOT, P>(slot_a, std::make_integer_sequence<int, P>{}, std::integral_constant<int, P>{});

  // B: rows n0 .. n0 + 31.  Wave instruction t (wave w issues t = w ND + d)
  // fills LDS bytes [1024 t, 1024 t + 1024) of the slot: lane L lands at
  // byte 1024 t + 16 L, i.e. row r = (1024 t + 16 L) / RB at chunk
  // position p; chunk g of row r is stored at position g ^ (r % 16), so the
  // lane fetches global chunk p ^ (r % 16) of its row segment.
  const uint32_t row_bytes = (uint32_t)ldb * 2u, a_row_bytes = (uint32_t)lda * 2u;
  // (row-major B: the workgroup's 32 columns of all K rows; K ldb 2 < 2^32
  // is checked on the host)
  const __amdgpu_buffer_rsrc_t rb =
      BROW ? make_rsrc(B + n0, (uint32_t)((int64_t)(K - 1) * ldb * 2 + 2 * CW)) : make_rsrc(B + (int64_t)n0 * ldb, 32u * row_bytes);
  // Row-major B: a k-row of the chunk is 2 CW bytes, so instruction t
  // fills k-rows RPI t .. RPI t + RPI - 1; lane L takes k-row RPI t + L / LPR,
  // bytes 16 (L % LPR) .. + 15.
  constexpr int LPR = CW / 8, RPI = 64 / LPR;
  const uint32_t vbr = (uint32_t)(lane / LPR) * row_bytes + (uint32_t)((lane % LPR) << 4);
  // A's chunk uses the same mapping, but with the whole row offset in the
  // per-lane part: the buffer's range check covers only that part, and it
  // is what turns rows past M into zeros.
  // kz: byte offset of the lane's 16-byte chunk within its row segment.
  uint32_t vb[ND], sb[ND], vas[ND], kz[ND];  // (ND = NDA)
  bool bmask[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const int t = wave * ND + d;
    const int r = (1024 * t + 16 * lane) / RB;
    const int p = ((1024 * t + 16 * lane) % RB) / 16;
    const int r0 = (1024 * t) / RB;  // first row of the instruction (wave-uniform)
    kz[d] = (uint32_t)((p ^ (r & 15)) << 4);
    vb[d] = (uint32_t)(r - r0) * row_bytes + kz[d];
    // rows past N (unshifted last workgroup): past the buffer's range, in
    // every chunk
    bmask[d] = RAG && n0 + r >= N;
    if (bmask[d]) vb[d] = 0xFFFFFFF0u;
    sb[d] = (uint32_t)r0 * row_bytes;
    vas[d] = (uint32_t)r * a_row_bytes + kz[d];
  }

  // A: rows past M read as zero (outside the buffer resource).  Wave w's
  // k-values of a chunk are [16 MF w, 16 MF (w + 1)).
  const int r = lane & 31, h = lane >> 5;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * a_row_bytes);

  // B fragment of MFMA q: row r, global chunk g = 2 (w MF + q) + h.
  int rd[MF];
#pragma unroll
  for (int q = 0; q < MF; ++q) rd[q] = r * RB + (((2 * (wi * MF + q) + h) ^ (r & 15)) << 4);

  f32x16 acc = f32x16{};

  // The shift is kept out of the buffer resources (whose ranges end at the
  // last row's end and, for A, make rows past M read as zero): chunk gc >= 1
  // starts 2 kpad bytes before gc RB in the wave-uniform offset (RB > 2 kpad);
  // in chunk 0 a lane whose 16 bytes lie at k < 0 takes a per-lane offset
  // past the end of the buffer, which the range check turns into zeros
  // without a memory access (kpad is a multiple of 8, so no lane straddles
  // k = 0), and the others move back by 2 kpad in their own offset.  Both
  // operands are masked, so that no value from before a row's start enters
  // a product.
  // Row-major B shifts whole k-rows: chunk gc >= 1 starts kpad rows early
  // in the wave-uniform offset; in chunk 0 rows below kpad load as zeros
  // and the others move back by kpad rows in their own offset.
  auto issue_brow = [&](int j, int gc) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int t = wave * NDB + d;
      if (gc == 0 && kpad != 0) {
        const int row = RPI * t + lane / LPR;
        const uint32_t v =
            row < kpad ? 0xFFFFFFF0u : (uint32_t)(row - kpad) * row_bytes + (uint32_t)((lane % LPR) << 4);
        load_lds16<BPOL>(rb, slot[j] + t * 1024, v, 0u);
      } else {
        load_lds16<BPOL>(rb, slot[j] + t * 1024, vbr, (uint32_t)(RPI * t + gc * KC - kpad) * row_bytes);
      }
    }
  };
  auto issue = [&](int j, int c) __attribute__((always_inline)) {
    const int gc = (c + rot) % nchunks + cbase;
    const uint32_t pad2 = 2u * (uint32_t)kpad;
    if constexpr (BROW) issue_brow(j, gc);
    if (gc == 0 && kpad != 0) {
      if constexpr (!BROW) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
          load_lds16<BPOL>(rb, slot[j] + (wave * ND + d) * 1024,
                           kz[d] < pad2 || bmask[d] ? 0xFFFFFFF0u : vb[d] - pad2, sb[d]);
      }
#pragma unroll
      for (int d = 0; d < ND; ++d)
        load_lds16(ra, slot_a[j] + (wave * ND + d) * 1024, kz[d] < pad2 ? 0xFFFFFFF0u : vas[d] - pad2, 0u);
    } else {
      const uint32_t kb = (uint32_t)gc * RB - pad2;
      if constexpr (!BROW) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
          load_lds16<BPOL>(rb, slot[j] + (wave * ND + d) * 1024, vb[d], sb[d] + kb);
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) load_lds16(ra, slot_a[j] + (wave * ND + d) * 1024, vas[d], kb);
    }
  };
  // Row-major B, MFMA q: lane (r, h) needs column r at k-rows
  // 16 (w MF + q) + 8 h .. + 7; lane s = l % 16 of its 16-lane group
  // addresses k-row 8 h + s / 4 (+ 4 for the second read), columns
  // 16 ((l / 16) % 2) + 4 (s % 4) .. + 3.
  const int rtr = (8 * h + ((lane & 15) >> 2)) * (2 * CW) + 64 * hc + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  auto compute = [&](int j) __attribute__((always_inline)) {
    u32x4 b[MF];
    if constexpr (BROW) {
      typedef short s4v __attribute__((vector_size(8)));
      typedef __attribute__((address_space(3))) s4v lds_s4v;
#pragma unroll
      for (int q = 0; q < MF; ++q) {
        char* p0 = slot[j] + 16 * (2 * CW) * (wi * MF + q) + rtr;
        const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(lds_ptr)p0);
        const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(lds_ptr)(p0 + 4 * (2 * CW)));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        b[q] = u32x4{l2.x, l2.y, h2.x, h2.y};
      }
    } else {
#pragma unroll
      for (int q = 0; q < MF; ++q) b[q] = *(const u32x4*)(slot[j] + rd[q]);
    }
    // A's slot has B's layout: lane (m, h) reads row m at B's positions
    u32x4 x[MF];
#pragma unroll
    for (int q = 0; q < MF; ++q) x[q] = *(const u32x4*)(slot_a[j] + rd[q]);
#pragma unroll
    for (int q = 0; q < MF; ++q) acc = mfma32<TIn>(b[q], x[q], acc);
  };
  // Output stage: output group t (0 .. 255) is (m = t / 8, n0 + 4 (t % 8)
  // .. +3), taken by threads t, t + 64 NW, ...; every group of a thread has
  // the same columns, whose bias values are loaded now so that the latency
  // hides behind the stream.
  constexpr int NG = 8 * CW;         // output groups: 32 rows x CW / 4 column quads
  const int oq = tid & (CW / 4 - 1);  // this thread's column quad
  u32x2 bias_q = u32x2{0u, 0u};
  if constexpr (epi_has_bias<EPI>())
    if (tid < NG) {
      const int nb = n0 + 4 * oq;
      if (!RAG || nb + 4 <= N) {
        bias_q = *(const u32x2*)(bias + nb);
      } else {
        // a quad reaching past N (unshifted last workgroup): element by element
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (nb + e < N) {
            const uint32_t v = bits16(bias[nb + e]);
            bias_q[e >> 1] |= (e & 1) ? (v << 16) : v;
          }
      }
    }
  __builtin_amdgcn_sched_barrier(0);

  // Chunk c lives in slot (c + off) % P, so that the last P chunks sit in
  // slots 0 .. P-1 in order whatever the chunk count; every slot index
  // below is a compile-time constant.
  const int off = (P - nchunks % P) % P;
  // chunks 0 .. P-2 in flight
  static_for<P>([&](auto oc) __attribute__((always_inline)) {
    constexpr int o = decltype(oc)::value;
    if (off == o) {
      static_for<P - 1>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        issue((j + o) % P, j);
      });
    }
  });

  // One chunk: wait for it (and prove every wave is past the previous
  // one), refill the slot just freed with the chunk P-1 ahead, multiply.
  int c0 = 0;
  // head: the first nchunks % P chunks, in slots off .. P-1
  static_for<P>([&](auto sc) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value;
    if constexpr (s > 0) {
      if (off != 0 && s >= off) {
        arrive<OPS * (P - 2)>();
        issue((s + P - 1) % P, c0 + P - 1);
        compute(s);
        __builtin_amdgcn_sched_barrier(0);
        ++c0;
      }
    }
  });
  // whole turns of the ring
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

  // Partial sums of the NW waves through LDS: once every wave is past the
  // barrier below the ring is free, and wave w's 4 KiB record goes to byte
  // 4096 w of the ring (spanning slots in order).  Lane l stores its 16
  // values as four 16-byte chunks, chunk c at position c ^ ((l >> 2) & 3)
  // of its 64 bytes, so each 16-lane group of a write covers 16 distinct
  // bank groups.
  static_assert(NW * 4096 <= P * SLOTB && SLOTB % 4096 == 0, "reduction records");
  auto record = [&](int w) __attribute__((always_inline)) -> char* {
    char* r = slot[0];
    static_for<P>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      if (w * 4096 / SLOTB == j) r = slot[j] + (w * 4096) % SLOTB;
    });
    return r;
  };
  __syncthreads();
  {
    char* rec = record(wave) + lane * 64;
    const int sw = (lane >> 2) & 3;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *(f32x4*)(rec + ((c ^ sw) << 4)) = f32x4{acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
  }
  __syncthreads();

  // Output (m, n0 + 4q + e), q = t % 8: accumulator v = 4 (q / 2) + e of
  // lane m + 32 (q % 2) in every wave's record, summed in wave order; then
  // finish() below.
  auto block_sum = [&](int om) __attribute__((always_inline)) -> f32x4 {
    const int qi = oq & 7, L = om + 32 * (qi & 1), c = qi >> 1;
    const int w0 = NWH * (oq >> 3);  // the waves of this quad's column half
    f32x4 z = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < NWH; ++w) z += *(const f32x4*)(record(w0 + w) + L * 64 + ((c ^ ((L >> 2) & 3)) << 4));
    return z;
  };
  // Column scale, bias, activation, residual, output scale, conversion and
  // one vector store of outputs (om, n0 + 4 oq .. + 3), if this workgroup
  // owns them.
  auto finish = [&](int om, f32x4 z) __attribute__((always_inline)) {
    const int n = n0 + 4 * oq;
    if (n < n_own) return;
    if constexpr (RAG) {
      if (n >= N) return;
    }
    if (RAG && (n + 4 > N || (ldc & 3) != 0)) {
      // a quad reaching past N, or rows of C not 4-element aligned:
      // element by element
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e >= N) break;
        float b = 0.0f;
        if constexpr (epi_has_bias<EPI>())
          b = to_f32(__builtin_bit_cast(TIn, (uint16_t)((e & 1) ? (bias_q[e >> 1] >> 16) : (bias_q[e >> 1] & 0xffffu))));
        const float s = scale ? scale[n + e] : 1.0f;
        const float rv = res ? out_to_f32(res[(int64_t)om * ldc + n + e]) : 0.0f;
        const float v = epilogue_ex<EPI>(z[e], b, scale != nullptr, s, res != nullptr, rv, out_scale != nullptr,
                                         out_scale ? *out_scale : 1.0f);
        C[(int64_t)om * ldc + n + e] = from_f32<TOut>(v);
      }
      return;
    }
    f32x4 sc = f32x4{1.0f, 1.0f, 1.0f, 1.0f}, r = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (scale) sc = *(const f32x4*)(scale + n);
    if (res) r = load4<TOut>(res + (int64_t)om * ldc + n);
    const float os = out_scale ? *out_scale : 1.0f;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float b = 0.0f;
      if constexpr (epi_has_bias<EPI>())
        b = to_f32(__builtin_bit_cast(TIn, (uint16_t)((e & 1) ? (bias_q[e >> 1] >> 16) : (bias_q[e >> 1] & 0xffffu))));
      v[e] = epilogue_ex<EPI>(z[e], b, scale != nullptr, sc[e], res != nullptr, r[e], out_scale != nullptr, os);
    }
    store4<TOut>(C + (int64_t)om * ldc + n, v[0], v[1], v[2], v[3]);
  };
  if (part != nullptr) {
    // Split K: store this workgroup's fp32 partial block (row-major 32 x 32
    // at part + 1024 (b splits + s)), then count the arrival.  The
    // workgroup that arrives last for its column block sums the splits'
    // partials in split order (the result does not depend on which one is
    // last), applies the epilogue, writes C and re-arms the counter for
    // the next run.
    //
    // The summing workgroup also clears the partials it read (the rows
    // below M, the only ones written), so that every completed run leaves
    // the whole workspace zero-filled, as it found it: a workspace may be
    // shared by plans whose partial and counter areas overlap.
    //
    // Visibility across XCDs.  The partials, the counter and the partial
    // reads are agent-scope atomic accesses, which go to the device-coherent
    // level.  The writing side has no release fence (one would write back
    // the XCD's whole L2 in every workgroup -- measured 1.7-4x slower, as
    // every workgroup then also lost A from L2): each thread waits for its
    // partial stores to be acknowledged (s_waitcnt vmcnt(0)) before the
    // workgroup barrier that precedes the relaxed count.  That the stores
    // are then visible device-wide before the count is a property of
    // gfx950's memory system (acknowledged agent-scope stores have reached
    // the coherent level), not a guarantee of the HIP memory model.  The
    // finishing workgroup does take an agent-scope acquire fence after the
    // count, so its partial reads are ordered after it.
    float* mine = part + (size_t)(blockIdx.x * nsplit + split) * (32 * CW);
    for (int t = tid; t < NG; t += NW * 64) {
      const int om = t / (CW / 4);
      if (om >= M) break;
      const f32x4 z = block_sum(om);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __hip_atomic_store(mine + om * CW + 4 * oq + e, z[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    // (the flag lives in A's first ring slot, unused since the k loop)
    int* is_last = (int*)slot_a[0];
    if (tid == 0)
      *is_last = __hip_atomic_fetch_add(arrivals + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (unsigned)(nsplit - 1);
    __syncthreads();
    if (!*is_last) return;
    // Acquire at agent scope, so that the partial reads below are ordered
    // after the count that saw every other split arrive (only the finishing
    // workgroup pays for the cache maintenance this implies).
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    float* blk = part + (size_t)blockIdx.x * nsplit * (32 * CW);
    for (int t = tid; t < NG; t += NW * 64) {
      const int om = t / (CW / 4);
      if (om >= M) break;
      f32x4 z = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int s = 0; s < nsplit; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          z[e] += __hip_atomic_load(blk + s * (32 * CW) + om * CW + 4 * oq + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int s = 0; s < nsplit; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __hip_atomic_store(blk + s * (32 * CW) + om * CW + 4 * oq + e, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      finish(om, z);
    }
    if (tid == 0) __hip_atomic_store(arrivals + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  for (int t = tid; t < NG; t += NW * 64) {
    const int om = t / (CW / 4);
    if (om >= M) break;
    finish(om, block_sum(om));
  }
}

template <typename TIn, typename TOut, int NW, int P, int KC, int EPI, bool BROW, int CW, int BPOL>
hipError_t launch_skinny(const LaunchArgs& a) {
  const bool rag = !BROW && (a.N % 8 != 0 || a.N < CW || a.ldc % 4 != 0);
  // split K when the caller gave a workspace: partial blocks, then one
  // arrival counter per column block
  const int nblocks = (a.N + CW - 1) / CW;
  float* part = a.split > 1 ? (float*)a.workspace : nullptr;
  unsigned* arrivals = a.split > 1 ? (unsigned*)((char*)a.workspace + (size_t)nblocks * a.split * (128 * CW)) : nullptr;
  const dim3 grid(nblocks, a.split > 1 ? a.split : 1), block(NW * 64);
  if constexpr (!BROW) {
    if (rag) {
      hipLaunchKernelGGL((gemm_skinny_kernel<TIn, TOut, NW, P, KC, EPI, BROW, CW, BPOL, true>), grid, block, 0,
                         a.stream, (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K,
                         a.lda, a.ldb, a.ldc, part, arrivals, a.scale, (const TOut*)a.residual, a.out_scale);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_skinny_kernel<TIn, TOut, NW, P, KC, EPI, BROW, CW, BPOL, false>), grid, block, 0, a.stream,
                     (const TIn*)a.A, (const TIn*)a.B, (const TIn*)a.bias, (TOut*)a.C, a.M, a.N, a.K, a.lda, a.ldb,
                     a.ldc, part, arrivals, a.scale, (const TOut*)a.residual, a.out_scale);
  return hipGetLastError();
}

template <typename TIn, typename TOut, int NW, int P, int KC, bool BROW, int CW, int BPOL>
LaunchFn pick_epi(int epi) {
  switch (epi) {
    case GEMM_EPI_NONE: return &launch_skinny<TIn, TOut, NW, P, KC, GEMM_EPI_NONE, BROW, CW, BPOL>;
    case GEMM_EPI_RELU: return &launch_skinny<TIn, TOut, NW, P, KC, GEMM_EPI_RELU, BROW, CW, BPOL>;
    case GEMM_EPI_BIAS_RELU: return &launch_skinny<TIn, TOut, NW, P, KC, GEMM_EPI_BIAS_RELU, BROW, CW, BPOL>;
    case GEMM_EPI_BIAS_GELU: return &launch_skinny<TIn, TOut, NW, P, KC, GEMM_EPI_BIAS_GELU, BROW, CW, BPOL>;
    case GEMM_EPI_BIAS: return &launch_skinny<TIn, TOut, NW, P, KC, GEMM_EPI_BIAS, BROW, CW, BPOL>;
    case GEMM_EPI_SILU: return &launch_skinny<TIn, TOut, NW, P, KC, GEMM_EPI_SILU, BROW, CW, BPOL>;
    case GEMM_EPI_BIAS_SILU: return &launch_skinny<TIn, TOut, NW, P, KC, GEMM_EPI_BIAS_SILU, BROW, CW, BPOL>;
    default: return nullptr;
  }
}

// The configurations of the table in gemm_skinny.hip, in its order (the
// indices are part of the ABI): waves, ring slots, k per chunk, B row-major,
// columns per workgroup.
template <typename TIn, typename TOut>
LaunchFn skinny_pick(int cfg, int epi) {
  switch (cfg) {
    case 0: return pick_epi<TIn, TOut, 8, 5, 256, false, 32, kStreamB>(epi);
    case 1: return pick_epi<TIn, TOut, 8, 4, 256, false, 32, kStreamB>(epi);
    case 2: return pick_epi<TIn, TOut, 4, 4, 256, false, 32, kStreamB>(epi);
    case 3: return pick_epi<TIn, TOut, 4, 8, 128, false, 32, kStreamB>(epi);
    case 4: return pick_epi<TIn, TOut, 4, 2, 256, false, 32, kStreamB>(epi);
    case 5: return pick_epi<TIn, TOut, 2, 2, 128, false, 32, kStreamB>(epi);
    case 6: return pick_epi<TIn, TOut, 8, 5, 256, true, 32, kStreamB>(epi);
    case 7: return pick_epi<TIn, TOut, 4, 8, 128, true, 32, kStreamB>(epi);
    case 8: return pick_epi<TIn, TOut, 2, 2, 128, true, 32, kStreamB>(epi);
    case 9: return pick_epi<TIn, TOut, 8, 6, 128, true, 64, kStreamB>(epi);
    default: return nullptr;
  }
}

}  // namespace
}  // namespace ge
