// attention.hip -- scaled dot-product attention forward, O = softmax(Q K^T /
// sqrt(D)) V per batch and head, Q/K/V/O laid out [B, S, H, D], fp16 or bf16,
// full or causal (key j visible to query i when j <= i).
//
// The blocked form with an online softmax: each workgroup owns 128 queries
// of one (batch, head) and streams the keys and values in blocks of 64
// through LDS, keeping per query a running maximum m, the running sum l
// and the unnormalised output o, rescaled by exp(m_old - m_new) whenever
// m moves, and divides by l at the end (csdn "从零开始学习
// TileLang", ch.13 "FlashAttention", sec. 13.6-13.8; ainew.jp "TileLang で
// GPU カーネル設計を解説", section 6).  Scores are scaled by log2(e) / sqrt(D)
// so that exp is the hardware exp2 (sec. 9.6 of the same tutorial).
//
// gfx950 layout.  Each wave owns 32 queries (and every other key block:
// two waves per query group, see the kernel) and every product is a
// v_mfma_f32_32x32x16 chain arranged so that no data crosses lanes except
// one max exchange per key block:
//   * S^T = K Q^T: first operand K (key rows from LDS), second Q (registers);
//     lane (i, h) = (lane % 32, lane / 32) receives, for query i, the scores
//     of 16 of every 32 keys.  Key rows are fed to the MFMA in the order
//     kappa(r) (bits 2 and 3 of r swapped) so that lane h holds keys
//     16 t + 8 h + 0..7 of each 32-key group in accumulator order 8 t + u;
//   * those 8 fp32 probabilities, rounded to the input format, are exactly
//     the lane's second operand of O^T = V^T P^T for 16 keys: P never leaves
//     the registers (bf16 adds a second operand, the rounded remainder, so
//     that the weights keep about 16 bits);
//   * O^T accumulates with V^T as first operand, so lane (i, h) holds 32 of
//     query i's 64 outputs: the rescale by exp(m_old - m_new) is per lane,
//     and the two halves of a query exchange their partial sums l once at
//     the end.
// K and V go to LDS as they are stored, by direct buffer loads (key rows of
// 128 bytes, 16-byte chunks XOR-swizzled by row); V^T's fragments -- eight
// consecutive keys of one d per lane -- come from gfx950's transposing LDS
// read ds_read_b64_tr_b16, two per fragment.  A ring of three LDS slots:
// the blocks of the next two iterations are in flight while one is
// multiplied.  Workgroups are renumbered so that each XCD takes a
// contiguous range of (batch, head, query block), the query blocks of a
// head together, and its L2 serves their common keys and values (B, S, H =
// 4, 1024, 8, fp16: 14.5 against 16.5 us with the blocks of a head spread
// over all eight XCDs).
#include "gemm_tile.hpp"

namespace ge {
namespace attn {

using tile::lds_ptr;
using tile::make_rsrc;
using tile::swz;

constexpr int kD = 64;        // head dimension
constexpr int kBM = 128;      // queries per workgroup (4 waves x 32)
constexpr int kBN = 64;       // keys per block
constexpr int kRow = kD * 2;  // bytes of one LDS row (64 16-bit values)
constexpr int kStage = kBN * kRow;

// a, b rounded to nearest even in T and packed (one v_cvt_pk_{f16,bf16}_f32)
// a.x + a.y + acc for two packed 16-bit values (v_dot2c_f32_{f16,bf16} with
// (1, 1)): the row sum of the rounded probabilities the MFMA multiplies
template <typename T>
__device__ __forceinline__ float add_pair(uint32_t a, float acc) {
  if constexpr (__is_same(T, f16)) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), (h2){(_Float16)1.0f, (_Float16)1.0f}, acc, false);
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, 0x3f803f80u), acc, false);
  }
}

// bf16 probabilities are split into a rounded part and its rounded
// remainder (see the kernel); fp16 ones are rounded once
template <typename T>
constexpr bool kSplitP = __is_same(T, bf16);

template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef T t2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, t2));
}

// The value of x in lane l ^ 32.  v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second; with x in
// both, the second result holds the partner's value in lanes 0..31 and the
// first in lanes 32..63.
__device__ __forceinline__ float partner32(float x, int upper) {
  const uint32_t a = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  return __builtin_bit_cast(float, upper ? r[0] : r[1]);
}

// V's LDS rows (one key, 64 d-values) keep 16-byte chunk c at position
// c ^ 4 ((key >> 1) & 1): a transposing read's half-wave takes four
// consecutive key rows at the same four chunks, which then fall on 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int vswz(int key) { return 4 * ((key >> 1) & 1); }

template <int J>
__device__ __forceinline__ char* kslot() {
  __shared__ __attribute__((aligned(1024))) char s[2 * kStage];
  return s;
}
template <int J>
__device__ __forceinline__ char* vslot() {
  __shared__ __attribute__((aligned(1024))) char s[2 * kStage];
  return s;
}

// RAGS: S not a multiple of 128 -- the last query block reaches past S
// (its query rows read row S - 1 and are not stored) and the last key block
// may too (rows past S load as zeros, their scores count as -inf).
template <typename T, bool CAUSAL, bool RAGS = false>
__global__ __launch_bounds__(512) void attn_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                       const T* __restrict__ V, T* __restrict__ O, int S, int H,
                                                       float scale_log2) {
  // Three ring slots of K and of V, each holding one block per key parity
  // (one __shared__ object per slot, so that the compiler can tell a read
  // of one slot from a direct load in flight into another).
  char* const sk[3] = {kslot<0>(), kslot<1>(), kslot<2>()};
  char* const sv[3] = {vslot<0>(), vslot<1>(), vslot<2>()};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // 8 waves: query group qg (32 queries) x key parity kp.  The two waves of
  // a query group take alternate key blocks -- two waves per SIMD, so one
  // can multiply while the other computes its softmax -- and merge their
  // partial results at the end.
  const int qg = wave & 3, kp = wave >> 2;
  const int il = lane & 31, h = lane >> 5;
  // Workgroup i runs on XCD i % 8 (round-robin dispatch): renumber so that
  // the query blocks of one (batch, head) share an XCD and its L2 holds
  // their keys and values once.
  const int nqb = gridDim.x, ntot = nqb * gridDim.y * gridDim.z;
  int lin = blockIdx.x + nqb * (blockIdx.y + gridDim.y * blockIdx.z);
  if ((ntot & 7) == 0) lin = (lin & 7) * (ntot >> 3) + (lin >> 3);
  const int q0 = (lin % nqb) * kBM, hd = (lin / nqb) % H, b = lin / nqb / H;
  const int64_t rs = (int64_t)H * kD;  // elements between consecutive sequence positions
  const int64_t base = ((int64_t)b * S * H + hd) * kD;
  const int qi = q0 + qg * 32 + il;  // this lane's query

  // Q fragments of this lane's query: d = 16 kk + 8 h .. + 7
  const int qrow = RAGS ? min(qi, S - 1) : qi;
  u32x4 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = *(const u32x4*)(Q + base + qrow * rs + 16 * kk + 8 * h);
  // pass them through an empty asm here, so that the wait for these loads
  // is placed before the key loop and not, conservatively, inside it (where
  // it would also wait for the next block's loads)
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) asm volatile("" : "+v"(qf[kk]));

  // K and V: direct loads, 8 wave instructions of 1 KiB per block and
  // operand, 2 per wave of the parity; instruction t fills rows 8 t ..
  // 8 t + 7, lane L row 8 t + L / 8 at chunk position L % 8, which holds
  // logical chunk (L % 8) ^ swz(row) for K and (L % 8) ^ vswz(row) for V.
  const uint32_t range = (uint32_t)(((int64_t)(S - 1) * rs + kD) * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, range);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + base, range);
  uint32_t kvoff[2], vvoff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 8 * (2 * qg + u) + (lane >> 3);
    kvoff[u] = (uint32_t)(row * rs * 2 + (((lane & 7) ^ swz(row)) << 4));
    vvoff[u] = (uint32_t)(row * rs * 2 + (((lane & 7) ^ vswz(row)) << 4));
  }
  const int poff = kp * kStage;
  auto load_kv = [&](auto jc, int kb) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    const uint32_t so = (uint32_t)((int64_t)kb * kBN * rs * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t ko = kvoff[u], vo = vvoff[u];
      // a key row at or past S: an offset past the buffer's range, which
      // loads zeros without a memory access (the check covers the
      // per-lane offset, not the block offset `so`)
      if constexpr (RAGS)
        if (kb * kBN + 8 * (2 * qg + u) + (lane >> 3) >= S) ko = vo = 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(kslot<j>() + poff + (2 * qg + u) * 1024), 16, ko, so, 0,
                                               0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(vslot<j>() + poff + (2 * qg + u) * 1024), 16, vo, so, 0,
                                               0);
    }
  };

  // MFMA operand reads.  S^T: lane (r, h) reads key row kappa(r) of group
  // g, chunk 2 kk + h.  O^T: V^T's fragment -- d-row 32 dt + r, keys
  // 32 g + 16 t + 8 h .. + 7 -- from two transposing reads of V's key rows:
  // in 16-lane group G = l / 16, lane 4 i + a addresses key row
  // 32 g + 16 t + 8 (G >> 1) + i (+ 4), d-values 32 dt + 16 (G & 1) + 4 a .. + 3.
  const int kr = (il & 0x13) | ((il & 4) << 1) | ((il & 8) >> 1);  // kappa: swap bits 2 and 3
  auto k_off = [&](int g, int kk) __attribute__((always_inline)) {
    const int row = 32 * g + kr;
    return row * kRow + (((2 * kk + h) ^ swz(row)) << 4);
  };
  // Key rows 8 (G >> 1) + i and + 4 have the same vswz (bit 1 of i), so
  // one byte offset per d-tile dt serves every (g, t) and both reads:
  // + (32 g + 16 t) rows, + 4 rows for the second read.
  const int tg = lane >> 4, ti = (lane >> 2) & 3, ta = lane & 3;
  int vt_base[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const int chunk = 4 * dt + 2 * (tg & 1) + (ta >> 1);
    vt_base[dt] = (8 * (tg >> 1) + ti) * kRow + ((chunk ^ vswz(ti)) << 4) + 8 * (ta & 1);
  }

  f32x16 acc_o[2] = {f32x16{}, f32x16{}};
  float m_run = -__builtin_inff();  // running maximum of the raw scores
  float l_run = 0.0f;               // this half's running sum of exp

  // key blocks (>= 2 unless RAGS with S <= 64: parity 1 then has none and
  // merges m = -inf, l = 0, o = 0)
  const int nkb = RAGS ? (S + kBN - 1) / kBN : S / kBN;
  const int nblk = CAUSAL ? (RAGS ? min((q0 + kBM) / kBN, nkb) : (q0 + kBM) / kBN) : nkb;

  auto block = [&](int kb, const char* skp, const char* svp) __attribute__((always_inline)) {
    // The block's operand fragments, all in one asm statement that waits
    // for them (one LDS round trip per block): K's eight for S^T -- g = 1
    // takes the g = 0 chunk of kk ^ 2, 32 rows down, since swz(32 + r) =
    // swz(r) ^ 4 -- and V^T's eight, [dt][g][t], two transposing reads
    // each.  The builtin form of the transposing read carries no alias
    // information, so the compiler would make it wait for every direct load
    // in flight, the next blocks' included.  (The block is in LDS: the
    // barrier before this iteration waited for it.)
    u32x2 vh[2][2][2][2];  // [dt][g][t][read]
    u32x4 kf[2][4];
    {
      uint32_t ka[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ka[kk] = (uint32_t)(uintptr_t)(lds_ptr)(skp + k_off(0, kk));
      const uint32_t b0 = (uint32_t)(uintptr_t)(lds_ptr)(svp + vt_base[0]);
      const uint32_t b1 = (uint32_t)(uintptr_t)(lds_ptr)(svp + vt_base[1]);
      asm volatile(
          "ds_read_b128 %16, %24 offset:0\n"
          "ds_read_b128 %17, %25 offset:0\n"
          "ds_read_b128 %18, %26 offset:0\n"
          "ds_read_b128 %19, %27 offset:0\n"
          "ds_read_b128 %20, %26 offset:4096\n"
          "ds_read_b128 %21, %27 offset:4096\n"
          "ds_read_b128 %22, %24 offset:4096\n"
          "ds_read_b128 %23, %25 offset:4096\n"
          "ds_read_b64_tr_b16 %0, %28 offset:0\n"
          "ds_read_b64_tr_b16 %1, %28 offset:512\n"
          "ds_read_b64_tr_b16 %2, %28 offset:2048\n"
          "ds_read_b64_tr_b16 %3, %28 offset:2560\n"
          "ds_read_b64_tr_b16 %4, %28 offset:4096\n"
          "ds_read_b64_tr_b16 %5, %28 offset:4608\n"
          "ds_read_b64_tr_b16 %6, %28 offset:6144\n"
          "ds_read_b64_tr_b16 %7, %28 offset:6656\n"
          "ds_read_b64_tr_b16 %8, %29 offset:0\n"
          "ds_read_b64_tr_b16 %9, %29 offset:512\n"
          "ds_read_b64_tr_b16 %10, %29 offset:2048\n"
          "ds_read_b64_tr_b16 %11, %29 offset:2560\n"
          "ds_read_b64_tr_b16 %12, %29 offset:4096\n"
          "ds_read_b64_tr_b16 %13, %29 offset:4608\n"
          "ds_read_b64_tr_b16 %14, %29 offset:6144\n"
          "ds_read_b64_tr_b16 %15, %29 offset:6656\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(vh[0][0][0][0]), "=&v"(vh[0][0][0][1]), "=&v"(vh[0][0][1][0]), "=&v"(vh[0][0][1][1]),
            "=&v"(vh[0][1][0][0]), "=&v"(vh[0][1][0][1]), "=&v"(vh[0][1][1][0]), "=&v"(vh[0][1][1][1]),
            "=&v"(vh[1][0][0][0]), "=&v"(vh[1][0][0][1]), "=&v"(vh[1][0][1][0]), "=&v"(vh[1][0][1][1]),
            "=&v"(vh[1][1][0][0]), "=&v"(vh[1][1][0][1]), "=&v"(vh[1][1][1][0]), "=&v"(vh[1][1][1][1]),
            "=&v"(kf[0][0]), "=&v"(kf[0][1]), "=&v"(kf[0][2]), "=&v"(kf[0][3]),
            "=&v"(kf[1][0]), "=&v"(kf[1][1]), "=&v"(kf[1][2]), "=&v"(kf[1][3])
          : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(b0), "v"(b1)
          : "memory");
    }
    // S^T for the two 32-key groups
    f32x16 s[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      s[g] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s[g] = mfma32<T>(kf[g][kk], qf[kk], s[g]);
    }
    // causal: keys after the query count as -inf
    if constexpr (CAUSAL) {
      if (kb * kBN + kBN - 1 > q0 + qg * 32) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int q = x >> 2, e = x & 3;
            const int key = kb * kBN + 32 * g + 16 * (q >> 1) + 8 * h + 4 * (q & 1) + e;
            if (key > qi) s[g][x] = -__builtin_inff();
          }
      }
    }
    // keys at or past S count as -inf
    if constexpr (RAGS) {
      if (kb * kBN + kBN > S) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int q = x >> 2, e = x & 3;
            const int key = kb * kBN + 32 * g + 16 * (q >> 1) + 8 * h + 4 * (q & 1) + e;
            if (key >= S) s[g][x] = -__builtin_inff();
          }
      }
    }
    // The block's probabilities p = 2^(s log2(e)/sqrt(D) - moff), rounded to
    // the input format as the MFMA multiplies them, and the lane's sum of
    // them.  bf16 keeps 8 significant bits, so its P is carried as two bf16
    // parts: p_hi = bf16(p) and p_lo = bf16(p - p_hi) (the difference is
    // exact in fp32), multiplied by two MFMAs into the same accumulator;
    // the weights then hold about 16 bits, like fp16's single part holds 11.
    u32x4 pp[2][2], pl[2][2];
    auto probs = [&](float moff) __attribute__((always_inline)) {
      float lb = 0.0f;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[g][8 * t + 2 * w], scale_log2, -moff));
            const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(s[g][8 * t + 2 * w + 1], scale_log2, -moff));
            pp[g][t][w] = pack2<T>(a, b);
            lb = add_pair<T>(pp[g][t][w], lb);
            if constexpr (kSplitP<T>) {
              const float ah = __builtin_bit_cast(float, pp[g][t][w] << 16);
              const float bh = __builtin_bit_cast(float, pp[g][t][w] & 0xffff0000u);
              pl[g][t][w] = pack2<T>(a - ah, b - bh);
              lb = add_pair<T>(pl[g][t][w], lb);
            }
          }
      return lb;
    };
    // The reference point m_run (a running maximum of the raw scores) moves
    // only when the probabilities at the current one would leave the range
    // kept for them.  First, with every lane's m_run set, the probabilities
    // at m_run: if each lane's sum of its 32 stays below 2^15, so does
    // every one of them (they are not negative), well inside the 16-bit
    // formats, and they are used as they are -- most blocks, with no block
    // maximum computed.
    float lb = 0.0f;
    bool done = false;
    if (!__builtin_amdgcn_ballot_w64(m_run == -__builtin_inff())) {
      lb = probs(m_run * scale_log2);
      done = !__builtin_amdgcn_ballot_w64(!(lb < 32768.0f));
    }
    if (!done) {
      // block maximum over the query's 64 scores (32 here, 32 in lane ^ 32)
      float mx = s[0][0];
#pragma unroll
      for (int x = 1; x < 16; ++x) mx = fmaxf(mx, s[0][x]);
#pragma unroll
      for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[1][x]);
      mx = fmaxf(mx, partner32(mx, h));
      // m_run moves where a score exceeds it by more than 2^8 in
      // probability (any lane of the wave): the probabilities then stay
      // below 256
      if (__builtin_amdgcn_ballot_w64((mx - m_run) * scale_log2 > 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        // (a causal query group can meet only masked keys in its parity's
        // first blocks: a lane whose m is still -inf keeps it, with alpha 1
        // and o = l = 0, when another lane moves)
        const float alpha =
            m_new == -__builtin_inff() ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) acc_o[dt] *= alpha;
      }
      lb = probs(m_run == -__builtin_inff() ? 0.0f : m_run * scale_log2);
    }
    l_run += lb;
    // O^T += V^T P^T, 16 keys at a time
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const u32x2 l2 = vh[dt][g][t][0], h2 = vh[dt][g][t][1];
          const u32x4 vf = u32x4{l2.x, l2.y, h2.x, h2.y};
          acc_o[dt] = mfma32<T>(vf, pp[g][t], acc_o[dt]);
          if constexpr (kSplitP<T>) acc_o[dt] = mfma32<T>(vf, pl[g][t], acc_o[dt]);
        }
  };

  // Ring of three slots: iteration it multiplies block 2 it + kp from slot
  // it % 3 after issuing the loads of block 2 (it + 2) + kp into slot
  // (it + 2) % 3, whose previous block (it - 1) every wave has finished (the
  // barrier that ended iteration it - 1).  Each barrier first waits until
  // at most that iteration's own loads (4 per wave) are outstanding: the
  // block of iteration it + 1 is then in LDS.  The loads are issued on
  // every iteration (past the last block, block kp again, never used): a
  // load under a condition leaves the compiler unsure which slot is in
  // flight, and it then waits for every load before each LDS read.
  auto barrier_vm = [&](bool keep) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    if (keep) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4) & ~(15 << 8));  // vmcnt(4) lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int niter = (nblk + 1) / 2;
  load_kv(std::integral_constant<int, 0>{}, kp);
  load_kv(std::integral_constant<int, 1>{}, 2 + kp < nblk ? 2 + kp : kp);
  barrier_vm(true);
  auto step = [&](auto jc, int it) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    const int kb = 2 * it + kp, nkb = kb + 4;
    load_kv(std::integral_constant<int, (j + 2) % 3>{}, nkb < nblk ? nkb : kp);
    if (kb < nblk) block(kb, kslot<j>() + poff, vslot<j>() + poff);
    barrier_vm(true);
  };
  // whole turns of the ring (one path around the back edge, so that the
  // compiler sees the same loads in flight at the loop head on every
  // entry), then the last one or two iterations
  int it = 0;
  for (; it + 3 <= niter; it += 3) {
    step(std::integral_constant<int, 0>{}, it);
    step(std::integral_constant<int, 1>{}, it + 1);
    step(std::integral_constant<int, 2>{}, it + 2);
  }
  if (it < niter) step(std::integral_constant<int, 0>{}, it);
  if (it + 1 < niter) step(std::integral_constant<int, 1>{}, it + 1);
  // the loads past the last block land before any wave reuses the slots
  barrier_vm(false);

  // Merge the two parities of each query group: parity 1 leaves (m, l, o)
  // in LDS (the slots are free after the last barrier), parity 0 combines
  // o = a0 o0 + a1 o1 and l = a0 l0 + a1 l1 with a = exp(m_p - max m).
  float* xo0 = (float*)sv[0] + qg * 16 * 64;  // o of d-tile 0: [qg][x][lane]
  float* xo1 = (float*)sv[1] + qg * 16 * 64;  // o of d-tile 1
  float* xm = (float*)sk[0] + qg * 2 * 64;    // m, l: [qg][2][lane]
  if (kp == 1) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      xo0[x * 64 + lane] = acc_o[0][x];
      xo1[x * 64 + lane] = acc_o[1][x];
    }
    xm[lane] = m_run;
    xm[64 + lane] = l_run;
  }
  barrier_vm(false);
  if (kp == 1) return;
  const float m1 = xm[lane], l1 = xm[64 + lane];
  const float m = fmaxf(m_run, m1);
  const float a0 = __builtin_amdgcn_exp2f((m_run - m) * scale_log2);
  const float a1 = __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
  const float lh = a0 * l_run + a1 * l1;
  // O = o / l, both halves' sums combined; lane (i, h) writes d = 32 dt +
  // 8 q + 4 h .. + 3 of its query
  const float inv = 1.0f / (lh + partner32(lh, h));
  const float c0 = a0 * inv, c1 = a1 * inv;
  if (RAGS && qi >= S) return;
  T* orow = O + base + qi * rs;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const float* xo = dt == 0 ? xo0 : xo1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc_o[dt][4 * q + e] * c0 + xo[(4 * q + e) * 64 + lane] * c1;
      u32x2 w;
      w.x = pack2<T>(v[0], v[1]);
      w.y = pack2<T>(v[2], v[3]);
      *(u32x2*)(orow + 32 * dt + 8 * q + 4 * h) = w;
    }
  }
}

template <typename T, bool CAUSAL>
hipError_t launch(const void* Q, const void* K, const void* V, void* O, int B, int S, int H, hipStream_t stream) {
  const float scale_log2 = (float)(1.4426950408889634 / 8.0);  // log2(e) / sqrt(64)
  if (S % kBM != 0)
    hipLaunchKernelGGL((attn_fwd_kernel<T, CAUSAL, true>), dim3((S + kBM - 1) / kBM, H, B), dim3(512), 0, stream,
                       (const T*)Q, (const T*)K, (const T*)V, (T*)O, S, H, scale_log2);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, CAUSAL>), dim3(S / kBM, H, B), dim3(512), 0, stream, (const T*)Q,
                       (const T*)K, (const T*)V, (T*)O, S, H, scale_log2);
  return hipGetLastError();
}

}  // namespace attn
}  // namespace ge

extern "C" gemm_epi_status gemm_epi_attention_fwd(const void* Q, const void* K, const void* V, void* O, int64_t B,
                                                   int64_t S, int64_t H, int64_t D, gemm_epi_dtype dtype, int causal,
                                                   void* stream) {
  if (!Q || !K || !V || !O || B <= 0 || S <= 0 || H <= 0 || D <= 0) return GEMM_EPI_ERR_INVALID_ARG;
  if (dtype != GEMM_EPI_F16 && dtype != GEMM_EPI_BF16) return GEMM_EPI_ERR_INVALID_ARG;
  const int64_t n = B * S * H * D;
  if (D != ge::attn::kD || n >= ((int64_t)1 << 31) || (S + ge::attn::kBM - 1) / ge::attn::kBM > 65535 ||
      H > 65535 || B > 65535)
    return GEMM_EPI_ERR_UNSUPPORTED;
  for (const void* p : {Q, K, V, (const void*)O})
    if (((uintptr_t)p & 15u) != 0) return GEMM_EPI_ERR_UNSUPPORTED;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dtype == GEMM_EPI_F16)
    e = causal ? ge::attn::launch<ge::f16, true>(Q, K, V, O, (int)B, (int)S, (int)H, s)
               : ge::attn::launch<ge::f16, false>(Q, K, V, O, (int)B, (int)S, (int)H, s);
  else
    e = causal ? ge::attn::launch<ge::bf16, true>(Q, K, V, O, (int)B, (int)S, (int)H, s)
               : ge::attn::launch<ge::bf16, false>(Q, K, V, O, (int)B, (int)S, (int)H, s);
  return e == hipSuccess ? GEMM_EPI_OK : GEMM_EPI_ERR_HIP;
}
