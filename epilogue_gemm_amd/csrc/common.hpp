// common.hpp -- shared device pieces of the gfx950 GEMM+epilogue kernels:
// element types, the fp32 epilogue and the output conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "../../include/gemm_epi.h"

namespace ge {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// FP8 E4M3 output element (OCP 8-bit floating point: bias 7, no
// infinities, largest finite 448), as gfx950's v_cvt_pk_fp8_f32 writes it.
struct fp8e4m3 {
  uint8_t bits;
};

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so that I is a
// compile-time constant inside f (for immediates such as s_waitcnt counts).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (LDS and export counters unconstrained).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Arguments every kernel family receives from the host side.
struct LaunchArgs {
  const void* A;
  const void* B;
  const void* bias;
  void* C;
  int M, N, K;
  int lda, ldb, ldc;  // leading dimensions (elements between rows of the stored layout)
  int epi;     // gemm_epi_epilogue
  int la, lb;  // gemm_epi_layout of A and B
  hipStream_t stream;
  // split-K skinny launches only: caller workspace (partials, then
  // arrival counters; zero-filled before first use, left zeroed) and the
  // number of K splits (1: no split, no workspace)
  void* workspace;
  int split;
  // optional epilogue operands (nullptr: absent): fp32 column scale (N),
  // residual (M x N row-major, output format) and fp32 output scale (one
  // value, read by every thread)
  const float* scale;
  const void* residual;
  const float* out_scale;
};

// ---------------------------------------------------------------------------
// 16-bit input element -> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
// an output element (16-bit, fp32 or E4M3) -> fp32
template <typename T>
__device__ __forceinline__ float out_to_f32(T x) {
  if constexpr (__is_same(T, fp8e4m3)) return __builtin_amdgcn_cvt_f32_fp8((int)x.bits, 0);
  else return (float)x;
}

// ---------------------------------------------------------------------------
// Epilogue on an fp32 accumulator value z with its column's bias b.
//   GELU: x / (1 + exp(-1.5957691216 (x + 0.044715 x^3))), the tanh form of
//   GELU as a logistic (ainew.jp "TileLang で GPU カーネル設計を解説",
//   section 4 "EPILOGUE FUSION").  The exponent is regrouped as
//   x (c1 + c2 x^2) with log2 e folded into c1 = -1.5957691216 log2 e and
//   c2 = -1.5957691216 * 0.044715 log2 e, so that exp is the hardware exp2
//   (v_exp_f32) of one product and the quotient is v_rcp_f32: seven
//   operations, each accurate to about one fp32 ulp, far below the 16-bit
//   output spacing.  Large negative x: 2^(+big) = +inf, 1/inf = 0, result
//   -0.  Large positive x: 2^(-big) = 0, result x.
// Bias is added first, then the activation (csdn tutorial ch.10
// sec. 10.8 "GEMM Epilogue 融合").
// ---------------------------------------------------------------------------
__device__ __forceinline__ float gelu_logistic(float x) {
  constexpr float c1 = (float)(-1.5957691216 * 1.4426950408889634);
  constexpr float c2 = (float)(-1.5957691216 * 0.044715 * 1.4426950408889634);
  const float e = __builtin_amdgcn_exp2f(x * __builtin_fmaf(c2, x * x, c1));
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// SiLU(x) = x / (1 + exp(-x)): exp as v_exp_f32 of -x log2 e, the quotient
// as v_rcp_f32.  Large negative x: 1/inf = 0, result -0; large positive x:
// result x.
__device__ __forceinline__ float silu_logistic(float x) {
  constexpr float c = (float)(-1.4426950408889634);
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * c));
}

template <int EPI>
__device__ __forceinline__ float epilogue(float z, float b) {
  if constexpr (EPI == GEMM_EPI_NONE) return z;
  else if constexpr (EPI == GEMM_EPI_RELU) return fmaxf(z, 0.0f);
  else if constexpr (EPI == GEMM_EPI_BIAS_RELU) return fmaxf(z + b, 0.0f);
  else if constexpr (EPI == GEMM_EPI_BIAS_GELU) return gelu_logistic(z + b);
  else if constexpr (EPI == GEMM_EPI_SILU) return silu_logistic(z);
  else if constexpr (EPI == GEMM_EPI_BIAS_SILU) return silu_logistic(z + b);
  else return z + b;  // GEMM_EPI_BIAS
}

template <int EPI>
constexpr bool epi_has_bias() {
  return EPI == GEMM_EPI_BIAS_RELU || EPI == GEMM_EPI_BIAS_GELU || EPI == GEMM_EPI_BIAS || EPI == GEMM_EPI_BIAS_SILU;
}

// The optional operands around the activation: q (act(s z + b) + r).  The
// flags are uniform across the launch, so the tests are scalar branches.
template <int EPI>
__device__ __forceinline__ float epilogue_ex(float z, float b, bool has_scale, float s, bool has_res, float r,
                                             bool has_q, float q) {
  if (has_scale) z *= s;
  float v = epilogue<EPI>(z, b);
  if (has_res) v += r;
  if (has_q) v *= q;
  return v;
}

// ---------------------------------------------------------------------------
// fp32 -> output element, round to nearest even (v_cvt_f16_f32 under the
// default round-to-nearest mode; v_cvt_pk_bf16_f32 for bf16).
// ---------------------------------------------------------------------------
template <typename TOut>
__device__ __forceinline__ TOut from_f32(float x) {
  return (TOut)x;
}

// E4M3 saturates: clamp to +-448 first (a NaN passes through both
// comparisons unchanged), then v_cvt_pk_fp8_f32 rounds to nearest even.
__device__ __forceinline__ float sat_e4m3(float x) { return x > 448.0f ? 448.0f : (x < -448.0f ? -448.0f : x); }

template <>
__device__ __forceinline__ fp8e4m3 from_f32<fp8e4m3>(float x) {
  const float c = sat_e4m3(x);
  return fp8e4m3{(uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xff)};
}

// Four E4M3 codes of v0..v3, byte i = v_i.
__device__ __forceinline__ uint32_t pack4_e4m3(float v0, float v1, float v2, float v3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v0), sat_e4m3(v1), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v2), sat_e4m3(v3), lo, true);
}

template <typename T>
__device__ __forceinline__ uint16_t bits16(T x) {
  return __builtin_bit_cast(uint16_t, x);
}

// Two outputs in a 16-bit format, rounded to nearest even and packed (a
// in the low half): one v_cvt_pk_{f16,bf16}_f32 for the pair, the same
// rounding as two single conversions.
template <typename TOut>
__device__ __forceinline__ uint32_t pack2_out(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef TOut t2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, t2));
}

// Four consecutive outputs of one row -> one vector store.
template <typename TOut>
__device__ __forceinline__ void store4(TOut* p, float v0, float v1, float v2, float v3) {
  if constexpr (sizeof(TOut) == 1) {
    *reinterpret_cast<uint32_t*>(p) = pack4_e4m3(v0, v1, v2, v3);
  } else if constexpr (sizeof(TOut) == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v0, v1, v2, v3};
  } else {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack2_out<TOut>(v0, v1), pack2_out<TOut>(v2, v3)};
  }
}

// Four consecutive elements (fp32, 16-bit or E4M3) as fp32; p 16-, 8- or
// 4-byte aligned respectively.
template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p) {
  if constexpr (sizeof(T) == 1) {
    const int w = *reinterpret_cast<const int*>(p);
    return f32x4{__builtin_amdgcn_cvt_f32_fp8(w, 0), __builtin_amdgcn_cvt_f32_fp8(w, 1),
                 __builtin_amdgcn_cvt_f32_fp8(w, 2), __builtin_amdgcn_cvt_f32_fp8(w, 3)};
  } else if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4*>(p);
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    f32x4 r;
    r.x = to_f32(__builtin_bit_cast(T, (uint16_t)(w.x & 0xffffu)));
    r.y = to_f32(__builtin_bit_cast(T, (uint16_t)(w.x >> 16)));
    r.z = to_f32(__builtin_bit_cast(T, (uint16_t)(w.y & 0xffffu)));
    r.w = to_f32(__builtin_bit_cast(T, (uint16_t)(w.y >> 16)));
    return r;
  }
}

// Four consecutive 16-bit bias values as fp32.
template <typename TIn>
__device__ __forceinline__ f32x4 load_bias4(const TIn* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  f32x4 r;
  r.x = to_f32(__builtin_bit_cast(TIn, (uint16_t)(w.x & 0xffffu)));
  r.y = to_f32(__builtin_bit_cast(TIn, (uint16_t)(w.x >> 16)));
  r.z = to_f32(__builtin_bit_cast(TIn, (uint16_t)(w.y & 0xffffu)));
  r.w = to_f32(__builtin_bit_cast(TIn, (uint16_t)(w.y >> 16)));
  return r;
}

// 32x32x16 MFMA, fp32 accumulate, for either 16-bit input format.  Each
// operand register holds 8 consecutive-in-k elements of one row (first
// operand) or one column (second operand).
template <typename TIn>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (__is_same(TIn, f16))
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
}

}  // namespace ge
