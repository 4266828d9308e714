/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for
 *             C = act(A.B [+ bias]).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library
 * never links, includes or calls it, and it shares no code, header or table
 * with the GPU library.
 *
 * What it computes (one definition, written out):
 *
 *   z[i][j] = s[j] * sum_{k<K} a(i,k) * b(k,j)   (+ bias[j] when the epilogue has a bias)
 *   y[i][j] = act(z[i][j])   (+ r[i][j] when a residual is given)
 *   C[i][j] = round_to_nearest_even(q * y[i][j], output format)
 *
 *   q is an optional fp32 output scale (1 when absent).  Output formats:
 *   the input format, fp32, or FP8 E4M3 (the quantised output the tutorial
 *   names as a fusion, ch.10 sec. 10.7 and the "GEMM + quantisation"
 *   list of its closing chapter).  E4M3 follows the OCP 8-bit floating
 *   point definition: 1 sign, 4 exponent (bias 7), 3 fraction bits, no
 *   infinities, S.1111.111 the only NaN, largest finite 448.  Encoding to
 *   E4M3 is, like every other output format, one round-to-nearest-even
 *   step straight from the fp64 value q y, saturating: |q y| >= 448 gives
 *   +-448.  A residual is not defined for FP8 output.
 *
 *   s[j] (an optional fp32 per-column scale, 1 when absent) and r[i][j] (an
 *   optional M x N row-major residual in the output format, 0 when absent)
 *   are the further epilogue fusions the csdn tutorial lists (ch.10 sec. 10.7
 *   "GEMM + other epilogue", and the operator table that pairs norms with
 *   residual fusion).  The pages give no formula for them; the reading taken
 *   is the common one: the scale multiplies the product before the bias (a
 *   per-output-channel dequantisation factor), the residual is added after
 *   the activation, once, before the single rounding.
 *
 *   - The GEMM is the textbook sum over k (TileLang tutorial on csdn,
 *     ch.10 "GEMM 矩阵乘法" sec. 10.1 definition and sec. 10.2 triple loop;
 *     second tutorial, sec. 八 "示例四：GEMM 矩阵乘法").
 *   - 16-bit inputs, wide accumulation, one conversion at output
 *     (same tutorial, sec. 10.6 "GEMM 的底层数据流").  The oracle widens
 *     to fp64: a product of two fp16 or two bf16 values is exact in fp64.
 *   - Bias is added before the activation, on the accumulator
 *     (same tutorial, sec. 10.8 "GEMM Epilogue 融合"; ainew.jp
 *     "TileLang で GPU カーネル設計を解説", section 4 "EPILOGUE FUSION").
 *   - ReLU(x) = max(x, 0) (atlascloud.ai "Writing high-performance kernels
 *     in TileLang", section "Écrivons un GEMM").
 *   - SiLU(x) = x / (1 + exp(-x)) = x * sigmoid(x), the activation taken for
 *     the tutorial's "other epilogues" (csdn ch.10 sec. 10.7).
 *   - GELU is the tanh form written as a logistic: x / (1 + exp(-c1*(x + c2*x^3)))
 *     with c1 = 1.5957691216 and c2 = 0.044715 as printed in ainew.jp
 *     section 4; the page's bullet between the last two factors is read as
 *     a multiplication.
 *   - Layouts: row-major element (r, c) of an R x C matrix sits at r*C + c,
 *     column-major at c*R + r (TileFusion "基础GEMM示例": A RowMajor<128,256>,
 *     B ColMajor<256,64>).  C is always row-major.
 *
 * Floating-point formats are decoded and encoded here from their bit-level
 * definitions (IEEE 754 binary16 and binary32; bfloat16 = the top 16 bits
 * of binary32).  Encoding is one round-to-nearest-even step straight from
 * fp64, overflow to +-inf, subnormals kept.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Format codes used by this file's entry points. */
#define ORC_F16 0
#define ORC_BF16 1
#define ORC_F32 2
#define ORC_FP8 3 /* OCP FP8 E4M3 */

#define ORC_ROW 0
#define ORC_COL 1

#define ORC_EPI_NONE 0
#define ORC_EPI_RELU 1
#define ORC_EPI_BIAS_RELU 2
#define ORC_EPI_BIAS_GELU 3
#define ORC_EPI_BIAS 4
#define ORC_EPI_SILU 5
#define ORC_EPI_BIAS_SILU 6

/* mantissa bits, exponent bits of each format */
static int fmt_mant(int fmt) { return fmt == ORC_F16 ? 10 : fmt == ORC_BF16 ? 7 : 23; }
static int fmt_expb(int fmt) { return fmt == ORC_F16 ? 5 : 8; }

/* Value of a bit pattern of a binary floating-point format with the given
 * field widths (sign | exponent | fraction). */
static double decode_bits(uint32_t bits, int mant, int expb) {
  uint32_t expmask = (1u << expb) - 1u;
  int bias = (1 << (expb - 1)) - 1;
  uint32_t sign = (bits >> (mant + expb)) & 1u;
  uint32_t e = (bits >> mant) & expmask;
  uint32_t f = bits & ((1u << mant) - 1u);
  double v;
  if (e == expmask) {
    if (f != 0) return NAN;
    v = INFINITY;
  } else if (e == 0) {
    v = ldexp((double)f, 1 - bias - mant); /* subnormal: f * 2^(emin - mant) */
  } else {
    v = ldexp((double)(f + (1u << mant)), (int)e - bias - mant);
  }
  return sign ? -v : v;
}

/* Bit pattern of x rounded once, to nearest with ties to even, into the
 * format with the given field widths.  Overflow gives +-inf; NaN gives the
 * canonical quiet NaN. */
static uint32_t encode_bits(double x, int mant, int expb) {
  uint32_t expmask = (1u << expb) - 1u;
  int bias = (1 << (expb - 1)) - 1;
  int emin = 1 - bias, emax = bias;
  uint32_t sign = signbit(x) ? 1u : 0u;
  uint32_t sbit = sign << (mant + expb);
  if (isnan(x)) return (expmask << mant) | (1u << (mant - 1));
  double a = fabs(x);
  if (isinf(a)) return sbit | (expmask << mant);
  if (a == 0.0) return sbit;
  int e2;
  frexp(a, &e2);          /* a = f * 2^e2 with f in [0.5, 1) */
  int E = e2 - 1;         /* a in [2^E, 2^(E+1)) */
  if (E < emin) E = emin; /* subnormal range shares the spacing of emin */
  /* representable values near a are integer multiples of 2^(E - mant);
   * scaling by a power of two is exact, so r is a exactly */
  double r = ldexp(a, mant - E);
  double n = nearbyint(r); /* default rounding mode: nearest, ties to even */
  if (n >= ldexp(1.0, mant + 1)) { /* carried into the next binade */
    n = ldexp(n, -1);
    E += 1;
  }
  if (E > emax) return sbit | (expmask << mant);
  if (n < ldexp(1.0, mant)) /* subnormal (only possible when E == emin) */
    return sbit | (uint32_t)n;
  return sbit | ((uint32_t)(E + bias) << mant) | ((uint32_t)n - (1u << mant));
}

/* E4M3 value of a byte: sign, exponent e (bias 7), fraction f; e = 0 is
 * subnormal (f * 2^-9); S.1111.111 is NaN; no infinities. */
static double decode_e4m3(uint32_t bits) {
  uint32_t sign = (bits >> 7) & 1u, e = (bits >> 3) & 15u, f = bits & 7u;
  if (e == 15u && f == 7u) return NAN;
  double v = e == 0 ? ldexp((double)f, -9) : ldexp((double)(8u + f), (int)e - 10);
  return sign ? -v : v;
}

/* E4M3 code of x: round to nearest even, saturating at +-448; NaN gives
 * 0x7F. */
static uint32_t encode_e4m3(double x) {
  if (isnan(x)) return 0x7Fu;
  uint32_t sbit = signbit(x) ? 0x80u : 0u;
  double a = fabs(x);
  if (a >= 448.0) return sbit | 0x7Eu; /* saturate (also +-inf) */
  if (a == 0.0) return sbit;
  int e2;
  frexp(a, &e2);
  int E = e2 - 1;      /* a in [2^E, 2^(E+1)) */
  if (E < -6) E = -6;  /* subnormals share the spacing 2^-9 */
  double n = nearbyint(ldexp(a, 3 - E)); /* a / 2^(E-3), ties to even */
  if (n >= 16.0) {     /* carried into the next binade */
    n = ldexp(n, -1);
    E += 1;
  }
  if (n < 8.0) return sbit | (uint32_t)n; /* subnormal (E == -6) */
  /* a < 448 rounds to at most 448 = 2^8 * 1.75: never the NaN code */
  return sbit | ((uint32_t)(E + 7) << 3) | ((uint32_t)n - 8u);
}

double oracle_decode(int fmt, uint32_t bits) {
  if (fmt == ORC_FP8) return decode_e4m3(bits);
  return decode_bits(bits, fmt_mant(fmt), fmt_expb(fmt));
}

uint32_t oracle_encode(int fmt, double x) {
  if (fmt == ORC_FP8) return encode_e4m3(x);
  return encode_bits(x, fmt_mant(fmt), fmt_expb(fmt));
}

/* Output code of y: one RNE step from fp64 to the output format
 * (saturating for E4M3). */
static uint32_t encode_out(int fmt, double y) { return oracle_encode(fmt, y); }

/* Element-wise forms of the two conversions above, for n values. */
void oracle_decode_n(int fmt, const uint32_t* bits, double* out, int64_t n) {
  for (int64_t p = 0; p < n; ++p) out[p] = oracle_decode(fmt, bits[p]);
}

void oracle_encode_n(int fmt, const double* x, uint32_t* out, int64_t n) {
  for (int64_t p = 0; p < n; ++p) out[p] = oracle_encode(fmt, x[p]);
}

/* GELU, tanh approximation in its logistic form, constants as printed. */
double oracle_gelu(double x) { return x / (1.0 + exp(-1.5957691216 * (x + 0.044715 * x * x * x))); }

/* SiLU: x times the logistic sigmoid of x. */
double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/* Activation applied to z (bias already added). */
static double apply_act(int epi, double z) {
  switch (epi) {
  case ORC_EPI_RELU:
  case ORC_EPI_BIAS_RELU:
    return z > 0.0 ? z : 0.0;
  case ORC_EPI_BIAS_GELU:
    return oracle_gelu(z);
  case ORC_EPI_SILU:
  case ORC_EPI_BIAS_SILU:
    return oracle_silu(z);
  default:
    return z;
  }
}

static int epi_has_bias(int epi) {
  return epi == ORC_EPI_BIAS_RELU || epi == ORC_EPI_BIAS_GELU || epi == ORC_EPI_BIAS || epi == ORC_EPI_BIAS_SILU;
}

static void store_bits(void* p, int fmt, int64_t idx, uint32_t v) {
  if (fmt == ORC_F32) ((uint32_t*)p)[idx] = v;
  else if (fmt == ORC_FP8) ((uint8_t*)p)[idx] = (uint8_t)v;
  else ((uint16_t*)p)[idx] = (uint16_t)v;
}

static uint32_t load_bits(const void* p, int fmt, int64_t idx) {
  return fmt == ORC_F32 ? ((const uint32_t*)p)[idx] : ((const uint16_t*)p)[idx];
}

/* Decoding table for a 16-bit input format: table[bits] = value. */
static double* make_table(int fmt) {
  double* t = (double*)malloc(65536 * sizeof(double));
  if (!t) return NULL;
  for (uint32_t b = 0; b < 65536; ++b) t[b] = oracle_decode(fmt, b);
  return t;
}

/* K = 0 is allowed: the sum over k is empty (0) and A and B may be NULL. */
static int check_args(int64_t M, int64_t N, int64_t K, int in_fmt, int out_fmt, int la, int lb, int epi) {
  if (M <= 0 || N <= 0 || K < 0) return -1;
  if (in_fmt != ORC_F16 && in_fmt != ORC_BF16) return -1;
  if (out_fmt != in_fmt && out_fmt != ORC_F32 && out_fmt != ORC_FP8) return -1;
  if ((la != ORC_ROW && la != ORC_COL) || (lb != ORC_ROW && lb != ORC_COL)) return -1;
  if (epi < ORC_EPI_NONE || epi > ORC_EPI_BIAS_SILU) return -1;
  return 0;
}

/* Optional epilogue operands: per-column fp32 scale (N bit patterns), a
 * residual (M x N row-major, output format) and the fp32 output scale (one
 * bit pattern).  Each may be NULL. */
typedef struct {
  const uint32_t* scale;
  const void* residual;
  const uint32_t* out_scale;
  int out_fmt;
} extras_t;

/* One output element: y = act(s_j * sum_k a(i,k) b(k,j) [+ bias_j]) [+ r_ij] in fp64. */
static double one_element(const double* tab, const uint16_t* A, const uint16_t* B, const uint16_t* bias,
                          const extras_t* ex, int64_t M, int64_t N, int64_t K, int la, int lb, int epi, int64_t i,
                          int64_t j) {
  double z = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double a = tab[A[la == ORC_ROW ? i * K + k : k * M + i]];
    double b = tab[B[lb == ORC_ROW ? k * N + j : j * K + k]];
    z += a * b;
  }
  if (ex->scale) z *= oracle_decode(ORC_F32, ex->scale[j]);
  if (epi_has_bias(epi)) z += tab[bias[j]];
  double y = apply_act(epi, z);
  if (ex->residual) y += oracle_decode(ex->out_fmt, load_bits(ex->residual, ex->out_fmt, i * N + j));
  if (ex->out_scale) y *= oracle_decode(ORC_F32, ex->out_scale[0]);
  return y;
}

/* Full product.  scale and residual are optional (NULL: absent).  y_out
 * (M*N doubles, row-major) and c_out (M*N elements of out_fmt, row-major)
 * may each be NULL.  nthreads <= 0 uses the OpenMP default.  Returns 0 on
 * success, -1 on bad arguments, -2 on no memory. */
int oracle_gemm_epi_ex(int64_t M, int64_t N, int64_t K, int in_fmt, int out_fmt, int la, int lb, int epi,
                       const void* A, const void* B, const void* bias, const uint32_t* scale, const void* residual,
                       const uint32_t* out_scale, double* y_out, void* c_out, int nthreads) {
  if (check_args(M, N, K, in_fmt, out_fmt, la, lb, epi)) return -1;
  if ((K > 0 && (!A || !B)) || (epi_has_bias(epi) && !bias)) return -1;
  if (residual && out_fmt == ORC_FP8) return -1;
  const extras_t ex = {scale, residual, out_scale, out_fmt};
  double* tab = make_table(in_fmt);
  if (!tab) return -2;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double y = one_element(tab, (const uint16_t*)A, (const uint16_t*)B, (const uint16_t*)bias, &ex, M, N, K, la,
                             lb, epi, i, j);
      if (y_out) y_out[i * N + j] = y;
      if (c_out) store_bits(c_out, out_fmt, i * N + j, encode_out(out_fmt, y));
    }
  }
  free(tab);
  return 0;
}

int oracle_gemm_epi(int64_t M, int64_t N, int64_t K, int in_fmt, int out_fmt, int la, int lb, int epi,
                    const void* A, const void* B, const void* bias, double* y_out, void* c_out, int nthreads) {
  return oracle_gemm_epi_ex(M, N, K, in_fmt, out_fmt, la, lb, epi, A, B, bias, NULL, NULL, NULL, y_out, c_out,
                            nthreads);
}

/* Selected elements only: for p < count, element (rows[p], cols[p]).
 * y_out[p] gets the fp64 value, bits_out[p] its rounded encoding. */
int oracle_gemm_epi_points_ex(int64_t M, int64_t N, int64_t K, int in_fmt, int out_fmt, int la, int lb, int epi,
                              const void* A, const void* B, const void* bias, const uint32_t* scale,
                              const void* residual, const uint32_t* out_scale, int64_t count, const int64_t* rows,
                              const int64_t* cols, double* y_out, uint32_t* bits_out, int nthreads) {
  if (check_args(M, N, K, in_fmt, out_fmt, la, lb, epi)) return -1;
  if ((K > 0 && (!A || !B)) || (epi_has_bias(epi) && !bias) || count < 0 || (count && (!rows || !cols))) return -1;
  if (residual && out_fmt == ORC_FP8) return -1;
  for (int64_t p = 0; p < count; ++p)
    if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -1;
  const extras_t ex = {scale, residual, out_scale, out_fmt};
  double* tab = make_table(in_fmt);
  if (!tab) return -2;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
#endif
  for (int64_t p = 0; p < count; ++p) {
    double y = one_element(tab, (const uint16_t*)A, (const uint16_t*)B, (const uint16_t*)bias, &ex, M, N, K, la, lb,
                           epi, rows[p], cols[p]);
    if (y_out) y_out[p] = y;
    if (bits_out) bits_out[p] = encode_out(out_fmt, y);
  }
  free(tab);
  return 0;
}

int oracle_gemm_epi_points(int64_t M, int64_t N, int64_t K, int in_fmt, int out_fmt, int la, int lb, int epi,
                           const void* A, const void* B, const void* bias, int64_t count, const int64_t* rows,
                           const int64_t* cols, double* y_out, uint32_t* bits_out, int nthreads) {
  return oracle_gemm_epi_points_ex(M, N, K, in_fmt, out_fmt, la, lb, epi, A, B, bias, NULL, NULL, NULL, count, rows,
                                   cols, y_out, bits_out, nthreads);
}

/* ------------------------------------------------------------------------
 * Attention forward (the second workload):
 *
 *   S[i][j] = (1 / sqrt(D)) * sum_d Q[i][d] K[j][d]
 *   P[i][j] = exp(S[i][j] - max_j' S[i][j']) / sum_j' exp(S[i][j'] - max_j' S[i][j'])
 *   O[i][d] = sum_j P[i][j] V[j][d]
 *
 * for every batch b and head h, with j (and j') running over all keys, or
 * over j <= i when causal; O rounded once (RNE) to the input format.
 * Scaled dot-product attention as the csdn tutorial defines it (ch.13
 * "FlashAttention", sec. 13.1), the layout [batch, seq, heads, dim] and the
 * causal rule (key j visible to query i when j <= i) of the ainew.jp page's
 * section 6 example.  The blocked, online form of the softmax (sec. 13.7) is
 * the GPU's business; this is the definition, in fp64.
 * ------------------------------------------------------------------------ */

/* One query row: y[d] for d < D (fp64), keys j < nk. */
static void attn_row(const double* tab, const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t S,
                     int64_t H, int64_t D, int64_t b, int64_t h, int64_t i, int causal, double* s, double* y) {
  const int64_t nk = causal ? i + 1 : S;
  const double scale = 1.0 / sqrt((double)D);
  const uint16_t* q = Q + ((b * S + i) * H + h) * D;
  double mx = -INFINITY;
  for (int64_t j = 0; j < nk; ++j) {
    const uint16_t* k = K + ((b * S + j) * H + h) * D;
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += tab[q[d]] * tab[k[d]];
    s[j] = acc * scale;
    if (s[j] > mx) mx = s[j];
  }
  double sum = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    s[j] = exp(s[j] - mx);
    sum += s[j];
  }
  for (int64_t d = 0; d < D; ++d) y[d] = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    const uint16_t* v = V + ((b * S + j) * H + h) * D;
    const double p = s[j] / sum;
    for (int64_t d = 0; d < D; ++d) y[d] += p * tab[v[d]];
  }
}

/* Rows (b[r], i[r], h[r]) for r < count, or every row when count < 0 (then
 * the outputs are laid out [B, S, H, D] like O).  y_out (fp64) and o_out
 * (bit patterns of fmt) may each be NULL.  Returns 0, -1 (bad arguments)
 * or -2 (no memory). */
int oracle_attention(int64_t B, int64_t S, int64_t H, int64_t D, int fmt, int causal, const void* Q,
                     const void* K, const void* V, int64_t count, const int64_t* rb, const int64_t* ri,
                     const int64_t* rh, double* y_out, void* o_out, int nthreads) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || (fmt != ORC_F16 && fmt != ORC_BF16) || !Q || !K || !V) return -1;
  if (count >= 0 && count > 0 && (!rb || !ri || !rh)) return -1;
  const int64_t rows = count < 0 ? B * S * H : count;
  for (int64_t r = 0; count >= 0 && r < count; ++r)
    if (rb[r] < 0 || rb[r] >= B || ri[r] < 0 || ri[r] >= S || rh[r] < 0 || rh[r] >= H) return -1;
  double* tab = make_table(fmt);
  if (!tab) return -2;
  int fail = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* s = (double*)malloc((size_t)S * sizeof(double));
    double* y = (double*)malloc((size_t)D * sizeof(double));
    if (!s || !y) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      fail = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
      for (int64_t r = 0; r < rows; ++r) {
        int64_t b, i, h;
        if (count < 0) {
          b = r / (S * H);
          i = (r / H) % S;
          h = r % H;
        } else {
          b = rb[r];
          i = ri[r];
          h = rh[r];
        }
        attn_row(tab, (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, S, H, D, b, h, i, causal, s, y);
        for (int64_t d = 0; d < D; ++d) {
          if (y_out) y_out[r * D + d] = y[d];
          if (o_out) ((uint16_t*)o_out)[r * D + d] = (uint16_t)oracle_encode(fmt, y[d]);
        }
      }
    }
    free(s);
    free(y);
  }
  free(tab);
  return fail ? -2 : 0;
}

/* Threads an OpenMP region of this library uses by default. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
