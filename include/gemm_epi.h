/*
 * gemm_epi.h -- C ABI of the MI355X (gfx950) GEMM with a fused epilogue:
 *
 *     C = act(s . (A . B) [+ bias]) [+ R]     fp16/bf16 inputs, fp32 accumulation
 *
 * The operation is the tiled GEMM whose epilogue (bias add, then ReLU or
 * GELU) runs on the fp32 accumulators before the single store of C:
 *   - GEMM definition and the fp16/bf16-in, fp32-accumulate, convert-on-output
 *     data flow: csdn "从零开始学习 TileLang" tutorial, ch.10 "GEMM 矩阵乘法",
 *     sec. 10.1 and 10.6;
 *   - epilogue on the accumulator before write-back (bias then ReLU):
 *     same chapter, sec. 10.8 "GEMM Epilogue 融合";
 *   - C = ReLU(A @ B): atlascloud.ai "Writing high-performance kernels in
 *     TileLang", section "Écrivons un GEMM";
 *   - C = GELU_tanh(A @ B + bias): ainew.jp "TileLang で GPU カーネル設計を解説",
 *     section 4 "EPILOGUE FUSION";
 *   - a row-major A with a column-major B and an fp32 C: TileFusion
 *     "基础GEMM示例" (xdnf.cn repost);
 *   - further epilogue fusions (another activation, a quantisation scale,
 *     a residual): csdn tutorial ch.10 sec. 10.7 (where hand-written GEMMs
 *     pay: GEMM with bias, activation, quantisation and other epilogues)
 *     and its operator table (residual fusion); the pages give no formula,
 *     the forms below are the common ones.
 *
 * Plain C: no HIP, torch or C++ types appear here.  Device buffers are plain
 * device pointers owned by the caller; the stream is a hipStream_t passed as
 * void* (NULL = the null stream).
 *
 * Errors never abort: every call returns a gemm_epi_status.
 */
#ifndef GEMM_EPI_H
#define GEMM_EPI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.  F32 and FP8_E4M3 are output formats only.  FP8_E4M3 is
 * the OCP 8-bit floating-point E4M3 format (bias 7, no infinities, largest
 * finite 448): the quantised output the tutorial lists among the fusions
 * (csdn ch.10 sec. 10.7, "GEMM + quantisation").  Conversion to it
 * saturates at +-448 and rounds to nearest even. */
typedef enum gemm_epi_dtype {
  GEMM_EPI_F16 = 0,      /* IEEE binary16 */
  GEMM_EPI_BF16 = 1,     /* bfloat16 (top half of binary32) */
  GEMM_EPI_F32 = 2,      /* IEEE binary32 */
  GEMM_EPI_FP8_E4M3 = 3  /* OCP FP8 E4M3, one byte */
} gemm_epi_dtype;

/* Storage order of an R x C operand: ROW_MAJOR puts (r, c) at r*C + c,
 * COL_MAJOR at c*R + r.  For B (logical K x N), COL_MAJOR is the N x K
 * "weight" layout with K contiguous.  C is always row-major M x N. */
typedef enum gemm_epi_layout { GEMM_EPI_ROW_MAJOR = 0, GEMM_EPI_COL_MAJOR = 1 } gemm_epi_layout;

/* Epilogue applied to the fp32 accumulator z before conversion:
 *   NONE       C = z
 *   RELU       C = max(z, 0)
 *   BIAS_RELU  C = max(z + bias[n], 0)
 *   BIAS_GELU  C = g(z + bias[n]),  g(x) = x / (1 + exp(-1.5957691216 (x + 0.044715 x^3)))
 *              (the tanh form of GELU written as a logistic)
 *   BIAS       C = z + bias[n]
 *   SILU       C = z / (1 + exp(-z))            (x times the logistic sigmoid)
 *   BIAS_SILU  C = silu(z + bias[n])
 * bias has N elements of the input format, broadcast over rows, and is
 * added before the activation.  gemm_epi_run_ex adds an optional column
 * scale (applied to z before the bias) and residual (added after the
 * activation). */
typedef enum gemm_epi_epilogue {
  GEMM_EPI_NONE = 0,
  GEMM_EPI_RELU = 1,
  GEMM_EPI_BIAS_RELU = 2,
  GEMM_EPI_BIAS_GELU = 3,
  GEMM_EPI_BIAS = 4,
  GEMM_EPI_SILU = 5,
  GEMM_EPI_BIAS_SILU = 6
} gemm_epi_epilogue;

typedef enum gemm_epi_status {
  GEMM_EPI_OK = 0,
  GEMM_EPI_ERR_INVALID_ARG = 1, /* null/ill-formed argument, bad enum, bad size */
  GEMM_EPI_ERR_UNSUPPORTED = 2, /* well-formed, but no kernel handles it */
  GEMM_EPI_ERR_HIP = 3,         /* the HIP runtime reported an error (see gemm_epi_last_hip_error) */
  GEMM_EPI_ERR_NO_MEMORY = 4    /* host allocation of the plan failed */
} gemm_epi_status;

/* Kernel families.  AUTO lets the plan choose. */
typedef enum gemm_epi_kernel {
  GEMM_EPI_KERNEL_AUTO = 0,
  GEMM_EPI_KERNEL_GENERIC = 1, /* any shape, layout and alignment; correctness anchor */
  GEMM_EPI_KERNEL_TILE = 2,    /* LDS-pipelined MFMA tile kernel (compute-bound shapes) */
  GEMM_EPI_KERNEL_SKINNY = 3   /* weight-streaming kernel for M <= 32 (HBM-bound shapes) */
} gemm_epi_kernel;

typedef struct gemm_epi_plan_s* gemm_epi_plan_t;

/* gemm_epi_plan -- validate a problem and choose its kernel.
 *
 * The per-shape build step: the pages build a kernel for fixed M, N, K and
 * block sizes once and get back a callable (atlascloud.ai "Writing
 * high-performance kernels in TileLang", section "Écrivons un GEMM", the
 * matmul(M, N, K, ...) call; csdn "从零开始学习 TileLang", ch.10 sec. 10.5,
 * the compile step before the call).  Here nothing is compiled at run time:
 * the plan picks one of the prebuilt kernels and its launch shape.
 *
 * A is M x K in layout_a, B is K x N in layout_b, C is M x N row-major,
 * all packed (leading dimension = the contiguous extent) unless
 * gemm_epi_plan_set_ld gives other leading dimensions.
 * in_dtype in {F16, BF16}; out_dtype in {in_dtype, F32, FP8_E4M3}.
 * Host only: no device allocation, no launch, no HIP call; allocates the
 * small host plan object only.  *out is written only on GEMM_EPI_OK.
 * The kernel is the tuning table's entry for this problem when there is one
 * that can run it (gemm_epi_tune), else the static rule.
 * K = 0 is the degenerate product: the sum over k is empty, so C =
 * act(bias) with the optional scale, residual and output scale applied to
 * zero products; it runs on the generic kernel, and A and B may be NULL.
 * Errors: INVALID_ARG (out == NULL, M or N <= 0, K < 0, unknown enum, out_dtype
 * not allowed), UNSUPPORTED (any of M*K, K*N, M*N >= 2^31 elements),
 * NO_MEMORY. */
gemm_epi_status gemm_epi_plan(gemm_epi_plan_t* out, int64_t M, int64_t N, int64_t K, gemm_epi_dtype in_dtype,
                              gemm_epi_dtype out_dtype, gemm_epi_layout layout_a, gemm_epi_layout layout_b,
                              gemm_epi_epilogue epilogue);

/* gemm_epi_plan_set_ld -- leading dimensions of the stored operands, for
 * products on sub-matrices of larger arrays.
 *
 * lda: elements between consecutive rows of A as stored (row-major: rows
 * of M x K, so >= K; column-major: columns, >= M); ldb likewise for B
 * (row-major >= N, column-major >= K); ldc between rows of C (>= N), which
 * a residual (gemm_epi_run_ex) shares.  0 keeps the packed value.  The
 * kernel is chosen again: the fast kernels need lda and ldb multiples of 8
 * elements; the decode-shape kernel and the 256 x 256 16x16x32 tiles with
 * a column-major B, and the 64 x 64 ring tiles, take any N and ldc, the
 * other tile kernels need them multiples of 8 (16 for FP8_E4M3 output),
 * else the generic kernel runs.
 * Padding between rows is never written; a fast kernel may read A's or B's
 * padding up to the next multiple of 8 elements of a row, which enters no
 * stored output.  Host only.
 * Errors: INVALID_ARG (NULL plan, a leading dimension below its minimum),
 * UNSUPPORTED (an operand then spans 2^31 elements or more); the plan is
 * unchanged on error. */
gemm_epi_status gemm_epi_plan_set_ld(gemm_epi_plan_t plan, int64_t lda, int64_t ldb, int64_t ldc);

/* gemm_epi_run -- enqueue C = act(A.B [+ bias]) on `stream` and return
 * without synchronising.
 *
 * The call of the built kernel on caller-allocated tensors, output
 * included (atlascloud.ai "Écrivons un GEMM", kernel(a, b, c) with c made
 * by the caller; csdn ch.10 sec. 10.5).
 *
 * A, B, bias, C are device pointers owned by the caller, who keeps them
 * alive until the stream has passed the kernel.  bias must be non-NULL
 * exactly when the epilogue uses it (A and B may be NULL when K = 0).
 * C must not overlap A, B or bias.
 * A plan is immutable during run, so concurrent runs of one plan on
 * different streams are safe.  Pointers that are not 16-byte aligned send
 * the call to the generic kernel.
 * Errors: INVALID_ARG (plan NULL, a required pointer NULL, bias given
 * without a bias epilogue), HIP (the launch failed; the code is kept per
 * thread for gemm_epi_last_hip_error). */
gemm_epi_status gemm_epi_run(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias, void* C,
                             void* stream);

/* gemm_epi_workspace_size -- bytes of device workspace that let
 * gemm_epi_run_ws split K across workgroups (0: this plan never splits).
 *
 * Only skinny plans (M <= 32) whose N gives fewer than 256 column blocks
 * split: a decode-like product with a narrow weight, e.g. one GPU's column
 * shard of a larger one, would otherwise leave most CUs idle.  A column
 * block is 32 columns (64 for the 64-column row-major-weight configuration,
 * skinny_rowb_64n_8w_6x128k); the workspace holds one fp32 32 x width
 * partial block (4 or 8 KiB) per column block and split, then one 32-bit
 * arrival counter per column block, rounded up to 256 bytes.
 * (Split-K as the remedy when one block's share of the work is too large:
 * csdn "从零开始学习 TileLang", ch.17 "常见性能问题", sec. 17.1.)
 * Host only.  0 for a NULL plan. */
size_t gemm_epi_workspace_size(gemm_epi_plan_t plan);

/* gemm_epi_run_ws -- gemm_epi_run with a caller-owned device workspace.
 *
 * When workspace_bytes >= gemm_epi_workspace_size(plan) > 0 and every
 * pointer (workspace included) is 16-byte aligned, K is split into
 * several ranges, each workgroup stores an fp32 partial block into the
 * workspace, and the last workgroup of each column block to finish sums
 * the partials in split order (so the result does not depend on timing),
 * applies the epilogue and writes C.  Otherwise this is gemm_epi_run and
 * the workspace is not touched.
 * The workspace must be zero-filled once before its first use; every run
 * that completes leaves it zero-filled again.  Runs that share a workspace
 * must not overlap in time (same stream, or ordered by events); the plan
 * itself is still read-only.  Same errors as gemm_epi_run. */
gemm_epi_status gemm_epi_run_ws(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias, void* C,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device array gemm_epi_run_noalloc uses on each GPU:
 * 4 MiB of split-K partial blocks plus room for the arrival counters.
 * (The largest workspace any plan asks for is under 4 MiB + 1 KiB.) */
#define GEMM_EPI_NOALLOC_SCRATCH_BYTES (4194304 + 4096)

/* gemm_epi_run_noalloc -- gemm_epi_run_ws for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing (no
 * hipMalloc, hipFree or allocating library call).
 *
 * A plan that splits K (gemm_epi_workspace_size > 0) uses, as its
 * workspace, a file-scope device array of GEMM_EPI_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends
 * (the current device's copy; the stream must belong to that device).
 * Before the split kernel, a small fill kernel on `stream` clears the part
 * of the array the run uses.  Every call on a GPU shares that GPU's array,
 * so calls that overlap in time on one GPU race: order them on one stream
 * or with events.  A plan with no split is exactly gemm_epi_run.
 * Same results as gemm_epi_run_ws with a workspace of the plan's size.
 * Errors: those of gemm_epi_run; UNSUPPORTED if the plan's workspace
 * exceeds GEMM_EPI_NOALLOC_SCRATCH_BYTES; HIP (the symbol lookup, the fill
 * or the launch failed). */
gemm_epi_status gemm_epi_run_noalloc(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias, void* C,
                                     void* stream);

/* Optional epilogue operands of gemm_epi_run_ex.  With them the output is
 *
 *     C[m][n] = out_scale * (act(col_scale[n] * (A.B)[m][n] + bias[n]) + residual[m][n])
 *
 * computed in fp32 and rounded once.
 *   col_scale  N fp32 values (a per-output-column factor such as a weight
 *              dequantisation scale), or NULL for 1.
 *   residual   M x N row-major elements of the output format (with C's
 *              leading dimension), or NULL for 0.  It must not overlap C: where M or N is not a multiple of
 *              a tile, neighbouring workgroups compute some outputs twice,
 *              and an in-place residual would then be added twice.  Not
 *              allowed with FP8_E4M3 output.
 *   out_scale  one fp32 value in device memory (the quantisation scale of
 *              an FP8_E4M3 output, or any final factor), or NULL for 1. */
typedef struct gemm_epi_extras {
  const float* col_scale;
  const void* residual;
  const float* out_scale;
} gemm_epi_extras;

/* gemm_epi_run_ex -- gemm_epi_run_ws with the optional epilogue operands of
 * gemm_epi_extras.  extras == NULL, or both of its pointers NULL, is exactly
 * gemm_epi_run_ws (workspace may be NULL with workspace_bytes 0).  A
 * col_scale or residual that is not 16-byte aligned sends the call to the
 * generic kernel, like any other unaligned pointer.  Same errors as
 * gemm_epi_run; INVALID_ARG also when residual overlaps C or the output is
 * FP8_E4M3. */
gemm_epi_status gemm_epi_run_ex(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias,
                                const gemm_epi_extras* extras, void* C, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Flags of gemm_epi_tune. */
#define GEMM_EPI_TUNE_COLD 1 /* evict the caches before every timed launch */

/* gemm_epi_tune -- measure every kernel configuration that can run the
 * plan's problem and make the fastest the plan's choice.
 *
 * The search runs on the GPU itself, on the caller's buffers and stream
 * (C is overwritten with the problem's result; the split-K workspace and
 * the extras are not used): each candidate is launched twice to warm up,
 * then `iters` times, and the mean time per launch decides.  Without
 * flags the timed launches run back to back between two events, so
 * operands that fit in the 256 MB last-level cache stay there; with
 * GEMM_EPI_TUNE_COLD every timed launch follows a kernel that reads a
 * 512 MiB scratch buffer (allocated and freed by this call) and is timed
 * by its own pair of events -- the condition of a weight streamed once per
 * step, which decides among HBM-bound configurations.  Candidates are the tile and skinny configurations the problem
 * meets (the generic kernel only when none does).  The choice is also
 * recorded in the process-wide tuning table, which every later
 * gemm_epi_plan of the same problem (shape, formats, layouts, epilogue)
 * consults before its static rule; the table can be saved to and loaded
 * from a text file.  (Search on the target, save the configuration, use it
 * online: csdn "从零开始学习 TileLang", ch.18 "自动调优", sec. 18.1, 18.3.)
 * Synchronises `stream`.  best_us (may be NULL) receives the winner's mean
 * microseconds per launch.
 * Errors: INVALID_ARG (NULL plan or buffer, iters <= 0, unknown flags,
 * bias given or missing for the epilogue, a buffer not 16-byte aligned),
 * NO_MEMORY (the cold-cache scratch buffer), HIP. */
gemm_epi_status gemm_epi_tune(gemm_epi_plan_t plan, const void* A, const void* B, const void* bias, void* C,
                              int iters, int flags, void* stream, float* best_us);

/* gemm_epi_tuning_save -- write the tuning table to a text file, one entry
 * per line: M N K in_dtype out_dtype layout_a layout_b epilogue kernel
 * config microseconds (enum values of this header; '#' starts a comment).
 * Host only.  INVALID_ARG if the path is NULL or cannot be written. */
gemm_epi_status gemm_epi_tuning_save(const char* path);

/* gemm_epi_tuning_load -- merge the entries of such a file into the table
 * (an entry replaces one of the same problem).  Host only.  INVALID_ARG if
 * the path is NULL or unreadable, or any line is malformed or out of range;
 * the table is then unchanged.  An entry whose configuration cannot run its
 * problem is ignored when a plan consults it. */
gemm_epi_status gemm_epi_tuning_load(const char* path);

/* Remove every entry of the tuning table. */
void gemm_epi_tuning_clear(void);

/* Number of entries in the tuning table. */
int gemm_epi_tuning_size(void);

/* gemm_epi_attention_fwd -- enqueue scaled dot-product attention forward,
 *
 *     O[b, i, h, :] = sum_j softmax_j(Q[b, i, h, :] . K[b, j, h, :] / sqrt(D)) V[b, j, h, :]
 *
 * on `stream` and return without synchronising.  Q, K, V, O are device
 * arrays laid out [B, S, H, D] (D contiguous) in the input format `dtype`
 * (F16 or BF16), caller-owned; O must not overlap the others.  causal != 0
 * lets query i see keys j <= i only.  fp32 scores and accumulation, an
 * online softmax over blocks of 64 keys, probabilities carried into the
 * second product as one fp16 value (F16) or as a bf16 value plus its bf16
 * remainder (BF16), O rounded once.  Any S >= 1: with S not a multiple of
 * 128 the last query block and key block are masked past S (nothing past
 * row S - 1 of a (b, h) slice is read into a result or written).  (Scaled
 * dot-product attention
 * and its blocked form with an online softmax: csdn "从零开始学习 TileLang",
 * ch.13 "FlashAttention", sec. 13.1, 13.6-13.8; layout, causal rule and the
 * B, H, S, D = 4, 8, 1024, 64 example: ainew.jp "TileLang で GPU カーネル設計を
 * 解説", section 6.)
 * Errors: INVALID_ARG (a NULL pointer, B/S/H/D <= 0, dtype not F16/BF16),
 * UNSUPPORTED (D != 64, more than 65535 blocks of 128 queries, B*S*H*D >=
 * 2^31, a pointer not 16-byte aligned), HIP (the launch failed). */
gemm_epi_status gemm_epi_attention_fwd(const void* Q, const void* K, const void* V, void* O, int64_t B, int64_t S,
                                       int64_t H, int64_t D, gemm_epi_dtype dtype, int causal, void* stream);

/* gemm_epi_destroy -- free the host plan object.  NULL is a no-op (OK).
 * No device synchronisation: runs already enqueued are unaffected. */
gemm_epi_status gemm_epi_destroy(gemm_epi_plan_t plan);

/* Static, NUL-terminated name of a status code. */
const char* gemm_epi_status_string(gemm_epi_status status);

/* hipError_t of the calling thread's last failed HIP call (0 if none). */
int gemm_epi_last_hip_error(void);

/* gemm_epi_plan_select -- force a kernel family and configuration index
 * (for tests and tuning).  kernel = AUTO restores the plan's own choice
 * (the tuning table's entry, else the static rule)
 * and ignores config.  Otherwise config indexes that family's table
 * (0 .. gemm_epi_num_configs-1), and -1 lets the family choose.
 * Errors: INVALID_ARG (NULL plan, bad enum or index), UNSUPPORTED (the
 * family cannot run this problem: its shape, layout or divisibility
 * requirements are not met; the plan is then unchanged). */
gemm_epi_status gemm_epi_plan_select(gemm_epi_plan_t plan, gemm_epi_kernel kernel, int config);

/* Number of configurations of a kernel family (0 for AUTO or unknown). */
int gemm_epi_num_configs(gemm_epi_kernel kernel);

/* The kernel family and configuration the plan will launch for 16-byte
 * aligned pointers; either out pointer may be NULL.  Returns the family's
 * static name (e.g. "tile_256x256x64"), or NULL for a NULL plan. */
const char* gemm_epi_plan_describe(gemm_epi_plan_t plan, gemm_epi_kernel* kernel, int* config);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPI_H */
