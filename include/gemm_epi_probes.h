/*
 * gemm_epi_probes.h -- measurement helpers of the gfx950 GEMM library: the
 * on-box ceilings that "% of peak" is reported against next to the
 * published ones (dense 16-bit MFMA 2.5 PFLOP/s, HBM3E 8 TB/s).  The pages
 * report throughput as a fraction of what the hardware can do (csdn
 * "从零开始学习 TileLang", ch.10 sec. 10.9 "GEMM 吞吐量", and the benchmark
 * template of ch.15); these two kernels measure that "can do" on the box
 * itself.  Not part of the GEMM's hot path.
 *
 * Plain C; device pointers owned by the caller; the stream is a
 * hipStream_t passed as void* (NULL = the null stream).  Calls enqueue and
 * return without synchronising; the caller times them (HIP events on the
 * same stream).
 */
#ifndef GEMM_EPI_PROBES_H
#define GEMM_EPI_PROBES_H

#include <stddef.h>

#include "gemm_epi.h"

#ifdef __cplusplus
extern "C" {
#endif

/* gemm_epi_probe_hbm_read -- read all `bytes` of `buf` once (16 bytes per
 * lane per load, four loads in flight per lane, 2048 workgroups of 256
 * threads looping over the buffer) and fold them into a word that is
 * written to `sink` only in a case no real data is expected to produce.
 * bytes / (kernel time) is the streaming read bandwidth; to measure HBM
 * rather than the 256 MB last-level cache, rotate through buffers whose
 * total exceeds it.
 * Errors: INVALID_ARG (NULL buf or sink, bytes not a positive multiple of
 * 16, buf not 16-byte or sink not 4-byte aligned), HIP. */
gemm_epi_status gemm_epi_probe_hbm_read(const void* buf, size_t bytes, void* sink, void* stream);

/* gemm_epi_probe_mfma -- `workgroups` workgroups of four waves, each wave
 * issuing iters x 8 v_mfma_f32_16x16x32_bf16 on register operands
 * (pseudo-random finite values, eight independent accumulator chains), and
 * one fp32 result per thread into out (workgroups x 256 floats).
 * FLOPs of a call: gemm_epi_probe_mfma_flops(iters, workgroups).
 * Errors: INVALID_ARG (NULL out, iters or workgroups <= 0), HIP. */
gemm_epi_status gemm_epi_probe_mfma(int iters, int workgroups, float* out, void* stream);

/* FLOPs of one gemm_epi_probe_mfma call: workgroups x 4 waves x iters x 8
 * MFMAs x 16 384 FLOP. */
double gemm_epi_probe_mfma_flops(int iters, int workgroups);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPI_PROBES_H */
