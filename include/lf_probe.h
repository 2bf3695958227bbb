/*
 * lf_probe.h -- measurement aids of the HSA library (liblf.so): the dense bf16
 * matrix-core ceiling and the shader clock that the attention kernel's roofline is
 * compared against, beside the published 2.5 PFLOP/s peak, and the achievable HBM read
 * rate that the pooling and prologue kernels are compared against, beside the published
 * 8 TB/s. Not part of the attention path; nothing in lf.h depends on them.
 */
#ifndef LF_PROBE_H
#define LF_PROBE_H

#include <stdint.h>

#include "lf.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------------------------
 * lf_probe_mfma_bf16 -- launches n_wg workgroups of 4 waves; every wave issues
 * 4 * iters v_mfma_f32_32x32x16_bf16 (four independent accumulator chains, operands in
 * registers, no memory traffic), i.e. n_wg * 16 * iters * 32768 FLOPs in total. Time the
 * launch on `stream` (e.g. with events) for the achieved dense rate.
 * sink: device, n_wg * 256 floats (each lane's folded result, so nothing is optimised
 *   away; values are meaningless).
 * clocks: device, 2 int64 entries, written by the first wave of workgroup 0: shader
 *   clock cycles and 100 MHz reference ticks over its loop (their ratio is the clock
 *   under matrix-core load).
 * Asynchronous on `stream`; caller-owned buffers; allocates nothing.
 * Errors: LF_ERR_INVALID_ARG (n_wg < 1, iters < 1, NULL or misaligned buffer),
 *   LF_ERR_HIP (launch).
 * ------------------------------------------------------------------------------- */
lf_status lf_probe_mfma_bf16(int32_t n_wg, int32_t iters, float* sink, int64_t* clocks, void* stream);

/* ---------------------------------------------------------------------------------
 * lf_probe_hbm_read -- a plain streaming read of `bytes` bytes at x by n_wg workgroups
 * of 256 threads: each thread reads 16-byte chunks with a grid stride, eight in flight,
 * and writes one folded value to sink. Time the launch on `stream` for the achieved read
 * rate (use a buffer well above the 256 MB Infinity Cache, e.g. >= 1 GiB).
 * x: device, 16-byte aligned, bytes > 0 and a multiple of 16 (read only).
 * sink: device, n_wg * 256 floats (values meaningless).
 * Asynchronous on `stream`; caller-owned buffers; allocates nothing.
 * Errors: LF_ERR_INVALID_ARG (n_wg < 1, bytes not a positive multiple of 16, NULL or
 *   misaligned buffer), LF_ERR_HIP (launch).
 * ------------------------------------------------------------------------------- */
lf_status lf_probe_hbm_read(const void* x, int64_t bytes, int32_t n_wg, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LF_PROBE_H */
