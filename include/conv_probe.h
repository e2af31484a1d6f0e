/*
 * conv_probe.h -- measurement probes of the MI355X conv2d library (same
 * shared library as conv_nhwc.h). They are not part of the convolution path:
 * they measure the ceilings that a roofline is drawn against on this machine,
 * beside the vendor's spec peaks, as the TSO paper measures its MAC and DRAM
 * roofs next to the theoretical ones because the rest of the machine keeps
 * either from being reached (TSO, roofline evaluation, Figure 11).
 *
 * Both only enqueue work on `stream` (a hipStream_t; NULL = default stream);
 * the caller times them with events.
 */
#ifndef CONV_PROBE_H
#define CONV_PROBE_H

#include <stdint.h>

#include "conv_nhwc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of 256 threads one conv_probe_mfma launch runs (4 per CU of a
 * 256-CU device, 4 waves each). */
#define kProbeMfmaWorkgroups 1024

/* Back-to-back independent matrix-core instructions on every SIMD:
 * v_mfma_f32_16x16x32_bf16 (dtype CONV_BF16) or v_mfma_i32_16x16x64_i8
 * (CONV_I8), `iters` rounds of 8 per wave, operands varying per lane.
 *   out : device float[4 * kProbeMfmaWorkgroups], 4-byte aligned; one value
 *         per wave is written (a checksum that keeps the work live).
 *   ops : host double; receives the multiply-add operations * 2 the launch
 *         performs (divide by its duration for FLOP/s or OP/s).
 * CONV_E_NULL for a NULL pointer, CONV_E_UNSUPPORTED for another dtype or
 * iters <= 0, CONV_E_ALIGN, CONV_E_HIP if the launch fails. */
conv_status conv_probe_mfma(int32_t dtype, int32_t iters, float* out, double* ops, void* stream);

/* A read + write stream: dst[i] = src[i] for `bytes` bytes (a multiple of
 * 16), 16 bytes per lane, four chunks in flight per lane, stores that bypass
 * the caches' retention. Both device pointers 16-byte aligned and the ranges
 * disjoint. Moves 2 * bytes through HBM. CONV_E_NULL, CONV_E_SHAPE (bytes <= 0
 * or not a multiple of 16), CONV_E_ALIGN, CONV_E_ALIAS, CONV_E_HIP. */
conv_status conv_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONV_PROBE_H */
