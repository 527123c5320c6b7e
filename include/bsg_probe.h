/*
 * bsg_probe.h -- C ABI of libbsg_probe.so, a measurement aid beside the GEMM
 * library (it computes nothing a GEMM caller needs).
 *
 * It measures the rate the matrix cores of one MI355X sustain when they do nothing
 * else: every SIMD runs two waves that only issue MFMAs, in the GEMM kernels'
 * register tile (a 128 x 64 output block per wave, 4 x 2 accumulators of 32 x 32)
 * and the GEMM kernels' occupancy (eight waves a workgroup, one workgroup a CU),
 * with no memory traffic and no LDS reads.  The published dense peaks assume the
 * top clock; under sustained load the chip holds the clock its power limit allows,
 * which depends on the operand data.  The GEMM kernels' rates are compared with
 * this rate, measured on the same kind of operand data, beside the published peak.
 *
 * Status codes are those of bsg.h.
 */
#ifndef BSG_PROBE_H
#define BSG_PROBE_H

#include <stdint.h>

#include "bsg.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Runs `iters` rounds of MFMAs on every wave of `workgroups` workgroups of 512
 * threads (each workgroup holds 160 KiB of LDS, so a CU runs one).
 *   kind: 0 BF16 (v_mfma_f32_32x32x16_bf16), 1 FP8 e4m3, 2 FP4 e2m1 (both
 *         v_mfma_scale_f32_32x32x64_f8f6f4 with UE8M0 scale operands).
 *   seed: 0 sets every operand value to 1.0 and every scale to 2^0, so each of a
 *         thread's 128 accumulators ends at exactly 2 * iters * Kmma (Kmma = 16
 *         for BF16, 64 for FP8 and FP4); any other seed draws the operand codes
 *         (BF16 magnitudes in [2^-3, 2^4), FP8 codes other than NaN, any FP4 code)
 *         and the scale bytes (2^-8 .. 2^4) from a hash of (seed, thread, register).
 *   workgroups: 1 .. 65535 (one per CU: the device's CU count).
 *   iters: 0 .. 2^24; a round is two k-steps of 8 MFMAs per wave, so a call
 *         performs workgroups * 8 * 16 * iters MFMAs (BF16 32768 flops each, FP8
 *         and FP4 131072).
 *   out: device float[workgroups * 512]: thread t's sum of its accumulators.
 *   stream: hipStream_t (NULL: the default stream); asynchronous like the GEMMs.
 * Returns BSG_OK, BSG_ERR_INVALID_ARG (kind, workgroups, iters out of range, or
 * out NULL or not 4-byte aligned) or BSG_ERR_HIP (the launch failed).
 */
int bsg_probe_mfma(int kind, uint32_t seed, int workgroups, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSG_PROBE_H */
