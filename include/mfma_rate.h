/*
 * mfma_rate.h -- C ABI of the matrix-core calibration library (libmfma_rate.so).
 *
 * Not part of the attention path: these kernels measure the dense MFMA rate that the device
 * sustains on random operands under its power limit, the practical ceiling that the attention
 * kernels' roofline fractions are read against.  Every wave of a workgroup of 8 (two per SIMD)
 * issues 16 * iters MFMAs back to back into four accumulators, the A operand read from LDS (or, for
 * attn_mfma_rate_regs, taken from registers).
 *
 *   table  : device pointer to 64 KiB of operand values (bf16 values for attn_mfma_rate, E4M3
 *            codes for attn_mfma_rate_fp8), 16-byte aligned, copied to LDS by every workgroup
 *   grid   : workgroups (the CU count gives one per CU), >= 1
 *   iters  : loop iterations, >= 1
 *   out    : device pointer to grid * 512 floats (one sum per thread, so nothing is optimised away)
 *   stream : hipStream_t or NULL
 * FLOP per launch: grid * 8 waves * 16 * iters * 32 * 32 * K * 2, K = 16 (bf16) or 64 (fp8).
 * Returns 0, 1 for a NULL pointer or a count below 1, or the hipError_t of the launch.  The
 * library allocates nothing.
 */
#ifndef MFMA_RATE_H
#define MFMA_RATE_H

#ifdef __cplusplus
extern "C" {
#endif

/* v_mfma_f32_32x32x16_bf16 */
int attn_mfma_rate(const void *table, int grid, int iters, float *out, void *stream);

/* v_mfma_f32_32x32x16_bf16 with the A operand from registers (no LDS reads): the rate without the
 * attention kernels' LDS operand traffic */
int attn_mfma_rate_regs(const void *table, int grid, int iters, float *out, void *stream);

/* v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, unit block scales */
int attn_mfma_rate_fp8(const void *table, int grid, int iters, float *out, void *stream);

/* the same with the A operand from registers (no LDS reads) */
int attn_mfma_rate_fp8_regs(const void *table, int grid, int iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif
