/* Measured machine peaks for the MLA benchmark (libmla_peaks.so).
 *
 * The rooflines of the MLA kernels are stated against the published MI355X peaks (8 TB/s of
 * HBM3E, 2.5 PFLOP/s dense bf16).  These three probes measure what one launch of a plain kernel
 * actually reaches on the same GPU, so a kernel's fraction can also be read against a ceiling
 * that was measured in the same run: a streaming read (the decode attention reads its cache and
 * writes little), a streaming copy, and a loop of dense bf16 matrix ops with no memory traffic
 * (the prefill projections and attention).
 *
 * Conventions: every pointer is device memory owned by the caller; calls enqueue on `stream`
 * (a hipStream_t, NULL = the null stream) and return at once; nothing is allocated; arguments
 * are checked before any launch.  Return value 0 on success, -1 for an invalid argument, -2 when
 * a HIP call failed.  Each probe writes one 32-bit value per launched thread into `sink`
 * (n_wg * threads entries), so that no load or matrix op can be optimised away; the values are
 * defined below, so a caller can check them.
 */
#ifndef MLA_PEAKS_H
#define MLA_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 16, 16-byte aligned) from `src` with 16-byte loads,
 * by n_wg workgroups of 256 threads, grid-strided with eight loads in flight per thread.
 * sink[t] (uint32, n_wg * 256 entries) = XOR of the 32-bit words thread t read, so the XOR of
 * all sink entries is the XOR of every word of the buffer. */
int mla_peak_read(const void* src, size_t bytes, uint32_t* sink, int n_wg, void* stream);

/* Streaming copy of `bytes` (a multiple of 16, both pointers 16-byte aligned, no overlap) with
 * 16-byte loads and stores, n_wg workgroups of 256 threads.  sink is not used (may be NULL). */
int mla_peak_copy(const void* src, void* dst, size_t bytes, int n_wg, void* stream);

/* `iters` rounds of four independent dense bf16 matrix ops per wave (shape 16 = the
 * 16x16x32 op, 32 = the 32x32x16 op, fp32 accumulation), all operands equal to bf16(value),
 * by n_wg workgroups of `threads` threads (256 or 512).  Per wave and round that is
 * 4 * 2*16*16*32 = 65,536 flop (shape 16) or 4 * 2*32*32*16 = 131,072 flop (shape 32).
 * sink[t] (float, n_wg * threads entries) = the sum of thread t's accumulator elements:
 * iters * 32 * v^2 * 16 (shape 16: 4 chains x 4 elements) or iters * 16 * v^2 * 64 (shape 32:
 * 4 chains x 16 elements), exact while it stays below 2^24, with v = bf16(value). */
int mla_peak_mfma_bf16(int shape, int iters, float value, float* sink, int n_wg, int threads, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PEAKS_H */
