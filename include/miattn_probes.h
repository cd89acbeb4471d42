/*
 * miattn_probes.h - peak probes of the running GPU (libmiattn_probes.so).
 *
 * Measurement aids for the roofline figures of the benchmark, not part of the attention
 * library: the dense bf16 matrix-core rate of the whole chip (back-to-back
 * v_mfma_f32_32x32x16_bf16 on independent accumulators, with random operands: the chip
 * clocks lower on random data than on constant operands), the bandwidth of a plain
 * streaming pass that reads two arrays and writes one, and the rate of random 256-byte row
 * gathers from a table that each XCD's L2 holds (the access of the CSR-sparse kernel), and
 * the issue rates of one or two waves per SIMD on matrix and vector instructions.  The caller times the launches
 * (e.g. with events on `stream`); the functions only enqueue work.  All pointers are device
 * pointers owned by the caller.  Each returns 0 on success or the HIP error code.
 */
#ifndef MIATTN_PROBES_H
#define MIATTN_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* blocks of 256 threads (4 waves); each wave runs `iters` rounds of 8 independent MFMAs.
 * out: float [blocks * 256] (one value per thread, written so that nothing is elided). */
int miattn_probe_mfma_bf16(float* out, int32_t blocks, int32_t iters, void* stream);

/* flop of one miattn_probe_mfma_bf16 launch: blocks * 4 * iters * 8 * 2 * 32 * 32 * 16. */
int64_t miattn_probe_mfma_bf16_flops(int32_t blocks, int32_t iters);

/* o[i] = a[i] ^ b[i] over `bytes` bytes (a multiple of 16; 16-byte aligned pointers), with
 * non-temporal 16-byte loads and stores: 3 * bytes of HBM traffic. */
int miattn_probe_stream_r2w1(const void* a, const void* b, void* o, int64_t bytes, void* stream);

/* Random row gathers: table holds 8 regions (one per XCD) of 2^rows_log2 rows of 256 bytes
 * (8 * 2^rows_log2 * 256 bytes, 16-byte aligned; 1 <= rows_log2 <= 20); workgroup b reads
 * region b % 8.  blocks of 256 threads; iters (a multiple of 8) 16-byte loads per thread,
 * one 256-byte row per 16 lanes per step.  out: uint32 [blocks * 256]. */
int miattn_probe_l2_gather(const void* table, int32_t rows_log2, int32_t blocks, int32_t iters,
                           uint32_t* out, void* stream);

/* bytes gathered by one miattn_probe_l2_gather launch: blocks * 256 * iters * 16. */
int64_t miattn_probe_l2_gather_bytes(int32_t blocks, int32_t iters);

/* Issue-rate probe: `blocks` workgroups of 256 * waves_per_simd threads (one per CU; 4 SIMDs),
 * each wave timing `iters` rounds of one pattern with the shader clock.  kind: 0 = 16 MFMA
 * (v_mfma_f32_32x32x16_bf16, two accumulators); 1 = 64 v_fma_f32; 2 = 32 v_exp_f32; 3 = the
 * 16 MFMAs each followed by 2 v_fma_f32 + 2 v_exp_f32 in the same wave; 5 = the 16 MFMAs
 * each followed by 4 v_fma_f32 + 2 v_exp_f32.  Two streams per SIMD (waves_per_simd 2 only;
 * waves 0-3 issue the 16 MFMAs, waves 4-7 vector work): 4 = 32 v_fma_f32 + 32 v_exp_f32;
 * 6 = as 4 with the MFMA waves at s_setprio 3; 7 = 48 v_fma_f32 + 16 v_exp_f32; 8 = as 7 with
 * the MFMA waves at s_setprio 3; 9 = 16 MFMAs on one accumulator (a dependent chain);
 * 10 = 64 v_fma_f32 in one dependent chain; 11 = 32 v_exp_f32, each followed by a
 * v_add_f32 of its result.  waves_per_simd: 1 or 2.  out: float
 * [blocks * 256 * waves_per_simd]; cycles: uint64 [blocks * 32], the start and end clock of
 * wave w of workgroup g at [32 g + 2 w] and [32 g + 2 w + 1] and the SIMD the wave ran on at
 * [32 g + 16 + w].  Returns 0 or the HIP error code (invalid arguments:
 * hipErrorInvalidValue, nothing launched). */
int miattn_probe_issue(int32_t kind, float* out, uint64_t* cycles, int32_t blocks, int32_t waves_per_simd,
                       int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_PROBES_H */
