/*
 * miattn_probes.h - peak probes of the running GPU (libmiattn_probes.so).
 *
 * Measurement aids for the roofline figures of the benchmark, not part of the attention
 * library: the dense bf16 matrix-core rate of the whole chip (back-to-back
 * v_mfma_f32_32x32x16_bf16 on independent accumulators, with random operands: the chip
 * clocks lower on random data than on constant operands) and the bandwidth of a plain
 * streaming pass that reads two arrays and writes one.  The caller times the launches
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

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_PROBES_H */
