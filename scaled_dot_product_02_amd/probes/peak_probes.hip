// Peak probes of the running GPU, declared in include/miattn_probes.h: the dense bf16 MFMA
// rate of the chip and the bandwidth of a plain 2-read / 1-write stream.  They give the
// benchmark measured ceilings beside the datasheet ones.
#include <hip/hip_runtime.h>

#include "miattn_probes.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChains = 8;   // independent accumulators: the matrix pipe never waits on a result

__device__ inline unsigned mix32(unsigned x)
{
    x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
    return x;
}

// eight bf16 values of magnitude in [0.5, 1) with random signs and mantissas.  The MFMA rate
// the chip sustains depends on the operand data: constant operands barely toggle the
// multipliers and run at a higher clock than the random data of a real workload.
__device__ inline bf16x8 random_operand(unsigned key)
{
    bf16x8 v;
    #pragma unroll
    for (int e = 0; e < 8; ++e) {
        const unsigned h = mix32(key * 8u + (unsigned)e);
        v[e] = __builtin_bit_cast(__bf16, (unsigned short)((h & 0x8000u) | (0x3f00u + ((h >> 4) & 0xffu))));
    }
    return v;
}

__global__ __launch_bounds__(kThreads) void mfma_bf16_loop(float* out, int iters)
{
    const unsigned key = (blockIdx.x * kThreads + threadIdx.x) * 8u;
    bf16x8 a[4], b[4];
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = random_operand(key + i);
        b[i] = random_operand(0x9e3779b9u + key + i);
    }
    f32x16 acc[kChains];
    #pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    for (int i = 0; i < iters; ++i) {
        // every MFMA takes a different operand pair from the one before it (the indices are
        // compile-time constants, so the operands stay in registers)
        #pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 3], b[(c + 1 + (c >> 2)) & 3], acc[c], 0, 0, 0);
    }
    float s = 0.f;
    #pragma unroll
    for (int c = 0; c < kChains; ++c)
        #pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void stream_r2w1(const u32x4* a, const u32x4* b, u32x4* o, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n)
        __builtin_nontemporal_store(__builtin_nontemporal_load(a + i) ^ __builtin_nontemporal_load(b + i), o + i);
}

}  // namespace

extern "C" {

int miattn_probe_mfma_bf16(float* out, int32_t blocks, int32_t iters, void* stream)
{
    if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_bf16_loop, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}

int64_t miattn_probe_mfma_bf16_flops(int32_t blocks, int32_t iters)
{
    return (int64_t)blocks * (kThreads / 64) * iters * kChains * 2 * 32 * 32 * 16;
}

int miattn_probe_stream_r2w1(const void* a, const void* b, void* o, int64_t bytes, void* stream)
{
    if (!a || !b || !o || bytes < 16 || bytes % 16) return (int)hipErrorInvalidValue;
    if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)o) % 16) return (int)hipErrorInvalidValue;
    const int64_t n = bytes / 16;
    hipLaunchKernelGGL(stream_r2w1, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       (hipStream_t)stream, (const u32x4*)a, (const u32x4*)b, (u32x4*)o, n);
    return (int)hipGetLastError();
}

}  // extern "C"
