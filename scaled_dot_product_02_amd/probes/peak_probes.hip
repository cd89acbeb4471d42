// Peak probes of the running GPU, declared in include/miattn_probes.h: the dense bf16 MFMA
// rate of the chip, the bandwidth of a plain 2-read / 1-write stream, the rate of random
// 256-byte row gathers from an L2-resident table, and the issue rates of single waves and
// wave pairs (how matrix and vector instructions overlap on a SIMD).  They give the
// benchmark measured ceilings beside the datasheet ones, and the attention kernels' phase
// design its measured basis.
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

// Random 256-byte row gathers from a table resident in L2: workgroup b reads region b % 8
// (the XCD that the round-robin dispatch places it on), 2^rows_log2 rows of 256 bytes.
// Each group of 16 lanes fetches one row per step (16 bytes a lane), eight rows in flight
// per group before any is used, like the dependent gathers of a CSR row.
__global__ __launch_bounds__(kThreads) void l2_gather(const u32x4* table, int rows_log2, int iters,
                                                      unsigned* out)
{
    const unsigned mask = (1u << rows_log2) - 1u;
    const u32x4* base = table + ((int64_t)(blockIdx.x & 7) << rows_log2) * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane & 15;
    const unsigned key = ((blockIdx.x * (kThreads / 64) + wave) * 4u + (lane >> 4)) * 0x9e3779b9u;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int i = 0; i < iters; i += 8) {
        u32x4 x[8];
        #pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = base[(int64_t)(mix32(key + (unsigned)(i + u)) & mask) * 16 + sub];
        #pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= x[u];
    }
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Issue-rate and overlap probe: one workgroup of 4 or 8 waves per CU (the static LDS array
// keeps a second workgroup off the CU), every wave timing `iters` rounds of one instruction
// pattern with the shader clock.  Each round issues, in the named encodings:
//   0: 16 v_mfma_f32_32x32x16_bf16 on two accumulators;
//   1: 64 independent v_fma_f32;
//   2: 32 independent v_exp_f32;
//   3: the 16 MFMAs of 0, each followed by 2 v_fma_f32 and 2 v_exp_f32 (one instruction stream);
//   4: waves 0-3 the 16 MFMAs, waves 4-7 the 32 v_fma_f32 and 32 v_exp_f32 (two streams on each
//      SIMD: one wave of matrix work, one of vector work);
//   5: the 16 MFMAs, each followed by 4 v_fma_f32 and 2 v_exp_f32;
//   6: as 4, with the MFMA waves at s_setprio 3;
//   7: waves 0-3 the 16 MFMAs, waves 4-7 48 v_fma_f32 and 16 v_exp_f32 (a softmax's mix of
//      vector work per 16 MFMAs);
//   8: as 7, with the MFMA waves at s_setprio 3;
//   9: 16 MFMAs on one accumulator (each depends on the one before);
//  10: 64 v_fma_f32 in one dependent chain;
//  11: 32 v_exp_f32, each followed by a v_add_f32 that reads its result (into 4 sums).
// In the two-stream patterns the role is taken from a wave-uniform (scalar) wave index
// outside the timed loop, so that each wave's loop holds its own instructions only.  The
// vector instructions are written as inline assembly so that the count and encoding are
// exactly these; none of them reads memory.
#define PROBE_MFMA(acc) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define PROBE_FMA(i) asm volatile("v_fma_f32 %0, %0, %1, -1.0" : "+v"(x[i]) : "s"(c))
#define PROBE_EXP(i) asm volatile("v_exp_f32_e32 %0, %0" : "+v"(x[i]))
template <int K>
__global__ __launch_bounds__(512) void issue_probe(float* out, unsigned long long* cyc, int iters, float seed)
{
    __shared__ float pad[24576];
    if (iters < 0) pad[threadIdx.x] = seed;   // never taken: the array only reserves LDS
    float x[64];
    #pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = seed * (float)(threadIdx.x + i);
    const float c = seed * 0.5f;
    bf16x8 a, b;
    #pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
        b[i] = (__bf16)(seed * (float)i);
    }
    f32x16 acc0 = {}, acc1 = {};
    constexpr bool SPLIT = K == 4 || (K >= 6 && K <= 8);
    const bool mfma_wave = !SPLIT || __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4;
    const unsigned long long t0 = __builtin_readcyclecounter();
    if (SPLIT && mfma_wave) {
        if constexpr (K == 6 || K == 8) __builtin_amdgcn_s_setprio(3);
        for (int it = 0; it < iters; ++it) {
            #pragma unroll
            for (int f = 0; f < 16; ++f) {
                if (f & 1) PROBE_MFMA(acc1); else PROBE_MFMA(acc0);
            }
        }
        if constexpr (K == 6 || K == 8) __builtin_amdgcn_s_setprio(0);
    } else if (SPLIT) {
        for (int it = 0; it < iters; ++it) {
            #pragma unroll
            for (int f = 0; f < 16; ++f) {
                if constexpr (K == 4 || K == 6) {
                    PROBE_FMA(2 * f); PROBE_FMA(2 * f + 1); PROBE_EXP(32 + 2 * f); PROBE_EXP(33 + 2 * f);
                } else {
                    PROBE_FMA(3 * f); PROBE_FMA(3 * f + 1); PROBE_FMA(3 * f + 2); PROBE_EXP(48 + f);
                }
            }
        }
    } else {
        for (int it = 0; it < iters; ++it) {
            #pragma unroll
            for (int f = 0; f < 16; ++f) {
                if constexpr (K == 0 || K == 3 || K == 5) {
                    if (f & 1) PROBE_MFMA(acc1); else PROBE_MFMA(acc0);
                }
                if constexpr (K == 9) PROBE_MFMA(acc0);
                if constexpr (K == 10) { PROBE_FMA(0); PROBE_FMA(0); PROBE_FMA(0); PROBE_FMA(0); }
                if constexpr (K == 11) {
                    PROBE_EXP(8 + 2 * f); asm volatile("v_add_f32_e32 %0, %0, %1" : "+v"(x[f & 3]) : "v"(x[8 + 2 * f]));
                    PROBE_EXP(9 + 2 * f); asm volatile("v_add_f32_e32 %0, %0, %1" : "+v"(x[(f + 2) & 3]) : "v"(x[9 + 2 * f]));
                }
                if constexpr (K == 1) { PROBE_FMA(4 * f); PROBE_FMA(4 * f + 1); PROBE_FMA(4 * f + 2); PROBE_FMA(4 * f + 3); }
                if constexpr (K == 2) { PROBE_EXP(2 * f); PROBE_EXP(2 * f + 1); }
                if constexpr (K == 3) { PROBE_FMA(2 * f); PROBE_FMA(2 * f + 1); PROBE_EXP(32 + 2 * f); PROBE_EXP(33 + 2 * f); }
                if constexpr (K == 5) {
                    PROBE_FMA(4 * f); PROBE_FMA(4 * f + 1); PROBE_FMA(4 * f + 2); PROBE_FMA(4 * f + 3);
                    PROBE_EXP(2 * f); PROBE_EXP(2 * f + 1);
                }
            }
        }
    }
    const unsigned long long t1 = __builtin_readcyclecounter();
    float r = 0.f;
    #pragma unroll
    for (int i = 0; i < 64; ++i) r += x[i];
    #pragma unroll
    for (int i = 0; i < 16; ++i) r += acc0[i] + acc1[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if ((threadIdx.x & 63) == 0) {
        cyc[32 * blockIdx.x + 2 * (threadIdx.x >> 6)] = t0;
        cyc[32 * blockIdx.x + 2 * (threadIdx.x >> 6) + 1] = t1;
        // SIMD of this wave: HW_ID bits 5:4 (s_getreg_b32 hwreg(HW_REG_HW_ID, 4, 2))
        cyc[32 * blockIdx.x + 16 + (threadIdx.x >> 6)] = (unsigned long long)__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);
    }
}
#undef PROBE_MFMA
#undef PROBE_FMA
#undef PROBE_EXP

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

int miattn_probe_l2_gather(const void* table, int32_t rows_log2, int32_t blocks, int32_t iters,
                           uint32_t* out, void* stream)
{
    if (!table || !out || rows_log2 < 1 || rows_log2 > 20 || blocks < 1 || iters < 8 || iters % 8)
        return (int)hipErrorInvalidValue;
    if ((uintptr_t)table % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(l2_gather, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4*)table, rows_log2, iters, (unsigned*)out);
    return (int)hipGetLastError();
}

int64_t miattn_probe_l2_gather_bytes(int32_t blocks, int32_t iters)
{
    return (int64_t)blocks * kThreads * iters * 16;
}

int miattn_probe_issue(int32_t kind, float* out, uint64_t* cycles, int32_t blocks, int32_t waves_per_simd,
                       int32_t iters, void* stream)
{
    if (!out || !cycles || blocks < 1 || iters < 1 || kind < 0 || kind > 11) return (int)hipErrorInvalidValue;
    if (waves_per_simd != 1 && waves_per_simd != 2) return (int)hipErrorInvalidValue;
    if ((kind == 4 || (kind >= 6 && kind <= 8)) && waves_per_simd != 2) return (int)hipErrorInvalidValue;
    const dim3 g(blocks), b(256 * waves_per_simd);
    const hipStream_t st = (hipStream_t)stream;
    unsigned long long* cy = (unsigned long long*)cycles;
    switch (kind) {
    case 0: hipLaunchKernelGGL(issue_probe<0>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 1: hipLaunchKernelGGL(issue_probe<1>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 2: hipLaunchKernelGGL(issue_probe<2>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 3: hipLaunchKernelGGL(issue_probe<3>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 4: hipLaunchKernelGGL(issue_probe<4>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 5: hipLaunchKernelGGL(issue_probe<5>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 6: hipLaunchKernelGGL(issue_probe<6>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 7: hipLaunchKernelGGL(issue_probe<7>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 8: hipLaunchKernelGGL(issue_probe<8>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 9: hipLaunchKernelGGL(issue_probe<9>, g, b, 0, st, out, cy, iters, 0.001f); break;
    case 10: hipLaunchKernelGGL(issue_probe<10>, g, b, 0, st, out, cy, iters, 0.001f); break;
    default: hipLaunchKernelGGL(issue_probe<11>, g, b, 0, st, out, cy, iters, 0.001f); break;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
