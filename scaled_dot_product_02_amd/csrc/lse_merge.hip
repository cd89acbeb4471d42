// Merge of two partial attention results (ring-attention update).
//
// For each (b, n, s), in the order of "npu_ring_attention_update对外接口" (equivalent
// small-operator logic): m = max(m1, m2); a = l1 exp(m1 - m); c = l2 exp(m2 - m);
// l = a + c; out = o1 (a/l) + o2 (c/l); statistics (m, l) are written out, and the
// output is rounded (RNE) to its storage type.  Both partials empty (m = -inf) gives
// (0, -inf, 0).
//
// HBM-bound elementwise work.  One workgroup of 1024 threads takes SB = 8 consecutive
// positions s of one batch entry b for all heads; its N x 8 x D output elements are walked
// as one flat range of 16-byte vectors (8 bf16 / fp16 or 4 fp32), one vector per thread and
// array per pass, with non-temporal loads and stores (nothing reads them again).
//   1. Each thread first requests the statistics of one of the N x 8 rows, then the
//      vectors of the first pass (indices clamped into the range, so the loads need no
//      branch), so the weights are formed while the vector loads are in flight.
//   2. The two weights of every row go to LDS and the merged statistics out; one barrier.
//   3. Every pass combines and stores its vectors.
// Statistics are [B, N, S] floats: the 8 positions of one head are 32 bytes, so four
// consecutive position blocks share each 128-byte line; those blocks are placed on one XCD.
#include "fa_params.h"

namespace miattn {
namespace {

constexpr int SB = 8;      // positions per workgroup
constexpr int UV = 1;      // vectors (or elements) per thread and array in one pass
constexpr int NT = 1024;   // threads per workgroup
constexpr int RG = 4;      // consecutive position blocks run on one XCD
constexpr int NMAX = 256;  // largest head count

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec;
template <> struct Vec<__bf16> { static constexpr int W = 8; };
template <> struct Vec<_Float16> { static constexpr int W = 8; };
template <> struct Vec<float> { static constexpr int W = 4; };

__device__ inline void unpack(const u32x4& x, float* f, __bf16*)
{
    #pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(x[e] << 16);
        f[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
    }
}
__device__ inline void unpack(const u32x4& x, float* f, _Float16*)
{
    #pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = (float)__builtin_bit_cast(_Float16, (unsigned short)(x[e] & 0xffffu));
        f[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(x[e] >> 16));
    }
}
__device__ inline void unpack(const u32x4& x, float* f, float*)
{
    #pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(x[e]);
}
__device__ inline u32x4 pack(const float* f, __bf16*)
{
    u32x4 r;
    #pragma unroll
    for (int e = 0; e < 4; ++e) {
        const __bf16 a = (__bf16)f[2 * e], b = (__bf16)f[2 * e + 1];
        r[e] = (unsigned)__builtin_bit_cast(unsigned short, a) |
               ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
    }
    return r;
}
__device__ inline u32x4 pack(const float* f, _Float16*)
{
    u32x4 r;
    #pragma unroll
    for (int e = 0; e < 4; ++e) {
        const _Float16 a = (_Float16)f[2 * e], b = (_Float16)f[2 * e + 1];
        r[e] = (unsigned)__builtin_bit_cast(unsigned short, a) |
               ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
    }
    return r;
}
__device__ inline u32x4 pack(const float* f, float*)
{
    u32x4 r;
    #pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __float_as_uint(f[e]);
    return r;
}

// VEC = true: 16-byte vectors (D a multiple of the vector width, aligned pointers and
// strides); VEC = false: one element per thread step, any D.
template <typename T, bool VEC>
__global__ __launch_bounds__(NT) void lse_merge_kernel(MergeParams p)
{
    __shared__ float w1s[NMAX * SB];
    __shared__ float w2s[NMAX * SB];
    // Position blocks are handed to the 8 XCDs round-robin; remap them so that RG
    // consecutive blocks (whose statistics share 128-byte lines: RG * SB floats) run on one
    // XCD, back to back, and each line is fetched and written back once through its L2.
    int pb = blockIdx.x;
    {
        const int full = gridDim.x - gridDim.x % (8 * RG);
        if (pb < full) {
            const int xcd = pb & 7, k = pb >> 3;
            pb = (k / RG) * (8 * RG) + xcd * RG + (k % RG);
        }
    }
    const int s0 = pb * SB;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int nrow = min(SB, p.S - s0);
    const int nst = p.N * SB;            // statistics rows (n, ds), ds >= nrow unused

    const int W = VEC ? Vec<T>::W : 1;
    const int per_row = p.N * p.D / W;   // vectors (or elements) per position
    const int total = nrow * per_row;

    auto stat_index = [&](int e) {
        const int n = e / SB, ds = min(e % SB, nrow - 1);
        return ((int64_t)b * p.N + n) * p.S + s0 + ds;
    };
    // weights of one row from its two (max, sum) pairs, and the merged statistics
    auto weights = [](float m1, float l1, float m2, float l2, float& w1, float& w2, float& m, float& l) {
        m = fmaxf(m1, m2);
        const bool any = m != -INFINITY;
        const float mr = any ? m : 0.f;
        const float a = l1 * expf(m1 - mr);
        const float c = l2 * expf(m2 - mr);
        l = any ? a + c : 0.f;
        w1 = any ? a / l : 0.f;
        w2 = any ? c / l : 0.f;
    };

    // 1. statistics of row tid requested first (rows tid + NT, ... come later)
    const int e0 = min(tid, nst - 1);
    const bool own = tid < nst && e0 % SB < nrow;
    const int64_t si0 = stat_index(e0);
    const float a_m1 = p.m1[si0], a_l1 = p.l1[si0], a_m2 = p.m2[si0], a_l2 = p.l2[si0];

    // 2. vectors of one pass: every thread loads (indices clamped into the range), only
    //    threads inside it store
    u32x4 x1[UV], x2[UV];
    float y1[UV], y2[UV];
    int64_t off[UV];
    int slot[UV];
    auto load_pass = [&](int base) {
        #pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int c = min(base + tid + NT * u, total - 1);
            // vector c: position s0 + ds, head n, dims d .. d + W - 1
            const int ds = c / per_row;
            const int cr = (c - ds * per_row) * W;
            const int n = cr / p.D;
            const int d = cr - n * p.D;
            slot[u] = n * SB + ds;
            off[u] = (int64_t)b * p.sb + (int64_t)(s0 + ds) * p.ss + (int64_t)n * p.sh + d;
            if constexpr (VEC) {
                x1[u] = __builtin_nontemporal_load((const u32x4*)((const T*)p.o1 + off[u]));
                x2[u] = __builtin_nontemporal_load((const u32x4*)((const T*)p.o2 + off[u]));
            } else {
                y1[u] = (float)((const T*)p.o1)[off[u]];
                y2[u] = (float)((const T*)p.o2)[off[u]];
            }
        }
    };
    auto combine_pass = [&](int base) {
        #pragma unroll
        for (int u = 0; u < UV; ++u) {
            if (base + tid + NT * u < total) {
                const float w1 = w1s[slot[u]], w2 = w2s[slot[u]];
                if constexpr (VEC) {
                    float f1[Vec<T>::W], f2[Vec<T>::W], y[Vec<T>::W];
                    unpack(x1[u], f1, (T*)nullptr);
                    unpack(x2[u], f2, (T*)nullptr);
                    #pragma unroll
                    for (int e = 0; e < Vec<T>::W; ++e) y[e] = __builtin_fmaf(f1[e], w1, f2[e] * w2);
                    __builtin_nontemporal_store(pack(y, (T*)nullptr), (u32x4*)((T*)p.out + off[u]));
                } else {
                    ((T*)p.out)[off[u]] = (T)__builtin_fmaf(y1[u], w1, y2[u] * w2);
                }
            }
        }
    };

    load_pass(0);
    __builtin_amdgcn_sched_barrier(0);

    // 3. weights of the N x SB rows into LDS, merged statistics out; each row's statistics
    //    are read and written by one thread, so outputs may alias the inputs
    {
        float w1, w2, m, l;
        weights(a_m1, a_l1, a_m2, a_l2, w1, w2, m, l);
        if (own) {
            w1s[tid] = w1;
            w2s[tid] = w2;
            p.mo[si0] = m;
            p.lo[si0] = l;
        }
    }
    for (int e = tid + NT; e < nst; e += NT) {
        if (e % SB >= nrow) continue;
        const int64_t si = stat_index(e);
        float w1, w2, m, l;
        weights(p.m1[si], p.l1[si], p.m2[si], p.l2[si], w1, w2, m, l);
        w1s[e] = w1;
        w2s[e] = w2;
        p.mo[si] = m;
        p.lo[si] = l;
    }
    __syncthreads();

    combine_pass(0);
    for (int base = NT * UV; base < total; base += NT * UV) {
        load_pass(base);
        combine_pass(base);
    }
}

template <typename T>
hipError_t launch_t(const MergeParams& p, hipStream_t stream)
{
    constexpr int W = Vec<T>::W;
    const bool vec = p.D % W == 0 && p.sb % W == 0 && p.sh % W == 0 && p.ss % W == 0 &&
                     ((uintptr_t)p.o1 % 16 == 0) && ((uintptr_t)p.o2 % 16 == 0) &&
                     ((uintptr_t)p.out % 16 == 0);
    dim3 grid((p.S + SB - 1) / SB, p.B), block(NT);
    if (vec)
        hipLaunchKernelGGL((lse_merge_kernel<T, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((lse_merge_kernel<T, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

// dtype: 0 = fp32, 1 = bf16, 2 = fp16 (the C-ABI enum values)
hipError_t launch_lse_merge(const MergeParams& p, int dtype, hipStream_t stream)
{
    if (dtype == 1) return launch_t<__bf16>(p, stream);
    if (dtype == 2) return launch_t<_Float16>(p, stream);
    if (dtype == 0) return launch_t<float>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace miattn
