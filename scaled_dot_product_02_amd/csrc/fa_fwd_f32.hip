// Attention forward in fp32 arithmetic on the vector ALUs.
//
// Same operation, batches, masks and statistics as the MFMA kernel.  It serves fp32
// inputs (the slower path the SDPA-pitfalls blog describes for FlashAttention backends,
// kept exact to fp32 rounding rather than rounded through bf16), and any input type when
// an explicit mask tensor is given (inputs widened to fp32 on load, output rounded to the
// input type).
//
// One workgroup = one wave = 64 query rows, one row per lane; K/V tiles of 32 keys are
// staged in LDS and read as broadcasts.  Keys are consumed in chunks of 16 with one
// online-softmax rescale per chunk.
#include "fa_common.h"

namespace miattn {
namespace {

constexpr int BM = kF32TileM;  // query rows per workgroup (one per lane)
constexpr int BN = 32;         // keys per LDS tile
constexpr int CH = 16;         // keys per softmax chunk

__device__ inline float4 load4(const float* x) { return *(const float4*)x; }
__device__ inline float4 load4(const __bf16* x)
{
    typedef __bf16 v4 __attribute__((ext_vector_type(4)));
    const v4 y = *(const v4*)x;
    return float4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
}
__device__ inline float4 load4(const _Float16* x)
{
    typedef _Float16 v4 __attribute__((ext_vector_type(4)));
    const v4 y = *(const v4*)x;
    return float4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
}
__device__ inline void store4(float* x, float4 v) { *(float4*)x = v; }
template <typename T>
__device__ inline void store4(T* x, float4 v)
{
    typedef T v4 __attribute__((ext_vector_type(4)));
    *(v4*)x = v4{(T)v.x, (T)v.y, (T)v.z, (T)v.w};
}

// T: input / output type; UPDATE = true: the epilogue merges the partial result into
// p.prev_* (ring update); MASKED = true: p.amask removes keys as well.
// D: head dim of Q and K; DV: head dim of V and the output (DV <= D).
// DROP = true: dropout on the probabilities (p.drop_*), the kept ones scaled in the epilogue.
template <typename T, int D, int DV, bool UPDATE, bool MASKED, bool DROP = false>
__global__ __launch_bounds__(64) void fa_fwd_f32_kernel(FaParams p)
{
    __shared__ __attribute__((aligned(16))) float Ks[BN * D];
    __shared__ __attribute__((aligned(16))) float Vs[BN * DV];

    const TileCoord tc = decode_tile(p, blockIdx.x, BM);
    if (!tc.live) return;
    const int lane = threadIdx.x;
    const int i0 = tc.r0;
    const int i1 = tc.r1;
    const int qi = i0 + lane;

    const T* qg = (const T*)p.q + (int64_t)tc.b * p.q_sb + tc.q0 * p.q_ss + (int64_t)tc.h * p.q_sh;
    const T* kg = (const T*)p.k + (int64_t)tc.b * p.k_sb + tc.kv0 * p.k_ss + (int64_t)tc.kvh * p.k_sh;
    const T* vg = (const T*)p.v + (int64_t)tc.b * p.v_sb + tc.kv0 * p.v_ss + (int64_t)tc.kvh * p.v_sh;
    T* og = (T*)p.out + (int64_t)tc.b * p.o_sb + tc.q0 * p.o_ss + (int64_t)tc.h * p.o_sh;
    const int64_t st_base = (int64_t)tc.b * p.st_sb + (int64_t)tc.h * p.st_sh + tc.q0;

    const Band bd = band_of(p, tc);
    int kv_lo, kv_hi;
    key_range(bd, i0, i1, tc.len_kv, kv_lo, kv_hi);
    // explicit mask row of this lane (rows / keys outside the mask count as masked)
    const bool mrow = MASKED && qi < p.Sq;
    const uint8_t* arow = MASKED ? p.amask + (int64_t)(mrow ? qi : 0) * p.amask_ld : nullptr;

    float q[D], o[DV];
    #pragma unroll
    for (int d = 0; d < D; d += 4) {
        float4 x = qi < tc.len_q ? load4(qg + (int64_t)qi * p.q_ss + d) : float4{0, 0, 0, 0};
        q[d] = x.x; q[d + 1] = x.y; q[d + 2] = x.z; q[d + 3] = x.w;
    }
    #pragma unroll
    for (int d = 0; d < DV; ++d) o[d] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int j0 = (kv_lo / BN) * BN; j0 < kv_hi; j0 += BN) {
        __syncthreads();
        for (int c = lane; c < BN * D / 4; c += 64) {
            const int row = c / (D / 4), col = 4 * (c % (D / 4));
            float4 kx{0, 0, 0, 0};
            if (j0 + row < tc.len_kv) kx = load4(kg + (int64_t)(j0 + row) * p.k_ss + col);
            *(float4*)(Ks + row * D + col) = kx;
        }
        for (int c = lane; c < BN * DV / 4; c += 64) {
            const int row = c / (DV / 4), col = 4 * (c % (DV / 4));
            float4 vx{0, 0, 0, 0};
            if (j0 + row < tc.len_kv) vx = load4(vg + (int64_t)(j0 + row) * p.v_ss + col);
            *(float4*)(Vs + row * DV + col) = vx;
        }
        __syncthreads();

        for (int c0 = 0; c0 < BN; c0 += CH) {
            float s[CH];
            float mx = -INFINITY;
            #pragma unroll
            for (int jj = 0; jj < CH; ++jj) {
                const float* kr = Ks + (c0 + jj) * D;
                float acc = 0.f;
                #pragma unroll
                for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], kr[d], acc);
                const int j = j0 + c0 + jj;
                const int64_t dj = (int64_t)j - qi;
                bool vis = j < tc.len_kv && ((dj <= bd.next && -dj <= bd.pre) || j < bd.pfx);
                if constexpr (MASKED) vis = vis && mrow && j < p.Skv && arow[j] == 0;
                s[jj] = vis ? acc * p.scale_log2 : -INFINITY;
                mx = fmaxf(mx, s[jj]);
            }
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            l_run *= alpha;
            #pragma unroll
            for (int d = 0; d < DV; ++d) o[d] *= alpha;
            uint32_t dw[4] = {0, 0, 0, 0};   // dropout bytes of the chunk's 16 keys
            if constexpr (DROP) {
                dw[0] = (uint32_t)((j0 + c0) >> 4);
                dw[1] = (uint32_t)qi;
                dw[2] = (uint32_t)(tc.h + 256 * tc.b);
                dw[3] = p.drop_offset;
                philox4x32_10(dw, p.seed_lo, p.seed_hi);
            }
            #pragma unroll
            for (int jj = 0; jj < CH; ++jj) {
                float e = __builtin_amdgcn_exp2f(s[jj] - m_use);
                l_run += e;
                if constexpr (DROP)
                    if (((dw[jj >> 2] >> (8 * (jj & 3))) & 0xffu) < p.drop_thr) e = 0.f;
                const float* vr = Vs + (c0 + jj) * DV;
                #pragma unroll
                for (int d = 0; d < DV; ++d) o[d] = __builtin_fmaf(e, vr[d], o[d]);
            }
            m_run = m_new;
        }
    }

    if (qi < i1) {
        // partial: O / l_run with max mc = m_run ln 2 and sum l_run; with UPDATE it is merged
        // into the prior (o_p, m_p, l_p): m = max(m_p, mc), a = l_p e^(m_p - m),
        // c = l_run e^(mc - m), out = o_p a / (a + c) + (O / l_run) c / (a + c)
        const bool any = l_run > 0.f;
        const float mc = any ? m_run * 0.69314718055994530942f : -INFINITY;
        float m_out = mc, l_out = l_run;
        float wc = any ? (DROP ? p.drop_scale : 1.f) / l_run : 0.f, wp = 0.f;
        if constexpr (UPDATE) {
            const float mp = p.prev_max[st_base + qi], lp = p.prev_sum[st_base + qi];
            const float m = fmaxf(mp, mc);
            wc = 0.f;
            l_out = 0.f;
            if (m != -INFINITY) {
                const float a = lp * __builtin_amdgcn_exp2f((mp - m) * 1.4426950408889634f);
                const float f = any ? __builtin_amdgcn_exp2f(m_run - m * 1.4426950408889634f) : 0.f;
                l_out = a + l_run * f;
                wp = a / l_out;
                wc = f / l_out;
            }
            m_out = m;
        }
        T* orow = og + (int64_t)qi * p.o_ss;
        #pragma unroll
        for (int d = 0; d < DV; d += 4) {
            float4 y{o[d] * wc, o[d + 1] * wc, o[d + 2] * wc, o[d + 3] * wc};
            if constexpr (UPDATE) {
                // an empty prior (weight 0) is not read: its buffer may hold anything
                if (wp != 0.f) {
                    const float4 po = load4((const T*)p.prev_out + (orow - (T*)p.out) + d);
                    y = float4{__builtin_fmaf(po.x, wp, y.x), __builtin_fmaf(po.y, wp, y.y),
                               __builtin_fmaf(po.z, wp, y.z), __builtin_fmaf(po.w, wp, y.w)};
                }
            }
            store4(orow + d, y);
        }
        if (p.smax) p.smax[st_base + qi] = m_out;
        if (p.ssum) p.ssum[st_base + qi] = l_out;
    }
}

template <typename T, bool UPDATE, bool MASKED>
hipError_t launch_t(const FaParams& p, int D, hipStream_t stream)
{
    dim3 grid(p.n_slots), block(64);
    if (p.drop_thr) {   // dropout: plain fp32 forward with Dv = D
        if constexpr (UPDATE || MASKED || sizeof(T) != 4) return hipErrorInvalidValue;
        else if (p.Dv != D) return hipErrorInvalidValue;
        else switch (D) {
        case 32: hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 32, 32, false, false, true>), grid, block, 0, stream, p); break;
        case 64: hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 64, 64, false, false, true>), grid, block, 0, stream, p); break;
        case 96: hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 96, 96, false, false, true>), grid, block, 0, stream, p); break;
        case 128: hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 128, 128, false, false, true>), grid, block, 0, stream, p); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (p.Dv != D) {   // value head dim below the Q/K head dim: plain fp32 forward only
        if constexpr (UPDATE || MASKED || sizeof(T) != 4) return hipErrorInvalidValue;
        else if (D == 64 && p.Dv == 32)
            hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 64, 32, false, false>), grid, block, 0, stream, p);
        else if (D == 96 && p.Dv == 64)
            hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 96, 64, false, false>), grid, block, 0, stream, p);
        else if (D == 128 && p.Dv == 64)
            hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 128, 64, false, false>), grid, block, 0, stream, p);
        else if (D == 128 && p.Dv == 96)
            hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 128, 96, false, false>), grid, block, 0, stream, p);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    switch (D) {
    case 32: hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 32, 32, UPDATE, MASKED>), grid, block, 0, stream, p); break;
    case 64: hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 64, 64, UPDATE, MASKED>), grid, block, 0, stream, p); break;
    case 96: hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 96, 96, UPDATE, MASKED>), grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL((fa_fwd_f32_kernel<T, 128, 128, UPDATE, MASKED>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_type(const FaParams& p, int D, hipStream_t stream)
{
    if (p.amask)
        return p.prev_out ? launch_t<T, true, true>(p, D, stream) : launch_t<T, false, true>(p, D, stream);
    return p.prev_out ? launch_t<T, true, false>(p, D, stream) : launch_t<T, false, false>(p, D, stream);
}

}  // namespace

// dtype: 0 = fp32, 1 = bf16, 2 = fp16 (the C-ABI enum values); bf16 / fp16 only with a mask
hipError_t launch_fa_fwd_f32(const FaParams& p, int D, int dtype, hipStream_t stream)
{
    if (dtype == 1 && p.amask) return launch_type<__bf16>(p, D, stream);
    if (dtype == 2 && p.amask) return launch_type<_Float16>(p, D, stream);
    if (dtype == 0) return launch_type<float>(p, D, stream);
    return hipErrorInvalidValue;
}

}  // namespace miattn
