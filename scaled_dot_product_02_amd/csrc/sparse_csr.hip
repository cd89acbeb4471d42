// CSR-sparse attention, fp32 (Paddle "sparse_attention": formula, parameters, example).
//
// Row i of slice (b, n) attends to the key rows listed in
// columns[b][n][offset[b][n][i] .. offset[b][n][i+1]).  One wave per query row:
//   * score phase: lane e takes entry e of a 64-entry chunk and forms the whole dot
//     product q . k_col (the query row is broadcast from LDS, the key row is gathered with
//     16-byte loads);
//   * chunk max and sum by wave butterflies; the running max / sum are rescaled once per
//     chunk (online softmax in the log2 domain);
//   * value phase: the chunk's (probability, column) pairs are broadcast lane by lane and
//     every lane accumulates its own head-dim slice of sum_c p_c v_c (coalesced row reads).
// Work per row is proportional to its entry count; four consecutive rows of one slice
// share a workgroup so their common columns are re-read from L1/L2.
#include "fa_params.h"

namespace miattn {
namespace {

constexpr int NT = 256;

__device__ inline float wave_max(float x)
{
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ inline float wave_sum(float x)
{
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D>
__global__ __launch_bounds__(NT) void sparse_csr_kernel(SparseParams p)
{
    constexpr int PL = D / 64;  // head-dim values per lane in the value phase
    __shared__ __attribute__((aligned(16))) float qs[NT / 64][D];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t total = (int64_t)p.B * p.N * p.S;
    const int64_t row = (int64_t)blockIdx.x * (NT / 64) + wave;
    const bool valid = row < total;
    if (valid)
        for (int d = lane; d < D; d += 64) qs[wave][d] = p.q[row * D + d];
    __syncthreads();
    if (!valid) return;

    const int64_t bn = row / p.S;
    const int i = (int)(row - bn * p.S);
    const int32_t* off = p.offset + bn * (p.S + 1);
    const int32_t* col = p.columns + bn * p.nnz;
    const float* kb = p.k + bn * p.S * D;
    const float* vb = p.v + bn * p.S * D;
    const int e0 = off[i], e1 = off[i + 1];

    float m_run = -INFINITY, l_run = 0.f;
    float o[PL];
    #pragma unroll
    for (int u = 0; u < PL; ++u) o[u] = 0.f;

    for (int base = e0; base < e1; base += 64) {
        const int cnt = min(64, e1 - base);
        float sc = -INFINITY;
        int c = 0;
        if (lane < cnt) {
            c = col[base + lane];
            const float4* kr = (const float4*)(kb + (int64_t)c * D);
            const float4* qr = (const float4*)qs[wave];
            float acc = 0.f;
            #pragma unroll
            for (int d4 = 0; d4 < D / 4; ++d4) {
                const float4 kx = kr[d4], qx = qr[d4];
                acc = __builtin_fmaf(qx.x, kx.x, acc);
                acc = __builtin_fmaf(qx.y, kx.y, acc);
                acc = __builtin_fmaf(qx.z, kx.z, acc);
                acc = __builtin_fmaf(qx.w, kx.w, acc);
            }
            sc = acc * p.scale_log2;
        }
        const float m_new = fmaxf(m_run, wave_max(sc));
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float pv = lane < cnt ? __builtin_amdgcn_exp2f(sc - m_new) : 0.f;
        l_run = l_run * alpha + wave_sum(pv);
        #pragma unroll
        for (int u = 0; u < PL; ++u) o[u] *= alpha;
        for (int e = 0; e < cnt; ++e) {
            const float pe = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), e));
            const int ce = __builtin_amdgcn_readlane(c, e);
            const float* vr = vb + (int64_t)ce * D;
            #pragma unroll
            for (int u = 0; u < PL; ++u) o[u] = __builtin_fmaf(pe, vr[lane + 64 * u], o[u]);
        }
        m_run = m_new;
    }
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    #pragma unroll
    for (int u = 0; u < PL; ++u) p.out[row * D + lane + 64 * u] = o[u] * inv;
}

}  // namespace

hipError_t launch_sparse_csr(const SparseParams& p, int D, hipStream_t stream)
{
    const int64_t rows = (int64_t)p.B * p.N * p.S;
    dim3 grid((unsigned)((rows + NT / 64 - 1) / (NT / 64))), block(NT);
    if (D == 64)
        hipLaunchKernelGGL(sparse_csr_kernel<64>, grid, block, 0, stream, p);
    else if (D == 128)
        hipLaunchKernelGGL(sparse_csr_kernel<128>, grid, block, 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace miattn
