// CSR-sparse attention, fp32 or fp64 (Paddle "sparse_attention": formula, parameters,
// example; the page lists float32 and float64 inputs).  All arithmetic is in the input type.
//
// Row i of slice (b, n) attends to the key rows listed in
// columns[b][n][offset[b][n][i] .. offset[b][n][i+1]).  One wave per query row:
//   * score phase: lane e takes entry e of a 64-entry chunk and forms the whole dot
//     product q . k_col (the query row is broadcast from LDS, the key row is gathered with
//     16-byte loads);
//   * chunk max and sum by wave butterflies; the running max / sum are rescaled once per
//     chunk (online softmax in the log2 domain);
//   * value phase: the chunk's (probability, column) pairs are broadcast lane by lane and
//     every lane accumulates its own head-dim slice of sum_c p_c v_c (coalesced row reads),
//     16 value rows per batch with all their loads in flight together.
// Work per row is proportional to its entry count; four consecutive rows of one slice
// share a workgroup so their common columns are re-read from L1/L2.
#include "fa_params.h"

namespace miattn {
namespace {

constexpr int NT = 256;

template <typename T>
__device__ inline T wave_max(T x)
{
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
    return x;
}
template <typename T>
__device__ inline T wave_sum(T x)
{
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ inline float exp2_t(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline double exp2_t(double x) { return exp2(x); }
__device__ inline float lane_value(float x, int e)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), e));
}
__device__ inline double lane_value(double x, int e)
{
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, e);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), e);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// T = float or double (all arithmetic in T); D a multiple of 32.
template <typename T, int D>
__global__ __launch_bounds__(NT) void sparse_csr_kernel(SparseParams p)
{
    constexpr int VW = 16 / sizeof(T);          // elements per 16-byte load
    typedef T V __attribute__((ext_vector_type(VW)));
    constexpr int PL = (D + 63) / 64;           // head-dim values per lane in the value phase
    __shared__ __attribute__((aligned(16))) T qs[NT / 64][D];
    const T* q = (const T*)p.q;
    const T* k = (const T*)p.k;
    const T* v = (const T*)p.v;
    T* out = (T*)p.out;
    const T scale_log2 = sizeof(T) == 8 ? (T)p.scale_log2_d : (T)p.scale_log2;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t total = (int64_t)p.B * p.N * p.S;
    // workgroups go to the 8 XCDs round-robin (id mod 8); XCD x takes the x-th eighth of
    // the row blocks in order, so that the rows resident on one XCD are consecutive rows of
    // one slice and share its K/V rows (the band, and the slice as a whole) in that XCD's L2
    const int64_t nblk = (total + NT / 64 - 1) / (NT / 64);
    const int64_t per = (nblk + 7) / 8;
    const int64_t blk = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    const int64_t row = blk * (NT / 64) + wave;
    const bool valid = row < total;
    if (valid)
        for (int d = lane; d < D; d += 64) qs[wave][d] = q[row * D + d];
    __syncthreads();
    if (!valid) return;

    const int64_t bn = row / p.S;
    const int i = (int)(row - bn * p.S);
    const int32_t* off = p.offset + bn * (p.S + 1);
    const int32_t* col = p.columns + bn * p.nnz;
    const T* kb = k + bn * p.S * D;
    const T* vb = v + bn * p.S * D;
    const int e0 = off[i], e1 = off[i + 1];

    T m_run = -INFINITY, l_run = 0;
    T o[PL];
    #pragma unroll
    for (int u = 0; u < PL; ++u) o[u] = 0;

    for (int base = e0; base < e1; base += 64) {
        const int cnt = min(64, e1 - base);
        T sc = -INFINITY;
        int c = 0;
        if (lane < cnt) {
            c = col[base + lane];
            const V* kr = (const V*)(kb + (int64_t)c * D);
            const V* qr = (const V*)qs[wave];
            T acc = 0;
            #pragma unroll
            for (int dv = 0; dv < D / VW; ++dv) {
                const V kx = kr[dv], qx = qr[dv];
                #pragma unroll
                for (int e = 0; e < VW; ++e) acc = fma(qx[e], kx[e], acc);
            }
            sc = acc * scale_log2;
        }
        const T m_new = fmax(m_run, wave_max(sc));
        const T alpha = exp2_t(m_run - m_new);
        const T pv = lane < cnt ? exp2_t(sc - m_new) : (T)0;
        l_run = l_run * alpha + wave_sum(pv);
        #pragma unroll
        for (int u = 0; u < PL; ++u) o[u] *= alpha;
        // value rows in batches of VB entries: all loads of a batch are in flight together
        // (one entry at a time would wait out a full memory latency per entry)
        constexpr int VB = 16;
        int e = 0;
        for (; e + VB <= cnt; e += VB) {
            T vv[VB][PL];
            #pragma unroll
            for (int x = 0; x < VB; ++x) {
                const T* vr = vb + (int64_t)__builtin_amdgcn_readlane(c, e + x) * D;
                #pragma unroll
                for (int u = 0; u < PL; ++u)
                    vv[x][u] = (D % 64 == 0 || lane + 64 * u < D) ? vr[lane + 64 * u] : (T)0;
            }
            #pragma unroll
            for (int x = 0; x < VB; ++x) {
                const T pe = lane_value(pv, e + x);
                #pragma unroll
                for (int u = 0; u < PL; ++u) o[u] = fma(pe, vv[x][u], o[u]);
            }
        }
        for (; e < cnt; ++e) {
            const T pe = lane_value(pv, e);
            const int ce = __builtin_amdgcn_readlane(c, e);
            const T* vr = vb + (int64_t)ce * D;
            #pragma unroll
            for (int u = 0; u < PL; ++u)
                if (D % 64 == 0 || lane + 64 * u < D) o[u] = fma(pe, vr[lane + 64 * u], o[u]);
        }
        m_run = m_new;
    }
    const T inv = l_run > 0 ? (T)1 / l_run : (T)0;
    #pragma unroll
    for (int u = 0; u < PL; ++u)
        if (D % 64 == 0 || lane + 64 * u < D) out[row * D + lane + 64 * u] = o[u] * inv;
}

template <typename T>
hipError_t launch_t(const SparseParams& p, int D, hipStream_t stream)
{
    const int64_t rows = (int64_t)p.B * p.N * p.S;
    dim3 grid((unsigned)(((rows + NT / 64 - 1) / (NT / 64) + 7) / 8 * 8)), block(NT);
    switch (D) {
    case 32: hipLaunchKernelGGL((sparse_csr_kernel<T, 32>), grid, block, 0, stream, p); break;
    case 64: hipLaunchKernelGGL((sparse_csr_kernel<T, 64>), grid, block, 0, stream, p); break;
    case 96: hipLaunchKernelGGL((sparse_csr_kernel<T, 96>), grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL((sparse_csr_kernel<T, 128>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_csr(const SparseParams& p, int D, bool f64, hipStream_t stream)
{
    return f64 ? launch_t<double>(p, D, stream) : launch_t<float>(p, D, stream);
}

}  // namespace miattn
