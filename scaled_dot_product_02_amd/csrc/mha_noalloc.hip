// The multi-head self-attention forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// mha_self_attn_fwd_noalloc, declared in include/miattn.h.  Same module as mha_self_attn_fwd
// (the MultiHeadAttention example of the page "flash attention的调用"), with two changes:
//   * its intermediates (q, k, v and the attention output) live in `scratch`, a file-scope
//     device array of kScratchBytes that each GPU holds until the process ends, instead of
//     a caller workspace;
//   * its projections run on linear_kernel below (no library GEMM, which may allocate its
//     own workspace or load code on first use).
// Nothing here calls hipMalloc, hipFree or an allocating library routine.  The address of a
// device's copy of `scratch` is looked up once per device with hipGetSymbolAddress, on that
// device's first call; host code uses only that address, never the array's name.
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>

#include "miattn.h"

namespace {

constexpr int64_t kScratchBytes = MIATTN_MHA_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (its device address), looked up on first use.
miattn_status_t scratch_of_device(int dev, void** ptr)
{
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MIATTN_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MIATTN_OK;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Operand fragment of one 32x32 MFMA step over 16 contraction indices: lane l holds
// k = 8 (l / 32) .. + 7 of its row.  fp32 runs the step as eight 32x32x2 MFMAs pairing
// element e of both operands (k = e on lanes 0..31, 8 + e on 32..63), which sums all 16 k.
template <typename T> struct Mma;
template <> struct Mma<__bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    __device__ static f32x16 step(const v8& a, const v8& b, const f32x16& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    __device__ static f32x16 step(const v8& a, const v8& b, const f32x16& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    typedef float v8 __attribute__((ext_vector_type(8)));
    __device__ static f32x16 step(const v8& a, const v8& b, f32x16 c)
    {
        #pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
};

constexpr int kLinThreads = 256;   // 4 waves
constexpr int LM = 128;            // rows of x (= rows of y) per workgroup
constexpr int LN = 128;            // rows of w (= columns of y) per workgroup
constexpr int LK = 32;             // contraction indices per staged chunk

// y[M][N] = x[M][K] w[N][K]^T + bias[N] (bias may be null), fp32 accumulation, one rounding
// to T; a linear layer with its weight stored [out, in].  K a multiple of 16 / sizeof(T) (so
// that 16-byte vectors never straddle the end of a row), rows 16-byte aligned.
// Wave (wm, wn) computes the 64 x 64 block y[64 wm ..][64 wn ..] of the workgroup's tile as
// y^T = w x^T: in the accumulator of a 32x32 MFMA a lane owns one row m of y and four
// consecutive columns n per group of four registers, so each group is one vector store.
// The x and w chunks pass through LDS (padded rows), the next chunk is loaded into
// registers while the current one is multiplied.
template <typename T>
__global__ __launch_bounds__(kLinThreads) void linear_kernel(const T* __restrict__ x,
                                                             const T* __restrict__ w,
                                                             const T* __restrict__ bias,
                                                             T* __restrict__ y, int64_t M, int N, int K)
{
    typedef typename Mma<T>::v8 v8;
    constexpr int EV = 16 / sizeof(T);        // elements per 16-byte vector
    constexpr int VPR = LK / EV;              // vectors per chunk row
    constexpr int RS = LK + 8;                // LDS row stride (elements): 8 of padding keeps
                                              // every 8-element fragment aligned to its size
    constexpr int VPT = LM * VPR / kLinThreads;   // vectors of each operand per thread per chunk
    __shared__ __attribute__((aligned(32))) T xs[LM * RS];
    __shared__ __attribute__((aligned(32))) T ws[LN * RS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.x * LM;
    const int n0 = blockIdx.y * LN;

    u32x4 sx[VPT], sw[VPT];
    auto load_chunk = [&](int k0) {
        #pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int c = tid + kLinThreads * u;
            const int r = c / VPR, kc = k0 + (c % VPR) * EV;
            const bool kin = kc < K;
            const int64_t xr = m0 + r;
            const int wr = n0 + r;
            sx[u] = kin && xr < M ? *(const u32x4*)(x + xr * K + kc) : u32x4{0u, 0u, 0u, 0u};
            sw[u] = kin && wr < N ? *(const u32x4*)(w + (int64_t)wr * K + kc) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_chunk = [&]() {
        #pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int c = tid + kLinThreads * u;
            const int r = c / VPR, kv = (c % VPR) * EV;
            *(u32x4*)(xs + r * RS + kv) = sx[u];
            *(u32x4*)(ws + r * RS + kv) = sw[u];
        }
    };

    f32x16 acc[2][2];
    #pragma unroll
    for (int a = 0; a < 2; ++a)
        #pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    const int lr = lane & 31, lg = lane >> 5;
    load_chunk(0);
    for (int k0 = 0; k0 < K; k0 += LK) {
        __syncthreads();            // the previous chunk's readers are done
        store_chunk();
        __syncthreads();
        if (k0 + LK < K) load_chunk(k0 + LK);
        #pragma unroll
        for (int ks = 0; ks < LK; ks += 16) {
            v8 fw[2], fx[2];
            #pragma unroll
            for (int a = 0; a < 2; ++a)
                fw[a] = *(const v8*)(ws + (64 * wn + 32 * a + lr) * RS + ks + 8 * lg);
            #pragma unroll
            for (int b = 0; b < 2; ++b)
                fx[b] = *(const v8*)(xs + (64 * wm + 32 * b + lr) * RS + ks + 8 * lg);
            #pragma unroll
            for (int a = 0; a < 2; ++a)
                #pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = Mma<T>::step(fw[a], fx[b], acc[a][b]);
        }
    }

    // accumulator register i of block (a, b): column n = 32 a + 8 (i / 4) + 4 lg + i % 4 of
    // the wave's block, row m = 32 b + lr
    typedef T v4 __attribute__((ext_vector_type(4)));
    #pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int64_t m = m0 + 64 * wm + 32 * b + lr;
        if (m >= M) continue;
        #pragma unroll
        for (int a = 0; a < 2; ++a)
            #pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + 64 * wn + 32 * a + 8 * g + 4 * lg;
                if (n >= N) continue;
                v4 o;
                #pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = (T)(acc[a][b][4 * g + e] + (bias ? (float)bias[n + e] : 0.f));
                *(v4*)(y + m * N + n) = o;
            }
    }
}

int64_t elem_bytes(int dtype)
{
    switch (dtype) {
    case MIATTN_F32: return 4;
    case MIATTN_BF16:
    case MIATTN_F16: return 2;
    default: return 0;
    }
}

template <typename T>
void launch_linear_t(const void* x, const void* w, const void* bias, void* y, int64_t M, int N, int K,
                     hipStream_t stream)
{
    const dim3 grid((unsigned)((M + LM - 1) / LM), (unsigned)((N + LN - 1) / LN));
    hipLaunchKernelGGL(linear_kernel<T>, grid, dim3(kLinThreads), 0, stream, (const T*)x, (const T*)w,
                       (const T*)bias, (T*)y, M, N, K);
}

miattn_status_t launch_linear(int dtype, const void* x, const void* w, const void* bias, void* y,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    if (dtype == MIATTN_BF16) launch_linear_t<__bf16>(x, w, bias, y, M, (int)N, (int)K, stream);
    else if (dtype == MIATTN_F16) launch_linear_t<_Float16>(x, w, bias, y, M, (int)N, (int)K, stream);
    else launch_linear_t<float>(x, w, bias, y, M, (int)N, (int)K, stream);
    return hipGetLastError() == hipSuccess ? MIATTN_OK : MIATTN_ERR_LAUNCH;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

miattn_status_t mha_self_attn_fwd_noalloc(const void* x, const void* w_qkv, const void* b_qkv,
                                          const void* w_out, const void* b_out, void* out,
                                          int64_t B, int64_t S, int64_t E, int64_t N,
                                          miattn_dtype_t dtype, const uint8_t* atten_mask,
                                          float dropout_p, uint64_t seed, uint32_t offset,
                                          void* stream)
{
    const int64_t eb = elem_bytes(dtype);
    if (eb == 0) return MIATTN_ERR_DTYPE;
    if (!x || !w_qkv || !w_out || !out) return MIATTN_ERR_NULL;
    if (B < 1 || S < 1 || N < 1 || N > 256 || E < N || E % N != 0 || B * S > INT32_MAX ||
        E > 32768)
        return MIATTN_ERR_SHAPE;
    const int64_t D = E / N;
    // head dims of the attention operator; rows of whole 16-byte vectors
    if (D > 768 || (E * eb) % 16 != 0) return MIATTN_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(w_out) || !aligned16(out))
        return MIATTN_ERR_SHAPE;   // operand and output rows move in 16-byte vectors
    const int64_t need = mha_workspace_bytes(B, S, E, dtype);
    if (need < 0) return MIATTN_ERR_SHAPE;
    if (need > kScratchBytes) return MIATTN_ERR_SCRATCH;
    if (!(dropout_p >= 0.f && dropout_p < 1.f)) return MIATTN_ERR_DROPOUT;
    if (dropout_p > 0.f && atten_mask) return MIATTN_ERR_UNSUPPORTED;
    // every check of the attention call, before the first launch
    const int32_t route = attn_fwd_route(B, N, N, S, S, D, D, dtype, MIATTN_BSND,
                                         MIATTN_MASK_NONE, atten_mask, dropout_p, 0);
    if (route < 0) return (miattn_status_t)(-route);

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MIATTN_ERR_LAUNCH;
    void* base = nullptr;
    const miattn_status_t sst = scratch_of_device(dev, &base);
    if (sst != MIATTN_OK) return sst;

    const hipStream_t st = (hipStream_t)stream;
    const int64_t M = B * S, plane = M * E * eb;
    char* ws = (char*)base;
    void* dst[3] = {ws, ws + plane, ws + 2 * plane};   // q, k, v
    void* ao = ws + 3 * plane;                         // attention output
    const char* wq = (const char*)w_qkv;
    const char* bq = (const char*)b_qkv;
    // the 3E outputs of the QKV layer split into thirds: rows [0, E), [E, 2E), [2E, 3E)
    for (int i = 0; i < 3; ++i) {
        const miattn_status_t s = launch_linear(dtype, x, wq + i * E * E * eb,
                                                bq ? bq + i * E * eb : nullptr, dst[i], M, E, E, st);
        if (s != MIATTN_OK) return s;
    }
    const miattn_status_t sa = attn_fwd_ext(dst[0], dst[1], dst[2], ao, nullptr, nullptr, B, N, N, S,
                                            S, D, D, dtype, MIATTN_BSND,
                                            (float)(1.0 / sqrt((double)D)), MIATTN_MASK_NONE, 0, 0,
                                            nullptr, atten_mask, dropout_p, seed, offset, stream);
    if (sa != MIATTN_OK) return sa;
    return launch_linear(dtype, ao, w_out, b_out, out, M, E, E, st);
}

}  // extern "C"
