// Multi-head self-attention module forward: the MultiHeadAttention example of the page
// "flash attention的调用" (a fused QKV linear layer, scaled dot-product attention per head
// without a causal mask, an optional mask and dropout, and the output linear layer).
//
// The two projections are plain GEMMs and go to rocBLAS (bf16 / fp16 / fp32 storage, fp32
// accumulation).  Each GEMM writes a buffer that a small kernel first fills with the bias
// broadcast over the rows, and runs with beta = 1, so the bias is added inside the GEMM's
// fp32 accumulation and every output is rounded once, as a linear layer with a fused bias
// does.  The attention in between is attn_fwd_ext on the BSND views of q, k and v.
// Declared in include/miattn.h.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <math.h>
#include <mutex>

#include "miattn.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxDevices = 64;
constexpr int kFillThreads = 256;

// y[r][:] = bias (or 0) for r < rows, in 16-byte vectors; vpr vectors per row.
__global__ __launch_bounds__(kFillThreads) void broadcast_rows(u32x4* y, const u32x4* bias, int64_t rows, int64_t vpr)
{
    const int64_t n = rows * vpr;
    for (int64_t i = (int64_t)blockIdx.x * kFillThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kFillThreads)
        y[i] = bias ? bias[i % vpr] : u32x4{0u, 0u, 0u, 0u};
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

rocblas_datatype blas_type(int dtype)
{
    return dtype == MIATTN_F32 ? rocblas_datatype_f32_r
         : dtype == MIATTN_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f16_r;
}

// One rocBLAS handle per device, created on first use and kept until the process ends; the
// mutex also serialises (set stream, enqueue GEMMs) sequences of concurrent callers.
std::mutex g_blas_mu;
rocblas_handle g_blas[kMaxDevices] = {};

// y[M, n_out] = x[M, k] w[n_out, k]^T + bias (row-major, bias may be NULL).  Caller holds the
// mutex and has set the handle's stream.
miattn_status_t linear(rocblas_handle h, hipStream_t stream, const void* x, const void* w,
                       const void* bias, void* y, int64_t M, int64_t n_out, int64_t k, int dtype)
{
    const int64_t vpr = n_out * elem_bytes(dtype) / 16;
    const int64_t vecs = M * vpr;
    const int64_t blocks = (vecs + kFillThreads - 1) / kFillThreads;
    hipLaunchKernelGGL(broadcast_rows, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(kFillThreads), 0,
                       stream, (u32x4*)y, (const u32x4*)bias, M, vpr);
    if (hipGetLastError() != hipSuccess) return MIATTN_ERR_LAUNCH;
    // row-major y = x w^T is column-major y^T = w^T(col-major, transposed) . x^T
    const float alpha = 1.f, beta = 1.f;
    const rocblas_datatype t = blas_type(dtype);
    const rocblas_status st = rocblas_gemm_ex(
        h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)n_out, (rocblas_int)M,
        (rocblas_int)k, &alpha, w, t, (rocblas_int)k, x, t, (rocblas_int)k, &beta, y, t,
        (rocblas_int)n_out, y, t, (rocblas_int)n_out, rocblas_datatype_f32_r,
        rocblas_gemm_algo_standard, 0, 0);
    return st == rocblas_status_success ? MIATTN_OK : MIATTN_ERR_BLAS;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

int64_t mha_workspace_bytes(int64_t B, int64_t S, int64_t E, miattn_dtype_t dtype)
{
    const int64_t eb = elem_bytes(dtype);
    if (eb == 0 || B < 1 || S < 1 || E < 1 || B > (int64_t(1) << 31) || S > (int64_t(1) << 31) ||
        E > 32768)
        return -1;
    return 4 * B * S * E * eb;   // q, k, v and the attention output
}

miattn_status_t mha_self_attn_fwd(const void* x, const void* w_qkv, const void* b_qkv,
                                  const void* w_out, const void* b_out, void* out,
                                  void* workspace, int64_t workspace_bytes,
                                  int64_t B, int64_t S, int64_t E, int64_t N,
                                  miattn_dtype_t dtype, const uint8_t* atten_mask,
                                  float dropout_p, uint64_t seed, uint32_t offset, void* stream)
{
    const int64_t eb = elem_bytes(dtype);
    if (eb == 0) return MIATTN_ERR_DTYPE;
    if (!x || !w_qkv || !w_out || !out) return MIATTN_ERR_NULL;
    if (B < 1 || S < 1 || N < 1 || N > 256 || E < N || E % N != 0 || B * S > INT32_MAX ||
        E > 32768)
        return MIATTN_ERR_SHAPE;
    const int64_t D = E / N;
    // head dims of the attention operator; rows of whole 16-byte vectors for the bias fill
    if (D > 768 || (E * eb) % 16 != 0) return MIATTN_ERR_SHAPE;
    const int64_t need = mha_workspace_bytes(B, S, E, dtype);
    if (!workspace || need < 0 || workspace_bytes < need) return MIATTN_ERR_WORKSPACE;
    if (!aligned16(workspace) || !aligned16(out) || (b_qkv && !aligned16(b_qkv)) ||
        (b_out && !aligned16(b_out)))
        return MIATTN_ERR_SHAPE;   // the bias rows and the filled outputs move in 16-byte vectors
    if (!(dropout_p >= 0.f && dropout_p < 1.f)) return MIATTN_ERR_DROPOUT;
    if (dropout_p > 0.f && atten_mask) return MIATTN_ERR_UNSUPPORTED;
    // every check of the attention call (dropout rounding, head dims, mask and dropout
    // combination) runs here, before the first launch, so that an error enqueues nothing
    const int32_t route = attn_fwd_route(B, N, N, S, S, D, D, dtype, MIATTN_BSND,
                                         MIATTN_MASK_NONE, atten_mask, dropout_p, 0);
    if (route < 0) return (miattn_status_t)(-route);

    const hipStream_t st = (hipStream_t)stream;
    const int64_t M = B * S, plane = M * E * eb;
    char* ws = (char*)workspace;
    void* q = ws;
    void* k = ws + plane;
    void* v = ws + 2 * plane;
    void* ao = ws + 3 * plane;
    const char* wq = (const char*)w_qkv;
    const char* bq = (const char*)b_qkv;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MIATTN_ERR_LAUNCH;
    {
        std::lock_guard<std::mutex> lock(g_blas_mu);
        if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
            g_blas[dev] = nullptr;
            return MIATTN_ERR_BLAS;
        }
        rocblas_handle h = g_blas[dev];
        if (rocblas_set_stream(h, st) != rocblas_status_success) return MIATTN_ERR_BLAS;
        // the 3E outputs of the QKV layer split into thirds: rows [0, E), [E, 2E), [2E, 3E)
        void* dst[3] = {q, k, v};
        for (int i = 0; i < 3; ++i) {
            const miattn_status_t s = linear(h, st, x, wq + i * E * E * eb, bq ? bq + i * E * eb : nullptr,
                                             dst[i], M, E, E, dtype);
            if (s != MIATTN_OK) return s;
        }
    }
    const miattn_status_t sa = attn_fwd_ext(q, k, v, ao, nullptr, nullptr, B, N, N, S, S, D, D, dtype,
                                            MIATTN_BSND, (float)(1.0 / sqrt((double)D)), MIATTN_MASK_NONE,
                                            0, 0, nullptr, atten_mask, dropout_p, seed, offset, stream);
    if (sa != MIATTN_OK) return sa;
    std::lock_guard<std::mutex> lock(g_blas_mu);
    rocblas_handle h = g_blas[dev];
    if (rocblas_set_stream(h, st) != rocblas_status_success) return MIATTN_ERR_BLAS;
    return linear(h, st, ao, w_out, b_out, out, M, E, E, dtype);
}

}  // extern "C"
