// Attention forward, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// What it computes: out = softmax(scale * Q K^T) V per (sequence, query head) (Paddle
// "sparse_attention" formula; manual_attention of the SDPA-pitfalls blog), over dense or
// packed (TND, cumulative END offsets) batches with GQA and band/causal masks
// (aclnnFlashAttentionVarLenScore, 功能说明 / 约束说明), emitting the per-row softmax max
// and sum that the ring-attention update consumes ("npu_ring_attention_update对外接口").
//
// How (one workgroup = 4 waves = 128 query rows of one head; 32 rows per wave):
//   * Q rows stay in VGPRs for the whole kernel as MFMA B operands.
//   * Per 64-key tile: K (row-major) and V (transposed, V^T[d][key]) are staged in LDS
//     from 128-bit global loads that were issued one tile ahead (register double buffer).
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane owns ONE query column and 16 keys
//     per 32x32 block, so the row max / row sum are in-lane reductions plus one exchange
//     with the lane 32 apart.
//   * Online softmax in the log2 domain (scale * log2(e) folded into one FMA before
//     v_exp_f32); running max and sum stay in registers; the sum is accumulated from
//     fp32 probabilities.
//   * O^T += V^T P^T: the probabilities are rounded to bf16 (RNE) and used straight from
//     the S^T accumulator registers as the B operand; the key order inside an MFMA is
//     permuted consistently on the V^T side, so no shuffle is needed.
//   * Tiles no visible pair touches are never loaded; the mask is evaluated only on
//     tiles that straddle the band edge or the sequence end.
#include "fa_common.h"

namespace miattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kBf16TileM;  // query rows per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int NT = 256;         // threads per workgroup

template <int D>
struct Cfg {
    static constexpr int KS = D + 8;          // K row stride in LDS (bf16): 16 B pad
    static constexpr int VS = BN + 4;         // V^T row stride in LDS (bf16): 8 B pad
    static constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
    static constexpr int KLOADS = BN * CPR / NT;   // K chunks per thread
    static constexpr int VUNITS = (BN / 4) * CPR;  // (4 keys x 8 dims) V units per tile
    static constexpr int KK = D / 16;         // MFMA k-steps over the head dim
    static constexpr int RT = D / 32;         // 32-row output tiles over the head dim
};

__device__ inline float xor32(float x) { return __shfl_xor(x, 32); }

template <int D>
__global__ __launch_bounds__(NT) void fa_fwd_bf16_kernel(FaParams p)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[BN * C::KS];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[D * C::VS];

    const TileCoord tc = decode_tile(p, blockIdx.x, BM);
    if (!tc.live) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lq = lane & 31;     // query column owned by this lane
    const int hf = lane >> 5;     // which half of the wave

    const int i0 = tc.t * BM;
    const int i1 = min(i0 + BM, tc.len_q);
    const int wr0 = i0 + 32 * wave;              // first row of this wave
    const int wr1 = min(wr0 + 32, i1);           // one past its last valid row
    const int qi = wr0 + lq;                     // this lane's query row

    const __bf16* qg = (const __bf16*)p.q + (int64_t)tc.b * p.q_sb + tc.q0 * p.q_ss + (int64_t)tc.h * p.q_sh;
    const __bf16* kg = (const __bf16*)p.k + (int64_t)tc.b * p.k_sb + tc.kv0 * p.k_ss + (int64_t)tc.kvh * p.k_sh;
    const __bf16* vg = (const __bf16*)p.v + (int64_t)tc.b * p.v_sb + tc.kv0 * p.v_ss + (int64_t)tc.kvh * p.v_sh;
    __bf16* og = (__bf16*)p.out + (int64_t)tc.b * p.o_sb + tc.q0 * p.o_ss + (int64_t)tc.h * p.o_sh;
    const int64_t st_base = (int64_t)tc.b * p.st_sb + (int64_t)tc.h * p.st_sh + tc.q0;

    int kv_lo, kv_hi;
    key_range(p, i0, i1, tc.len_kv, kv_lo, kv_hi);

    // ---- Q fragment: B operand of S^T = K Q^T; lane (lq, hf) holds d = 16kk + 8hf + 0..7
    bf16x8 qf[C::KK];
    #pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
        if (qi < tc.len_q)
            qf[kk] = *(const bf16x8*)(qg + (int64_t)qi * p.q_ss + 16 * kk + 8 * hf);
        else
            qf[kk] = bf16x8{};
    }

    f32x16 o[C::RT];
    #pragma unroll
    for (int r = 0; r < C::RT; ++r) o[r] = f32x16{};
    float m_run = -INFINITY;   // running max of scale*log2(e)*s over visible keys
    float l_run = 0.f;         // this lane's half of the running sum

    // ---- register staging of one K/V tile
    u32x4 kreg[C::KLOADS];
    u32x4 vreg[4];
    const int vq = tid % (BN / 4);   // key quad of this thread's V unit
    const int vc = tid / (BN / 4);   // 8-dim chunk of this thread's V unit
    const bool v_active = tid < C::VUNITS;

    auto load_tile = [&](int j0) {
        #pragma unroll
        for (int u = 0; u < C::KLOADS; ++u) {
            const int c = tid + NT * u;
            const int row = j0 + c / C::CPR;
            if (row < tc.len_kv)
                kreg[u] = *(const u32x4*)(kg + (int64_t)row * p.k_ss + 8 * (c % C::CPR));
            else
                kreg[u] = u32x4{};
        }
        if (v_active) {
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = j0 + 4 * vq + r;
                if (row < tc.len_kv)
                    vreg[r] = *(const u32x4*)(vg + (int64_t)row * p.v_ss + 8 * vc);
                else
                    vreg[r] = u32x4{};
            }
        }
    };
    auto store_tile = [&]() {
        #pragma unroll
        for (int u = 0; u < C::KLOADS; ++u) {
            const int c = tid + NT * u;
            *(u32x4*)(Ks + (c / C::CPR) * C::KS + 8 * (c % C::CPR)) = kreg[u];
        }
        if (v_active) {
            // transpose 4 keys x 8 dims into 8 rows of V^T holding 4 keys each
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32x2 lo, hi;
                lo[0] = (vreg[0][e] & 0xffffu) | (vreg[1][e] << 16);
                lo[1] = (vreg[2][e] & 0xffffu) | (vreg[3][e] << 16);
                hi[0] = (vreg[0][e] >> 16) | (vreg[1][e] & 0xffff0000u);
                hi[1] = (vreg[2][e] >> 16) | (vreg[3][e] & 0xffff0000u);
                *(u32x2*)(Vt + (8 * vc + 2 * e) * C::VS + 4 * vq) = lo;
                *(u32x2*)(Vt + (8 * vc + 2 * e + 1) * C::VS + 4 * vq) = hi;
            }
        }
    };

    const int j_start = (kv_lo / BN) * BN;
    if (kv_lo < kv_hi) load_tile(j_start);

    for (int j0 = j_start; j0 < kv_hi; j0 += BN) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (j0 + BN < kv_hi) load_tile(j0 + BN);

        // does any pair of this wave's rows and this tile lie inside the band?
        const bool wave_rows = wr0 < wr1;
        const int64_t dmax = (int64_t)(j0 + BN - 1) - wr0;      // largest j - i
        const int64_t dmin = (int64_t)j0 - (wr1 - 1);           // smallest j - i
        const bool any_vis = wave_rows && j0 < tc.len_kv && dmin <= p.next && -dmax <= p.pre;
        if (!any_vis) continue;
        const bool full = (j0 + BN <= tc.len_kv) && dmax <= p.next && -dmin <= p.pre;

        // ---- S^T = K Q^T : two 32(key) x 32(query) blocks
        f32x16 s[2] = {f32x16{}, f32x16{}};
        #pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
            #pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 a = *(const bf16x8*)(Ks + (32 * kb + lq) * C::KS + 16 * kk + 8 * hf);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
            }
        }
        // key of accumulator element i of block kb: j0 + 32kb + 8(i/4) + 4hf + i%4
        if (!full) {
            #pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                #pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = j0 + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
                    const int64_t dj = (int64_t)j - qi;
                    if (!(j < tc.len_kv && dj <= p.next && -dj <= p.pre)) s[kb][i] = -INFINITY;
                }
            }
        }

        // ---- online softmax (log2 domain)
        float mx = -INFINITY;
        #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            #pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx * p.scale_log2);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float rs = 0.f;
        #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            #pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], p.scale_log2, -m_use));
                s[kb][i] = e;
                rs += e;
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
        #pragma unroll
        for (int r = 0; r < C::RT; ++r)
            #pragma unroll
            for (int i = 0; i < 16; ++i) o[r][i] *= alpha;

        // ---- P (bf16) as B operand: slot t of MFMA j holds key 16j + 8(t/4) + 4hf + t%4
        bf16x8 pf[4];
        #pragma unroll
        for (int j = 0; j < 4; ++j)
            #pragma unroll
            for (int t = 0; t < 8; ++t) pf[j][t] = (__bf16)s[j >> 1][8 * (j & 1) + t];

        // ---- O^T += V^T P^T
        #pragma unroll
        for (int r = 0; r < C::RT; ++r) {
            #pragma unroll
            for (int j = 0; j < 4; ++j) {
                const __bf16* vr = Vt + (32 * r + lq) * C::VS + 16 * j + 4 * hf;
                const bf16x4 lo = *(const bf16x4*)vr;
                const bf16x4 hi = *(const bf16x4*)(vr + 8);
                const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], o[r], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: normalize, round to bf16, store; emit the row statistics
    const float lt = l_run + xor32(l_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qi < wr1) {
        __bf16* orow = og + (int64_t)qi * p.o_ss;
        #pragma unroll
        for (int r = 0; r < C::RT; ++r)
            #pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 w;
                #pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[r][4 * g4 + e] * inv);
                *(bf16x4*)(orow + 32 * r + 8 * g4 + 4 * hf) = w;
            }
        if (hf == 0) {
            if (p.smax) p.smax[st_base + qi] = lt > 0.f ? m_run * 0.69314718055994530942f : -INFINITY;
            if (p.ssum) p.ssum[st_base + qi] = lt;
        }
    }
}

}  // namespace

hipError_t launch_fa_fwd_bf16(const FaParams& p, int D, hipStream_t stream)
{
    dim3 grid(p.n_slots), block(NT);
    if (D == 64)
        hipLaunchKernelGGL(fa_fwd_bf16_kernel<64>, grid, block, 0, stream, p);
    else if (D == 128)
        hipLaunchKernelGGL(fa_fwd_bf16_kernel<128>, grid, block, 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace miattn
