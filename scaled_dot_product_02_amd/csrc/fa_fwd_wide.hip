// Attention forward for any head dims 1 <= Dv <= D <= 768 in every dtype: the path for
// fp32 inputs, and for bf16 / fp16 at the (D, Dv) pairs and feature combinations that the
// tiled kernel is not built for (the operator of "aclnnFlashAttentionVarLenScore" allows
// head dims 1..768 with the V head dim at most the Q/K one; the tiled kernel covers 32..256
// in steps of 32).
//
// Same operation, batches, masks, statistics, fused update and dropout as the other
// kernels.  A workgroup of 8 waves owns BM query rows (32 for fp32, 64 for bf16 / fp16)
// and walks 32-key tiles, splitting the head dims across its waves:
//   * for S^T = K Q^T the waves form RB row blocks of 32 rows x 8 / RB slices of the Q/K
//     head dim (zero past D); each contracts its slice on the matrix cores, with its Q rows
//     held in registers and K read from global memory (L2) straight into MFMA operand
//     layout;
//   * the partial score tiles meet in LDS; each wave then owns BM / 8 rows: it sums the
//     partials, applies scale and masks, and runs the online-softmax step (running max,
//     rescale factor, exponentials, running sum) and writes P and the factor back;
//   * wave w accumulates O^T = V^T P^T for all BM rows over its slice of the V head dim
//     (32 VB columns).  bf16 / fp16 stage that slice in LDS from 16-byte loads issued at
//     the start of the tile (for VB = 2 a tile ahead, into a second buffer) and read it
//     back transposed (ds_read_b64_tr_b16) as the A operand.
// Two barriers per tile.  bf16 / fp16 use v_mfma_f32_32x32x16 with P rounded to the input
// type (as the tiled MFMA kernel); fp32 uses v_mfma_f32_32x32x2f32 with P kept in fp32 and
// V^T fragments read from global memory.
#include "fa_common.h"

namespace miattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int NW = 8;          // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int BN = 32;         // keys per tile
constexpr int RS = BN + 4;     // row stride of the partial-score tiles in LDS (floats)

// Operand fragments: 8 consecutive elements of the contraction index per lane (lane l holds
// k = 8 (l / 32) .. +7 of a 16-wide step), and one 32x32 MFMA step over them.
template <typename T> struct Frag;
template <> struct Frag<__bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    static constexpr int PS = BN + 8;   // P row stride in LDS (elements)
    __device__ static f32x16 mma(const v8& a, const v8& b, const f32x16& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Frag<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    static constexpr int PS = BN + 8;
    __device__ static f32x16 mma(const v8& a, const v8& b, const f32x16& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Frag<float> {
    typedef float v8 __attribute__((ext_vector_type(8)));
    static constexpr int PS = BN + 4;
    // element e of every lane forms one K = 2 step: k = e (lanes 0..31) and 8 + e (32..63),
    // the same pairing on both operands, so the eight steps sum over all 16 k
    __device__ static f32x16 mma(const v8& a, const v8& b, f32x16 c)
    {
        #pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
};

// x[0 .. n) of a row as an 8-element fragment, zero from n on (n may be <= 0).  vec: the
// row is 8-element aligned (D % 8 == 0 and an aligned base), so a full fragment is one
// vector load.
template <typename T>
__device__ inline typename Frag<T>::v8 load_frag(const T* x, int n, bool vec)
{
    typedef typename Frag<T>::v8 v8;
    if (vec && n >= 8) return *(const v8*)x;
    v8 r;
    #pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = e < n ? x[e] : (T)0.f;
    return r;
}

// 32-row blocks per workgroup: one for fp32 (to keep the operands and accumulators of a
// wave within 256 registers), else two.
constexpr int wide_row_blocks(bool f32) { return f32 ? 1 : 2; }

// ds_read_b64_tr_b16 over four rows of 16-bit elements: lane l, slot e receives element
// l % 4 of the 8-byte block read by lane 16 (l / 16) + 4 e + (l % 16) / 4.  The V tile of a
// wave sits in LDS as [key][dv]; lane r reads the four dv 16 ((r / 16) % 2) + 4 (r % 4) ..
// + 3 of key (r % 16) / 4 (+ 4 for the second read), so lane l ends up with
// V[key 8 (l / 32) + e][dv l % 32] for e = 0..7: the A operand of O^T += V^T P^T.
__device__ inline i16x4 ds_read_tr16(const void* lds)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds);
}

// T: input / output type.  KC: the workgroup covers 128 KC >= D columns of the Q/K head
// dim; VB: 32-column blocks of the V head dim per wave (256 VB >= Dv).
// flags: 1 = Q and K rows allow vector loads, 2 = output rows allow 4-element stores,
// 4 = V rows allow 8-element vector loads.
template <typename T, int KC, int VB>
__global__ __launch_bounds__(NT, 1) void fa_fwd_wide_kernel(FaParams p, int D, int flags)
{
    typedef typename Frag<T>::v8 v8;
    constexpr int RB = wide_row_blocks(sizeof(T) == 4);   // 32-row blocks per workgroup
    constexpr int BM = 32 * RB;
    constexpr int RPW = BM / NW;                 // softmax rows per wave
    constexpr int LPR = 64 / RPW;                // lanes per softmax row
    constexpr int KPL = BN / LPR;                // keys per lane in the softmax
    constexpr int PS = Frag<T>::PS;
    // for S^T = K Q^T the waves split into RG row groups (of RBW 32-row blocks) x NDS
    // slices of the Q/K head dim (16 KQ columns each); for O^T = V^T P^T into NW slices of
    // the V head dim.  Head dims up to 256 split the rows too (RG = RB), which halves the
    // partial-score tiles in LDS so that two workgroups fit a CU; larger ones keep every
    // row block in each wave, so that K is read once per workgroup.
    constexpr int RG = KC <= 2 ? RB : 1;
    constexpr int RBW = RB / RG;
    constexpr int NDS = NW / RG;
    constexpr int KQ = KC * RG;
    constexpr int DS = 16 * KQ, DVS = 32 * VB;
    // 16-bit types stage each wave's V slice in LDS ([key][dv], row stride VSS) from 16-byte
    // loads and read it back transposed; fp32 reads V^T fragments from global memory
    constexpr bool TR = sizeof(T) == 2;
    // row pitch of the slice: a ds_read_b64_tr_b16 gathers four key rows and two 16-dim
    // halves for 32 lanes, which fall in disjoint bank ranges when the pitch is 32 or 96
    // modulo 128 elements; slices of 32 or 96 dims meet that unpadded, 64-dim ones (two
    // buffers, no room for a 96 pitch) keep a pitch of 72
    constexpr int VSS = (DVS % 128 == 32 || DVS % 128 == 96) ? DVS : DVS + 8;
    constexpr int VCH = DVS / 8;                 // 16-byte chunks per key of a wave's slice
    constexpr int VU = TR ? BN * VCH / 64 : 1;   // chunks per lane per tile (= 2 VB)
    // V buffers: two (the next tile's slice loaded and stored during this one) for VB = 2;
    // one for VB = 1, which keeps the workgroup within half the LDS (two per CU), and for
    // VB = 3, where two would not fit beside the partial-score tiles
    constexpr int NB = VB == 2 ? 2 : 1;

    __shared__ __attribute__((aligned(16))) float red[NDS][BM][RS];
    __shared__ __attribute__((aligned(16))) T ps[BM][PS];
    __shared__ float alpha_s[BM];
    __shared__ float wfin[2][BM];
    __shared__ __attribute__((aligned(16))) T vs[NB][TR ? NW : 1][TR ? BN : 1][TR ? VSS : 8];

    const TileCoord tc = decode_tile(p, blockIdx.x, BM);
    if (!tc.live) return;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, hi = lane >> 5;
    const int i0 = tc.r0, i1 = tc.r1;
    const int Dv = p.Dv;
    const bool vec_qk = flags & 1, vec_o = flags & 2, vec_v = flags & 4;

    const T* qg = (const T*)p.q + (int64_t)tc.b * p.q_sb + tc.q0 * p.q_ss + (int64_t)tc.h * p.q_sh;
    const T* kg = (const T*)p.k + (int64_t)tc.b * p.k_sb + tc.kv0 * p.k_ss + (int64_t)tc.kvh * p.k_sh;
    const T* vg = (const T*)p.v + (int64_t)tc.b * p.v_sb + tc.kv0 * p.v_ss + (int64_t)tc.kvh * p.v_sh;
    T* og = (T*)p.out + (int64_t)tc.b * p.o_sb + tc.q0 * p.o_ss + (int64_t)tc.h * p.o_sh;
    const int64_t st_base = (int64_t)tc.b * p.st_sb + (int64_t)tc.h * p.st_sh + tc.q0;

    const Band bd = band_of(p, tc);
    int kv_lo, kv_hi;
    key_range(bd, i0, i1, tc.len_kv, kv_lo, kv_hi);

    // this wave's row block and head-dim slices; waves past the end of one skip that
    // contraction
    const int rg = w / NDS, ds = w % NDS;
    const int d0 = ds * DS, dv0 = w * DVS;
    const int nq = (D + DS - 1) / DS;            // slices holding part of the Q/K head dim
    const bool qk_on = d0 < D, pv_on = dv0 < Dv;
    const int dlane = d0 + 8 * hi;               // first of the lane's 8 head-dim columns

    v8 qf[RBW][KQ];
    #pragma unroll
    for (int r = 0; r < RBW; ++r) {
        const int qi = i0 + 32 * (rg * RBW + r) + col;
        #pragma unroll
        for (int c = 0; c < KQ; ++c)
            qf[r][c] = qk_on && qi < i1 ? load_frag(qg + (int64_t)qi * p.q_ss + dlane + 16 * c, D - dlane - 16 * c, vec_qk)
                                        : load_frag(qg, 0, false);
    }
    auto load_k = [&](int j0, v8 (&kf)[KQ]) {
        const int j = j0 + col;
        #pragma unroll
        for (int c = 0; c < KQ; ++c)
            kf[c] = qk_on && j < tc.len_kv ? load_frag(kg + (int64_t)j * p.k_ss + dlane + 16 * c, D - dlane - 16 * c, vec_qk)
                                           : load_frag(kg, 0, false);
    };

    f32x16 o[VB][RB];
    #pragma unroll
    for (int vb = 0; vb < VB; ++vb)
        #pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            #pragma unroll
            for (int r = 0; r < 16; ++r) o[vb][rb][r] = 0.f;

    // softmax ownership: row srow of the tile, keys skey .. skey + KPL - 1
    const int srow = w * RPW + lane / LPR, skey = (lane % LPR) * KPL;
    const int sqi = i0 + srow;
    const bool mrow = p.amask && sqi < p.Sq;
    const uint8_t* arow = mrow ? p.amask + (int64_t)sqi * p.amask_ld : nullptr;
    float m_run = -INFINITY, l_run = 0.f;

    // V slice of the tile at key j0 (16-bit types): chunk u of the lane = key u / VCH, dims
    // 8 (u % VCH) .. + 7 of the wave's slice; only this wave reads its slice, so its LDS
    // writes need no barrier
    u32x4 vst[VU];
    auto load_v = [&](int j0) {
        #pragma unroll
        for (int i = 0; i < VU; ++i) {
            const int u = lane + 64 * i, j = j0 + u / VCH, dv = dv0 + 8 * (u % VCH);
            const T* src = vg + (int64_t)j * p.v_ss + dv;
            vst[i] = u32x4{0u, 0u, 0u, 0u};
            if (pv_on && j < tc.len_kv && dv < Dv) {
                if (vec_v) {
                    vst[i] = *(const u32x4*)src;
                } else {
                    T x[8];
                    #pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = dv + e < Dv ? src[e] : (T)0.f;
                    vst[i] = *(const u32x4*)x;
                }
            }
        }
    };
    auto store_v = [&](int buf) {
        #pragma unroll
        for (int i = 0; i < VU; ++i) {
            const int u = lane + 64 * i;
            *(u32x4*)&vs[buf][w][u / VCH][8 * (u % VCH)] = vst[i];
        }
    };

    const int jfirst = (kv_lo / BN) * BN;
    v8 kf[KQ];
    load_k(jfirst, kf);
    if constexpr (TR && NB == 2) {
        load_v(jfirst);
        store_v(0);
    }
    for (int j0 = jfirst; j0 < kv_hi; j0 += BN) {
        const int buf = NB == 2 ? ((j0 - jfirst) / BN) & 1 : 0;
        if constexpr (TR) {
            if (NB == 1) load_v(j0);
            else if (j0 + BN < kv_hi) load_v(j0 + BN);
        }
        // partial S^T of the wave's row blocks over its head-dim slice -> red[ds][row][key]
        if (qk_on) {
            #pragma unroll
            for (int r = 0; r < RBW; ++r) {
                f32x16 s;
                #pragma unroll
                for (int x = 0; x < 16; ++x) s[x] = 0.f;
                #pragma unroll
                for (int c = 0; c < KQ; ++c) s = Frag<T>::mma(kf[c], qf[r][c], s);
                #pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    *(f32x4*)&red[ds][32 * (rg * RBW + r) + col][8 * jj + 4 * hi] =
                        f32x4{s[4 * jj], s[4 * jj + 1], s[4 * jj + 2], s[4 * jj + 3]};
            }
            if (j0 + BN < kv_hi) load_k(j0 + BN, kf);
        }
        __syncthreads();

        // fp32: V^T fragments of this tile (consumed after the softmax): lane holds
        // V[key 16 kc + 8 hi + e][dv0 + 32 vb + col]
        v8 vf[TR ? 1 : VB][2];
        if constexpr (!TR)
        #pragma unroll
        for (int vb = 0; vb < VB; ++vb)
            #pragma unroll
            for (int kc = 0; kc < 2; ++kc)
                #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = j0 + 16 * kc + 8 * hi + e, dv = dv0 + 32 * vb + col;
                    vf[vb][kc][e] = pv_on && j < tc.len_kv && dv < Dv ? vg[(int64_t)j * p.v_ss + dv] : (T)0.f;
                }

        // online softmax over the wave's rows
        {
            float s[KPL];
            #pragma unroll
            for (int e = 0; e < KPL; ++e) s[e] = 0.f;
            for (int u = 0; u < nq; ++u)
                #pragma unroll
                for (int e = 0; e < KPL; ++e) s[e] += red[u][srow][skey + e];
            float mx = -INFINITY;
            #pragma unroll
            for (int e = 0; e < KPL; ++e) {
                const int j = j0 + skey + e;
                const int64_t dj = (int64_t)j - sqi;
                bool vis = j < tc.len_kv && ((dj <= bd.next && -dj <= bd.pre) || j < bd.pfx);
                if (p.amask) vis = vis && mrow && j < p.Skv && arow[j] == 0;
                s[e] = vis ? s[e] * p.scale_log2 : -INFINITY;
                mx = fmaxf(mx, s[e]);
            }
            #pragma unroll
            for (int m = 1; m < LPR; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            uint32_t word = 0;
            if (p.drop_thr) {
                // the lane's keys lie in one 16-key group: one Philox call per lane
                const int j = j0 + skey;
                uint32_t c[4] = {(uint32_t)(j >> 4), (uint32_t)sqi, (uint32_t)(tc.h + 256 * tc.b), p.drop_offset};
                philox4x32_10(c, p.seed_lo, p.seed_hi);
                const int wi = (j & 15) >> 2;
                word = wi == 0 ? c[0] : wi == 1 ? c[1] : wi == 2 ? c[2] : c[3];
            }
            float sum = 0.f;
            #pragma unroll
            for (int e = 0; e < KPL; ++e) {
                float x = __builtin_amdgcn_exp2f(s[e] - m_use);
                sum += x;
                if (p.drop_thr && ((word >> (8 * ((skey + e) & 3))) & 0xffu) < p.drop_thr) x = 0.f;
                ps[srow][skey + e] = (T)x;
            }
            #pragma unroll
            for (int m = 1; m < LPR; m <<= 1) sum += __shfl_xor(sum, m, 64);
            l_run = l_run * alpha + sum;
            m_run = m_new;
            if (lane % LPR == 0) alpha_s[srow] = alpha;
        }
        // this tile's V slice (one buffer), or the next tile's into the other buffer; the
        // last reader of either, this wave's own PV, came earlier in program order
        if constexpr (TR) {
            if (NB == 1) store_v(0);
            else if (j0 + BN < kv_hi) store_v(buf ^ 1);
        }
        __syncthreads();

        // O^T += V^T P^T over this wave's V head-dim slice
        if (pv_on) {
            #pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float a = alpha_s[32 * rb + col];
                #pragma unroll
                for (int vb = 0; vb < VB; ++vb) o[vb][rb] *= a;
                #pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const v8 pf = *(const v8*)&ps[32 * rb + col][16 * kc + 8 * hi];
                    #pragma unroll
                    for (int vb = 0; vb < VB; ++vb) {
                        v8 a;
                        if constexpr (TR) {
                            const int key = 16 * kc + 8 * hi + ((lane & 15) >> 2);
                            const int dv = 32 * vb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                            const i16x4 lo = ds_read_tr16(&vs[buf][w][key][dv]);
                            const i16x4 up = ds_read_tr16(&vs[buf][w][key + 4][dv]);
                            a = __builtin_bit_cast(v8, i16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
                        } else {
                            a = vf[vb][kc];
                        }
                        o[vb][rb] = Frag<T>::mma(a, pf, o[vb][rb]);
                    }
                }
            }
        }
    }

    // statistics and output weights of the wave's softmax rows: the partial is O / l_run with
    // max mc = m_run ln 2; with a prior (o_p, m_p, l_p) it is merged: m = max(m_p, mc),
    // a = l_p e^(m_p - m), c = l_run e^(mc - m), out = o_p a / (a + c) + (O / l_run) c / (a + c)
    if (lane % LPR == 0) {
        const bool any = l_run > 0.f;
        const float mc = any ? m_run * 0.69314718055994530942f : -INFINITY;
        float m_out = mc, l_out = l_run;
        float wc = any ? (p.drop_thr ? p.drop_scale : 1.f) / l_run : 0.f, wp = 0.f;
        if (p.prev_out && sqi < i1) {
            const float mp = p.prev_max[st_base + sqi], lp = p.prev_sum[st_base + sqi];
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
        wfin[0][srow] = wc;
        wfin[1][srow] = wp;
        if (sqi < i1) {
            if (p.smax) p.smax[st_base + sqi] = m_out;
            if (p.ssum) p.ssum[st_base + sqi] = l_out;
        }
    }
    __syncthreads();

    if (pv_on) {
        #pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = 32 * rb + col, qi = i0 + r;
            if (qi >= i1) continue;
            const float wc = wfin[0][r], wp = wfin[1][r];
            T* orow = og + (int64_t)qi * p.o_ss;
            const T* prow = p.prev_out ? (const T*)p.prev_out + (orow - (T*)p.out) : nullptr;
            #pragma unroll
            for (int vb = 0; vb < VB; ++vb)
                #pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int dv = dv0 + 32 * vb + 8 * jj + 4 * hi;
                    if (dv >= Dv) continue;
                    float y[4];
                    #pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = o[vb][rb][4 * jj + e] * wc;
                    // an empty prior (weight 0) is not read: its buffer may hold anything
                    if (prow && wp != 0.f)
                        #pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (dv + e < Dv) y[e] = __builtin_fmaf((float)prow[dv + e], wp, y[e]);
                    if (vec_o && dv + 4 <= Dv) {
                        typedef T v4 __attribute__((ext_vector_type(4)));
                        *(v4*)(orow + dv) = v4{(T)y[0], (T)y[1], (T)y[2], (T)y[3]};
                    } else {
                        #pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (dv + e < Dv) orow[dv + e] = (T)y[e];
                    }
                }
        }
    }
}

template <typename T, int KC, int VB>
hipError_t launch_kv(const FaParams& p, int D, int flags, hipStream_t stream)
{
    hipLaunchKernelGGL((fa_fwd_wide_kernel<T, KC, VB>), dim3(p.n_slots), dim3(NT), 0, stream, p, D, flags);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_type(const FaParams& p, int D, int flags, hipStream_t stream)
{
    const int kc = (D + 127) / 128, vb = (p.Dv + 255) / 256;
    switch (kc * 4 + vb) {
    case 1 * 4 + 1: return launch_kv<T, 1, 1>(p, D, flags, stream);
    case 2 * 4 + 1: return launch_kv<T, 2, 1>(p, D, flags, stream);
    case 3 * 4 + 1: return launch_kv<T, 3, 1>(p, D, flags, stream);
    case 3 * 4 + 2: return launch_kv<T, 3, 2>(p, D, flags, stream);
    case 4 * 4 + 1: return launch_kv<T, 4, 1>(p, D, flags, stream);
    case 4 * 4 + 2: return launch_kv<T, 4, 2>(p, D, flags, stream);
    case 5 * 4 + 1: return launch_kv<T, 5, 1>(p, D, flags, stream);
    case 5 * 4 + 2: return launch_kv<T, 5, 2>(p, D, flags, stream);
    case 5 * 4 + 3: return launch_kv<T, 5, 3>(p, D, flags, stream);
    case 6 * 4 + 1: return launch_kv<T, 6, 1>(p, D, flags, stream);
    case 6 * 4 + 2: return launch_kv<T, 6, 2>(p, D, flags, stream);
    case 6 * 4 + 3: return launch_kv<T, 6, 3>(p, D, flags, stream);
    default: return hipErrorInvalidValue;
    }
}

bool aligned16(const void* x) { return ((uintptr_t)x & 15u) == 0; }

}  // namespace

int fa_wide_tile_m(int dtype) { return 32 * wide_row_blocks(dtype == 0); }

// dtype: 0 = fp32, 1 = bf16, 2 = fp16 (the C-ABI enum values)
hipError_t launch_fa_fwd_wide(const FaParams& p, int D, int dtype, hipStream_t stream)
{
    if (D < 1 || D > 768 || p.Dv < 1 || p.Dv > D) return hipErrorInvalidValue;
    const int flags = (D % 8 == 0 && aligned16(p.q) && aligned16(p.k) ? 1 : 0) |
                      (p.Dv % 4 == 0 && aligned16(p.out) && (!p.prev_out || aligned16(p.prev_out)) ? 2 : 0) |
                      (p.Dv % 8 == 0 && aligned16(p.v) ? 4 : 0);
    switch (dtype) {
    case 0: return launch_type<float>(p, D, flags, stream);
    case 1: return launch_type<__bf16>(p, D, flags, stream);
    case 2: return launch_type<_Float16>(p, D, flags, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miattn
