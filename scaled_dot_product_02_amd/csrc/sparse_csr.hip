// CSR-sparse attention, fp32 or fp64, any head dim 1..768 (Paddle "sparse_attention":
// formula, parameters, example; the page lists float32 and float64 inputs and puts no
// bound on the head dim).  All arithmetic is in the input type.
//
// Row i of slice (b, n) attends to the key rows listed in
// columns[b][n][offset[b][n][i] .. offset[b][n][i+1]).
//
// A workgroup (8 waves) takes RB = 64 consecutive rows of one slice.  Rows that are
// close to each other mostly list the same nearby keys (a sliding-window band is the
// common pattern, e.g. the page's example and local + random layouts), so the workgroup
// first copies the K and V rows of a key window into LDS with coalesced loads: the WL keys
// that end at the block's last row (the 128 keys before each row of the block, when they
// fit the LDS).  Every entry whose column falls in the window then reads its K / V row
// from LDS; the others are gathered from global memory (L2), so any CSR pattern is served
// and one without locality costs only the window copy.
//
// Each wave takes rows of the block in turn.  fp32 rows of 32, 64 or 128 and fp64 rows of
// 32 or 64 take the grouped layout described at grouped_row below; every other row:
//   * score phase: lane e takes entry e of a 64-entry chunk and forms the whole dot
//     product q . k_col (the query row is broadcast from LDS, the key row comes from the
//     window or from global memory through one generic pointer, so a chunk that mixes
//     both has no divergent branch);
//   * chunk max and sum by wave reductions; the running max / sum are rescaled once per
//     chunk (online softmax in the log2 domain);
//   * value phase: the chunk's (probability, column) pairs are broadcast lane by lane and
//     every lane accumulates its own head-dim slice of sum_c p_c v_c (coalesced row reads
//     from the window or global memory), several value rows per batch with all their
//     loads in flight together.
#include <type_traits>

#include "fa_params.h"

namespace miattn {
namespace {

constexpr int NT = 512;                   // threads per workgroup (8 waves)
constexpr int NW = NT / 64;
constexpr int RB = kSparseRowBlock;       // rows per workgroup
constexpr int kBand = 128;                // keys before a row that the window aims to hold
constexpr int kLdsBytes = 144 * 1024;     // LDS of a workgroup (query rows + K / V window)

// x combined (max or sum) over the lanes that agree with this one in the lane-index bits
// below FROM (FROM = 1: the whole wave).  fp32: rotations inside 16-lane rows (DPP), then
// v_permlane16_swap / v_permlane32_swap across rows, no LDS traffic; fp64: shuffles.
template <int N>
__device__ inline float row_ror(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}
template <int FROM, bool MAX>
__device__ inline float lane_reduce(float x)
{
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if constexpr (FROM <= 1) x = op(x, row_ror<1>(x));
    if constexpr (FROM <= 2) x = op(x, row_ror<2>(x));
    if constexpr (FROM <= 4) x = op(x, row_ror<4>(x));
    if constexpr (FROM <= 8) x = op(x, row_ror<8>(x));
    if constexpr (FROM <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (FROM <= 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
}
template <int FROM, bool MAX>
__device__ inline double lane_reduce(double x)
{
    #pragma unroll
    for (int o = FROM; o < 64; o <<= 1) {
        const double y = __shfl_xor(x, o);
        x = MAX ? fmax(x, y) : x + y;
    }
    return x;
}
// x summed over the DL lanes that share lane / DL (DL = 2, 4, 8 or 16): DPP quad swaps, then
// half-row and row mirrors; fp64: shuffles
template <int DL>
__device__ inline float group_sum(float x)
{
    if constexpr (DL >= 2)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
    if constexpr (DL >= 4)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
    if constexpr (DL >= 8)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
    if constexpr (DL >= 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));
    return x;
}
template <int DL>
__device__ inline double group_sum(double x)
{
    #pragma unroll
    for (int o = 1; o < DL; o <<= 1) x += __shfl_xor(x, o);
    return x;
}
template <typename T>
__device__ inline T wave_max(T x) { return lane_reduce<1, true>(x); }
template <typename T>
__device__ inline T wave_sum(T x) { return lane_reduce<1, false>(x); }
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

// The layout of a workgroup's LDS for head dim D: per wave one query row, then the K
// window (row stride KS, padded by 16 bytes so that lanes reading consecutive window rows
// at the same offset hit different banks) and the V window (row stride VS, padded by 64
// bytes: the grouped layout below reads 64-byte pieces of 16 rows at once, and consecutive
// rows then start 16 banks apart; grouped rows read K that way too).
struct SparseLds {
    int QS, KS, VS, WL;
};

__host__ __device__ inline SparseLds sparse_lds(int D, int esz, int ve, bool grouped)
{
    SparseLds l;
    l.QS = grouped ? 0 : (D + ve - 1) / ve * ve;     // grouped rows keep the query in registers
    l.KS = grouped ? D + 64 / esz : D + (ve > 1 ? ve : 1);
    l.VS = D + 64 / esz;
    const int room = kLdsBytes / esz - NW * l.QS;
    const int wl = room / (l.KS + l.VS);
    l.WL = wl < RB + kBand ? wl : RB + kBand;
    return l;
}

// T = float or double (all arithmetic in T).  DC = the head dim when it is fixed at compile
// time (0: the head dim p.D at run time, at most 64 * PL).  VE = elements per vector access
// of a K / Q row (the head dim and the K pointer are multiples of it).
template <typename T, int DC, int PL, int VE>
__global__ __launch_bounds__(NT) void sparse_csr_kernel(SparseParams p)
{
    typedef T V __attribute__((ext_vector_type(VE)));
    typedef __attribute__((address_space(3))) const V LVc;    // LDS
    typedef __attribute__((address_space(1))) const V GVc;    // global
    // grouped rows (compile-time head dims whose rows are whole 64-byte slices that tile a
    // wave): DL lanes per row, NV elements per lane, EG entry groups, JB entries of a group
    // loaded per batch
    constexpr int RBYTES = DC * (int)sizeof(T);
    // (fp64 rows of 1 KB would need 16 lanes of scores and spill: they take the other path)
    constexpr bool GV = DC > 0 && VE > 1 && RBYTES % 64 == 0 && RBYTES <= 512 &&
                        64 % (RBYTES / 64 ? RBYTES / 64 : 1) == 0;
    constexpr int DL = GV ? RBYTES / 64 : 1;
    constexpr int NV = 64 / (int)sizeof(T);
    constexpr int EG = 64 / DL;
    constexpr int JB = sizeof(T) == 8 ? 1 : DL < 2 ? DL : 2;
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
    const int D = DC ? DC : p.D;
    const SparseLds L = sparse_lds(D, (int)sizeof(T), VE, GV);
    T* qs_all = (T*)lds;
    T* ks = qs_all + NW * L.QS;
    T* vs = ks + L.WL * L.KS;
    const T* q = (const T*)p.q;
    const T* k = (const T*)p.k;
    const T* v = (const T*)p.v;
    T* out = (T*)p.out;
    const T scale_log2 = sizeof(T) == 8 ? (T)p.scale_log2_d : (T)p.scale_log2;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

    // workgroups go to the 8 XCDs round-robin (id mod 8); XCD x takes the x-th eighth of
    // the row blocks in order, so that the blocks resident on one XCD are consecutive
    // blocks of one slice and share its gathered K/V rows in that XCD's L2
    const int nblk_s = (p.S + RB - 1) / RB;
    const int64_t nblk = (int64_t)p.B * p.N * nblk_s;
    const int64_t per = (nblk + 7) / 8;
    const int64_t blk = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (blk >= nblk) return;     // uniform over the workgroup
    const int64_t bn = blk / nblk_s;
    const int r0 = (int)(blk - bn * nblk_s) * RB;
    const int r1 = min(p.S, r0 + RB);
    const int w1 = r1, w0 = max(0, r1 - L.WL);
    const int wl = w1 - w0;
    const T* kb = k + bn * p.S * D;
    const T* vb = v + bn * p.S * D;

    // the key window: K rows [w0, w1) into ks (padded rows), V rows into vs
    {
        const T* ksrc = kb + (int64_t)w0 * D;
        const T* vsrc = vb + (int64_t)w0 * D;
        const int n = wl * D;
        for (int x = threadIdx.x; x < n; x += NT) {
            const int r = x / D, d = x - r * D;
            ks[r * L.KS + d] = ksrc[x];
            vs[r * L.VS + d] = vsrc[x];
        }
    }
    __syncthreads();

    const int32_t* off = p.offset + bn * (p.S + 1);
    typedef __attribute__((address_space(1))) const int32_t GI;
    GI* colg = (GI*)(p.columns + bn * p.nnz);
    T* qs = qs_all + wave * L.QS;

    // Grouped rows (compile-time head dims whose rows tile a wave in 64-byte pieces): lane =
    // (entry group eg, position dg among the DL lanes of a row).  Group eg takes entries eg,
    // eg + EG, ... of a 64-entry chunk; lane dg holds the 16-byte pieces dg, dg + DL,
    // dg + 2 DL, dg + 3 DL of the query row and reads the same pieces of those entries' K
    // and V rows (each load instruction reads 16 DL contiguous bytes of a row).  A score is
    // the group's sum of its lanes' partial dot products; every lane of a group then holds
    // the group's scores and probabilities, so no value moves between lanes until the end
    // of the row, where the groups' partial outputs are added up.  Entries past the chunk
    // take the window's first key with probability 0.
    auto grouped_row = [&](int i, int64_t row) {
        typedef T V16 __attribute__((ext_vector_type(16 / sizeof(T))));
        typedef __attribute__((address_space(3))) const V16 LV16;
        typedef __attribute__((address_space(1))) const V16 GV16;
        constexpr int EPV = 16 / (int)sizeof(T);
        const int eg = lane / DL, dg = lane % DL;
        V16 qv[4];
        GV16* qrow = (GV16*)(q + row * DC) + dg;
        #pragma unroll
        for (int x = 0; x < 4; ++x) qv[x] = qrow[x * DL];
        const int e0 = off[i], e1 = off[i + 1];
        T m_run = -INFINITY, l_run = 0;
        T ga[NV];
        #pragma unroll
        for (int u = 0; u < NV; ++u) ga[u] = 0;
        for (int base = e0; base < e1; base += 64) {
            const int cnt = min(64, e1 - base);
            int cj[DL];
            bool any_in = false, all_in_l = true;
            #pragma unroll
            for (int j = 0; j < DL; ++j) {
                const int e = eg + EG * j;
                cj[j] = e < cnt ? colg[base + e] : w0;
                const bool in = (unsigned)(cj[j] - w0) < (unsigned)wl;
                any_in |= in;
                all_in_l &= in;
            }
            // chunk-wide: every row in the window (LDS reads), none (global reads), or both
            // (generic reads); one straight-line body per case
            const bool all_in = __all(all_in_l), none_in = !__any(any_in);
            auto body = [&](auto mode) {
                constexpr int M = decltype(mode)::value;   // 0 LDS, 1 global, 2 either
                auto load4 = [&](V16 (&dst)[4], const T* win, int stride, const T* glob, int c) {
                    if constexpr (M == 0) {
                        LV16* r = (LV16*)(win + (c - w0) * stride) + dg;
                        #pragma unroll
                        for (int x = 0; x < 4; ++x) dst[x] = r[x * DL];
                    } else if constexpr (M == 1) {
                        GV16* r = (GV16*)(glob + (int64_t)c * DC) + dg;
                        #pragma unroll
                        for (int x = 0; x < 4; ++x) dst[x] = r[x * DL];
                    } else {
                        const int wr = c - w0;
                        const V16* r = (const V16*)((unsigned)wr < (unsigned)wl ? win + wr * stride
                                                                                : glob + (int64_t)c * DC) + dg;
                        #pragma unroll
                        for (int x = 0; x < 4; ++x) dst[x] = r[x * DL];
                    }
                };
                T sj[DL];
                #pragma unroll
                for (int j0 = 0; j0 < DL; j0 += JB) {
                    V16 kk[JB][4];
                    #pragma unroll
                    for (int j = 0; j < JB; ++j) load4(kk[j], ks, L.KS, kb, cj[j0 + j]);
                    #pragma unroll
                    for (int j = 0; j < JB; ++j) {
                        T acc = 0;
                        #pragma unroll
                        for (int x = 0; x < 4; ++x)
                            #pragma unroll
                            for (int y = 0; y < EPV; ++y) acc = fma(qv[x][y], kk[j][x][y], acc);
                        sj[j0 + j] = acc;
                    }
                    // keep the next batch's loads behind this one (registers)
                    __builtin_amdgcn_sched_barrier(0);
                }
                T mloc = -INFINITY;
                #pragma unroll
                for (int j = 0; j < DL; ++j) {
                    sj[j] = eg + EG * j < cnt ? group_sum<DL>(sj[j]) * scale_log2 : (T)-INFINITY;
                    mloc = fmax(mloc, sj[j]);
                }
                const T m_new = fmax(m_run, lane_reduce<DL, true>(mloc));
                const T alpha = exp2_t(m_run - m_new);
                T psum = 0;
                #pragma unroll
                for (int j = 0; j < DL; ++j) {
                    sj[j] = exp2_t(sj[j] - m_new);
                    psum += sj[j];
                }
                l_run = l_run * alpha + lane_reduce<DL, false>(psum);
                #pragma unroll
                for (int u = 0; u < NV; ++u) ga[u] *= alpha;
                #pragma unroll
                for (int j0 = 0; j0 < DL; j0 += JB) {
                    V16 vv[JB][4];
                    #pragma unroll
                    for (int j = 0; j < JB; ++j) load4(vv[j], vs, L.VS, vb, cj[j0 + j]);
                    #pragma unroll
                    for (int j = 0; j < JB; ++j)
                        #pragma unroll
                        for (int x = 0; x < 4; ++x)
                            #pragma unroll
                            for (int y = 0; y < EPV; ++y)
                                ga[x * EPV + y] = fma(sj[j0 + j], vv[j][x][y], ga[x * EPV + y]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                m_run = m_new;
            };
            if (all_in)
                body(std::integral_constant<int, 0>{});
            else if (none_in)
                body(std::integral_constant<int, 1>{});
            else
                body(std::integral_constant<int, 2>{});
        }
        // add up the entry groups' partial sums (lanes with the same dg) and store
        const T inv = l_run > 0 ? (T)1 / l_run : (T)0;
        #pragma unroll
        for (int u = 0; u < NV; ++u) ga[u] = lane_reduce<DL, false>(ga[u]);
        if (lane < DL) {
            V16* dst = (V16*)(out + row * DC) + lane;
            #pragma unroll
            for (int x = 0; x < 4; ++x) {
                V16 r;
                #pragma unroll
                for (int y = 0; y < EPV; ++y) r[y] = ga[x * EPV + y] * inv;
                dst[x * DL] = r;
            }
        }
    };

    for (int i = r0 + wave; i < r1; i += NW) {
        const int64_t row = bn * p.S + i;
        if constexpr (GV) {
            grouped_row(i, row);
            continue;
        }
        // the wave's query row (LDS operations of one wave complete in order, so the
        // previous row's reads are done before these writes land)
        for (int d = lane; d < D; d += 64) qs[d] = q[row * D + d];
        const int e0 = off[i], e1 = off[i + 1];
        T m_run = -INFINITY, l_run = 0;
        T o[PL];
        #pragma unroll
        for (int u = 0; u < PL; ++u) o[u] = 0;

        for (int base = e0; base < e1; base += 64) {
            const int cnt = min(64, e1 - base);
            // lanes past cnt take the window's first key (any valid row: their p is 0)
            const int c = lane < cnt ? colg[base + lane] : w0;
            const int wr = c - w0;
            const bool in = (unsigned)wr < (unsigned)wl;
            // chunk-wide: every entry in the window (LDS reads), none (global reads), or
            // both (generic reads); band + random rows give mostly one-sided chunks
            const bool all_in = __all(in), none_in = !__any(in);
            const V* qr = (const V*)qs;
            auto dot = [&](auto kr) {
                T acc = 0;
                if constexpr (DC != 0 && RBYTES <= 256) {
                    #pragma unroll
                    for (int dv = 0; dv < (DC ? DC : VE) / VE; ++dv) {
                        const V kx = kr[dv], qx = qr[dv];
                        #pragma unroll
                        for (int e = 0; e < VE; ++e) acc = fma(qx[e], kx[e], acc);
                    }
                } else if constexpr (DC != 0) {
                    // longer rows: 128 bytes of the row per unrolled step (registers)
                    #pragma unroll 8
                    for (int dv = 0; dv < (DC ? DC : VE) / VE; ++dv) {
                        const V kx = kr[dv], qx = qr[dv];
                        #pragma unroll
                        for (int e = 0; e < VE; ++e) acc = fma(qx[e], kx[e], acc);
                    }
                } else {
                    #pragma unroll 4
                    for (int dv = 0; dv < D / VE; ++dv) {
                        const V kx = kr[dv], qx = qr[dv];
                        #pragma unroll
                        for (int e = 0; e < VE; ++e) acc = fma(qx[e], kx[e], acc);
                    }
                }
                return acc;
            };
            T sc = -INFINITY;
            if (lane < cnt) {
                T acc;
                if (all_in)
                    acc = dot((LVc*)(ks + wr * L.KS));
                else if (none_in)
                    acc = dot((GVc*)(kb + (int64_t)c * D));
                else
                    acc = dot(in ? (const V*)(ks + wr * L.KS) : (const V*)(kb + (int64_t)c * D));
                sc = acc * scale_log2;
            }
            const T m_new = fmax(m_run, wave_max(sc));
            const T alpha = exp2_t(m_run - m_new);
            const T pv = lane < cnt ? exp2_t(sc - m_new) : (T)0;
            l_run = l_run * alpha + wave_sum(pv);
            #pragma unroll
            for (int u = 0; u < PL; ++u) o[u] *= alpha;
            // value rows in batches of VB entries: all loads of a batch are in flight
            // together (one entry at a time would wait out a full latency per entry)
            constexpr int VREGS = PL * (int)sizeof(T) / 4;     // registers per value row
            constexpr int VB = VREGS >= 32 ? 1 : 32 / VREGS > 16 ? 16 : 32 / VREGS;
            int e = 0;
            for (; e + VB <= cnt; e += VB) {
                T vv[VB][PL];
                #pragma unroll
                for (int x = 0; x < VB; ++x) {
                    const int ce = __builtin_amdgcn_readlane(c, e + x);
                    const int wr = ce - w0;
                    const T* vr = (unsigned)wr < (unsigned)wl ? vs + wr * L.VS : vb + (int64_t)ce * D;
                    #pragma unroll
                    for (int u = 0; u < PL; ++u)
                        vv[x][u] = (DC % 64 == 0 && DC) || lane + 64 * u < D ? vr[lane + 64 * u] : (T)0;
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
                const int wr = ce - w0;
                const T* vr = (unsigned)wr < (unsigned)wl ? vs + wr * L.VS : vb + (int64_t)ce * D;
                #pragma unroll
                for (int u = 0; u < PL; ++u)
                    if ((DC % 64 == 0 && DC) || lane + 64 * u < D) o[u] = fma(pe, vr[lane + 64 * u], o[u]);
            }
            m_run = m_new;
        }
        const T inv = l_run > 0 ? (T)1 / l_run : (T)0;
        #pragma unroll
        for (int u = 0; u < PL; ++u)
            if ((DC % 64 == 0 && DC) || lane + 64 * u < D) out[row * D + lane + 64 * u] = o[u] * inv;
    }
}

template <typename T, int DC, int PL, int VE>
hipError_t launch_one(const SparseParams& p, hipStream_t stream)
{
    const int64_t nblk = (int64_t)p.B * p.N * ((p.S + RB - 1) / RB);
    dim3 grid((unsigned)((nblk + 7) / 8 * 8)), block(NT);
    hipLaunchKernelGGL((sparse_csr_kernel<T, DC, PL, VE>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// the head dim at run time: PL = values per lane of the output row (D <= 64 PL)
template <typename T, int VE>
hipError_t launch_general(const SparseParams& p, hipStream_t stream)
{
    const int D = p.D;
    if (D <= 64) return launch_one<T, 0, 1, VE>(p, stream);
    if (D <= 128) return launch_one<T, 0, 2, VE>(p, stream);
    if (D <= 256) return launch_one<T, 0, 4, VE>(p, stream);
    if (D <= 512) return launch_one<T, 0, 8, VE>(p, stream);
    return launch_one<T, 0, 12, VE>(p, stream);
}

template <typename T>
hipError_t launch_t(const SparseParams& p, bool aligned16, hipStream_t stream)
{
    constexpr int VE = 16 / sizeof(T);
    const bool vec = aligned16 && p.D % VE == 0;
    if (vec) {
        switch (p.D) {
        case 32: return launch_one<T, 32, 1, VE>(p, stream);
        case 64: return launch_one<T, 64, 1, VE>(p, stream);
        case 96: return launch_one<T, 96, 2, VE>(p, stream);
        case 128: return launch_one<T, 128, 2, VE>(p, stream);
        default: return launch_general<T, VE>(p, stream);
        }
    }
    return launch_general<T, 1>(p, stream);
}

}  // namespace

int sparse_window_keys(int D, bool f64, bool aligned16)
{
    const int ve = f64 ? 2 : 4;
    // compile-time head dims whose rows tile a wave in 64-byte pieces take the grouped layout
    const int rb = D * (f64 ? 8 : 4);
    const bool grouped = aligned16 && (D == 32 || D == 64 || D == 128) && rb % 64 == 0 && rb <= 512 &&
                         64 % (rb / 64) == 0;
    return sparse_lds(D, f64 ? 8 : 4, aligned16 && D % ve == 0 ? ve : 1, grouped).WL;
}

bool sparse_head_dim_fits(int D, bool f64)
{
    // the window must hold at least one key row beside the query rows
    return D >= 1 && D <= 768 && sparse_lds(D, f64 ? 8 : 4, f64 ? 2 : 4, false).WL >= 1 &&
           sparse_lds(D, f64 ? 8 : 4, 1, false).WL >= 1;
}

hipError_t launch_sparse_csr(const SparseParams& p, bool f64, bool aligned16, hipStream_t stream)
{
    return f64 ? launch_t<double>(p, aligned16, stream) : launch_t<float>(p, aligned16, stream);
}

}  // namespace miattn
