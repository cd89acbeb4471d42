// Attention forward, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// What it computes: out = softmax(scale * Q K^T) V per (sequence, query head) (Paddle
// "sparse_attention" formula; manual_attention of the SDPA-pitfalls blog), over dense or
// packed (TND, cumulative END offsets) batches with GQA and band/causal masks
// (aclnnFlashAttentionVarLenScore, 功能说明 / 约束说明), emitting the per-row softmax max
// and sum that the ring-attention update consumes ("npu_ring_attention_update对外接口").
//
// Design (one workgroup = 8 waves = 256 query rows of one head; two waves per SIMD):
//   * Each wave owns one 32-row query block, held in VGPRs for the whole kernel as MFMA
//     B operands.  A wave needs under 256 registers with every accumulator in ordinary
//     VGPRs, so two waves share each SIMD.  Waves w and w + 4 share a SIMD, which evens
//     out the causal triangle across the four SIMDs, and they run one phase apart (below)
//     so that one wave's softmax (vector ALU) overlaps the other's matrix-core work.
//   * Keys advance in tiles of 64.  K (row-major) and V (transposed, V^T[d][key]; row-
//     major for head dims above 128, below) tiles are staged from 128-bit buffer loads
//     through registers into a 4-deep ring of LDS buffers; a tile's loads are issued two
//     steps before its LDS stores (two register sets), which covers the memory latency
//     under load.  Every thread stages the same share of each tile, with no branch.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane owns ONE query column and 16 of the
//     32 keys, so the row max / row sum are in-lane reductions plus one exchange with the
//     lane 32 apart.
//   * O^T += V^T P^T: the probabilities are rounded to bf16 (RNE) and used straight from
//     the S^T accumulator registers as the B operand.  The order of keys inside each MFMA
//     follows the S^T register layout; the V^T rows in LDS store their keys in that same
//     order (bits 2 and 3 of the key index swapped), so each A operand is one 128-bit read.
//   * Software pipeline: step t issues QK(t) and PV(t-1) on the matrix cores (phase M) and
//     then runs the softmax of tile t on the vector ALUs (phase S), each phase closed by a
//     barrier.  Waves 4-7 run one phase behind waves 0-3, so each SIMD always has one wave
//     in each phase; the M phase runs at raised wave priority so that the matrix issue is
//     not starved by the partner's vector work.
//   * Online softmax in the log2 domain (scale * log2(e) folded into one FMA before
//     v_exp_f32).  The reference max m_ref moves only when a tile's max exceeds it by more
//     than 2^8 (probabilities stay <= 256, safe in bf16 and fp32), so the O accumulator is
//     almost never rescaled; the true running max is tracked separately and the emitted
//     softmax_sum is re-referenced to it at the end.  The row sum is accumulated from the
//     fp32 probabilities.
//   * Tiles no visible pair touches are never loaded or computed; masks are evaluated
//     only on tiles that straddle the band edge or the sequence end.
#include "fa_common.h"
#include "fa_mfma.h"

namespace miattn {
namespace {

constexpr int BM = kBf16TileM;  // 256 query rows per workgroup
#ifndef FA_BN
#define FA_BN 64
#endif
#ifndef FA_PREFETCH
#define FA_PREFETCH 3
#endif
constexpr int BN = FA_BN;       // keys per tile
constexpr int NKB = BN / 32;    // 32-key blocks per tile
constexpr int PF = FA_PREFETCH; // tiles in flight ahead of the one in softmax (2 or 3)
#ifndef FA_LDSD
#define FA_LDSD 6
#endif
#ifndef FA_SCHED
#define FA_SCHED 1
#endif
constexpr int LDSD = FA_LDSD;   // LDS fragment reads kept in flight ahead of their MFMAs
constexpr int NT = 512;         // threads per workgroup (8 waves)
constexpr int NBUF = 4;         // LDS ring depth (tiles)
constexpr float kLazyThresh = 8.0f;  // log2 units
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3: 32-bit data format, raw

// Row pitch (elements) of V staged as [key][dim] for transposed reads: the four key rows and
// two 16-dim halves that a ds_read_b64_tr_b16 gathers for 32 lanes fall in disjoint bank
// ranges when the pitch is 32 or 96 modulo 128 elements.
constexpr int vrow_pitch(int dv)
{
    int p = dv + 8;
    while (p % 128 != 32 && p % 128 != 96) p += 8;
    return p;
}

// D: head dim of Q and K; DV: head dim of V and the output (DV <= D).
// Head dims up to 128 run 8 waves (two per SIMD) on 64-key tiles.  Larger ones (160..256)
// run 4 waves, one per SIMD, so that a wave may hold up to 512 registers (the O
// accumulators of D 256 alone take 128), on 32-key tiles so that the 4-deep K and V
// rings fit in LDS (138 KB at D 256); there V is staged row-major like K and read back
// transposed as the matrix operand.

template <int D, int DV, bool FOUR = (D > 128)>
struct Cfg {
    static constexpr bool BIG = FOUR;
    static constexpr int NW = BIG ? 4 : 8;            // waves per workgroup
    static constexpr int NT = 64 * NW;                // threads per workgroup
    static constexpr int BM = 32 * NW;                // query rows per workgroup
    static constexpr int BN = BIG ? 32 : ::miattn::BN; // keys per tile
    static constexpr int NKB = BN / 32;               // 32-key blocks per tile
    static constexpr int KS = D + 8;                  // K row stride in LDS (bf16)
    static constexpr int VS = BN + 8;                 // V^T row stride in LDS (bf16)
    static constexpr int CPR = D / 8;                 // 16-byte chunks per K row
    static constexpr int KCH = BN * CPR;              // K chunks per tile
    static constexpr int KPT = (KCH + NT - 1) / NT;   // K chunks per thread (some repeat)
    static constexpr int VUNITS = (BN / 2) * (DV / 8); // V units (2 keys x 8 dims) per tile
    static constexpr int VPT = (VUNITS + NT - 1) / NT; // V units per thread (some repeat)
    // one wave per SIMD: V staged as [key][dim] (16-byte chunks like K) and read back
    // transposed as the P V operand, instead of transposed into V^T by the staging threads
    static constexpr bool VROW = BIG;
    static constexpr int VP = vrow_pitch(DV);         // V row pitch in LDS (VROW)
    static constexpr int CPRV = DV / 8;               // 16-byte chunks per V row
    static constexpr int VCH = BN * CPRV;             // V chunks per tile (VROW)
    static constexpr int VRT = (VCH + NT - 1) / NT;   // V chunks per thread (VROW; some repeat)
    static constexpr int SREG = KPT + (VROW ? VRT : 2 * VPT);  // staging registers (16 B each)
    static constexpr int KK = D / 16;                 // MFMA k-steps over the Q/K head dim
    static constexpr int RT = DV / 32;                // 32-row output tiles over the V head dim
    static constexpr int KBUF = BN * KS;
    static constexpr int VBUF = VROW ? BN * VP : DV * VS;
};

// UPDATE = true: the epilogue merges the partial result into p.prev_* (ring update).
// MASKED = true: the explicit mask p.amask (rows 4-byte aligned) removes keys as well;
// each tile's mask bytes are loaded in the previous tile's matrix-core phase and set the
// initial value of its score accumulators.
// DROP = true: dropout on the probabilities (p.drop_*), the kept ones scaled in the epilogue.
template <int D, int DV, bool MASKED, bool DROP>
using KCfg = Cfg<D, DV, fa_four_waves(D, MASKED || DROP)>;

template <int D, int DV, typename T, bool UPDATE, bool MASKED, bool DROP = false>
__global__ __launch_bounds__((KCfg<D, DV, MASKED, DROP>::NT), (KCfg<D, DV, MASKED, DROP>::BIG && D <= 128 ? 2 : 1))
void fa_fwd_bf16_kernel(FaParams p)
{
    using C = KCfg<D, DV, MASKED, DROP>;
    constexpr int NT = C::NT, BM = C::BM, BN = C::BN, NKB = C::NKB;
    static_assert(!(C::BIG && (MASKED || DROP)), "the mask tensor and dropout assume 64-key tiles");
    constexpr int PF = ::miattn::PF;
    constexpr int LDSD = ::miattn::LDSD;
    using X8 = typename Elem<T>::v8;   // one MFMA operand: 8 elements
    using X4 = typename Elem<T>::v4;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[NBUF * C::KBUF];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[NBUF * C::VBUF];

    const TileCoord tc = decode_tile(p, blockIdx.x, BM);
    if (!tc.live) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31;   // query column owned by this lane
    const int hf = lane >> 5;   // half of the wave

    const int len_q = tc.len_q, len_kv = tc.len_kv;
    const int i0 = tc.r0;
    const int i1 = tc.r1;

    const __bf16* qg = (const __bf16*)p.q + (int64_t)tc.b * p.q_sb + tc.q0 * p.q_ss + (int64_t)tc.h * p.q_sh;
    const __bf16* kg = (const __bf16*)p.k + (int64_t)tc.b * p.k_sb + tc.kv0 * p.k_ss + (int64_t)tc.kvh * p.k_sh;
    const __bf16* vg = (const __bf16*)p.v + (int64_t)tc.b * p.v_sb + tc.kv0 * p.v_ss + (int64_t)tc.kvh * p.v_sh;
    T* og = (T*)p.out + (int64_t)tc.b * p.o_sb + tc.q0 * p.o_ss + (int64_t)tc.h * p.o_sh;
    const int64_t st_base = (int64_t)tc.b * p.st_sb + (int64_t)tc.h * p.st_sh + tc.q0;

    // ---- key tiles of the workgroup
    int kv_lo, kv_hi;
    const Band bd = band_of(p, tc);
    key_range(bd, i0, i1, len_kv, kv_lo, kv_hi);
    const int T0 = kv_lo / BN;
    const int T1 = kv_lo < kv_hi ? (kv_hi + BN - 1) / BN : T0;
    if constexpr (UPDATE) {
        if (T0 >= T1 && p.out == p.prev_out && p.smax == p.prev_max && p.ssum == p.prev_sum) {
            // An in-place update by a key chunk that no row of this tile sees: every row
            // keeps its value (the update leaves a non-empty prior unchanged), except that a
            // row with an empty prior takes the empty result (out 0, sum 0).
            for (int r = tid; r < i1 - i0; r += NT) {
                const int64_t si = st_base + i0 + r;
                if (p.prev_max[si] == -INFINITY) {
                    p.ssum[si] = 0.f;
                    T* orow = og + (int64_t)(i0 + r) * p.o_ss;
                    for (int d = 0; d < DV; d += 4) *(X4*)(orow + d) = X4{};
                }
            }
            return;
        }
    }

    // ---- this wave's rows [rb, re): active tiles, unmasked tiles, per-lane key bounds
    const int rb = i0 + 32 * wave;
    const int re = min(rb + 32, i1);
    int w_lo = 0, w_hi = 0;   // tiles [w_lo, w_hi) hold a visible key of this wave
    int full_lo = 0, full_hi = 0;   // tiles [full_lo, full_hi) need no mask
    int jlo = 0, jhi = -1;          // keys [jlo, jhi] are visible from this lane's row
    if (rb < re) {
        int lo, hi;
        key_range(bd, rb, re, len_kv, lo, hi);
        if (lo < hi) {
            w_lo = lo / BN;
            w_hi = (hi + BN - 1) / BN;
        }
        const int64_t flo = bd.pfx > 0 ? 0 : (int64_t)(re - 1) - bd.pre;   // first key seen by every row
        const int64_t fhi = max((int64_t)rb + bd.next, bd.pfx - 1);        // last key seen by every row
        const int64_t fl = flo <= 0 ? 0 : (flo + BN - 1) / BN;
        const int64_t fh = fhi < 0 ? 0 : (min(fhi, (int64_t)len_kv - 1) + 1) / BN;
        full_lo = (int)min(fl, (int64_t)1 << 30);
        full_hi = (int)fh;
        const int qi = rb + lq;
        const int64_t a = bd.pfx > 0 ? 0 : (int64_t)qi - bd.pre;
        const int64_t z = max((int64_t)qi + bd.next, bd.pfx - 1);
        jlo = (int)max((int64_t)0, min(a, (int64_t)len_kv));
        jhi = (int)max((int64_t)-1, min(z, (int64_t)len_kv - 1));
    }
    auto wave_active = [&](int t) { return t >= w_lo && t < w_hi; };

    // ---- Q fragment: B operand of S^T = K Q^T; lane (lq, hf) holds d = 16kk + 8hf + 0..7
    X8 qf[C::KK];
    {
        const int qi = min(rb + lq, len_q - 1);
        const __bf16* qrow = qg + (int64_t)qi * p.q_ss + 8 * hf;
        #pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) qf[kk] = *(const X8*)(qrow + 16 * kk);
    }

    f32x16 o[C::RT];
    #pragma unroll
    for (int r = 0; r < C::RT; ++r) o[r] = f32x16{};
    float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;
    const float cl2 = p.scale_log2;

    // ---- global -> register -> LDS staging of one tile.  Every thread takes KPT K chunks
    //      (16 B of one key row) and one V unit (2 keys x 8 dims), so the staging work is
    //      the same in every wave and has no branch (a branch would also make the compiler
    //      wait for the loads where the paths join).  The loads are buffer loads whose
    //      descriptor spans only the tile's rows inside the sequence: rows past its end
    //      (or a whole tile past the key range) read as zero, and each thread's byte offset
    //      inside a tile is a constant.  With fewer V units than threads, threads repeat a
    //      unit and store identical values.
    u32x4 stA[C::SREG], stB[C::SREG];
    int kp[C::VPT], vc[C::VPT];   // V unit u of this thread: keys 2 kp, 2 kp + 1, dims 8 vc ..
    #pragma unroll
    for (int u = 0; u < C::VPT; ++u) {
        const int vu = (tid + NT * u) % C::VUNITS;
        kp[u] = vu % (BN / 2);
        vc[u] = vu / (BN / 2);
    }
    const int64_t krb = 2 * p.k_ss, vrb = 2 * p.v_ss;   // row strides in bytes
    uint32_t koff[C::KPT], voff[C::VROW ? C::VRT : 2 * C::VPT];
    #pragma unroll
    for (int u = 0; u < C::KPT; ++u) {
        const int c = C::KCH % NT ? (tid + NT * u) % C::KCH : tid + NT * u;
        koff[u] = (uint32_t)((c / C::CPR) * krb + 16 * (c % C::CPR));
    }
    if constexpr (C::VROW) {
        #pragma unroll
        for (int u = 0; u < C::VRT; ++u) {
            const int c = C::VCH % NT ? (tid + NT * u) % C::VCH : tid + NT * u;
            voff[u] = (uint32_t)((c / C::CPRV) * vrb + 16 * (c % C::CPRV));
        }
    } else {
        #pragma unroll
        for (int u = 0; u < C::VPT; ++u)
            #pragma unroll
            for (int r = 0; r < 2; ++r) voff[2 * u + r] = (uint32_t)((2 * kp[u] + r) * vrb + 16 * vc[u]);
    }

    // descriptor inputs are workgroup-uniform; readfirstlane keeps them in scalar registers
    // (a descriptor the compiler thinks divergent would be looped over lane by lane)
    auto rsrc = [](const void* base, int64_t bytes) {
        const uint64_t a = (uint64_t)base;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
        const int n = __builtin_amdgcn_readfirstlane((int)bytes);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, kBufferFlags);
    };
    // explicit mask: this lane's row, loaded a step before its Q K^T products as two
    // 16-byte pieces: lane (lq, hf) reads the 32 bytes of 32-key block hf of the tile (word
    // j: keys 4j .. 4j + 3 of the block).  The scores of the lane need, in word 4b + g, the
    // bytes of keys 32b + 8g + 4hf .. + 3 (byte e: key + e), so lane hf keeps words 2g + hf
    // of both blocks: one lane-pair exchange per g trades block 0's odd words (held by the
    // hf = 0 lanes) for block 1's even words (held by the hf = 1 lanes).  Two wide loads
    // touch a quarter of the cache lines that eight 4-byte loads do.
    u32x4 mraw[2] = {u32x4{}, u32x4{}};
    __amdgpu_buffer_rsrc_t rmask;
    uint32_t moff = 0;
    if constexpr (MASKED) {
        rmask = rsrc(p.amask, (int64_t)p.Sq * p.amask_ld);
        moff = (uint32_t)((int64_t)min(rb + lq, p.Sq - 1) * p.amask_ld) + 32 * hf;
    }
    auto load_mask = [&](int t) {
        #pragma unroll
        for (int k = 0; k < 2; ++k)
            mraw[k] = __builtin_amdgcn_raw_buffer_load_b128(rmask, moff + t * BN + 16 * k, 0, 0);
    };
    // the words in score order (byte e of word 4b + g: key 32b + 8g + 4hf + e)
    auto mask_words = [&](unsigned (&mw)[8]) {
        #pragma unroll
        for (int g = 0; g < 4; ++g) {
            const unsigned even = mraw[g >> 1][2 * (g & 1)], odd = mraw[g >> 1][2 * (g & 1) + 1];
            // lanes 32-63 of the first operand trade with lanes 0-31 of the second
            const auto x = __builtin_amdgcn_permlane32_swap(even, odd, false, false);
            mw[g] = x[0];
            mw[4 + g] = x[1];
        }
    };
    auto load_tile = [&](int t, u32x4 (&stage)[C::SREG]) {
        const int j0 = t * BN;
        const int rows = max(0, min(BN, len_kv - j0));
        const __amdgpu_buffer_rsrc_t rk = rsrc((const char*)kg + (int64_t)j0 * krb, rows * krb);
        const __amdgpu_buffer_rsrc_t rv = rsrc((const char*)vg + (int64_t)j0 * vrb, rows * vrb);
        #pragma unroll
        for (int u = 0; u < C::KPT; ++u) stage[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[u], 0, 0);
        #pragma unroll
        for (int r = 0; r < (C::VROW ? C::VRT : 2 * C::VPT); ++r)
            stage[C::KPT + r] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[r], 0, 0);
    };
    // staged chunk u (K chunks, then V chunks) of tile t into LDS (the V-as-rows layout)
    auto store_chunk = [&](int t, const u32x4 (&stage)[C::SREG], int u) __attribute__((always_inline)) {
        const int bf = t & (NBUF - 1);
        if (u < C::KPT) {
            const int c = C::KCH % NT ? (tid + NT * u) % C::KCH : tid + NT * u;
            *(u32x4*)(Ks + bf * C::KBUF + (c / C::CPR) * C::KS + 8 * (c % C::CPR)) = stage[u];
        } else {
            const int c = C::VCH % NT ? (tid + NT * (u - C::KPT)) % C::VCH : tid + NT * (u - C::KPT);
            *(u32x4*)(Vt + bf * C::VBUF + (c / C::CPRV) * C::VP + 8 * (c % C::CPRV)) = stage[u];
        }
    };
    auto store_tile = [&](int t, const u32x4 (&stage)[C::SREG]) {
        const int bf = t & (NBUF - 1);
        __bf16* kb = Ks + bf * C::KBUF;
        if constexpr (C::VROW) {
            #pragma unroll
            for (int u = 0; u < C::SREG; ++u) store_chunk(t, stage, u);
            return;
        }
        #pragma unroll
        for (int u = 0; u < C::KPT; ++u) {
            const int c = C::KCH % NT ? (tid + NT * u) % C::KCH : tid + NT * u;
            *(u32x4*)(kb + (c / C::CPR) * C::KS + 8 * (c % C::CPR)) = stage[u];
        }
        // dims 8 vc + e of keys 2 kp, 2 kp + 1 -> one 32-bit word of V^T row 8 vc + e
        #pragma unroll
        for (int u = 0; u < C::VPT; ++u) {
            __bf16* vb = Vt + bf * C::VBUF + 8 * vc[u] * C::VS + vt_pos(2 * kp[u]);
            const u32x4 x0 = stage[C::KPT + 2 * u], x1 = stage[C::KPT + 2 * u + 1];
            #pragma unroll
            for (int e = 0; e < 8; ++e) {
                // low halves (even e) or high halves (odd e) of the two keys' words:
                // v_perm_b32 takes bytes 0-3 from its second operand and 4-7 from its first
                const unsigned w = __builtin_amdgcn_perm(x1[e >> 1], x0[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
                *(unsigned*)(vb + e * C::VS) = w;
            }
        }
    };

    // ---- S^T = K Q^T for tile t (NKB blocks of 32 keys x 32 queries)
    auto qk = [&](int t, f32x16 (&s)[NKB]) {
        const __bf16* kb = Ks + (t & (NBUF - 1)) * C::KBUF + lq * C::KS + 8 * hf;
        constexpr int NF = C::KK * NKB;   // fragments (= MFMAs)
        // fragment f: block b and k-step kk.  The plain instance alternates the blocks; the
        // mask tensor instance takes block 0's MFMAs first, so that block 1's initial values
        // are formed while they run
        auto fb = [](int f) { return MASKED ? f / C::KK : f % NKB; };
        auto fk = [](int f) { return MASKED ? f % C::KK : f / NKB; };
        X8 a[NF];
        #pragma unroll
        for (int f = 0; f < LDSD && f < NF; ++f)
            a[f] = *(const X8*)(kb + 32 * fb(f) * C::KS + 16 * fk(f));
        if constexpr (MASKED) {
            // the mask tensor enters as the scores' initial value: -inf for a removed key
            // (-inf plus the finite dot product stays -inf), 0 otherwise; the byte tests run
            // beside this wave's own MFMAs instead of in the softmax phase.  Element i of
            // block b is byte i % 4 of word 4b + i / 4
            unsigned mw[8];
            mask_words(mw);
            #pragma unroll
            for (int b = 0; b < NKB; ++b)
                #pragma unroll
                for (int i = 0; i < 16; ++i)
                    s[b][i] = (mw[4 * b + (i >> 2)] >> (8 * (i & 3)) & 0xffu) != 0u ? -INFINITY : 0.f;
        } else {
            #pragma unroll
            for (int b = 0; b < NKB; ++b) s[b] = f32x16{};
        }
        #pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + LDSD < NF)
                a[f + LDSD] = *(const X8*)(kb + 32 * fb(f + LDSD) * C::KS + 16 * fk(f + LDSD));
            s[fb(f)] = Elem<T>::mfma(a[f], qf[fk(f)], s[fb(f)]);
        }
#if FA_SCHED
        // keep LDSD reads in flight ahead of the MFMAs that consume them
        constexpr int AH = LDSD < NF ? LDSD : NF;
        __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
        #pragma unroll
        for (int f = 0; f < NF - AH; ++f) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
#endif
    };

    // ---- V^T fragment f of tile t from V staged as [key][dim] (VROW): two
    //      ds_read_b64_tr_b16.  Lane l, slot e of a transposed read receives element l % 4 of
    //      the 8-byte block read by lane 16 (l / 16) + 4 e + (l % 16) / 4, so lane l reading
    //      dims 32 r + 16 ((l / 16) % 2) + 4 (l % 4) .. + 3 of key 16 j + 4 hf + (l % 16) / 4
    //      (then 8 keys further) leaves lane (lq, hf) with V[16 j + 8 (e / 4) + 4 hf + e % 4]
    //      [32 r + lq], e = 0..7: the key order of the P operand (r = f / (2 NKB),
    //      j = f % (2 NKB))
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const int v_lane = (4 * hf + ((lane & 15) >> 2)) * C::VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto vfrag_rows = [&](int t, int f) __attribute__((always_inline)) -> X8 {
        const __bf16* v = Vt + (t & (NBUF - 1)) * C::VBUF + v_lane + 16 * (f % (2 * NKB)) * C::VP + 32 * (f / (2 * NKB));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)v);
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(v + 8 * C::VP));
        return __builtin_bit_cast(X8, i16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    };
    // O^T += V^T P^T for tile t (VROW) with work(f) issued after MFMA f
    auto pv_rows = [&](int t, const X8 (&pp)[2 * NKB], auto&& work) __attribute__((always_inline)) {
        constexpr int NF = C::RT * 2 * NKB;
        X8 a[NF];
        #pragma unroll
        for (int f = 0; f < LDSD && f < NF; ++f) a[f] = vfrag_rows(t, f);
        #pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + LDSD < NF) a[f + LDSD] = vfrag_rows(t, f + LDSD);
            o[f / (2 * NKB)] = Elem<T>::mfma(a[f], pp[f % (2 * NKB)], o[f / (2 * NKB)]);
            work(f);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- O^T += V^T P^T for tile t
    auto pv = [&](int t, const X8 (&pp)[2 * NKB]) {
        if constexpr (C::VROW) {
            pv_rows(t, pp, [](int) {});
            return;
        }
        const __bf16* vb = Vt + (t & (NBUF - 1)) * C::VBUF + lq * C::VS + 8 * hf;
        constexpr int NF = C::RT * 2 * NKB;   // fragment f: r = f / (2 NKB), j = f % (2 NKB)
        X8 a[NF];
        #pragma unroll
        for (int f = 0; f < LDSD && f < NF; ++f)
            a[f] = *(const X8*)(vb + 32 * (f / (2 * NKB)) * C::VS + 16 * (f % (2 * NKB)));
        #pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + LDSD < NF)
                a[f + LDSD] = *(const X8*)(vb + 32 * ((f + LDSD) / (2 * NKB)) * C::VS + 16 * ((f + LDSD) % (2 * NKB)));
            o[f / (2 * NKB)] = Elem<T>::mfma(a[f], pp[f % (2 * NKB)], o[f / (2 * NKB)]);
        }
#if FA_SCHED
        constexpr int AH = LDSD < NF ? LDSD : NF;
        __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
        #pragma unroll
        for (int f = 0; f < NF - AH; ++f) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
#endif
    };

    // ---- online softmax of tile t; leaves bf16 probabilities in pp
    auto softmax = [&](int t, f32x16 (&s)[NKB], X8 (&pp)[2 * NKB]) {
        const int jb = t * BN + 4 * hf;   // key of element i of block b: jb + 32b + 8(i/4) + i%4
        if (t < full_lo || t >= full_hi) {
            #pragma unroll
            for (int b = 0; b < NKB; ++b)
                #pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = jb + 32 * b + 8 * (i >> 2) + (i & 3);
                    if (j < jlo || j > jhi) s[b][i] = -INFINITY;
                }
        }
        // tree reductions keep the dependent chains short
        // four independent chains, each folding two values per step (v_max3)
        float mq[4];
        #pragma unroll
        for (int c = 0; c < 4; ++c) {
            float m = s[0][4 * c];
            #pragma unroll
            for (int k = 1; k < 4 * NKB; k += 2) {
                const int b0 = k / 4, i0 = k % 4, b1 = (k + 1) / 4, i1 = (k + 1) % 4;
                m = (k + 1 < 4 * NKB) ? fmaxf(fmaxf(m, s[b0][4 * c + i0]), s[b1][4 * c + i1])
                                      : fmaxf(m, s[b0][4 * c + i0]);
            }
            mq[c] = m;
        }
        float mx = pair_max(fmaxf(fmaxf(fmaxf(mq[0], mq[1]), mq[2]), mq[3]));
        const float mt = mx * cl2;
        m_true = fmaxf(m_true, mt);
        const bool need = mt > m_ref + kLazyThresh;
        if (__any(need)) {
            const float m_new = need ? mt : m_ref;
            const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
            l_run *= alpha;
            #pragma unroll
            for (int r = 0; r < C::RT; ++r)
                #pragma unroll
                for (int i = 0; i < 16; ++i) o[r][i] *= alpha;
            m_ref = m_new;
        }
        const float mu = m_ref == -INFINITY ? 0.f : m_ref;
        // four partial row sums, each starting from its first term (no add of 0)
        float rq[4];
        #pragma unroll
        for (int b = 0; b < NKB; ++b)
            #pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][i], cl2, -mu));
                s[b][i] = e;
                if (b == 0 && i < 4)
                    rq[i] = e;
                else
                    rq[i & 3] += e;
            }
        l_run += (rq[0] + rq[1]) + (rq[2] + rq[3]);
        // slot e of MFMA j holds key 16j + 8(e/4) + 4hf + e%4 = element 8(j%2) + e of block j/2
        if constexpr (DROP) {
            // MFMA j covers the 16 keys of Philox block 4t + j; slot e takes byte e%4 of
            // word 2(e/4) + hf.  Lanes l and l + 32 hold the same query row: each computes
            // the blocks j = hf + 2k and hands the partner the two words it needs.
            static_assert(2 * NKB == 4, "dropout assumes four 16-key blocks per tile");
            uint32_t W[2][4];
            #pragma unroll
            for (int k = 0; k < 2; ++k) {
                W[k][0] = (uint32_t)(t * (BN / 16) + hf + 2 * k);
                W[k][1] = (uint32_t)(rb + lq);
                W[k][2] = (uint32_t)(tc.h + 256 * tc.b);
                W[k][3] = p.drop_offset;
                philox4x32_10(W[k], p.seed_lo, p.seed_hi);
            }
            uint32_t got[4];   // the partner's words hf and 2 + hf of its blocks
            #pragma unroll
            for (int k = 0; k < 2; ++k)
                #pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const uint32_t x = hf ? W[k][2 * w] : W[k][2 * w + 1];
                    auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
                    got[2 * k + w] = hf ? r[0] : r[1];
                }
            #pragma unroll
            for (int j = 0; j < 2 * NKB; ++j) {
                const int k = j >> 1;
                const bool own = (j & 1) == hf;
                const uint32_t wa = own ? (hf ? W[k][1] : W[k][0]) : got[2 * k];
                const uint32_t wb = own ? (hf ? W[k][3] : W[k][2]) : got[2 * k + 1];
                #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t byte = ((e < 4 ? wa : wb) >> (8 * (e & 3))) & 0xffu;
                    pp[j][e] = byte >= p.drop_thr ? (T)s[j >> 1][8 * (j & 1) + e] : (T)0.f;
                }
            }
        } else {
            #pragma unroll
            for (int j = 0; j < 2 * NKB; ++j)
                #pragma unroll
                for (int e = 0; e < 8; ++e) pp[j][e] = (T)s[j >> 1][8 * (j & 1) + e];
        }
    };

    // Step t is two phases, each closed by a barrier:
    //   M: prefetch tile t+PF into registers; S(t) = K(t) Q^T and O += P(t-1) V(t-1) on the
    //      matrix cores (the P V MFMAs cover the latency of S(t));
    //   S: land tile t+2 in LDS (its buffer's last reader finished before this phase
    //      began), then softmax(t) on the vector ALUs (the mask tensor instance, whose
    //      prefetch is one tile shallower, lands the tile after the softmax).
    // Waves 4-7 run the same code one phase behind waves 0-3, so on every SIMD one wave is
    // in its M phase while the other is in its S phase and the matrix cores and the vector
    // ALUs work at the same time.  The M phase runs at raised wave priority: the SIMD
    // otherwise favours the older wave, and a softmax of waves 0-3 would starve the MFMA
    // issue of waves 4-7.  Tile t+2 is complete after the barrier that closes the late
    // waves' S phase of step t, two phases before the first read of it, and overwrites the
    // buffer of tile t-2, whose last reader (P V in the late waves' M phase of step t-1)
    // finished one barrier earlier.
    X8 pp[2 * NKB];
    f32x16 sa[NKB];
    const bool late = C::NW == 8 && wave >= 4;   // one wave per SIMD: no partner to skew against
    auto step = [&](int t, u32x4 (&ld)[C::SREG], u32x4 (&sto)[C::SREG]) {
        __builtin_amdgcn_s_setprio(3);
        load_tile(t + PF, ld);
        if (wave_active(t)) qk(t, sa);
        // the mask bytes of the next tile, which its Q K^T products start from a step later
        if constexpr (MASKED)
            if (t + 1 < T1) load_mask(t + 1);
        if (t - 1 >= T0 && wave_active(t - 1)) pv(t - 1, pp);
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        // the staged tile goes to LDS first, so that the writes complete under the softmax
        // (with a shallower prefetch its loads were issued only one phase earlier: there it
        // goes last)
        if constexpr (PF == 3) store_tile(t + 2, sto);
        if (wave_active(t)) softmax(t, sa, pp);
        if constexpr (PF != 3) store_tile(t + 2, sto);
        __syncthreads();
    };

    if constexpr (C::BIG) {
        // ---- one wave per SIMD (head dims above 128): no partner wave overlaps the softmax
        //      with the matrix core, so each wave overlaps its own: step t issues
        //      S(t+1) = K(t+1) Q^T with the softmax of tile t between the MFMAs, then O and
        //      the row sum move to the new reference max where it changed (rare), then
        //      O += P(t) V(t).  One barrier per step: tile t+2 lands in LDS during step t
        //      (its slot's last reader, P V of tile t-2, finished before the previous
        //      barrier) and tile t+3 is loaded.  A tile that a wave does not see is
        //      computed as fully masked (its probabilities are zero), which keeps the
        //      interleaved block free of branches.
        if (T0 < T1) {
            load_tile(T0, stA);
            load_tile(T0 + 1, stB);
            __builtin_amdgcn_s_waitcnt(0);
            store_tile(T0, stA);
            store_tile(T0 + 1, stB);
            if (PF == 3) load_tile(T0 + 2, stB);
            __syncthreads();
            f32x16 sa[NKB], sb[NKB];
            X8 pp[2 * NKB];
            qk(T0, sa);
            float mq[2], mu = 0.f, rq[4] = {0.f, 0.f, 0.f, 0.f}, ex[4];
            float m_ref_n = -INFINITY, m_true_n = -INFINITY;
            // the softmax of tile t (16 scores per lane in s[0]) in slots: max over
            // elements 0-7 and 8-15, the reduction and reference update, then the eight
            // pairs with each pair's exponentials one slot before its sums and rounding.
            // The empty asm statements pin the work to its slot.
            auto sm_slot = [&](int f, f32x16 (&sx)[NKB]) __attribute__((always_inline)) {
                if (f < 2) {
                    float m = sx[0][8 * f];
                    #pragma unroll
                    for (int k = 1; k < 8; k += 2)
                        m = k + 1 < 8 ? fmaxf(fmaxf(m, sx[0][8 * f + k]), sx[0][8 * f + k + 1]) : fmaxf(m, sx[0][8 * f + k]);
                    mq[f] = m;
                    asm volatile("" : "+v"(mq[f]));
                } else if (f == 2) {
                    const float mx = pair_max(fmaxf(mq[0], mq[1]));
                    const float mt = mx * cl2;
                    m_true_n = fmaxf(m_true, mt);
                    m_ref_n = mt > m_ref + kLazyThresh ? mt : m_ref;
                    mu = m_ref_n == -INFINITY ? 0.f : m_ref_n;
                    asm volatile("" : "+v"(mu), "+v"(m_ref_n), "+v"(m_true_n));
                } else {
                    const int k = f - 3;
                    if (k >= 1 && k <= 8) {
                        const int q = k - 1, i = 2 * q;
                        const float x0 = ex[2 * (q & 1)], x1 = ex[2 * (q & 1) + 1];
                        if (q < 2) {
                            rq[i & 3] = x0;
                            rq[(i + 1) & 3] = x1;
                        } else {
                            rq[i & 3] += x0;
                            rq[(i + 1) & 3] += x1;
                        }
                        pp[i >> 3][i & 7] = (T)x0;
                        pp[i >> 3][(i & 7) + 1] = (T)x1;
                        asm volatile("" : "+v"(rq[i & 3]), "+v"(rq[(i + 1) & 3]));
                    }
                    if (k < 8) {
                        float y0 = sx[0][2 * k], y1 = sx[0][2 * k + 1];
                        asm volatile("" : "+v"(y0), "+v"(y1));
                        float& x0 = ex[2 * (k & 1)];
                        float& x1 = ex[2 * (k & 1) + 1];
                        x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(y0, cl2, -mu));
                        x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(y1, cl2, -mu));
                        asm volatile("" : "+v"(x0), "+v"(x1));
                    }
                }
            };
            constexpr int NSL = 12;   // softmax slots
            // tile t's scores in cur; S(t+1) into nxt
            auto big_step = [&](int t, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB], u32x4 (&ld)[C::SREG],
                                u32x4 (&sto)[C::SREG]) __attribute__((always_inline)) {
                load_tile(t + PF, ld);
                // keys past each lane's last visible one, and tiles the wave does not see
                if (!wave_active(t) || t < full_lo || t >= full_hi) {
                    const bool act = wave_active(t);
                    const int lo = act ? jlo : 1 << 30, hi = act ? jhi : -1;
                    const int jb = t * BN + 4 * hf;
                    #pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int j = jb + 8 * (i >> 2) + (i & 3);
                        if (j < lo || j > hi) cur[0][i] = -INFINITY;
                    }
                }
                {
                    const __bf16* kb = Ks + ((t + 1) & (NBUF - 1)) * C::KBUF + lq * C::KS + 8 * hf;
                    X8 a[C::KK];
                    nxt[0] = f32x16{};
                    #pragma unroll
                    for (int f = 0; f < LDSD && f < C::KK; ++f) a[f] = *(const X8*)(kb + 16 * f);
                    #pragma unroll
                    for (int f = 0; f < C::KK; ++f) {
                        if (f + LDSD < C::KK) a[f + LDSD] = *(const X8*)(kb + 16 * (f + LDSD));
                        nxt[0] = Elem<T>::mfma(a[f], qf[f], nxt[0]);
                        if (f < NSL) sm_slot(f, cur);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    #pragma unroll
                    for (int f = C::KK; f < NSL; ++f) sm_slot(f, cur);
                }
                if (__any(m_ref_n != m_ref)) {
                    const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_ref_n);
                    l_run *= alpha;
                    // the output accumulators live in the matrix core's registers (AGPRs);
                    // the pins keep their copies to vector registers and back inside this
                    // rare branch (unpinned, the compiler hoisted the copies out of it, into
                    // every step)
                    #pragma unroll
                    for (int r = 0; r < C::RT; ++r) asm volatile("" : "+a"(o[r]));
                    #pragma unroll
                    for (int r = 0; r < C::RT; ++r)
                        #pragma unroll
                        for (int i = 0; i < 16; ++i) o[r][i] *= alpha;
                    #pragma unroll
                    for (int r = 0; r < C::RT; ++r) asm volatile("" : "+a"(o[r]));
                }
                m_ref = m_ref_n;
                m_true = m_true_n;
                l_run += (rq[0] + rq[1]) + (rq[2] + rq[3]);
                // the staged tile t+2 lands in LDS one chunk per P V MFMA
                pv_rows(t, pp, [&](int f) __attribute__((always_inline)) {
                    if (f < C::SREG) store_chunk(t + 2, sto, f);
                });
                #pragma unroll
                for (int u = C::RT * 2 * NKB; u < C::SREG; ++u) store_chunk(t + 2, sto, u);
                __syncthreads();
            };
            int t = T0;
            u32x4 (&sB)[C::SREG] = PF == 3 ? stB : stA;
            for (; t + 1 < T1; t += 2) {
                big_step(t, sa, sb, stA, sB);
                big_step(t + 1, sb, sa, sB, stA);
            }
            if (t < T1) big_step(t, sa, sb, stA, sB);
        }
    } else if (T0 < T1) {
        // Q and the first two tiles in one memory round trip; the wait also drains Q, so
        // no wait on it is left for the key loop (where it would also wait for prefetches)
        if constexpr (MASKED) load_mask(T0);
        load_tile(T0, stA);
        load_tile(T0 + 1, stB);
        __builtin_amdgcn_s_waitcnt(0);
        store_tile(T0, stA);
        store_tile(T0 + 1, stB);
        if (PF == 3) load_tile(T0 + 2, stB);
        __syncthreads();
        if (late) __syncthreads();    // the late waves' first phase is empty
        int t = T0;
        // tile t+2 sits in the register set loaded one step earlier when PF == 3
        u32x4 (&sB)[C::SREG] = PF == 3 ? stB : stA;
        for (; t + 1 < T1; t += 2) {
            step(t, stA, sB);
            step(t + 1, sB, stA);
        }
        if (t < T1) step(t, stA, sB);
        if (wave_active(T1 - 1)) pv(T1 - 1, pp);
        if (!late) __syncthreads();   // the early waves' last phase is empty
    }

    // ---- epilogue: normalize, round to the storage type, store; emit the row statistics.
    //      This partial is O / lt with max mc = m_true ln 2 and sum l_c = lt 2^(m_ref - m_true).
    //      With UPDATE it is merged into the prior (o_p, m_p, l_p) as the ring-attention
    //      update does: m = max(m_p, mc), a = l_p e^(m_p - m), c = l_c e^(mc - m),
    //      out = o_p a / (a + c) + (O / lt) c / (a + c), before the single rounding.
    const float lt = pair_sum(l_run);
    const int qi = rb + lq;
    const bool valid = qi < re;          // both lanes of a row share it
    const bool any = lt > 0.f;
    const float mc = any ? m_true * 0.69314718055994530942f : -INFINITY;
    float m_out = mc;
    float l_out = any ? lt * __builtin_amdgcn_exp2f(m_ref - m_true) : 0.f;
    float wc = any ? (DROP ? p.drop_scale : 1.f) / lt : 0.f;   // weight of the accumulator O
    float wp = 0.f;                    // weight of the prior output
    if constexpr (UPDATE) {
        const float mp = valid ? p.prev_max[st_base + qi] : -INFINITY;
        const float lp = valid ? p.prev_sum[st_base + qi] : 0.f;
        const float m = fmaxf(mp, mc);
        wc = 0.f;
        l_out = 0.f;
        if (m != -INFINITY) {
            const float a = lp * __builtin_amdgcn_exp2f((mp - m) * 1.4426950408889634f);
            const float f = any ? __builtin_amdgcn_exp2f(m_ref - m * 1.4426950408889634f) : 0.f;
            l_out = a + lt * f;
            wp = a / l_out;
            wc = f / l_out;
        }
        m_out = m;
    }
    // Lane (lq, hf) holds dims 8 g + 4 hf .. + 3 of its row in group g of each 32-dim block;
    // one exchange with the lane 32 apart per pair of groups (lanes 32-63 of the first
    // operand trade with lanes 0-31 of the second) leaves lane (lq, 0) with dims 16 p .. + 7
    // and lane (lq, 1) with dims 16 p + 8 .. + 15 of pair p: each row then takes 32
    // contiguous bytes per 16-byte-per-lane store.  Every lane takes part in the exchange;
    // the reads of the prior and the stores are guarded by the row bound.
    T* orow = og + (int64_t)qi * p.o_ss + 4 * hf;    // this lane's 8-byte pieces
    T* orow16 = og + (int64_t)qi * p.o_ss + 8 * hf;  // this lane's 16-byte pieces
    #pragma unroll
    for (int r = 0; r < C::RT; ++r) {
        uint32_t d[4][2];
        #pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            X4 w;
            if constexpr (UPDATE) {
                // an empty prior (weight 0) is not read: its buffer may hold anything
                const T* prow = (const T*)p.prev_out + (orow - (T*)p.out);
                X4 po{};
                if (valid && wp != 0.f) po = *(const X4*)(prow + 32 * r + 8 * g4);
                #pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = (T)__builtin_fmaf((float)po[e], wp, o[r][4 * g4 + e] * wc);
            } else {
                #pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (T)(o[r][4 * g4 + e] * wc);
            }
            const auto wd = __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))), w);
            d[g4][0] = wd[0];
            d[g4][1] = wd[1];
        }
        #pragma unroll
        for (int pr = 0; pr < 2; ++pr)
            #pragma unroll
            for (int h = 0; h < 2; ++h) {
                const auto x = __builtin_amdgcn_permlane32_swap(d[2 * pr][h], d[2 * pr + 1][h], false, false);
                d[2 * pr][h] = x[0];
                d[2 * pr + 1][h] = x[1];
            }
        if (valid) {
            #pragma unroll
            for (int pr = 0; pr < 2; ++pr)
                *(X8*)(orow16 + 32 * r + 16 * pr) =
                    __builtin_bit_cast(X8, u32x4{d[2 * pr][0], d[2 * pr][1], d[2 * pr + 1][0], d[2 * pr + 1][1]});
        }
    }
    if (valid && hf == 0) {
        if (p.smax) p.smax[st_base + qi] = m_out;
        if (p.ssum) p.ssum[st_base + qi] = l_out;
    }
}

template <int D, typename T, bool UPDATE, bool MASKED>
void launch_d(const FaParams& p, hipStream_t stream)
{
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, D, T, UPDATE, MASKED>), dim3(p.n_slots),
                       dim3(KCfg<D, D, MASKED, false>::NT), 0, stream, p);
}

template <typename T, bool UPDATE, bool MASKED>
hipError_t launch_t(const FaParams& p, int D, hipStream_t stream)
{
    switch (D) {
    case 32: launch_d<32, T, UPDATE, MASKED>(p, stream); break;
    case 64: launch_d<64, T, UPDATE, MASKED>(p, stream); break;
    case 96: launch_d<96, T, UPDATE, MASKED>(p, stream); break;
    case 128: launch_d<128, T, UPDATE, MASKED>(p, stream); break;
    default:
        // head dims above 128 (4-wave workgroups, 32-key tiles): no mask tensor
        if constexpr (MASKED) return hipErrorInvalidValue;
        else switch (D) {
            case 160: launch_d<160, T, UPDATE, false>(p, stream); break;
            case 192: launch_d<192, T, UPDATE, false>(p, stream); break;
            case 224: launch_d<224, T, UPDATE, false>(p, stream); break;
            case 256: launch_d<256, T, UPDATE, false>(p, stream); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

// dropout on the probabilities (plain forward, value head dim = head dim)
template <typename T>
hipError_t launch_drop(const FaParams& p, int D, hipStream_t stream)
{
    dim3 grid(p.n_slots), block(NT);
    switch (D) {
    case 32: hipLaunchKernelGGL((fa_fwd_bf16_kernel<32, 32, T, false, false, true>), grid, block, 0, stream, p); break;
    case 64: hipLaunchKernelGGL((fa_fwd_bf16_kernel<64, 64, T, false, false, true>), grid, block, 0, stream, p); break;
    case 96: hipLaunchKernelGGL((fa_fwd_bf16_kernel<96, 96, T, false, false, true>), grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL((fa_fwd_bf16_kernel<128, 128, T, false, false, true>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// value head dim below the Q/K head dim (plain forward only)
template <int D, int DV, typename T>
void launch_dv_pair(const FaParams& p, hipStream_t stream)
{
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, DV, T, false, false>), dim3(p.n_slots),
                       dim3(KCfg<D, DV, false, false>::NT), 0, stream, p);
}

template <typename T>
hipError_t launch_dv(const FaParams& p, int D, int Dv, hipStream_t stream)
{
    if (D == 64 && Dv == 32) launch_dv_pair<64, 32, T>(p, stream);
    else if (D == 96 && Dv == 64) launch_dv_pair<96, 64, T>(p, stream);
    else if (D == 128 && Dv == 64) launch_dv_pair<128, 64, T>(p, stream);
    else if (D == 128 && Dv == 96) launch_dv_pair<128, 96, T>(p, stream);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fa_fwd_bf16(const FaParams& p, int D, bool f16, hipStream_t stream)
{
    const bool upd = p.prev_out != nullptr;
    if (p.drop_thr) {
        if (upd || p.amask || p.Dv != D) return hipErrorInvalidValue;
        return f16 ? launch_drop<_Float16>(p, D, stream) : launch_drop<__bf16>(p, D, stream);
    }
    if (p.Dv != D) {
        if (upd || p.amask) return hipErrorInvalidValue;
        return f16 ? launch_dv<_Float16>(p, D, p.Dv, stream) : launch_dv<__bf16>(p, D, p.Dv, stream);
    }
    if (p.amask) {   // the masked variant has no fused update
        if (upd) return hipErrorInvalidValue;
        return f16 ? launch_t<_Float16, false, true>(p, D, stream) : launch_t<__bf16, false, true>(p, D, stream);
    }
    if (f16) return upd ? launch_t<_Float16, true, false>(p, D, stream) : launch_t<_Float16, false, false>(p, D, stream);
    return upd ? launch_t<__bf16, true, false>(p, D, stream) : launch_t<__bf16, false, false>(p, D, stream);
}

}  // namespace miattn
