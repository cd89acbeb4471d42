// Attention forward, bf16 / fp16 inputs, masks whose visible keys start at key 0 (causal
// either way round, with or without a per-sequence prefix, no mask, or a band with no lower
// bound), with or without dropout: the persistent form of the tiled MFMA kernel, for packed
// (TND) and dense forwards with GQA.
//
// What it computes is what the tiled kernel computes (out = softmax(scale * Q K^T) V per
// sequence and query head with the per-row softmax max and sum; Paddle "sparse_attention"
// formula, the packing, GQA and causal mask of "aclnnFlashAttentionVarLenScore" 功能说明 /
// 约束说明, the statistics of "npu_ring_attention_update对外接口").  Only the way the work is
// cut and scheduled differs:
//   * A work item is R = 256 / HPI query rows of HPI query heads that share one kv head
//     (HPI = the largest power of two dividing the GQA ratio, at most 8), so the 8 waves
//     of a workgroup (32 rows each) cover R rows x HPI heads and every K / V tile staged in
//     LDS serves HPI heads at once.  Query tiles start at the sequence start, so with 64-
//     row items the causal diagonal of an item is a single 64-key tile: the diagonal costs
//     one step per item instead of four.
//   * One workgroup per CU walks a static list of items.  Under a causal mask the work of
//     an item grows with its query-tile index, so the global order takes query-tile
//     indices from the largest down (all sequences long enough for that index, longest
//     first) and hands item i to workgroup i mod G in even rounds and G - 1 - (i mod G) in
//     odd ones (a snake, which keeps the per-workgroup sums within about 2% of each other
//     on mixed lengths).  Every workgroup derives the same list from the sequence lengths,
//     which it sorts in LDS, so no scheduling state lives in device memory.
//   * The key tiles of consecutive items form one stream: tiles of the next item are
//     prefetched while the current one finishes, the next item's Q is loaded as soon as the
//     current item's last Q K^T product is issued, and an item's epilogue runs in the first
//     softmax phase of the next item.  The per-workgroup start-up (Q and first-tile latency,
//     the first LDS stores) and the tail of the last phase are paid once per CU instead of
//     once per item.
// Within a step everything is as in the tiled kernel: S^T = K Q^T on
// v_mfma_f32_32x32x16 with the scores of a query row in one lane pair, the online softmax
// in the log2 domain with a lazily moved reference max, P used as the B operand of
// O^T += V^T P^T straight from the accumulators, K and V staged row-major through a 4-deep
// LDS ring three tiles ahead (V read back transposed as the matrix operand), and the two
// waves of each SIMD one phase apart (matrix-core phase M, softmax phase S).
#include "fa_common.h"
#include "fa_mfma.h"

namespace miattn {
namespace {

constexpr int PT = 512;          // threads per workgroup (8 waves)
constexpr int PBN = 64;          // keys per tile
constexpr int PNKB = 2;          // 32-key blocks per tile
constexpr int PNBUF = 4;         // LDS ring depth (tiles)
constexpr int PLDSD = 6;         // LDS fragment reads in flight ahead of their MFMAs
constexpr float kPLazy = 8.0f;   // lazy rescale threshold (log2 units)
constexpr int kPRsrcFlags = 0x00020000;   // buffer descriptor word 3: 32-bit data, raw

template <int D>
struct PCfg {
    static constexpr int KS = D + 8;                   // K row stride in LDS (elements)
    static constexpr int VP = D + 32;                  // V row stride in LDS (elements): the
                                                       // rows of a transposed read fall in
                                                       // disjoint bank ranges
    static constexpr int CPR = D / 8;                  // 16-byte chunks per K row
    static constexpr int KCH = PBN * CPR;              // K chunks per tile
    static constexpr int KPT = KCH / PT;               // K chunks per thread
    static constexpr int SREG = 2 * KPT;               // staging registers (16 B each): K, then V
    static constexpr int KK = D / 16;                  // MFMA k-steps over the head dim
    static constexpr int RT = D / 32;                  // 32-row output tiles
    static constexpr int KBUF = PBN * KS;
    static constexpr int VBUF = PBN * VP;
    static_assert(KCH % PT == 0, "K chunks split evenly over the threads");
};

// One work item: rows [r0, r1) of query tile t of sequence b, heads [HPI g, HPI g + HPI).
struct PItem {
    int b, g, t;
    int64_t q0, kv0;        // first packed row of the sequence (0 for dense batches)
    int len_q, len_kv;
    int r0, r1;
    int T0, T1;             // key tiles [T0, T1) seen by some row of the item
    int off;                // causal diagonal: row i sees keys 0 .. i + off
    int pfx;                // and keys 0 .. pfx - 1 (the prefix; 0 without one)
};

// What the key loop needs of an item, computed once when the workgroup lists its items
// (64 bytes in LDS): byte addresses of K / V row 0 of the item's sequence and kv head, of
// Q / out row r0 of its first head, the statistics index of that row, and its bounds.
struct PRec {
    int64_t kaddr, vaddr, qaddr, oaddr, st;
    int32_t len_kv;         // keys of the sequence
    int32_t rows;           // r1 - r0
    int32_t diag;           // r0 + off: item row i sees keys 0 .. diag + i
    int32_t T0, T1;         // key tiles
    int32_t pfx;            // keys 0 .. pfx - 1 are visible from every row (the prefix)
};
static_assert(sizeof(PRec) == 64, "one LDS record per item");

// With dropout the record also carries the item's first row (sequence-local) and the third
// Philox counter word of its first head, h0 + 256 b: 80 bytes.
template <bool DROP> struct PRecT : PRec {};
template <> struct PRecT<true> : PRec {
    int32_t r0;
    uint32_t hb0;
    int32_t pad[2];
};
static_assert(sizeof(PRecT<true>) == 80, "dropout record");

// LDS of a workgroup beside the K / V ring: the item records (the packed batch's
// sequence tables, needed only while the records are built, share the ring's space).
template <int D, bool DROP>
constexpr int persist_max_items()
{
    return (160 * 1024 - PNBUF * (PCfg<D>::KBUF + PCfg<D>::VBUF) * 2 - 64) / (int)sizeof(PRecT<DROP>);
}

// DROP: dropout on the probabilities (the tiled kernel's Philox4x32-10 counters and byte
// test, so both kernels drop the same entries), the kept ones scaled in the epilogue.
template <int D, typename T, int HPI, bool VARLEN, bool DROP>
__global__ __launch_bounds__(PT, 1) void fa_fwd_persist_kernel(FaParams p)
{
    using C = PCfg<D>;
    using X8 = typename Elem<T>::v8;
    using X4 = typename Elem<T>::v4;
    // Q, out and the statistics are accessed through global-address-space pointers: the
    // compiler must assume that generic (flat) loads complete out of order with the buffer
    // loads of the tile prefetch, and would make each use of Q wait for all of them
    typedef __attribute__((address_space(1))) const X8 GX8;
    typedef __attribute__((address_space(1))) X8 GX8w;
    typedef __attribute__((address_space(1))) const T GT_c;
    typedef __attribute__((address_space(1))) T GT;
    typedef __attribute__((address_space(1))) float GF;
    constexpr int R = 256 / HPI;     // query rows per item
    constexpr int WPH = 8 / HPI;     // waves per head
    constexpr int MAXI = persist_max_items<D, DROP>();
    __shared__ __attribute__((aligned(16))) __bf16 ring[PNBUF * (C::KBUF + C::VBUF)];
    __shared__ PRecT<DROP> s_rec[MAXI];
    __shared__ int s_nitems, s_nsteps;
    __bf16* Ks = ring;
    __bf16* Vs = ring + PNBUF * C::KBUF;
    // sequence tables of a packed batch: bounds, and the sequences sorted by query tiles
    // (descending, ties by index) so that every workgroup derives the same item order
    int* s_q0 = (int*)ring;
    int* s_kv0 = s_q0 + kPersistMaxSeq;
    int* s_lq = s_kv0 + kPersistMaxSeq;
    int* s_lkv = s_lq + kPersistMaxSeq;
    int* s_nts = s_lkv + kPersistMaxSeq;
    int* s_perm = s_nts + kPersistMaxSeq;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31;        // query column owned by this lane
    const int hf = lane >> 5;        // half of the wave
    const int hgi = wave / WPH;      // head of the item's group that this wave computes
    const int wrow = 32 * (wave % WPH);
    const bool late = wave >= 4;     // waves 4-7 run one phase behind
    const int n_groups = p.Nq / HPI;
    const int nseq = p.B;

    // ---- the workgroup's items
    {
        int ntd = 0;   // dense batches: query tiles of every sequence
        if constexpr (VARLEN) {
            for (int b = tid; b < nseq; b += PT) {
                const int64_t qs = b ? p.cu_q[b - 1] : 0, ks = b ? p.cu_kv[b - 1] : 0;
                s_q0[b] = (int)qs;
                s_kv0[b] = (int)ks;
                s_lq[b] = (int)(p.cu_q[b] - qs);
                s_lkv[b] = (int)(p.cu_kv[b] - ks);
            }
            __syncthreads();
            for (int b = tid; b < nseq; b += PT) {
                const int nb = (s_lq[b] + R - 1) / R;
                int rank = 0;
                for (int j = 0; j < nseq; ++j) {
                    const int nj = (s_lq[j] + R - 1) / R;
                    rank += nj > nb || (nj == nb && j < b);
                }
                s_perm[rank] = b;
                s_nts[rank] = nb;
            }
            __syncthreads();
        } else {
            ntd = (p.Sq + R - 1) / R;
        }
        // Item i of the global order goes to workgroup i mod G in even rounds and
        // G - 1 - (i mod G) in odd ones.  Wave 0 first lists the groups of query-tile levels
        // that hold the same sequences (level t holds kp x n_groups items, kp the sequences
        // with more than t tiles, from the largest t down), then every lane takes one of the
        // workgroup's items and finds its level, sequence and head group from that table;
        // items that see no key get the empty result.  Batches of up to 64 sequences keep
        // the sorted tile counts in wave 0's lanes for the table walk.
        if (wave == 0) {
            const int nwg = gridDim.x, wg = blockIdx.x;
            int* s_gbase = s_perm + kPersistMaxSeq;    // group x: index of its first item,
            int* s_gtop = s_gbase + kPersistMaxSeq;    //   its top level,
            int* s_gper = s_gtop + kPersistMaxSeq;     //   and items per level
            int n_grp = 1, total = 0;
            if constexpr (VARLEN) {
                const bool regs = nseq <= 64;
                const int r_nts = regs && lane < nseq ? s_nts[lane] : 0;
                auto tiles_sorted = [&](int k) -> int {
                    return regs ? __builtin_amdgcn_readlane(r_nts, k) : __builtin_amdgcn_readfirstlane(s_nts[k]);
                };
                int t = nseq > 0 ? tiles_sorted(0) - 1 : -1;
                int kp = 0, base = 0;
                while (kp < nseq && tiles_sorted(kp) > t) ++kp;
                n_grp = 0;
                while (t >= 0) {
                    const int per = kp * n_groups;
                    const int stop = kp < nseq ? tiles_sorted(kp) : 0;
                    if (lane == 0) {
                        s_gbase[n_grp] = base;
                        s_gtop[n_grp] = t;
                        s_gper[n_grp] = per;
                    }
                    ++n_grp;
                    base += (t - stop + 1) * per;
                    t = stop - 1;
                    while (kp < nseq && tiles_sorted(kp) > t) ++kp;
                }
                total = base;
            } else {
                total = ntd * nseq * n_groups;
            }
            int n = 0, steps = 0;
            for (int k0 = 0;; k0 += 64) {
                const int k = k0 + lane;
                const int i = k * nwg + ((k & 1) ? nwg - 1 - wg : wg);
                const bool valid = k0 * nwg < total && i < total;
                if (!__any(valid)) break;
                PItem it{};
                it.T1 = 0;
                if (valid) {
                    int base = 0, top = ntd - 1, per = nseq * n_groups;
                    if constexpr (VARLEN) {
                        // the last group that starts at or before item i
                        int lo = 0, hi = n_grp - 1;
                        while (lo < hi) {
                            const int mid = (lo + hi + 1) >> 1;
                            if (s_gbase[mid] <= i) lo = mid;
                            else hi = mid - 1;
                        }
                        base = s_gbase[lo];
                        top = s_gtop[lo];
                        per = s_gper[lo];
                    }
                    const int d = (i - base) / per;
                    const int j = i - base - d * per;
                    const int kk = j / n_groups;
                    it.g = j - kk * n_groups;
                    it.t = top - d;
                    if constexpr (VARLEN) {
                        it.b = s_perm[kk];
                        it.q0 = s_q0[it.b];
                        it.kv0 = s_kv0[it.b];
                        it.len_q = s_lq[it.b];
                        it.len_kv = s_lkv[it.b];
                    } else {
                        it.b = kk;
                        it.q0 = it.kv0 = 0;
                        it.len_q = p.Sq;
                        it.len_kv = p.Skv;
                    }
                    it.r0 = it.t * R;
                    it.r1 = min(it.len_q, it.r0 + R);
                    // row i sees keys 0 .. i + off: the diagonal (top-left or bottom-right)
                    // moved by the band's upper bound (causal: 0; no mask: every key),
                    // clamped to the sequence so that it stays a 32-bit value
                    {
                        const int64_t off64 = (p.align_br ? (int64_t)it.len_kv - it.len_q : 0) + p.next;
                        it.off = (int)(off64 > it.len_kv ? it.len_kv : (off64 < -(int64_t)it.len_q - 1 ? -it.len_q - 1 : off64));
                    }
                    // a per-sequence prefix: keys below it are visible from every row
                    it.pfx = 0;
                    if (p.prefix) {
                        const int64_t x = p.prefix[it.b];
                        it.pfx = x < 0 ? 0 : (x > it.len_kv ? it.len_kv : (int)x);
                    }
                    // rows [r0, r1) see keys 0 .. max(r1 - 1 + off, pfx - 1)
                    const int vis = max(0, min(max(it.r1 + it.off, it.pfx), it.len_kv));
                    it.T0 = 0;
                    it.T1 = (vis + PBN - 1) / PBN;
                }
                const bool live = valid && it.T1 > 0;
                // records of the live items in item order (lanes below this one first)
                const uint64_t live_mask = __ballot(live);
                const int pos = n + __builtin_amdgcn_mbcnt_hi((uint32_t)(live_mask >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)live_mask, 0u));
                if (live && pos < MAXI) {
                    const int h0 = it.g * HPI;
                    const int kvh = h0 / p.group;
                    PRecT<DROP>& rc = s_rec[pos];
                    rc.kaddr = (int64_t)p.k + ((int64_t)it.b * p.k_sb + it.kv0 * p.k_ss + (int64_t)kvh * p.k_sh) * 2;
                    rc.vaddr = (int64_t)p.v + ((int64_t)it.b * p.v_sb + it.kv0 * p.v_ss + (int64_t)kvh * p.v_sh) * 2;
                    rc.qaddr = (int64_t)p.q + ((int64_t)it.b * p.q_sb + (it.q0 + it.r0) * p.q_ss + (int64_t)h0 * p.q_sh) * 2;
                    rc.oaddr = (int64_t)p.out + ((int64_t)it.b * p.o_sb + (it.q0 + it.r0) * p.o_ss + (int64_t)h0 * p.o_sh) * 2;
                    rc.st = (int64_t)it.b * p.st_sb + (int64_t)h0 * p.st_sh + it.q0 + it.r0;
                    rc.len_kv = it.len_kv;
                    rc.rows = it.r1 - it.r0;
                    rc.diag = it.r0 + it.off;
                    rc.T0 = it.T0;
                    rc.T1 = it.T1;
                    rc.pfx = it.pfx;
                    if constexpr (DROP) {
                        rc.r0 = it.r0;
                        rc.hb0 = (uint32_t)h0 + 256u * (uint32_t)it.b;
                    }
                }
                int st = live && pos < MAXI ? it.T1 - it.T0 : 0;
                #pragma unroll
                for (int o = 32; o > 0; o >>= 1) st += __shfl_xor(st, o);
                steps += st;
                n = min(MAXI, n + (int)__builtin_popcountll(live_mask));
                // items that see no key (rare): the wave writes their empty result one by one
                uint64_t empty_mask = __ballot(valid && it.T1 == 0);
                while (empty_mask) {
                    const int e = __builtin_ctzll(empty_mask);
                    empty_mask &= empty_mask - 1;
                    const int eb = __builtin_amdgcn_readlane(it.b, e);
                    const int eg = __builtin_amdgcn_readlane(it.g, e);
                    const int er0 = __builtin_amdgcn_readlane(it.r0, e);
                    const int er1 = __builtin_amdgcn_readlane(it.r1, e);
                    const int64_t eq0 = __builtin_amdgcn_readlane((int)it.q0, e);
                    const int h0 = eg * HPI;
                    for (int hh = 0; hh < HPI; ++hh)
                        for (int qi = er0 + lq; qi < er1; qi += 32) {
                            T* orow = (T*)p.out + (int64_t)eb * p.o_sb + (eq0 + qi) * p.o_ss +
                                      (int64_t)(h0 + hh) * p.o_sh + 4 * hf;
                            #pragma unroll
                            for (int r = 0; r < C::RT; ++r)
                                #pragma unroll
                                for (int g4 = 0; g4 < 4; ++g4) *(X4*)(orow + 32 * r + 8 * g4) = X4{};
                            if (hf == 0) {
                                const int64_t si = (int64_t)eb * p.st_sb + (int64_t)(h0 + hh) * p.st_sh + eq0 + qi;
                                if (p.smax) p.smax[si] = -INFINITY;
                                if (p.ssum) p.ssum[si] = 0.f;
                            }
                        }
                }
            }
            if (lane == 0) {
                s_nitems = n;
                s_nsteps = steps;
            }
        }
        __syncthreads();
    }
    const int n_items = __builtin_amdgcn_readfirstlane(s_nitems);
    if (n_items == 0) return;
    const int n_steps = __builtin_amdgcn_readfirstlane(s_nsteps);

    auto rec64 = [&](const int64_t& x) -> int64_t {
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    auto rec32 = [&](const int32_t& x) -> int { return __builtin_amdgcn_readfirstlane(x); };

    // per-wave and per-lane offsets from an item's row r0 / first head (bytes; stats in
    // elements), the same for every item
    const int64_t q_wave = ((int64_t)wrow * p.q_ss + (int64_t)hgi * p.q_sh) * 2;
    const int64_t o_wave = ((int64_t)wrow * p.o_ss + (int64_t)hgi * p.o_sh) * 2;
    const int64_t st_wave = (int64_t)hgi * p.st_sh + wrow;
    const int64_t q_row = p.q_ss * 2, o_row = p.o_ss * 2;   // bytes per row
    // row strides of K and V in bytes (a 64-row tile spans under 2^31 bytes: the host routes
    // larger strides elsewhere)
    const int krb = (int)(2 * p.k_ss), vrb = (int)(2 * p.v_ss);
    const bool want_max = p.smax != nullptr, want_sum = p.ssum != nullptr;
    float* const smax = p.smax;
    float* const ssum = p.ssum;

    // ---- the loader: item l_k and its next tile l_tile
    int l_k = 0, l_tile = 0, l_T1 = 0, l_len = 0;
    int64_t l_kb = 0, l_vb = 0;
    auto loader_item = [&](int k) {
        l_kb = rec64(s_rec[k].kaddr);
        l_vb = rec64(s_rec[k].vaddr);
        l_len = rec32(s_rec[k].len_kv);
        l_tile = rec32(s_rec[k].T0);
        l_T1 = rec32(s_rec[k].T1);
    };
    loader_item(0);

    // ---- buffer descriptors (workgroup-uniform inputs kept in scalar registers)
    auto rsrc = [](int64_t base, int64_t bytes) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)base >> 32));
        const int n = __builtin_amdgcn_readfirstlane((int)bytes);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, kPRsrcFlags);
    };

    // ---- staging of one tile: every thread takes KPT K chunks (16 B of a key row) and one
    //      V unit (2 keys x 8 dims); rows past the sequence end read as zero
    u32x4 stA[C::SREG], stB[C::SREG];
    uint32_t koff[C::KPT], voff[C::KPT];
    #pragma unroll
    for (int u = 0; u < C::KPT; ++u) {
        const int c = tid + PT * u;
        koff[u] = (uint32_t)((c / C::CPR) * krb + 16 * (c % C::CPR));
        voff[u] = (uint32_t)((c / C::CPR) * vrb + 16 * (c % C::CPR));
    }

    // load the loader's next tile (zeros past the list) and advance the loader; the row
    // count is clamped with scalar instructions (the compiler would form a vector
    // v_med3_i32 and multiply on the vector ALU, which the softmax of the partner wave needs)
    auto load_next = [&](u32x4 (&stage)[C::SREG]) {
        if (l_tile == l_T1 && l_k + 1 < n_items) loader_item(++l_k);
        const int j0 = l_tile * PBN;
        int rows = l_len - j0;
        asm("s_max_i32 %0, %0, 0\n\ts_min_i32 %0, %0, %1" : "+s"(rows) : "n"(PBN));
        if (l_tile >= l_T1) rows = 0;
        const __amdgpu_buffer_rsrc_t rk = rsrc(l_kb + (int64_t)j0 * krb, rows * krb);
        const __amdgpu_buffer_rsrc_t rv = rsrc(l_vb + (int64_t)j0 * vrb, rows * vrb);
        #pragma unroll
        for (int u = 0; u < C::KPT; ++u) stage[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[u], 0, 0);
        #pragma unroll
        for (int u = 0; u < C::KPT; ++u) stage[C::KPT + u] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[u], 0, 0);
        ++l_tile;
    };
    auto store_tile = [&](int slot, const u32x4 (&stage)[C::SREG]) {
        __bf16* kb = Ks + slot * C::KBUF;
        __bf16* vb = Vs + slot * C::VBUF;
        #pragma unroll
        for (int u = 0; u < C::KPT; ++u) {
            const int c = tid + PT * u;
            *(u32x4*)(kb + (c / C::CPR) * C::KS + 8 * (c % C::CPR)) = stage[u];
            *(u32x4*)(vb + (c / C::CPR) * C::VP + 8 * (c % C::CPR)) = stage[C::KPT + u];
        }
    };

    // ---- compute-side state of the current item: key tiles, this wave's causal bounds
    X8 qf[C::KK];
    f32x16 o[C::RT];
    float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;
    const float cl2 = p.scale_log2;
    int c_T0 = 0, c_T1 = 0;
    int w_hi = 0;        // tiles [0, w_hi) hold a visible key of this wave's rows
    int full_hi = 0;     // tiles [0, full_hi) are visible in full from every row of the wave
    int jhi = -1;        // keys [0, jhi] are visible from this lane's row
    uint32_t d_row = 0, d_hb = 0;   // dropout counter words of this lane's row and head

    // bounds of item k for this wave (causal: item row i sees keys 0 .. max(diag + i, pfx - 1))
    auto item_bounds = [&](int k) {
        const int rows = rec32(s_rec[k].rows);
        const int diag = rec32(s_rec[k].diag);
        const int len_kv = rec32(s_rec[k].len_kv);
        const int pfx = rec32(s_rec[k].pfx);
        c_T0 = rec32(s_rec[k].T0);
        c_T1 = rec32(s_rec[k].T1);
        if constexpr (DROP) {
            d_row = (uint32_t)(rec32(s_rec[k].r0) + wrow + lq);
            d_hb = (uint32_t)rec32((int32_t)s_rec[k].hb0) + (uint32_t)hgi;
        }
        const int re = min(wrow + 32, rows);   // this wave's item rows [wrow, re)
        w_hi = full_hi = 0;
        jhi = -1;
        if (wrow < re) {
            w_hi = (max(0, min(max(diag + re, pfx), len_kv)) + PBN - 1) / PBN;
            full_hi = max(0, min(max(diag + wrow + 1, pfx), len_kv)) / PBN;
            jhi = min(max(diag + wrow + lq, pfx - 1), len_kv - 1);
        }
    };
    // Q rows of item k for this wave: B operand of S^T = K Q^T, lane (lq, hf) holds
    // d = 16 kk + 8 hf .. + 7 of its row (rows past the item's end repeat its last row)
    auto load_q = [&](int k) {
        const int rows = rec32(s_rec[k].rows);
        const int qi = min(wrow + lq, rows - 1) - wrow;
        const GX8* qrow = (const GX8*)((GT_c*)(rec64(s_rec[k].qaddr) + q_wave + qi * q_row) + 8 * hf);
        #pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) qf[kk] = qrow[2 * kk];
    };

    // ---- S^T = K Q^T for the tile in LDS slot `slot`
    auto qk = [&](int slot, f32x16 (&s)[PNKB]) {
        const __bf16* kb = Ks + slot * C::KBUF + lq * C::KS + 8 * hf;
        constexpr int NF = C::KK * PNKB;
        X8 a[NF];
        #pragma unroll
        for (int b = 0; b < PNKB; ++b) s[b] = f32x16{};
        #pragma unroll
        for (int f = 0; f < PLDSD && f < NF; ++f)
            a[f] = *(const X8*)(kb + 32 * (f % PNKB) * C::KS + 16 * (f / PNKB));
        #pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + PLDSD < NF)
                a[f + PLDSD] = *(const X8*)(kb + 32 * ((f + PLDSD) % PNKB) * C::KS + 16 * ((f + PLDSD) / PNKB));
            s[f % PNKB] = Elem<T>::mfma(a[f], qf[f / PNKB], s[f % PNKB]);
        }
        constexpr int AH = PLDSD < NF ? PLDSD : NF;
        __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
        #pragma unroll
        for (int f = 0; f < NF - AH; ++f) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
    };

    // ---- O^T += V^T P^T for the tile in LDS slot `slot`.  Fragment f is 32-dim block
    //      r = f % RT and 16-key block j = f / RT, so consecutive MFMAs feed different
    //      accumulators while each accumulator still takes its key blocks in order.  V sits
    //      in LDS as [key][dim]; the A operand of fragment (r, j) comes from
    //      two ds_read_b64_tr_b16: lane l, slot e of a transposed read receives element l % 4
    //      of the 8-byte block read by lane 16 (l / 16) + 4 e + (l % 16) / 4, so lane l reading
    //      dims 32 r + 16 ((l / 16) % 2) + 4 (l % 4) .. + 3 of key 16 j + 4 hf + (l % 16) / 4
    //      (then 8 keys further) leaves lane (lq, hf) with V[16 j + 8 (e / 4) + 4 hf + e % 4]
    //      [32 r + lq], e = 0..7: the key order of the P operand taken from the S accumulators
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const int v_lane = (4 * hf + ((lane & 15) >> 2)) * C::VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto vfrag = [&](int slot, int f) -> X8 {
        const __bf16* v = Vs + slot * C::VBUF + v_lane + 16 * (f / C::RT) * C::VP + 32 * (f % C::RT);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)v);
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(v + 8 * C::VP));
        return __builtin_bit_cast(X8, i16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    };
    auto pv = [&](int slot, const X8 (&pp)[2 * PNKB]) {
        constexpr int NF = C::RT * 2 * PNKB;
        X8 a[NF];
        #pragma unroll
        for (int f = 0; f < PLDSD && f < NF; ++f) a[f] = vfrag(slot, f);
        #pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f + PLDSD < NF) a[f + PLDSD] = vfrag(slot, f + PLDSD);
            o[f % C::RT] = Elem<T>::mfma(a[f], pp[f / C::RT], o[f % C::RT]);
        }
        constexpr int AH = PLDSD < NF ? PLDSD : NF;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
        #pragma unroll
        for (int f = 0; f < NF - AH; ++f) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
    };

    // ---- online softmax of key tile t; leaves the rounded probabilities in pp
    auto softmax = [&](int t, f32x16 (&s)[PNKB], X8 (&pp)[2 * PNKB]) {
        if (t >= full_hi) {
            const int jb = t * PBN + 4 * hf;   // key of element i of block b: jb + 32b + 8(i/4) + i%4
            #pragma unroll
            for (int b = 0; b < PNKB; ++b)
                #pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (jb + 32 * b + 8 * (i >> 2) + (i & 3) > jhi) s[b][i] = -INFINITY;
        }
        float mq[4];
        #pragma unroll
        for (int c = 0; c < 4; ++c) {
            float m = s[0][4 * c];
            #pragma unroll
            for (int k = 1; k < 4 * PNKB; k += 2) {
                const int b0 = k / 4, i0 = k % 4, b1 = (k + 1) / 4, i1 = (k + 1) % 4;
                m = (k + 1 < 4 * PNKB) ? fmaxf(fmaxf(m, s[b0][4 * c + i0]), s[b1][4 * c + i1])
                                       : fmaxf(m, s[b0][4 * c + i0]);
            }
            mq[c] = m;
        }
        const float mx = pair_max(fmaxf(fmaxf(fmaxf(mq[0], mq[1]), mq[2]), mq[3]));
        const float mt = mx * cl2;
        m_true = fmaxf(m_true, mt);
        const bool need = mt > m_ref + kPLazy;
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
        for (int b = 0; b < PNKB; ++b)
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
        if constexpr (DROP) {
            // slot e of MFMA j holds key 16j + 8(e/4) + 4hf + e%4 of the tile, the 16 keys of
            // Philox block 4t + j; slot e takes byte e%4 of word 2(e/4) + hf.  Lanes l and
            // l + 32 hold the same query row: each computes the blocks j = hf + 2k and hands
            // the partner the two words it needs
            uint32_t W[2][4];
            #pragma unroll
            for (int k = 0; k < 2; ++k) {
                W[k][0] = (uint32_t)(t * (PBN / 16) + hf + 2 * k);
                W[k][1] = d_row;
                W[k][2] = d_hb;
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
            for (int j = 0; j < 2 * PNKB; ++j) {
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
            for (int j = 0; j < 2 * PNKB; ++j)
                #pragma unroll
                for (int e = 0; e < 8; ++e) pp[j][e] = (T)s[j >> 1][8 * (j & 1) + e];
        }
    };

    // ---- epilogue of item k: O / l rounded to the storage type, the statistics in
    //      natural-log units (sum re-referenced from m_ref to the true max); then the row
    //      state starts over for the next item
    auto epilogue = [&](int k) {
        const int rows = rec32(s_rec[k].rows);
        const float lt = pair_sum(l_run);
        const int qi = wrow + lq;
        const bool any = lt > 0.f;
        const float wc = any ? (DROP ? p.drop_scale : 1.f) / lt : 0.f;
        // Lane (lq, hf) holds dims 8 g + 4 hf .. + 3 of its row in group g of each 32-dim
        // block.  One exchange with the lane 32 apart (lanes 32-63 of the first operand
        // trade with lanes 0-31 of the second) per pair of groups leaves lane (lq, 0) with
        // dims 16 p .. + 7 and lane (lq, 1) with dims 16 p + 8 .. + 15 of the pair p, so
        // each row takes 32 contiguous bytes per 16-byte-per-lane store, in half the
        // store instructions of 8-byte pieces.  Every lane takes part in the exchange;
        // only the stores are guarded by the row bound (both lanes of a row share it).
        GT* orow = (GT*)(rec64(s_rec[k].oaddr) + o_wave + lq * o_row) + 8 * hf;
        #pragma unroll
        for (int r = 0; r < C::RT; ++r) {
            uint32_t d[4][2];
            #pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                X4 w;
                #pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (T)(o[r][4 * g4 + e] * wc);
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
            if (qi < rows) {
                #pragma unroll
                for (int pr = 0; pr < 2; ++pr)
                    *(GX8w*)(orow + 32 * r + 16 * pr) =
                        __builtin_bit_cast(X8, u32x4{d[2 * pr][0], d[2 * pr][1], d[2 * pr + 1][0], d[2 * pr + 1][1]});
            }
        }
        if (qi < rows && hf == 0) {
            const float m_out = any ? m_true * 0.69314718055994530942f : -INFINITY;
            const float l_out = any ? lt * __builtin_amdgcn_exp2f(m_ref - m_true) : 0.f;
            const int64_t si = rec64(s_rec[k].st) + st_wave + lq;
            if (want_max) ((GF*)smax)[si] = m_out;
            if (want_sum) ((GF*)ssum)[si] = l_out;
        }
        m_ref = m_true = -INFINITY;
        l_run = 0.f;
        #pragma unroll
        for (int r = 0; r < C::RT; ++r) o[r] = f32x16{};
    };

    // ---- prologue: the first item's Q and its first two tiles in one memory round trip
    item_bounds(0);
    load_q(0);
    int c_tile = c_T0;
    load_next(stA);
    load_next(stB);
    __builtin_amdgcn_s_waitcnt(0);
    store_tile(0, stA);
    store_tile(1, stB);
    load_next(stB);
    #pragma unroll
    for (int r = 0; r < C::RT; ++r) o[r] = f32x16{};
    __syncthreads();
    if (late) __syncthreads();   // the late waves' first phase is empty

    // Step s (stream position s, LDS slot s % 4) is two phases, each closed by a barrier:
    //   M: load stream position s + 3; S(s) = K(s) Q^T; O += P(s-1) V(s-1) (at an item's
    //      first tile, that is the previous item's last P V);
    //   S: land position s + 2 in LDS (its slot's last reader finished before this
    //      phase began); at an item's first tile, the previous item's epilogue; softmax(s).
    // The next item's Q is loaded at the start of the item's last softmax phase, once the
    // current item's last S = K Q^T has been issued.
    // Waves 4-7 run one phase behind waves 0-3, so each SIMD always has one wave in each
    // phase; the ring argument of the tiled kernel holds on stream positions.
    X8 pp[2 * PNKB];
    f32x16 sa[PNKB];
    int s = 0;
    int c_k = 0;
    bool p_act = false;    // the previous step left a P V to do
    bool first = false;    // this step starts an item after another one (its epilogue is due)
    auto step = [&](u32x4 (&ld)[C::SREG], u32x4 (&sto)[C::SREG]) {
        const bool act = c_tile < w_hi;
        __builtin_amdgcn_s_setprio(3);
        load_next(ld);
        if (act) qk(s & (PNBUF - 1), sa);
        if (p_act) pv((s - 1) & (PNBUF - 1), pp);
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        // the staged tile goes to LDS first, so that the writes complete under the softmax
        store_tile((s + 2) & (PNBUF - 1), sto);
        const bool last = c_tile + 1 == c_T1;
        if (last && c_k + 1 < n_items) load_q(c_k + 1);
        if (first) {
            epilogue(c_k - 1);
            first = false;
        }
        if (act) softmax(c_tile, sa, pp);
        p_act = act;
        ++c_tile;
        if (last && ++c_k < n_items) {
            item_bounds(c_k);
            c_tile = c_T0;
            first = true;
        }
        ++s;
        __syncthreads();
    };

    // every workgroup knows its number of steps, so the loop has no exit inside a pair of
    // steps (the two register sets of the staged tiles swap roles from one step to the next)
    int left = n_steps;
    for (; left >= 2; left -= 2) {
        step(stA, stB);
        step(stB, stA);
    }
    if (left) step(stA, stB);
    // the last item: its last P V, then (after the barrier that closes the late waves' last
    // softmax phase for the early ones) its epilogue
    if (p_act) pv((s - 1) & (PNBUF - 1), pp);
    if (!late) __syncthreads();   // the early waves' last phase is empty
    epilogue(n_items - 1);
}

template <int D, typename T, int HPI, bool DROP>
hipError_t launch_hpi_d(const FaParams& p, hipStream_t stream)
{
    if (p.cu_q)
        hipLaunchKernelGGL((fa_fwd_persist_kernel<D, T, HPI, true, DROP>), dim3(p.n_slots), dim3(PT), 0, stream, p);
    else
        hipLaunchKernelGGL((fa_fwd_persist_kernel<D, T, HPI, false, DROP>), dim3(p.n_slots), dim3(PT), 0, stream, p);
    return hipGetLastError();
}

template <int D, typename T, int HPI>
hipError_t launch_hpi(const FaParams& p, hipStream_t stream)
{
    return p.drop_thr ? launch_hpi_d<D, T, HPI, true>(p, stream) : launch_hpi_d<D, T, HPI, false>(p, stream);
}

template <int D, typename T>
hipError_t launch_dt(const FaParams& p, hipStream_t stream)
{
    switch (p.persist_hpi) {
    case 1: return launch_hpi<D, T, 1>(p, stream);
    case 2: return launch_hpi<D, T, 2>(p, stream);
    case 4: return launch_hpi<D, T, 4>(p, stream);
    case 8: return launch_hpi<D, T, 8>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int fa_persist_heads_per_item(int group)
{
    int h = 1;
    while (h < 8 && group % (2 * h) == 0) h *= 2;
    return h;
}

int fa_persist_max_items(int D, bool drop)
{
    if (drop) return D == 64 ? persist_max_items<64, true>() : persist_max_items<128, true>();
    return D == 64 ? persist_max_items<64, false>() : persist_max_items<128, false>();
}

hipError_t launch_fa_fwd_persist(const FaParams& p, int D, bool f16, hipStream_t stream)
{
    if (D == 128) return f16 ? launch_dt<128, _Float16>(p, stream) : launch_dt<128, __bf16>(p, stream);
    if (D == 64) return f16 ? launch_dt<64, _Float16>(p, stream) : launch_dt<64, __bf16>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace miattn
