/*
 * miattn.h - C ABI of the MI355X (gfx950) fused scaled-dot-product attention forward.
 *
 * The library computes  out = softmax(scale * Q K^T) V  FlashAttention-style: score tiles
 * live in registers and the S x S score matrix never reaches device memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named q, k, v, out, prev_*, cur_*, softmax_*, cu_seqlens_*, csr_* are DEVICE
 *    pointers.  The caller owns every buffer; the library never allocates, frees or
 *    synchronizes, and keeps no state between calls besides its loaded code objects.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.  Every call
 *    only enqueues work on that stream and returns; results are ready when the stream is.
 *  - Every host-checkable condition is validated before any HIP call; on failure nothing
 *    is enqueued and a status other than MIATTN_OK is returned.  A failed launch returns
 *    MIATTN_ERR_LAUNCH.  No exception crosses the ABI.
 *  - Device-resident metadata (cumulative lengths, CSR offsets/columns) is a caller
 *    contract: monotone non-decreasing, last entry = total rows, columns in [0, S).
 *    Contents violating it give undefined results (the library cannot read device
 *    memory without a synchronization).
 *  - Outputs are fully overwritten.  Inputs must not alias outputs except where noted.
 *  - Results are bitwise reproducible run to run: no atomics, fixed reduction orders
 *    (the determinism the aclnnFlashAttentionVarLenScore constraints ask for by default).
 *  - Element (b, n, s, d) of a 4-D tensor sits at:
 *      BNSD: ((b*N + n)*S + s)*D + d          (batch, heads, seq, head_dim)
 *      BSND: ((b*S + s)*N + n)*D + d
 *      BSH : same memory as BSND with H = N*D
 *      SBH : ((s*B + b)*N + n)*D + d          (H = N*D; head n owns columns n*D..n*D+D-1)
 *  - Masks act on sequence-local positions i (query) and j (key):
 *      MIATTN_MASK_NONE      : every key is visible;
 *      MIATTN_MASK_CAUSAL    : j <= i                                  (top-left aligned);
 *      MIATTN_MASK_BAND      : -pre_tokens <= j - i <= next_tokens     (top-left; pre/next
 *                              signed; the band must be non-empty: pre_tokens + next_tokens
 *                              >= 0, the band rule of the aclnnFlashAttentionVarLenScore
 *                              constraints);
 *      MIATTN_MASK_CAUSAL_BR : j - i <= Skv - Sq                        (bottom-right aligned:
 *                              the diagonal ends at the last query / last key of the
 *                              sequence; the reading of that page's sparseMode 3, which
 *                              needs Sq <= Skv so that no row is empty);
 *      MIATTN_MASK_BAND_BR   : -pre_tokens <= j - i - (Skv - Sq) <= next_tokens.
 *    Sq / Skv are the lengths of each sequence.  Tiles that no visible pair touches are
 *    never loaded.  attn_fwd_ext / attn_fwd_varlen_ext add a prefix and an explicit
 *    mask tensor.
 *  - Softmax statistics (fp32, optional, each may be NULL):
 *      softmax_max[row] = max over visible keys of scale * q.k   (natural-log units);
 *      softmax_sum[row] = sum over visible keys of exp(scale * q.k - softmax_max[row]).
 *    A row with no visible key yields out = 0, softmax_max = -inf, softmax_sum = 0.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below are int-sized.  In C++ they take int as their fixed underlying type, so
 * that every int a caller passes is a value of the type and the entry points can reject an
 * unknown one (without a fixed type a C++ enum holds only the range of its enumerators). */
#ifdef __cplusplus
#define MIATTN_ENUM enum : int
#else
#define MIATTN_ENUM enum
#endif

typedef MIATTN_ENUM {
    MIATTN_OK = 0,
    MIATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    MIATTN_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    MIATTN_ERR_DTYPE = 3,       /* unknown dtype, or one this entry point does not take */
    MIATTN_ERR_LAYOUT = 4,      /* unknown layout */
    MIATTN_ERR_GQA_RATIO = 5,   /* Nq is not a non-zero integer multiple of Nkv */
    MIATTN_ERR_MASK = 6,        /* unknown mask, or an empty band (pre + next < 0) */
    MIATTN_ERR_UNSUPPORTED = 7, /* valid per the operator spec but not built (e.g. head_dim) */
    MIATTN_ERR_LAUNCH = 8,      /* the HIP launch failed */
    MIATTN_ERR_SCALE = 9,       /* scale is not a finite positive number */
    MIATTN_ERR_DROPOUT = 10,    /* dropout_p is not in [0, 1) (or rounds to 256/256) */
    MIATTN_ERR_BLAS = 11,       /* a rocBLAS call (handle creation or GEMM) failed */
    MIATTN_ERR_WORKSPACE = 12,  /* the workspace is NULL or smaller than required */
    MIATTN_ERR_SCRATCH = 13     /* larger than the static scratch of a no-allocation entry point */
} miattn_status_t;

/* MIATTN_F64 is taken by sparse_csr_attn only (the Paddle page lists float32 and float64). */
typedef MIATTN_ENUM { MIATTN_F32 = 0, MIATTN_BF16 = 1, MIATTN_F16 = 2, MIATTN_F64 = 3 } miattn_dtype_t;
typedef MIATTN_ENUM { MIATTN_BNSD = 0, MIATTN_BSND = 1, MIATTN_BSH = 2, MIATTN_SBH = 3 } miattn_layout_t;
typedef MIATTN_ENUM {
    MIATTN_MASK_NONE = 0,
    MIATTN_MASK_CAUSAL = 1,
    MIATTN_MASK_BAND = 2,
    MIATTN_MASK_CAUSAL_BR = 3,
    MIATTN_MASK_BAND_BR = 4
} miattn_mask_t;

/* Kernels a dense forward may run on (attn_fwd_route). */
typedef MIATTN_ENUM {
    MIATTN_KERNEL_TILED = 1,      /* the tiled MFMA kernel, one workgroup per query tile */
    MIATTN_KERNEL_GENERAL = 2,    /* the head-dim-general kernel */
    MIATTN_KERNEL_PERSISTENT = 3  /* the tiled kernel's persistent causal form */
} miattn_kernel_t;

/*
 * attn_fwd - dense attention forward over a batch of equal-length sequences.
 *
 * Defines: out = softmax(scale * Q K^T) V per (batch, query head), the formula of the
 * Paddle "sparse_attention" page and of manual_attention in the blog "高效 AI 模型开发：
 * PyTorch torch.nn.attention 报错排查与高效替代方法"; the (batch, heads, seq, head_dim)
 * layout that blog requires; GQA/MQA (query head h reads kv head h / (Nq/Nkv)) and the
 * band mask from the aclnnFlashAttentionVarLenScore constraints.
 *
 *   q    [B, Nq,  Sq,  D] in `layout`;   k, v [B, Nkv, Skv, D] in `layout`;
 *   out  [B, Nq,  Sq,  D] in `layout` (same dtype as q);
 *   softmax_max, softmax_sum: fp32 [B, Nq, Sq] contiguous, or NULL.
 *   dtype: MIATTN_BF16 or MIATTN_F16 (fp32 accumulation, the softmax weights rounded to
 *   the input type for the P V product, RNE output) or MIATTN_F32 (fp32 matrix-core
 *   products, softmax weights kept in fp32); all on the matrix cores.
 *   D: any of 1..768, the operator spec's range (aclnnFlashAttentionVarLenScore 约束说明),
 *   in every dtype; outside it -> MIATTN_ERR_SHAPE.  The tiled kernels serve 32, 64, 96
 *   and 128 (and 160, 192, 224, 256 in bf16 / fp16 without a mask tensor or dropout);
 *   every other head dim and combination runs on a head-dim-general MFMA kernel (the head
 *   dim split over the waves of a workgroup, partial scores summed in LDS), same results
 *   to rounding, slower.
 *   Ranges: B >= 1, 1 <= Nq, Nkv <= 256, 1 <= Sq, Skv <= 2^30 with B*Sq and
 *   B*Skv <= 2^31.  Shapes whose K / V row stride is too large for the tiled kernels'
 *   32-bit tile offsets (64 rows x stride x element size >= 2^31 bytes: the SBH layout
 *   with B*Nkv*D >= 2^24 in bf16 / fp16) run on the head-dim-general kernel, which indexes
 *   in 64 bits; attn_fwd_route reports the choice.
 *   scale: finite and > 0 (callers pass 1/sqrt(D)).
 *   Pass pre_tokens/next_tokens for the band modes; they are ignored otherwise.
 *   Returns MIATTN_OK or an error status; nothing is enqueued on error.
 */
miattn_status_t attn_fwd(const void* q, const void* k, const void* v, void* out,
                         float* softmax_max, float* softmax_sum,
                         int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                         miattn_dtype_t dtype, miattn_layout_t layout, float scale,
                         miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens,
                         void* stream);

/*
 * attn_fwd_varlen - attention forward over a packed batch of variable-length sequences.
 *
 * Defines: the TND packing and per-sequence computation of aclnnFlashAttentionVarLenScore
 * (功能说明 and 约束说明): all sequences are stacked along T with no padding; sequence b
 * owns query rows [cu_seqlens_q[b-1], cu_seqlens_q[b]) and key rows
 * [cu_seqlens_kv[b-1], cu_seqlens_kv[b]) (cu[-1] = 0: the vectors are END offsets with no
 * leading zero, so lengths [2,2,0,2,2] are passed as [2,4,4,6,8]); zero-length sequences
 * are allowed; mask positions are local to each sequence.
 *
 *   q   [Tq,  Nq,  D];  k, v [Tkv, Nkv, D];  out [Tq, Nq, D]   (row-major, dtype `dtype`);
 *   softmax_max, softmax_sum: fp32 [Nq, Tq] contiguous, or NULL;
 *   cu_seqlens_q, cu_seqlens_kv: DEVICE int64 [B], monotone, last = Tq / Tkv;
 *   max_seqlen_q, max_seqlen_kv: host upper bounds of the sequence lengths (the grid is
 *   sized from max_seqlen_q; rows of a longer sequence are NOT computed).
 *   Ranges: 1 <= B <= 2048, 1 <= Tq, Tkv <= 2^20, 1 <= Nq, Nkv <= 256, D as attn_fwd.
 *   dtype, scale, mask, pre/next: as for attn_fwd.
 */
miattn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v, void* out,
                                float* softmax_max, float* softmax_sum,
                                const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                                int64_t B, int64_t Tq, int64_t Tkv,
                                int64_t max_seqlen_q, int64_t max_seqlen_kv,
                                int64_t Nq, int64_t Nkv, int64_t D,
                                miattn_dtype_t dtype, float scale,
                                miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens,
                                void* stream);

/*
 * attn_lse_merge - merge two partial attention results of the same queries over disjoint
 * key sets into one (the ring-attention update of "npu_ring_attention_update对外接口",
 * equivalent small-operator logic): with m = max(prev_max, cur_max),
 *   a = prev_sum * exp(prev_max - m),  c = cur_sum * exp(cur_max - m),  l = a + c,
 *   out = prev_out * (a / l) + cur_out * (c / l),  out_max = m,  out_sum = l,
 * computed in fp32 and rounded (RNE) to the output dtype.  If both partials are empty
 * (m = -inf) the row becomes out = 0, out_max = -inf, out_sum = 0.
 *
 *   prev_out, cur_out, out: [B, N, S, D] in `layout`, dtype `dtype` (BF16, F16, F32);
 *   prev_max, prev_sum, cur_max, cur_sum, out_max, out_sum: fp32 [B, N, S] contiguous
 *   (a packed TND batch is B = 1, S = T with layout BSND; its stats are then [N, T]).
 *   out may alias prev_out or cur_out; out_max/out_sum may alias the matching input stats
 *   (the update is elementwise and each element is read before it is written by the same
 *   thread).  Any D >= 1; limits: N <= 256, B <= 65535, N * D <= 2^27, S <= 2^30,
 *   B * N * S * D <= 2^40 (else MIATTN_ERR_SHAPE).
 */
miattn_status_t attn_lse_merge(const void* prev_out, const float* prev_max, const float* prev_sum,
                               const void* cur_out, const float* cur_max, const float* cur_sum,
                               void* out, float* out_max, float* out_sum,
                               int64_t B, int64_t N, int64_t S, int64_t D,
                               miattn_dtype_t dtype, miattn_layout_t layout, void* stream);

/*
 * attn_fwd_update - attention of q over ONE chunk of keys, merged into a running result
 * in the same launch: the forward of attn_fwd followed by the ring-attention update of
 * attn_lse_merge ("npu_ring_attention_update对外接口"), with the chunk's partial result kept
 * in fp32 registers instead of being stored, re-read and rounded in between.  With
 * m_c, l_c, o_c the chunk's softmax max, sum and normalized output (attn_fwd's outputs):
 *   m = max(prev_max, m_c),  a = prev_sum * exp(prev_max - m),  c = l_c * exp(m_c - m),
 *   out = prev_out * a / (a + c) + o_c * c / (a + c),  out_max = m,  out_sum = a + c,
 * rounded once (RNE) to the dtype.  Calling it once per key chunk, with the chunk's band
 * offset in pre/next (e.g. causal over keys [j0, j0 + Skv): MIATTN_MASK_BAND with
 * pre_tokens = 2^40, next_tokens = -j0), accumulates attention over all the chunks.
 * A row that sees no key of this chunk keeps the prior bit for bit, given that a
 * non-empty prior row has prev_sum > 0 (as every attention output has); an empty prior
 * row (prev_max = -inf, prev_sum = 0) gives attn_fwd's result, and its prev_out is not
 * read (it may hold anything, e.g. an uninitialized buffer before the first chunk).
 *
 *   q, k, v, layout, sizes, dtype, scale, mask, pre/next: as for attn_fwd;
 *   prev_out, out: [B, Nq, Sq, D] in `layout`, dtype `dtype`;
 *   prev_max, prev_sum, out_max, out_sum: fp32 [B, Nq, Sq] contiguous (none may be NULL).
 *   out may alias prev_out and out_max / out_sum may alias prev_max / prev_sum (each
 *   element is read and then written by the same thread), which is the usual in-place
 *   accumulation.  Returns as attn_fwd (MIATTN_ERR_NULL for a NULL prior or statistics).
 */
miattn_status_t attn_fwd_update(const void* q, const void* k, const void* v,
                                const void* prev_out, const float* prev_max, const float* prev_sum,
                                void* out, float* out_max, float* out_sum,
                                int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                                miattn_dtype_t dtype, miattn_layout_t layout, float scale,
                                miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens,
                                void* stream);

/*
 * attn_fwd_varlen_update - attn_fwd_update over a packed (TND) batch: the key chunk of
 * sequence b is rows [cu_seqlens_kv[b-1], cu_seqlens_kv[b]) of k / v (a chunk packed
 * with its own cumulative lengths, as one ring step holds it); the running result is
 * [Tq, Nq, D] with statistics [Nq, Tq] (the TND form of the ring update, with
 * actual_seq_qlen given by cu_seqlens_q).  Arguments and limits as attn_fwd_varlen, plus
 * the prior and aliasing rules of attn_fwd_update.
 */
miattn_status_t attn_fwd_varlen_update(const void* q, const void* k, const void* v,
                                       const void* prev_out, const float* prev_max,
                                       const float* prev_sum, void* out, float* out_max,
                                       float* out_sum,
                                       const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                                       int64_t B, int64_t Tq, int64_t Tkv,
                                       int64_t max_seqlen_q, int64_t max_seqlen_kv,
                                       int64_t Nq, int64_t Nkv, int64_t D,
                                       miattn_dtype_t dtype, float scale,
                                       miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens,
                                       void* stream);

/*
 * attn_fwd_ext / attn_fwd_varlen_ext - attn_fwd / attn_fwd_varlen with the rest of
 * the mask surface and the value head dim of aclnnFlashAttentionVarLenScore, and dropout (约束说明: sparseMode, prefixOptional,
 * attenMaskOptional), under these readings (the page's mode definitions were not part of
 * the extracted text):
 *   prefix: DEVICE int64 [B] or NULL.  Keys j < prefix[b] are visible from every row of
 *     sequence b, in addition to the causal keys (sparseMode 6 is prefix + bottom-right
 *     causal: use mask MIATTN_MASK_CAUSAL_BR).  Only with MIATTN_MASK_CAUSAL or
 *     MIATTN_MASK_CAUSAL_BR (else MIATTN_ERR_MASK); values are clamped to [0, Skv].
 *   atten_mask: DEVICE uint8 [Sq, Skv] (dense) or [max_seqlen_q, max_seqlen_kv] (packed),
 *     row-major, or NULL.  A nonzero byte at (i, j) removes key j from query i (sequence-local
 *     positions, top-left), on top of the mask mode and the prefix; it is shared by all
 *     batch entries / sequences and heads.  The page forbids rows that are entirely masked;
 *     here such a row gives the empty result (out 0, max -inf, sum 0).
 *   bf16 / fp16 with atten_mask run on the tiled kernel like attn_fwd when the mask pointer
 *   is 4-byte aligned, its row length (Skv, resp. max_seqlen_kv) a multiple of 4 and its
 *   size under 2^31 bytes; otherwise on the head-dim-general kernel (byte reads of the
 *   mask), same results to rounding.  Other arguments, limits and errors as attn_fwd /
 *   attn_fwd_varlen.
 *   Dv: head dim of v and out (aclnnFlashAttentionVarLenScore 约束说明: qD == kD >= vD);
 *     v is [B, Nkv, Skv, Dv] / [Tkv, Nkv, Dv] and out [B, Nq, Sq, Dv] / [Tq, Nq, Dv] in the
 *     same layout.  Any 1 <= Dv <= D (else MIATTN_ERR_SHAPE).
 *   dropout_p, seed, offset: dropout on the probabilities (the dropout_p of the
 *     MultiHeadAttention page and the SDPA-pitfalls blog); the pages name no generator, so
 *     it is defined here: probability (i, j) of query head h in batch entry / sequence b is
 *     dropped when byte j % 4 of word (j % 16) / 4 of Philox4x32-10 (Salmon et al., SC 2011)
 *     with counter (j / 16, i, h + 256 b, offset) and key (seed & 0xffffffff, seed >> 32)
 *     is below thr = round(256 dropout_p); kept probabilities are scaled by 256 / (256 - thr)
 *     (so E[out] = attention without dropout).  i, j are sequence-local.  softmax_max /
 *     softmax_sum stay those of the undropped softmax.  dropout_p = 0 (thr 0) is no dropout;
 *     not finite, < 0, or thr = 256 -> MIATTN_ERR_DROPOUT; dropout with atten_mask or Dv < D
 *     -> MIATTN_ERR_UNSUPPORTED.
 */
miattn_status_t attn_fwd_ext(const void* q, const void* k, const void* v, void* out,
                                float* softmax_max, float* softmax_sum,
                                int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                                int64_t Dv, miattn_dtype_t dtype, miattn_layout_t layout, float scale,
                                miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens,
                                const int64_t* prefix, const uint8_t* atten_mask,
                                float dropout_p, uint64_t seed, uint32_t offset, void* stream);

miattn_status_t attn_fwd_varlen_ext(const void* q, const void* k, const void* v, void* out,
                                       float* softmax_max, float* softmax_sum,
                                       const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                                       int64_t B, int64_t Tq, int64_t Tkv,
                                       int64_t max_seqlen_q, int64_t max_seqlen_kv,
                                       int64_t Nq, int64_t Nkv, int64_t D, int64_t Dv,
                                       miattn_dtype_t dtype, float scale,
                                       miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens,
                                       const int64_t* prefix, const uint8_t* atten_mask,
                                       float dropout_p, uint64_t seed, uint32_t offset,
                                       void* stream);

/*
 * attn_fwd_route - which kernel a dense forward with these arguments runs on, without any
 * HIP call (a query for callers and tests of the routing that attn_fwd_ext and
 * attn_fwd_update apply; the routing is a property of this implementation, not of the
 * pages).  Arguments as attn_fwd_ext; update != 0 asks about attn_fwd_update; atten_mask
 * is only inspected for its alignment, never read.
 *   Returns MIATTN_KERNEL_TILED, MIATTN_KERNEL_PERSISTENT or MIATTN_KERNEL_GENERAL, or
 *   minus the status the forward would return for these arguments (e.g. -MIATTN_ERR_SHAPE).
 *   The environment variable MIATTN_PERSIST=0 turns the persistent route off (the tiled
 *   kernel then serves those calls, with identical results).
 */
int32_t attn_fwd_route(int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                       int64_t Dv, miattn_dtype_t dtype, miattn_layout_t layout,
                       miattn_mask_t mask, const uint8_t* atten_mask, float dropout_p,
                       int32_t update);

/*
 * sparse_csr_attn - CSR-sparse attention (Paddle "sparse_attention": formula, parameters
 * and code example): row i of slice (b, n) attends only to the key rows listed in
 * csr_columns[b][n][csr_offset[b][n][i] .. csr_offset[b][n][i+1]) of the same slice,
 * softmax(scale * q_i . k_c) over those entries, times v_c.  `csr_offset` is a row pointer
 * (offset[0] = 0, offset[S] = entries used).  Every stored entry counts once (a repeated
 * column counts as often as it is stored); an empty row gives 0.
 *
 *   q, k, v, out: fp32 or fp64 [B, N, S, D] (BNSD) contiguous (all arithmetic in that type;
 *   the fp64 path uses `scale` widened to double);
 *   csr_offset: DEVICE int32 [B, N, S+1];  csr_columns: DEVICE int32 [B, N, nnz];
 *   dtype: MIATTN_F32 or MIATTN_F64 (bf16/fp16 -> UNSUPPORTED).  Any head dim 1 <= D <= 768
 *   (the page bounds none; 768 is the dense entry points' limit); D > 768 -> SHAPE.
 *   nnz >= 0.  Entries whose column lies among the keys just before a block of 64 rows
 *   are read from a copy in LDS, the rest gathered from global memory: a banded pattern
 *   runs fastest, any pattern runs.
 */
miattn_status_t sparse_csr_attn(const void* q, const void* k, const void* v, void* out,
                                const int32_t* csr_offset, const int32_t* csr_columns,
                                int64_t nnz, int64_t B, int64_t N, int64_t S, int64_t D,
                                miattn_dtype_t dtype, float scale, void* stream);

/*
 * sparse_csr_window - how many keys sparse_csr_attn serves from LDS: rows are taken in
 * blocks of 64 ([64 j, 64 j + 64) of each slice, the last one ragged), and an entry of a row
 * in a block that ends at row r1 (exclusive) is read from the LDS copy when its column lies
 * in [max(0, r1 - W), r1), W the value returned; every other entry is gathered from global
 * memory.  For 16-byte aligned Q, K, V and out (the value may differ for unaligned ones).
 * A property of this implementation (for measurement), not of the Paddle page.
 *   Returns W >= 1, or minus the status sparse_csr_attn would return for this D and dtype.
 */
int32_t sparse_csr_window(int64_t D, miattn_dtype_t dtype);

/*
 * mha_self_attn_fwd - forward of the multi-head self-attention module of the page "flash
 * attention的调用" (its MultiHeadAttention example): a fused QKV projection, scaled dot-product
 * attention per head with scale 1/sqrt(D), no causal mask, optional attention mask and
 * dropout on the probabilities, and the output projection:
 *     [q | k | v] = x W_qkv^T + b_qkv          (the 3E outputs split into thirds)
 *     o_h         = attention(q_h, k_h, v_h)   (heads h = 0..N-1 of D = E/N columns each)
 *     out         = [o_0 .. o_{N-1}] W_out^T + b_out
 * The projections are rocBLAS GEMMs (fp32 accumulation, one rounding to the storage type:
 * the output buffer is first filled with the broadcast bias and the GEMM runs with
 * beta = 1); the attention is attn_fwd_ext on the BSND views of q, k, v.
 *
 *   x: DEVICE [B, S, E] contiguous;  out: DEVICE [B, S, E] contiguous (must not alias x);
 *   w_qkv: DEVICE [3E, E] row-major (out_features x in_features, as a linear layer stores
 *   it);  b_qkv: DEVICE [3E] or NULL (no bias);  w_out: DEVICE [E, E];  b_out: DEVICE [E] or
 *   NULL.  All of the storage type `dtype`: MIATTN_BF16, MIATTN_F16 or MIATTN_F32.
 *   workspace: DEVICE scratch of at least mha_workspace_bytes(B, S, E, dtype) bytes (q, k, v
 *   and the attention output), owned by the caller; its contents are overwritten.
 *   N divides E with D = E / N <= 768; rows of E elements are whole 16-byte vectors (E a
 *   multiple of 8 for bf16 / fp16, of 4 for fp32); 1 <= N <= 256; B * S <= 2^31 - 1.
 *   atten_mask: DEVICE uint8 [S, S] or NULL, nonzero = the pair is masked out (the
 *   convention of attn_fwd_ext), with the same alignment rules as there.
 *   dropout_p, seed, offset: as attn_fwd_ext (dropout is not combined with atten_mask).
 * Errors are reported before any work is enqueued, except MIATTN_ERR_BLAS / _LAUNCH.  The
 * first call on a device creates that device's rocBLAS handle (kept until the process ends).
 */
int64_t mha_workspace_bytes(int64_t B, int64_t S, int64_t E, miattn_dtype_t dtype);

miattn_status_t mha_self_attn_fwd(const void* x, const void* w_qkv, const void* b_qkv,
                                  const void* w_out, const void* b_out, void* out,
                                  void* workspace, int64_t workspace_bytes,
                                  int64_t B, int64_t S, int64_t E, int64_t N,
                                  miattn_dtype_t dtype, const uint8_t* atten_mask,
                                  float dropout_p, uint64_t seed, uint32_t offset, void* stream);

/*
 * mha_self_attn_fwd_noalloc - mha_self_attn_fwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same module and arguments without the workspace; it allocates nothing:
 *   - q, k, v and the attention output live in a static device array of
 *     MIATTN_MHA_SCRATCH_BYTES that each GPU the library runs on holds until the process
 *     ends (the first call on a device only looks up that device's copy);
 *   - the projections run on this library's own GEMM kernel (fp32 accumulation, the bias
 *     added in fp32 before the one rounding to the storage type), not rocBLAS, so outputs
 *     can differ from mha_self_attn_fwd's by the rounding of a different summation order.
 * Limit: mha_workspace_bytes(B, S, E, dtype) <= MIATTN_MHA_SCRATCH_BYTES, else
 * MIATTN_ERR_SCRATCH (bf16: B * S * E <= 8 Mi elements).  x, w_qkv, w_out and out must be
 * 16-byte aligned.  Other arguments, limits and errors as mha_self_attn_fwd; errors are
 * reported before any work is enqueued, except MIATTN_ERR_LAUNCH.
 * Every call on one GPU uses that GPU's one array, so calls that overlap on a GPU (on
 * different streams, or from different threads) race and must be serialized by the
 * caller; nothing in the array needs to start at zero (each call overwrites what it reads).
 */
#define MIATTN_MHA_SCRATCH_BYTES (64ll << 20)

miattn_status_t mha_self_attn_fwd_noalloc(const void* x, const void* w_qkv, const void* b_qkv,
                                          const void* w_out, const void* b_out, void* out,
                                          int64_t B, int64_t S, int64_t E, int64_t N,
                                          miattn_dtype_t dtype, const uint8_t* atten_mask,
                                          float dropout_p, uint64_t seed, uint32_t offset,
                                          void* stream);

/* Static, human-readable name of a status code. */
const char* miattn_status_str(miattn_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
