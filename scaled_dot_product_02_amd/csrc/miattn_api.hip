// C ABI of the attention-forward library: argument validation, layout strides, grid
// sizing and launches on the caller's stream.  Declared in include/miattn.h.
#include <math.h>
#include <stdlib.h>

#include <atomic>

#include "miattn.h"
#include "fa_params.h"

using namespace miattn;

namespace {

constexpr int64_t kTokensClamp = int64_t(1) << 40;  // |pre|, |next| beyond this change nothing
// Longest dense sequence: positions, tile bounds and key indices are 32-bit in the kernels
constexpr int64_t kMaxLen = int64_t(1) << 30;

struct Strides { int64_t sb, ss, sh; };

bool layout_ok(int layout) { return layout >= MIATTN_BNSD && layout <= MIATTN_SBH; }

Strides strides_of(int layout, int64_t B, int64_t N, int64_t S, int64_t D)
{
    switch (layout) {
    case MIATTN_BNSD: return {N * S * D, D, S * D};
    case MIATTN_BSND:
    case MIATTN_BSH: return {S * N * D, N * D, D};
    default: /* SBH */ return {N * D, B * N * D, D};
    }
}

// Band of a mask mode; the bottom-right modes shift it per sequence (FaParams::align_br).
miattn_status_t check_mask(int mask, int64_t pre, int64_t next, FaParams& p)
{
    auto clamp = [](int64_t x) { return x > kTokensClamp ? kTokensClamp : (x < -kTokensClamp ? -kTokensClamp : x); };
    int64_t& pre_c = p.pre;
    int64_t& next_c = p.next;
    p.align_br = mask == MIATTN_MASK_CAUSAL_BR || mask == MIATTN_MASK_BAND_BR;
    if (mask == MIATTN_MASK_NONE) {
        pre_c = next_c = kTokensClamp;
    } else if (mask == MIATTN_MASK_CAUSAL || mask == MIATTN_MASK_CAUSAL_BR) {
        pre_c = kTokensClamp;
        next_c = 0;
    } else if (mask == MIATTN_MASK_BAND || mask == MIATTN_MASK_BAND_BR) {
        // the band must be non-empty: pre + next >= 0 (evaluated without overflow)
        if ((__int128)pre + (__int128)next < 0) return MIATTN_ERR_MASK;
        pre_c = clamp(pre);
        next_c = clamp(next);
    } else {
        return MIATTN_ERR_MASK;
    }
    return MIATTN_OK;
}

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

// head dims of the tiled kernels in every dtype (the sparse kernel: these only)
bool head_dim_built(int64_t D) { return D == 32 || D == 64 || D == 96 || D == 128; }

// larger head dims of the tiled MFMA kernel: bf16 / fp16, V head dim equal, no mask tensor
// and no dropout
bool big_head_dim(int64_t D) { return D == 160 || D == 192 || D == 224 || D == 256; }

// Whether the tiled MFMA kernel serves this forward (bf16 / fp16); every other valid one,
// fp32 included, runs on the head-dim-general kernel.
bool tiled_forward(int64_t D, int64_t Dv, int dtype, bool update, bool amask, bool drop)
{
    if (dtype != MIATTN_BF16 && dtype != MIATTN_F16) return false;
    if (head_dim_built(D)) {
        if (Dv == D) return true;
        const bool pair = (D == 64 && Dv == 32) || (D == 96 && Dv == 64) || (D == 128 && Dv == 64) ||
                          (D == 128 && Dv == 96);
        return pair && !update && !amask && !drop;
    }
    return big_head_dim(D) && Dv == D && !amask && !drop;
}

// Dropout probability p -> byte threshold round(256 p) and the scale of kept probabilities;
// p must be finite in [0, 1) with threshold < 256.  Threshold 0 is no dropout.
miattn_status_t set_dropout(FaParams& p, float prob, uint64_t seed, uint32_t offset)
{
    if (!(prob >= 0.f && prob < 1.f)) return MIATTN_ERR_DROPOUT;
    const int thr = (int)lrintf(prob * 256.f);
    if (thr >= 256) return MIATTN_ERR_DROPOUT;
    p.drop_thr = (uint32_t)thr;
    p.drop_scale = 256.f / (float)(256 - thr);
    p.seed_lo = (uint32_t)seed;
    p.seed_hi = (uint32_t)(seed >> 32);
    p.drop_offset = offset;
    return MIATTN_OK;
}

// V head dim: 1..D (the varlen operator: kD >= vD); D itself is checked against 1..768
miattn_status_t check_head_dims(int64_t D, int64_t Dv)
{
    return Dv < 1 || Dv > D ? MIATTN_ERR_SHAPE : MIATTN_OK;
}

miattn_status_t check_dtype_fa(int dtype)
{
    if (dtype == MIATTN_F32 || dtype == MIATTN_BF16 || dtype == MIATTN_F16) return MIATTN_OK;
    return MIATTN_ERR_DTYPE;
}

// Grid of the attention kernels: levels x batch x kv heads groups, padded to a
// multiple of 8 groups, times the GQA group size.
miattn_status_t size_grid(FaParams& p, int64_t max_len_q, int tile_m)
{
    const int64_t levels = (max_len_q + tile_m - 1) / tile_m;
    const int64_t groups = levels * p.B * p.Nkv;
    const int64_t slots = ((groups + 7) / 8) * 8 * p.group;
    if (slots >= (int64_t(1) << 31)) return MIATTN_ERR_UNSUPPORTED;
    p.n_levels = (int32_t)levels;
    p.n_slots = (int32_t)slots;
    return MIATTN_OK;
}

// Whether a validated forward runs on the tiled MFMA kernel (else the general one).
bool use_tiled(const FaParams& p, int dtype, int64_t D)
{
    // an explicit mask stays on the tiled kernel when its rows are 4-byte aligned words
    // (read as 32-bit buffer loads with 32-bit offsets); otherwise it takes the general one
    const bool mask_words = !p.amask || ((uintptr_t)p.amask % 4 == 0 && p.amask_ld % 4 == 0 &&
                                         (int64_t)p.Sq * p.amask_ld < (int64_t(1) << 31));
    // the tiled kernel addresses a key tile through a buffer descriptor whose byte range
    // (64 rows of K or V) and per-lane offsets are 32-bit; larger row strides (the SBH
    // layout with B * Nkv * D >= 2^24 elements) take the general kernel, which indexes in
    // 64 bits
    const int64_t esz = dtype == MIATTN_F32 ? 4 : 2;
    const bool tile_fits = 64 * esz * (p.k_ss > p.v_ss ? p.k_ss : p.v_ss) < (int64_t(1) << 31);
    return mask_words && tile_fits &&
           tiled_forward(D, p.Dv, dtype, p.prev_out != nullptr, p.amask != nullptr, p.drop_thr != 0);
}

// Compute units of the current device (the persistent kernel runs one workgroup per CU),
// queried once per device.
int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        return 0;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// MIATTN_PERSIST=0 in the environment turns the persistent kernel off (the tiled kernel
// then takes its forwards), for comparisons; read at every call.
bool persist_enabled()
{
    const char* e = getenv("MIATTN_PERSIST");
    return !(e && e[0] == '0' && e[1] == 0);
}

// Whether a forward that the tiled kernel would serve runs on the persistent one: causal
// (either alignment, with or without a prefix or dropout) without a mask tensor or prior,
// head dim 64 or 128 with V of the same head dim, packed batches of at most
// kPersistMaxSeq sequences.
bool use_persistent(const FaParams& p, int64_t D, int64_t Tq, int n_wg)
{
    if (D != 64 && D != 128) return false;
    if (p.Dv != D || p.prev_out || p.amask) return false;
    // every row's visible keys start at key 0 (no mask, causal with or without a prefix,
    // or a band with no lower bound): the kernel moves the causal diagonal by the band's
    // upper bound and extends each row's keys to the prefix
    if (p.pre != kTokensClamp) return false;
    if (p.cu_q && p.B > kPersistMaxSeq) return false;
    // items: sum over sequences of their query tiles, times the head groups; packed
    // batches have at most Tq / rows + B tiles.  Each workgroup lists its items in LDS.
    const int64_t hpi = fa_persist_heads_per_item(p.group);
    const int64_t rows = 256 / hpi;
    const int64_t tiles = p.cu_q ? (Tq + rows - 1) / rows + p.B : p.B * ((p.Sq + rows - 1) / rows);
    const int64_t items = tiles * (p.Nq / hpi);
    if (n_wg < 1 || items >= (int64_t(1) << 30) || (items + n_wg - 1) / n_wg > fa_persist_max_items((int)D, p.drop_thr != 0))
        return false;
    return persist_enabled();
}

miattn_status_t launch_fa(FaParams& p, int dtype, int64_t D, hipStream_t stream, int64_t max_len_q)
{
    const bool tiled = use_tiled(p, dtype, D);
    const int n = tiled ? cu_count() : 0;
    if (tiled && use_persistent(p, D, p.cu_q ? p.st_sh : 0, n)) {
        p.persist_hpi = fa_persist_heads_per_item(p.group);
        p.n_slots = n;
        return launch_fa_fwd_persist(p, (int)D, dtype == MIATTN_F16, stream) == hipSuccess
                   ? MIATTN_OK : MIATTN_ERR_LAUNCH;
    }
    const int tile_m = !tiled ? fa_wide_tile_m(dtype)
                     : fa_four_waves((int)D, p.amask != nullptr || p.drop_thr != 0) ? kBf16TileMBig : kBf16TileM;
    miattn_status_t st = size_grid(p, max_len_q, tile_m);
    if (st != MIATTN_OK) return st;
    hipError_t e = tiled ? launch_fa_fwd_bf16(p, (int)D, dtype == MIATTN_F16, stream)
                         : launch_fa_fwd_wide(p, (int)D, dtype, stream);
    return e == hipSuccess ? MIATTN_OK : MIATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

const char* miattn_status_str(miattn_status_t s)
{
    switch (s) {
    case MIATTN_OK: return "ok";
    case MIATTN_ERR_NULL: return "a required pointer is null";
    case MIATTN_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MIATTN_ERR_DTYPE: return "unknown or unsupported dtype for this entry point";
    case MIATTN_ERR_LAYOUT: return "unknown layout";
    case MIATTN_ERR_GQA_RATIO: return "Nq must be a non-zero integer multiple of Nkv";
    case MIATTN_ERR_MASK: return "unknown mask or empty band (pre_tokens + next_tokens < 0)";
    case MIATTN_ERR_UNSUPPORTED: return "valid but not built (head_dim, dtype or grid size)";
    case MIATTN_ERR_LAUNCH: return "kernel launch failed";
    case MIATTN_ERR_SCALE: return "scale must be finite and positive";
    case MIATTN_ERR_DROPOUT: return "dropout_p must be in [0, 1) with round(256 p) < 256";
    case MIATTN_ERR_BLAS: return "a rocBLAS call failed";
    case MIATTN_ERR_WORKSPACE: return "workspace missing or smaller than mha_workspace_bytes()";
    case MIATTN_ERR_SCRATCH: return "problem larger than the static scratch of the no-allocation entry point";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

// Validation and launch parameters of a dense forward (no HIP call); with prev_out set,
// the partial result is merged into the prior.
miattn_status_t prepare_dense(FaParams& p, const void* q, const void* k, const void* v,
                              const void* prev_out, const float* prev_max, const float* prev_sum,
                              void* out, float* softmax_max, float* softmax_sum,
                              int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv,
                              int64_t D, int64_t Dv, int dtype, int layout, float scale,
                              int mask, int64_t pre_tokens, int64_t next_tokens,
                              const int64_t* prefix, const uint8_t* atten_mask,
                              float dropout_p, uint64_t seed, uint32_t offset)
{
    if (!q || !k || !v || !out) return MIATTN_ERR_NULL;
    miattn_status_t st = check_dtype_fa(dtype);
    if (st == MIATTN_ERR_DTYPE) return st;
    if (!layout_ok(layout)) return MIATTN_ERR_LAYOUT;
    if (B < 1 || Nq < 1 || Nkv < 1 || Sq < 1 || Skv < 1 || D < 1) return MIATTN_ERR_SHAPE;
    if (Nq > 256 || Nkv > 256 || D > 768) return MIATTN_ERR_SHAPE;
    if (Sq > kMaxLen || Skv > kMaxLen) return MIATTN_ERR_SHAPE;
    if (B * Sq > (int64_t(1) << 31) || B * Skv > (int64_t(1) << 31)) return MIATTN_ERR_SHAPE;
    if (Nq % Nkv != 0) return MIATTN_ERR_GQA_RATIO;
    p = FaParams{};
    st = check_mask(mask, pre_tokens, next_tokens, p);
    if (st != MIATTN_OK) return st;
    if (prefix && mask != MIATTN_MASK_CAUSAL && mask != MIATTN_MASK_CAUSAL_BR)
        return MIATTN_ERR_MASK;   // a prefix goes with the causal modes only
    if (!scale_ok(scale)) return MIATTN_ERR_SCALE;
    st = check_head_dims(D, Dv);
    if (st != MIATTN_OK) return st;
    p.Dv = (int32_t)Dv;
    st = set_dropout(p, dropout_p, seed, offset);
    if (st != MIATTN_OK) return st;
    p.prefix = prefix;
    p.amask = atten_mask;
    p.amask_ld = Skv;
    if (p.drop_thr && (prev_out || atten_mask || Dv != D)) return MIATTN_ERR_UNSUPPORTED;

    const Strides sq = strides_of(layout, B, Nq, Sq, D), skv = strides_of(layout, B, Nkv, Skv, D);
    const Strides so = strides_of(layout, B, Nq, Sq, Dv), sv = strides_of(layout, B, Nkv, Skv, Dv);
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.smax = softmax_max; p.ssum = softmax_sum;
    p.prev_out = prev_out; p.prev_max = prev_max; p.prev_sum = prev_sum;
    p.cu_q = p.cu_kv = nullptr;
    p.q_sb = sq.sb; p.q_ss = sq.ss; p.q_sh = sq.sh;
    p.o_sb = so.sb; p.o_ss = so.ss; p.o_sh = so.sh;
    p.k_sb = skv.sb; p.k_ss = skv.ss; p.k_sh = skv.sh;
    p.v_sb = sv.sb; p.v_ss = sv.ss; p.v_sh = sv.sh;
    p.st_sb = Nq * Sq; p.st_sh = Sq;
    p.B = (int32_t)B; p.Nq = (int32_t)Nq; p.Nkv = (int32_t)Nkv; p.group = (int32_t)(Nq / Nkv);
    p.Sq = (int32_t)Sq; p.Skv = (int32_t)Skv;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    return MIATTN_OK;
}

miattn_status_t fwd_dense(const void* q, const void* k, const void* v,
                          const void* prev_out, const float* prev_max, const float* prev_sum,
                          void* out, float* softmax_max, float* softmax_sum,
                          int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                          int64_t Dv, int dtype, int layout, float scale,
                          int mask, int64_t pre_tokens, int64_t next_tokens,
                          const int64_t* prefix, const uint8_t* atten_mask,
                          float dropout_p, uint64_t seed, uint32_t offset, void* stream)
{
    FaParams p;
    const miattn_status_t st = prepare_dense(p, q, k, v, prev_out, prev_max, prev_sum, out,
                                             softmax_max, softmax_sum, B, Nq, Nkv, Sq, Skv, D, Dv,
                                             dtype, layout, scale, mask, pre_tokens, next_tokens,
                                             prefix, atten_mask, dropout_p, seed, offset);
    if (st != MIATTN_OK) return st;
    return launch_fa(p, dtype, D, (hipStream_t)stream, Sq);
}

// Packed (TND) forward; with prev_out set, the partial result is merged into the prior.
miattn_status_t fwd_varlen(const void* q, const void* k, const void* v,
                           const void* prev_out, const float* prev_max, const float* prev_sum,
                           void* out, float* softmax_max, float* softmax_sum,
                           const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                           int64_t B, int64_t Tq, int64_t Tkv,
                           int64_t max_seqlen_q, int64_t max_seqlen_kv,
                           int64_t Nq, int64_t Nkv, int64_t D, int64_t Dv,
                           int dtype, float scale,
                           int mask, int64_t pre_tokens, int64_t next_tokens,
                           const int64_t* prefix, const uint8_t* atten_mask,
                          float dropout_p, uint64_t seed, uint32_t offset, void* stream)
{
    if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_kv) return MIATTN_ERR_NULL;
    miattn_status_t st = check_dtype_fa(dtype);
    if (st == MIATTN_ERR_DTYPE) return st;
    if (B < 1 || B > 2048) return MIATTN_ERR_SHAPE;
    if (Tq < 1 || Tkv < 1 || Tq > (int64_t(1) << 20) || Tkv > (int64_t(1) << 20)) return MIATTN_ERR_SHAPE;
    if (max_seqlen_q < 1 || max_seqlen_q > Tq || max_seqlen_kv < 1 || max_seqlen_kv > Tkv)
        return MIATTN_ERR_SHAPE;
    if (Nq < 1 || Nkv < 1 || Nq > 256 || Nkv > 256 || D < 1 || D > 768) return MIATTN_ERR_SHAPE;
    if (Nq % Nkv != 0) return MIATTN_ERR_GQA_RATIO;
    FaParams p{};
    st = check_mask(mask, pre_tokens, next_tokens, p);
    if (st != MIATTN_OK) return st;
    if (prefix && mask != MIATTN_MASK_CAUSAL && mask != MIATTN_MASK_CAUSAL_BR)
        return MIATTN_ERR_MASK;   // a prefix goes with the causal modes only
    if (!scale_ok(scale)) return MIATTN_ERR_SCALE;
    st = check_head_dims(D, Dv);
    if (st != MIATTN_OK) return st;
    p.Dv = (int32_t)Dv;
    st = set_dropout(p, dropout_p, seed, offset);
    if (st != MIATTN_OK) return st;
    p.prefix = prefix;
    p.amask = atten_mask;
    p.amask_ld = max_seqlen_kv;
    if (p.drop_thr && (prev_out || atten_mask || Dv != D)) return MIATTN_ERR_UNSUPPORTED;

    p.q = q; p.k = k; p.v = v; p.out = out;
    p.smax = softmax_max; p.ssum = softmax_sum;
    p.prev_out = prev_out; p.prev_max = prev_max; p.prev_sum = prev_sum;
    p.cu_q = cu_seqlens_q; p.cu_kv = cu_seqlens_kv;
    p.q_sb = 0; p.q_ss = Nq * D; p.q_sh = D;
    p.o_sb = 0; p.o_ss = Nq * Dv; p.o_sh = Dv;
    p.k_sb = 0; p.k_ss = Nkv * D; p.k_sh = D;
    p.v_sb = 0; p.v_ss = Nkv * Dv; p.v_sh = Dv;
    p.st_sb = 0; p.st_sh = Tq;
    p.B = (int32_t)B; p.Nq = (int32_t)Nq; p.Nkv = (int32_t)Nkv; p.group = (int32_t)(Nq / Nkv);
    p.Sq = (int32_t)max_seqlen_q; p.Skv = (int32_t)max_seqlen_kv;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    return launch_fa(p, dtype, D, (hipStream_t)stream, max_seqlen_q);
}

}  // namespace

extern "C" {

miattn_status_t attn_fwd(const void* q, const void* k, const void* v, void* out,
                         float* softmax_max, float* softmax_sum,
                         int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                         miattn_dtype_t dtype, miattn_layout_t layout, float scale,
                         miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens, void* stream)
{
    return fwd_dense(q, k, v, nullptr, nullptr, nullptr, out, softmax_max, softmax_sum, B, Nq, Nkv,
                     Sq, Skv, D, D, dtype, layout, scale, mask, pre_tokens, next_tokens, nullptr,
                     nullptr, 0.f, 0, 0, stream);
}

miattn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v, void* out,
                                float* softmax_max, float* softmax_sum,
                                const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                                int64_t B, int64_t Tq, int64_t Tkv,
                                int64_t max_seqlen_q, int64_t max_seqlen_kv,
                                int64_t Nq, int64_t Nkv, int64_t D,
                                miattn_dtype_t dtype, float scale,
                                miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens, void* stream)
{
    return fwd_varlen(q, k, v, nullptr, nullptr, nullptr, out, softmax_max, softmax_sum,
                      cu_seqlens_q, cu_seqlens_kv, B, Tq, Tkv, max_seqlen_q, max_seqlen_kv, Nq, Nkv,
                      D, D, dtype, scale, mask, pre_tokens, next_tokens, nullptr, nullptr, 0.f, 0,
                      0, stream);
}

miattn_status_t attn_fwd_update(const void* q, const void* k, const void* v,
                                const void* prev_out, const float* prev_max, const float* prev_sum,
                                void* out, float* out_max, float* out_sum,
                                int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                                miattn_dtype_t dtype, miattn_layout_t layout, float scale,
                                miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens, void* stream)
{
    if (!prev_out || !prev_max || !prev_sum || !out_max || !out_sum) return MIATTN_ERR_NULL;
    return fwd_dense(q, k, v, prev_out, prev_max, prev_sum, out, out_max, out_sum, B, Nq, Nkv,
                     Sq, Skv, D, D, dtype, layout, scale, mask, pre_tokens, next_tokens, nullptr,
                     nullptr, 0.f, 0, 0, stream);
}

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
                                       void* stream)
{
    if (!prev_out || !prev_max || !prev_sum || !out_max || !out_sum) return MIATTN_ERR_NULL;
    return fwd_varlen(q, k, v, prev_out, prev_max, prev_sum, out, out_max, out_sum,
                      cu_seqlens_q, cu_seqlens_kv, B, Tq, Tkv, max_seqlen_q, max_seqlen_kv, Nq, Nkv,
                      D, D, dtype, scale, mask, pre_tokens, next_tokens, nullptr, nullptr, 0.f, 0,
                      0, stream);
}

miattn_status_t attn_fwd_ext(const void* q, const void* k, const void* v, void* out,
                                float* softmax_max, float* softmax_sum,
                                int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                                int64_t Dv, miattn_dtype_t dtype, miattn_layout_t layout, float scale,
                                miattn_mask_t mask, int64_t pre_tokens, int64_t next_tokens,
                                const int64_t* prefix, const uint8_t* atten_mask,
                                float dropout_p, uint64_t seed, uint32_t offset, void* stream)
{
    return fwd_dense(q, k, v, nullptr, nullptr, nullptr, out, softmax_max, softmax_sum, B, Nq, Nkv,
                     Sq, Skv, D, Dv, dtype, layout, scale, mask, pre_tokens, next_tokens, prefix,
                     atten_mask, dropout_p, seed, offset, stream);
}

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
                                       void* stream)
{
    return fwd_varlen(q, k, v, nullptr, nullptr, nullptr, out, softmax_max, softmax_sum,
                      cu_seqlens_q, cu_seqlens_kv, B, Tq, Tkv, max_seqlen_q, max_seqlen_kv, Nq, Nkv,
                      D, Dv, dtype, scale, mask, pre_tokens, next_tokens, prefix, atten_mask,
                      dropout_p, seed, offset, stream);
}

int32_t attn_fwd_route(int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                       int64_t Dv, miattn_dtype_t dtype, miattn_layout_t layout,
                       miattn_mask_t mask, const uint8_t* atten_mask, float dropout_p,
                       int32_t update)
{
    // the same validation and routing as attn_fwd_ext / attn_fwd_update; the data pointers
    // are stand-ins that are never dereferenced
    char dummy[16];
    float* fs = (float*)dummy;
    FaParams p;
    const miattn_status_t st = prepare_dense(
        p, dummy, dummy, dummy, update ? dummy : nullptr, update ? fs : nullptr,
        update ? fs : nullptr, dummy, fs, fs, B, Nq, Nkv, Sq, Skv, D, Dv, dtype, layout, 1.f,
        mask, 0, 0, nullptr, atten_mask, dropout_p, 0, 0);
    if (st != MIATTN_OK) return -(int32_t)st;
    if (!use_tiled(p, dtype, D)) return MIATTN_KERNEL_GENERAL;
    // the routing is decided for a device of 256 compute units (this query makes no HIP call)
    return use_persistent(p, D, 0, 256) ? MIATTN_KERNEL_PERSISTENT : MIATTN_KERNEL_TILED;
}

miattn_status_t attn_lse_merge(const void* prev_out, const float* prev_max, const float* prev_sum,
                               const void* cur_out, const float* cur_max, const float* cur_sum,
                               void* out, float* out_max, float* out_sum,
                               int64_t B, int64_t N, int64_t S, int64_t D,
                               miattn_dtype_t dtype, miattn_layout_t layout, void* stream)
{
    if (!prev_out || !prev_max || !prev_sum || !cur_out || !cur_max || !cur_sum || !out ||
        !out_max || !out_sum)
        return MIATTN_ERR_NULL;
    if (dtype != MIATTN_F32 && dtype != MIATTN_BF16 && dtype != MIATTN_F16) return MIATTN_ERR_DTYPE;
    if (!layout_ok(layout)) return MIATTN_ERR_LAYOUT;
    if (B < 1 || N < 1 || S < 1 || D < 1 || N > 256 || B > 65535) return MIATTN_ERR_SHAPE;
    if (B * N * S * D > (int64_t(1) << 40) || S > (int64_t(1) << 30) || N * D > (int64_t(1) << 27))
        return MIATTN_ERR_SHAPE;
    const Strides s = strides_of(layout, B, N, S, D);
    MergeParams p{};
    p.o1 = prev_out; p.m1 = prev_max; p.l1 = prev_sum;
    p.o2 = cur_out; p.m2 = cur_max; p.l2 = cur_sum;
    p.out = out; p.mo = out_max; p.lo = out_sum;
    p.sb = s.sb; p.ss = s.ss; p.sh = s.sh;
    p.B = (int32_t)B; p.N = (int32_t)N; p.S = (int32_t)S; p.D = (int32_t)D;
    return launch_lse_merge(p, dtype, (hipStream_t)stream) == hipSuccess ? MIATTN_OK : MIATTN_ERR_LAUNCH;
}

int32_t sparse_csr_window(int64_t D, miattn_dtype_t dtype)
{
    if (dtype != MIATTN_F32 && dtype != MIATTN_F64)
        return -(int32_t)((dtype == MIATTN_BF16 || dtype == MIATTN_F16) ? MIATTN_ERR_UNSUPPORTED
                                                                        : MIATTN_ERR_DTYPE);
    if (D < 1 || D > 768) return -(int32_t)MIATTN_ERR_SHAPE;
    if (!sparse_head_dim_fits((int)D, dtype == MIATTN_F64)) return -(int32_t)MIATTN_ERR_UNSUPPORTED;
    return sparse_window_keys((int)D, dtype == MIATTN_F64, true);
}

miattn_status_t sparse_csr_attn(const void* q, const void* k, const void* v, void* out,
                                const int32_t* csr_offset, const int32_t* csr_columns,
                                int64_t nnz, int64_t B, int64_t N, int64_t S, int64_t D,
                                miattn_dtype_t dtype, float scale, void* stream)
{
    if (!q || !k || !v || !out || !csr_offset) return MIATTN_ERR_NULL;
    if (nnz > 0 && !csr_columns) return MIATTN_ERR_NULL;
    if (dtype != MIATTN_F32 && dtype != MIATTN_F64)
        return (dtype == MIATTN_BF16 || dtype == MIATTN_F16) ? MIATTN_ERR_UNSUPPORTED : MIATTN_ERR_DTYPE;
    if (B < 1 || N < 1 || S < 1 || D < 1 || nnz < 0 || D > 768) return MIATTN_ERR_SHAPE;
    if (S >= (int64_t(1) << 31) - 1 || nnz >= (int64_t(1) << 31) || B * N * S >= (int64_t(1) << 33))
        return MIATTN_ERR_SHAPE;
    if (!scale_ok(scale)) return MIATTN_ERR_SCALE;
    if (!sparse_head_dim_fits((int)D, dtype == MIATTN_F64)) return MIATTN_ERR_UNSUPPORTED;
    SparseParams p{};
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.offset = csr_offset; p.columns = csr_columns; p.nnz = nnz;
    p.B = (int32_t)B; p.N = (int32_t)N; p.S = (int32_t)S; p.D = (int32_t)D;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.scale_log2_d = (double)scale * 1.4426950408889634074;
    // vector reads of Q / K / V rows and vector stores of output rows
    const bool aligned16 = (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) == 0;
    return launch_sparse_csr(p, dtype == MIATTN_F64, aligned16, (hipStream_t)stream) == hipSuccess
               ? MIATTN_OK : MIATTN_ERR_LAUNCH;
}

}  // extern "C"
