// Internal launch parameters shared by the C-ABI layer and the kernels (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

// One attention forward launch.  Dense batches use stride_b and implicit sequence
// starts of 0; packed (TND) batches read the sequence bounds from cu_q / cu_kv
// (END offsets, no leading zero) and use stride_b = 0.
struct FaParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* smax;            // may be null (never null when prev_out is set)
    float* ssum;            // may be null (never null when prev_out is set)
    // Running result that this launch's partial is merged into (ring-attention update in
    // the epilogue); null for a plain forward.  prev_out has the strides of out, the
    // statistics the indexing of smax / ssum; out / smax / ssum may alias them.
    const void* prev_out;
    const float* prev_max;
    const float* prev_sum;
    const int64_t* cu_q;    // null for dense batches
    const int64_t* cu_kv;
    int64_t q_sb, q_ss, q_sh;   // element strides: batch, sequence position, head
    int64_t k_sb, k_ss, k_sh;
    int64_t v_sb, v_ss, v_sh;
    int64_t o_sb, o_ss, o_sh;
    int64_t st_sb, st_sh;       // stats element index = b*st_sb + h*st_sh + (seq start + i)
    int32_t B, Nq, Nkv, group;  // group = Nq / Nkv
    int32_t Sq, Skv;            // dense: lengths; packed: upper bounds (max_seqlen)
    int32_t Dv;                 // head dim of V and the output (<= the Q/K head dim)
    int32_t n_levels;           // q tiles per sequence at the longest length
    int32_t n_slots;            // workgroups in the grid (multiple of 8 * group)
    int64_t pre, next;          // visible band: -pre <= j - i - off <= next (clamped)
    int32_t align_br;           // off = len_kv - len_q of the sequence (bottom-right), else 0
    const int64_t* prefix;      // device [B] or null: keys j < prefix[b] are seen by every row
                                // (only with pre unbounded, so the visible keys stay a range)
    const uint8_t* amask;       // device [Sq][Skv] bytes or null: nonzero = masked out,
                                // sequence-local positions
    int64_t amask_ld;           // row stride of amask
    uint32_t drop_thr;          // dropout: a probability is dropped when its byte < drop_thr
    float drop_scale;           // 256 / (256 - drop_thr), applied to the kept ones
    uint32_t seed_lo, seed_hi;  // Philox4x32-10 key
    uint32_t drop_offset;       // fourth counter word
    float scale;                // softmax scale
    float scale_log2;           // scale * log2(e)
    int32_t persist_hpi;        // persistent kernel: query heads per work item (1, 2, 4, 8)
};

struct MergeParams {
    const void* o1;
    const float* m1;
    const float* l1;
    const void* o2;
    const float* m2;
    const float* l2;
    void* out;
    float* mo;
    float* lo;
    int64_t sb, sh, ss;         // element strides of the outputs (head_dim contiguous)
    int32_t B, N, S, D;
};

struct SparseParams {
    const void* q;          // float or double, as `out`
    const void* k;
    const void* v;
    void* out;
    const int32_t* offset;
    const int32_t* columns;
    int64_t nnz;
    int32_t B, N, S, D;
    float scale_log2;
    double scale_log2_d;        // the same in double precision (fp64 inputs)
};

// Launchers (defined next to their kernels).  Each returns the launch status.
// the MFMA forward for bf16 (f16 = false) or fp16 (f16 = true) inputs; both forwards
// merge into p.prev_* when p.prev_out is set
hipError_t launch_fa_fwd_bf16(const FaParams& p, int D, bool f16, hipStream_t stream);
// the head-dim-general forward: any 1 <= p.Dv <= D <= 768, every dtype and feature; rows per
// workgroup fa_wide_tile_m(dtype)
hipError_t launch_fa_fwd_wide(const FaParams& p, int D, int dtype, hipStream_t stream);
// the persistent causal forward (bf16 / fp16, head dim 64 or 128): p.n_slots workgroups
// (one per CU) walk the work items; p.persist_hpi = fa_persist_heads_per_item(p.group)
hipError_t launch_fa_fwd_persist(const FaParams& p, int D, bool f16, hipStream_t stream);
// query heads of one GQA group that a persistent work item covers: the largest power of two
// dividing the group size, at most 8
int fa_persist_heads_per_item(int group);
int fa_wide_tile_m(int dtype);
hipError_t launch_lse_merge(const MergeParams& p, int dtype, hipStream_t stream);
// the CSR kernel; aligned16: Q, K, V and out are 16-byte aligned (vector row accesses)
hipError_t launch_sparse_csr(const SparseParams& p, bool f64, bool aligned16, hipStream_t stream);
// whether the CSR kernel takes head dim D (1..768; fp64 at 768 still fits its LDS)
bool sparse_head_dim_fits(int D, bool f64);
// keys of the CSR kernel's LDS window (the keys before the end of each block of
// kSparseRowBlock rows that it reads from LDS instead of global memory)
int sparse_window_keys(int D, bool f64, bool aligned16);
constexpr int kSparseRowBlock = 64;

// Longest packed batch (sequences) of the persistent kernel, whose workgroups sort the
// sequence lengths in LDS.
constexpr int kPersistMaxSeq = 512;
// the most work items one workgroup of the persistent kernel may own at head dim D, with
// or without dropout (its item records live in LDS; dropout makes them larger)
int fa_persist_max_items(int D, bool drop);

// Row tile heights, used by the C-ABI layer to size the grids.
constexpr int kBf16TileM = 256;
constexpr int kBf16TileMBig = 128;   // the MFMA kernel's 4-wave configuration

#ifndef FA_FOUR_WAVE_MIN_D
#define FA_FOUR_WAVE_MIN_D 129
#endif
// Whether the MFMA kernel runs its 4-wave, 32-key-tile configuration (128-row tiles) for
// head dim D: always above 128; from FA_FOUR_WAVE_MIN_D up for the plain and update
// instances (the mask-tensor and dropout instances assume 64-key tiles).
constexpr bool fa_four_waves(int D, bool mask_or_dropout)
{
    return D > 128 || (!mask_or_dropout && D >= FA_FOUR_WAVE_MIN_D);
}

}  // namespace miattn
