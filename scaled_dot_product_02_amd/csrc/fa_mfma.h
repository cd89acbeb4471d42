// Device helpers of the tiled MFMA attention kernels (bf16 / fp16 inputs, fp32
// accumulation on v_mfma_f32_32x32x16): operand types, the MFMA itself, the lane-pair
// reductions of the transposed score layout and the key order of the V^T tiles.
#pragma once
#include "fa_common.h"

namespace miattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Element type of the MFMA path: bf16 or fp16 inputs, outputs and probabilities; fp32
// accumulation either way.  Conversions from fp32 round to nearest even.
template <typename T> struct Elem;
template <> struct Elem<__bf16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    __device__ static f32x16 mfma(const v8& a, const v8& b, const f32x16& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Elem<_Float16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
    __device__ static f32x16 mfma(const v8& a, const v8& b, const f32x16& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// max / sum of x over the lane pair (l, l ^ 32); v_permlane32_swap(x, x) leaves
// (x[l % 32], x[l % 32 + 32]) in every lane, so both lanes get the same result.
__device__ inline float pair_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of key k (0..31 inside a tile) in a V^T row: bits 2 and 3 swapped, matching
// the key order of the P operand taken from the S^T accumulator layout.
__device__ inline int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

}  // namespace
}  // namespace miattn
