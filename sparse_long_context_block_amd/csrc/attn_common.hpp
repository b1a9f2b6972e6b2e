// Device helpers shared by the two attention kernels (sparse_attn.hip,
// attn_union.hip): constants of the online softmax, bf16 packing and the
// cross-lane reductions of the MFMA result layouts.
#pragma once

#include "sgqa_internal.hpp"

namespace sgqa {
namespace attn {

using namespace dev;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;          // log2 units

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Reductions across lanes through v_permlane16_swap / v_permlane32_swap
// (VALU ops: no LDS round trip as with ds_bpermute): xor16 combines lanes
// l and l ^ 16, xor32 lanes l and l ^ 32.
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace attn
}  // namespace sgqa
