// Small device helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace octo {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulation.  Per lane l
// (n = l % 32, g = l / 32): A supplies row n and 8 of the 16 k values, B supplies
// column n and the same 8 k values, and the result holds column n, rows
// 8*(j/4) + 4*g + (j%4) for j = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld16(const bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ void st16(bf16* p, bf16x8 v) {
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
}
__device__ __forceinline__ bf16x4 ld8(const bf16* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ void st8(bf16* p, bf16x4 v) {
    *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ bf16x8 zero8() {
    return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = 0.f;
    return z;
}

// 2^x on the hardware exponential unit (exact 0 for -inf).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Map a block index onto (group, member) so that the `members` blocks of one group
// run on the same XCD (workgroups are dealt to the 8 XCDs round-robin by index) and
// groups keep their launch order.  Returns false for padding blocks.
__device__ __forceinline__ bool xcd_group(int bid, int members, int n_groups, int& group,
                                          int& member) {
    const int per = 8 * members;
    const int i8 = bid / per;
    const int rem = bid - i8 * per;
    group = i8 * 8 + (rem & 7);
    member = rem >> 3;
    return group < n_groups;
}

inline int xcd_grid(int n_groups, int members) { return (n_groups + 7) / 8 * 8 * members; }

}  // namespace octo
