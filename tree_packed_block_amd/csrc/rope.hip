// Rotary position embedding at the packed tokens' DAG positions, on gfx950.
//
// The positions come out of the plan (Octopus project page, card "02 · Memory": a
// mounted key keeps the position it was written at, and a reader's positions jump to
// max(p_B, e_A + 1), so keys are never re-rotated when mounted).  Pairs (x_i, x_{i+D/2})
// turn by pos * base^(-2i/D).  This is an HBM-bound pass: one group of D/2 lanes per
// token computes the token's D/2 angles once (in float64 before the reduction to
// [-pi, pi], since pos * theta reaches ~10^5 radians) and turns every head of the token.
#include "device_common.h"
#include "kernels.h"

namespace octo {

template <typename T>
__device__ __forceinline__ float to_f(T v) { return (float)v; }

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(int rows, int H, int D, double log2_base,
                                                   float sign, const int32_t* __restrict__ pos,
                                                   const T* x, T* out) {
    const int half = D / 2;
    const int per_block = 256 / half;
    const int i = threadIdx.x % half;
    const int row = blockIdx.x * per_block + threadIdx.x / half;
    if (row >= rows) return;
    const double theta = exp2(-2.0 * (double)i / (double)D * log2_base);
    const double ang = (double)pos[row] * theta;
    const double two_pi = 6.283185307179586476925286766559;
    const float r = (float)(ang - two_pi * rint(ang / two_pi));
    float sn, cs;
    sincosf(r, &sn, &cs);
    sn *= sign;
    const size_t base = (size_t)row * H * D;
    for (int h = 0; h < H; ++h) {
        const size_t o = base + (size_t)h * D + i;
        const float x1 = to_f(x[o]), x2 = to_f(x[o + half]);
        out[o] = (T)(x1 * cs - x2 * sn);
        out[o + half] = (T)(x2 * cs + x1 * sn);
    }
}

hipError_t launch_rope(bool bf16_, int rows, int H, int D, float base, bool inverse,
                       const int32_t* pos, const void* x, void* out, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int per_block = 256 / (D / 2);
    const dim3 grid((rows + per_block - 1) / per_block), block(256);
    const double lb = std::log2((double)base);
    const float sign = inverse ? -1.f : 1.f;
    if (bf16_)
        hipLaunchKernelGGL(rope_kernel<bf16>, grid, block, 0, s, rows, H, D, lb, sign, pos,
                           (const bf16*)x, (bf16*)out);
    else
        hipLaunchKernelGGL(rope_kernel<float>, grid, block, 0, s, rows, H, D, lb, sign, pos,
                           (const float*)x, (float*)out);
    return hipGetLastError();
}

}  // namespace octo
