// Rotary position embedding at the packed tokens' DAG positions, on gfx950.
//
// The positions come out of the plan (Octopus project page, card "02 · Memory": a
// mounted key keeps the position it was written at, and a reader's positions jump to
// max(p_B, e_A + 1), so keys are never re-rotated when mounted).  Pairs (x_i, x_{i+D/2})
// turn by pos * base^(-2i/D).  This is an HBM-bound pass: D/16 lanes per token compute
// the token's D/2 angles once (in float64 before the reduction to [-pi, pi], since
// pos * theta reaches ~10^5 radians) and turn every head of the token.
#include "device_common.h"
#include "kernels.h"

namespace octo {

// Pair frequencies base^(-2i/D), i < D/2, computed on the host in float64.
struct RopeFreqs {
    double theta[64];
};

// Each lane owns 8 consecutive pair indices of one token (16-byte accesses in bf16),
// computes their 8 angles once and applies them to every head of the token, in x (H
// heads) and then, if given, in x2 (H2 heads).
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(int rows, int D, RopeFreqs f, float sign,
                                                   const int32_t* __restrict__ pos, int H,
                                                   const T* x, T* out, int H2, const T* x2,
                                                   T* out2) {
    const int half = D / 2;
    const int lanes = half / 8;  // lanes per token
    const int per_block = 256 / lanes;
    const int i0 = (threadIdx.x % lanes) * 8;
    const int row = blockIdx.x * per_block + threadIdx.x / lanes;
    if (row >= rows) return;
    const double p = (double)pos[row];
    const double two_pi = 6.283185307179586476925286766559;
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double ang = p * f.theta[i0 + e];
        const float r = (float)(ang - two_pi * rint(ang * (1.0 / two_pi)));
        sincosf(r, &sn[e], &cs[e]);
        sn[e] *= sign;
    }
    auto turn = [&](int nh, const T* src, T* dst) {
        const size_t base = (size_t)row * nh * D + i0;
        for (int h = 0; h < nh; ++h) {
            const size_t o = base + (size_t)h * D;
            T a[8], b[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a[e] = src[o + e];
                b[e] = src[o + half + e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x1 = (float)a[e], y1 = (float)b[e];
                a[e] = (T)(x1 * cs[e] - y1 * sn[e]);
                b[e] = (T)(y1 * cs[e] + x1 * sn[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dst[o + e] = a[e];
                dst[o + half + e] = b[e];
            }
        }
    };
    turn(H, x, out);
    if (x2 != nullptr) turn(H2, x2, out2);
}

hipError_t launch_rope2(bool bf16_, int rows, int D, float base, bool inverse,
                        const int32_t* pos, int H, const void* x, void* out, int H2,
                        const void* x2, void* out2, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    RopeFreqs f{};
    const double lb = std::log2((double)base);
    for (int i = 0; i < D / 2; ++i) f.theta[i] = std::exp2(-2.0 * i / D * lb);
    const int per_block = 256 / (D / 16);
    const dim3 grid((rows + per_block - 1) / per_block), block(256);
    const float sign = inverse ? -1.f : 1.f;
    if (bf16_)
        hipLaunchKernelGGL(rope_kernel<bf16>, grid, block, 0, s, rows, D, f, sign, pos, H,
                           (const bf16*)x, (bf16*)out, H2, (const bf16*)x2, (bf16*)out2);
    else
        hipLaunchKernelGGL(rope_kernel<float>, grid, block, 0, s, rows, D, f, sign, pos, H,
                           (const float*)x, (float*)out, H2, (const float*)x2, (float*)out2);
    return hipGetLastError();
}

hipError_t launch_rope(bool bf16_, int rows, int H, int D, float base, bool inverse,
                       const int32_t* pos, const void* x, void* out, hipStream_t s) {
    return launch_rope2(bf16_, rows, D, base, inverse, pos, H, x, out, 0, nullptr, nullptr, s);
}

}  // namespace octo
