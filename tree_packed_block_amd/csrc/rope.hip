// Rotary position embedding at the packed tokens' DAG positions, on gfx950.
//
// The positions come out of the plan (Octopus project page, card "02 · Memory": a
// mounted key keeps the position it was written at, and a reader's positions jump to
// max(p_B, e_A + 1), so keys are never re-rotated when mounted).  Pairs (x_i, x_{i+D/2})
// turn by pos * base^(-2i/D).  This is an HBM-bound pass: D/16 lanes per token compute
// the token's D/2 angles once (reduced in float64, since pos * theta reaches 2^24
// radians) and turn every head of the token.  The attention kernels turn query rows and
// gradients in registers themselves (rope_operand, rope_accum); this pass serves keys,
// the serving side's queries, and the float32 path.
#include "device_common.h"
#include "kernels.h"

namespace octo {

RopeFreq rope_freq(int D, float base) {
    RopeFreq f;
    f.turn0 = 1.0 / 6.283185307179586476925286766559;
    f.ratio = std::exp2(-2.0 / D * std::log2((double)base));
    return f;
}

// Eight consecutive elements of a row, moved as 16-byte vectors.
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16* p) { v = ld16(p); }
    __device__ __forceinline__ void store(bf16* p) const { st16(p, v); }
    __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
    __device__ __forceinline__ void set(int e, float x) { v[e] = (bf16)x; }
};
template <>
struct Vec8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const float4*>(p)[0];
        b = reinterpret_cast<const float4*>(p)[1];
    }
    __device__ __forceinline__ void store(float* p) const {
        reinterpret_cast<float4*>(p)[0] = a;
        reinterpret_cast<float4*>(p)[1] = b;
    }
    __device__ __forceinline__ float get(int e) const {
        const float4& q = e < 4 ? a : b;
        const int k = e & 3;
        return k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
    }
    __device__ __forceinline__ void set(int e, float x) {
        float4& q = e < 4 ? a : b;
        const int k = e & 3;
        if (k == 0) q.x = x; else if (k == 1) q.y = x; else if (k == 2) q.z = x; else q.w = x;
    }
};

// One thread per (token, run of 8 consecutive pair indices): it computes the run's 8
// angles once, then turns that run in every head of the token, in x (H heads) and then,
// if given, in x2 (H2 heads).  Heads go four at a time with all their loads issued before
// any store (out may equal x, and each thread touches only its own elements), so every
// thread keeps eight 16-byte reads in flight.
template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(int rows, RopeFreq f, float sign,
                                                   const int32_t* __restrict__ pos, int H,
                                                   const T* x, T* out, int H2, const T* x2,
                                                   T* out2) {
    constexpr int HALF = D / 2, RUNS = HALF / 8, HB = 4;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int row = (int)(gid / RUNS), i0 = (int)(gid % RUNS) * 8;
    if (row >= rows) return;
    const int p = pos[row];
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        rope_angle(p, f, i0 + e, cs[e], sn[e]);
        sn[e] *= sign;
    }
    auto turn = [&](int nh, const T* src, T* dst) {
        const size_t base = (size_t)row * nh * D + i0;
        for (int h0 = 0; h0 < nh; h0 += HB) {
            Vec8<T> a[HB], b[HB];
#pragma unroll
            for (int u = 0; u < HB; ++u)
                if (h0 + u < nh) {
                    const size_t o = base + (size_t)(h0 + u) * D;
                    a[u].load(src + o);
                    b[u].load(src + o + HALF);
                }
#pragma unroll
            for (int u = 0; u < HB; ++u)
                if (h0 + u < nh) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x1 = a[u].get(e), y1 = b[u].get(e);
                        a[u].set(e, x1 * cs[e] - y1 * sn[e]);
                        b[u].set(e, y1 * cs[e] + x1 * sn[e]);
                    }
                    const size_t o = base + (size_t)(h0 + u) * D;
                    a[u].store(dst + o);
                    b[u].store(dst + o + HALF);
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
    const RopeFreq f = rope_freq(D, base);
    const long long threads = (long long)rows * (D / 16);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    const float sign = inverse ? -1.f : 1.f;
    if (bf16_) {
        if (D == 128)
            hipLaunchKernelGGL((rope_kernel<bf16, 128>), grid, block, 0, s, rows, f, sign, pos, H,
                               (const bf16*)x, (bf16*)out, H2, (const bf16*)x2, (bf16*)out2);
        else
            hipLaunchKernelGGL((rope_kernel<bf16, 64>), grid, block, 0, s, rows, f, sign, pos, H,
                               (const bf16*)x, (bf16*)out, H2, (const bf16*)x2, (bf16*)out2);
    } else {
        if (D == 128)
            hipLaunchKernelGGL((rope_kernel<float, 128>), grid, block, 0, s, rows, f, sign, pos,
                               H, (const float*)x, (float*)out, H2, (const float*)x2,
                               (float*)out2);
        else
            hipLaunchKernelGGL((rope_kernel<float, 64>), grid, block, 0, s, rows, f, sign, pos, H,
                               (const float*)x, (float*)out, H2, (const float*)x2, (float*)out2);
    }
    return hipGetLastError();
}

hipError_t launch_rope(bool bf16_, int rows, int H, int D, float base, bool inverse,
                       const int32_t* pos, const void* x, void* out, hipStream_t s) {
    return launch_rope2(bf16_, rows, D, base, inverse, pos, H, x, out, 0, nullptr, nullptr, s);
}

}  // namespace octo
