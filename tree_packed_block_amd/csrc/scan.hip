// Branch-aware gated delta-rule scan over the packed episode DAG, on gfx950.
//
// The hybrid backbone's recurrent layers (Gated DeltaNet) keep a mutable state per
// branch; `fork` clones the parent's recurrent checkpoint at the fork point and mounted
// spans bypass the recurrent layers (Octopus project page, primitives table; the packed
// trainer compiles these boundary checkpoints into its one pass).  Per head, with state
// S (Dv x Dk), the gated delta rule (Yang, Kautz and Hatamizadeh, 2024) is
//     S_t = alpha_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T,
//     o_t = S_t q_t.
// A branch starts from its parent's state just before the parent's own token `fork`
// (a checkpoint slot) and scans its own tokens; the branches of one depth run in one
// launch, levels in order.  One workgroup per (branch, head) keeps the 128 x 128 float32
// state in registers, 8 lanes per state row (16 columns each): a token costs 48 fused
// multiply-adds per lane and two 8-lane reductions, with the next token's inputs loaded
// while the current one is applied.  This is a sequential form, bound by the latency of
// one token's dependent arithmetic.
#include "device_common.h"
#include "kernels.h"

namespace octo {

namespace {
constexpr int kDim = 128;             // Dk = Dv
constexpr int kParts = 8;             // lanes per state row
constexpr int kCols = kDim / kParts;  // columns per lane
}  // namespace

__global__ __launch_bounds__(1024) void gdn_scan_kernel(DevPlan P, int l0, int H,
                                                        const bf16* __restrict__ Q,
                                                        const bf16* __restrict__ K,
                                                        const bf16* __restrict__ V,
                                                        const float* __restrict__ A,
                                                        const float* __restrict__ Bt,
                                                        bf16* __restrict__ O,
                                                        float* __restrict__ states) {
    const int b = ld_const(P.sc_level_br + l0 + blockIdx.x / H);
    const int h = blockIdx.x % H;
    const int t = threadIdx.x;
    const int i = t / kParts;           // value row
    const int c0 = (t % kParts) * kCols;  // first key column of this lane
    const int start = ld_const(P.sc_start + b), len = ld_const(P.sc_len + b);
    const int init = ld_const(P.sc_init + b);
    const size_t rstride = (size_t)H * kDim;  // elements per token in q, k, v, o

    float s[kCols];
    if (init >= 0) {
        const float4* src = reinterpret_cast<const float4*>(
            states + (((size_t)init * H + h) * kDim + i) * kDim + c0);
#pragma unroll
        for (int j = 0; j < kCols / 4; ++j) {
            const float4 x = src[j];
            s[4 * j] = x.x;
            s[4 * j + 1] = x.y;
            s[4 * j + 2] = x.z;
            s[4 * j + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kCols; ++j) s[j] = 0.f;
    }
    int ck = ld_const(P.sc_ck_ptr + b);
    const int ck_end = ld_const(P.sc_ck_ptr + b + 1);
    int next_ck = ck < ck_end ? ld_const(P.sc_ck_off + ck) : -1;
    auto save = [&]() {
        const int slot = ld_const(P.sc_ck_slot + ck);
        float4* dst = reinterpret_cast<float4*>(states + (((size_t)slot * H + h) * kDim + i) * kDim + c0);
#pragma unroll
        for (int j = 0; j < kCols / 4; ++j)
            dst[j] = make_float4(s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]);
        ++ck;
        next_ck = ck < ck_end ? ld_const(P.sc_ck_off + ck) : -1;
    };

    // Inputs of one token for this lane: its 16 key and query columns, its value row,
    // the head's gate and step size.
    struct Tok {
        bf16x8 k[2], q[2];
        float v, a, bt;
    };
    auto load = [&](int r) {
        Tok x;
        const size_t row = (size_t)(start + r);
        const bf16* kp = K + row * rstride + (size_t)h * kDim + c0;
        const bf16* qp = Q + row * rstride + (size_t)h * kDim + c0;
        x.k[0] = ld16(kp);
        x.k[1] = ld16(kp + 8);
        x.q[0] = ld16(qp);
        x.q[1] = ld16(qp + 8);
        x.v = (float)V[row * rstride + (size_t)h * kDim + i];
        x.a = A[row * H + h];
        x.bt = Bt[row * H + h];
        return x;
    };

    Tok cur = load(0);
    for (int r = 0; r < len; ++r) {
        while (r == next_ck) save();
        const Tok nxt = load(r + 1 < len ? r + 1 : r);
        float kf[kCols], qf[kCols];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            kf[j] = (float)cur.k[0][j];
            kf[8 + j] = (float)cur.k[1][j];
            qf[j] = (float)cur.q[0][j];
            qf[8 + j] = (float)cur.q[1][j];
        }
        float sk = 0.f;
#pragma unroll
        for (int j = 0; j < kCols; ++j) sk = fmaf(s[j], kf[j], sk);
        sk += __shfl_xor(sk, 1);
        sk += __shfl_xor(sk, 2);
        sk += __shfl_xor(sk, 4);
        // S <- alpha S + beta (v - alpha S k) k^T
        const float c = cur.bt * (cur.v - cur.a * sk);
        float oi = 0.f;
#pragma unroll
        for (int j = 0; j < kCols; ++j) {
            s[j] = fmaf(cur.a, s[j], c * kf[j]);
            oi = fmaf(s[j], qf[j], oi);
        }
        oi += __shfl_xor(oi, 1);
        oi += __shfl_xor(oi, 2);
        oi += __shfl_xor(oi, 4);
        if ((t % kParts) == 0) O[(size_t)(start + r) * rstride + (size_t)h * kDim + i] = (bf16)oi;
        cur = nxt;
    }
    while (len == next_ck) save();
}

hipError_t launch_gdn_scan(const DevPlan& p, int l0, int n_br, int H, const void* q,
                           const void* k, const void* v, const float* alpha,
                           const float* beta, void* o, float* states, hipStream_t s) {
    if (n_br <= 0) return hipSuccess;
    hipLaunchKernelGGL(gdn_scan_kernel, dim3(n_br * H), dim3(kParts * kDim), 0, s, p, l0, H,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta, (bf16*)o,
                       states);
    return hipGetLastError();
}

}  // namespace octo
