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
// launch, levels in order.  State rows evolve independently (row i needs only itself,
// k, v_i, alpha and beta), so each (branch, head) is split over 4 workgroups of 32 rows,
// the float32 state in registers, 8 lanes per row (16 columns each): a token costs 64
// multiply-adds per lane and two 8-lane DPP reductions.  The inputs of 32 tokens at a
// time are copied to LDS asynchronously (k, q, the slice's v, alpha, beta) while the
// previous 32 are applied.  This is a sequential form (no chunked matrix products),
// bound by the fp32 vector throughput the tree's widest level can use.
#include "device_common.h"
#include "kernels.h"

namespace octo {

namespace {
constexpr int kDim = 128;             // Dk = Dv
constexpr int kParts = 8;             // lanes per state row
constexpr int kCols = kDim / kParts;  // columns per lane
constexpr int kChunk = 32;            // tokens staged in LDS per step
constexpr int kSplit = 4;             // workgroups per (branch, head), each a slice of rows
constexpr int kRows = kDim / kSplit;  // state rows per workgroup
constexpr int kThreads = kRows * kParts;

// Sum over each aligned group of 8 lanes, with DPP moves (no LDS round trip): swap
// neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), then mirror each half
// row of 8 lanes, which pairs every lane of one quad with one of the other.
__device__ __forceinline__ float sum8(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1,
                                                            0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E,
                                                            0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141,
                                                            0xF, 0xF, true));
    return x;
}
}  // namespace

__global__ __launch_bounds__(kThreads) void gdn_scan_kernel(DevPlan P, int l0, int H,
                                                        const bf16* __restrict__ Q,
                                                        const bf16* __restrict__ K,
                                                        const bf16* __restrict__ V,
                                                        const float* __restrict__ A,
                                                        const float* __restrict__ Bt,
                                                        bf16* __restrict__ O,
                                                        float* __restrict__ states) {
    // LDS: two stages of a chunk of kChunk tokens: k, q ([kChunk][128] bf16 each), this
    // workgroup's slice of v ([kChunk][kRows] bf16) and alpha, beta ([kChunk] floats each).
    constexpr int TILE = kChunk * kDim * 2;
    constexpr int VT = kChunk * kRows * 2;
    constexpr int STAGE = 2 * TILE + VT + 2 * kChunk * 4;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

    const int item = blockIdx.x / kSplit, slice = blockIdx.x % kSplit;
    const int b = ld_const(P.sc_level_br + l0 + item / H);
    const int h = item % H;
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int il = t / kParts;            // row within the slice
    const int i = slice * kRows + il;     // value row
    const int c0 = (t % kParts) * kCols;  // first key column of this lane
    const int start = ld_const(P.sc_start + b), len = ld_const(P.sc_len + b);
    const int init = ld_const(P.sc_init + b);
    const size_t rstride = (size_t)H * kDim;  // elements per token in q, k, v, o
    const unsigned smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

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

    // Copies of chunk c into stage st: piece p (16 bytes) of the k and q tiles is token
    // p / 16, columns 8 (p % 16) ..; piece p of the v slice is token p / (kRows / 8),
    // rows slice * kRows + 8 (p % (kRows / 8)) ..; tokens past the branch's end are
    // clamped to its last token.  Lanes below 2 kChunk fetch alpha (t < kChunk) or beta.
    const int n_chunks = (len + kChunk - 1) / kChunk;
    constexpr int KQ_PER = TILE / 16 / kThreads;  // k (and q) pieces per thread
    constexpr int VP = VT / 16;                   // v pieces in all
    static_assert(KQ_PER * kThreads * 16 == TILE, "k and q tiles split evenly over threads");
    static_assert(VP % 64 == 0 && VP <= kThreads, "the v slice is copied by whole waves");
    float ab = 0.f;
    auto issue = [&](int c, int st) {
        const int last = len - 1 - c * kChunk;  // last valid token within the chunk
        const size_t base = (size_t)(start + c * kChunk) * rstride + (size_t)h * kDim;
        const unsigned dst = smem_base + st * STAGE + w * 64 * 16;
#pragma unroll
        for (int u = 0; u < KQ_PER; ++u) {
            const int p = u * kThreads + t;
            const int tok = min(p / 16, last);
            const unsigned off = (unsigned)(((size_t)tok * rstride + 8 * (p % 16)) * 2);
            dma16_s(K + base, off, dst + u * kThreads * 16);
            dma16_s(Q + base, off, dst + TILE + u * kThreads * 16);
        }
        if (w * 64 < VP) {  // whole waves: VP is a multiple of 64
            const int tok = min(t / (kRows / 8), last);
            const unsigned off = (unsigned)(((size_t)tok * rstride + slice * kRows +
                                             8 * (t % (kRows / 8))) * 2);
            dma16_s(V + base, off, dst + 2 * TILE);
        }
        if (t < 2 * kChunk) {
            const int tk = min(c * kChunk + t % kChunk, len - 1);
            ab = (t < kChunk ? A : Bt)[(size_t)(start + tk) * H + h];
        }
    };
    auto put_ab = [&](int st) {
        if (t < 2 * kChunk)
            *reinterpret_cast<float*>(smem + st * STAGE + 2 * TILE + VT + t * 4) = ab;
    };

    issue(0, 0);
    put_ab(0);
    wait_vmem<0>();
    barrier();
    for (int c = 0; c < n_chunks; ++c) {
        const int st = c & 1;
        if (c + 1 < n_chunks) issue(c + 1, st ^ 1);
        const unsigned char* sk_ = smem + st * STAGE;
        const int r0 = c * kChunk, r1 = min(len, r0 + kChunk);
        for (int r = r0; r < r1; ++r) {
            while (r == next_ck) save();
            const int rr = r - r0;
            const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(sk_ + rr * kDim * 2 + c0 * 2);
            const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(sk_ + rr * kDim * 2 + c0 * 2 + 16);
            const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(sk_ + TILE + rr * kDim * 2 + c0 * 2);
            const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(sk_ + TILE + rr * kDim * 2 + c0 * 2 + 16);
            const float vi = (float)*reinterpret_cast<const bf16*>(sk_ + 2 * TILE + (rr * kRows + il) * 2);
            const float a = *reinterpret_cast<const float*>(sk_ + 2 * TILE + VT + rr * 4);
            const float bt = *reinterpret_cast<const float*>(sk_ + 2 * TILE + VT + (kChunk + rr) * 4);
            float kf[kCols], qf[kCols];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                kf[j] = (float)k0[j];
                kf[8 + j] = (float)k1[j];
                qf[j] = (float)q0[j];
                qf[8 + j] = (float)q1[j];
            }
            float skv = 0.f;
#pragma unroll
            for (int j = 0; j < kCols; ++j) skv = fmaf(s[j], kf[j], skv);
            skv = sum8(skv);
            // S <- alpha S + beta (v - alpha S k) k^T
            const float cc = bt * (vi - a * skv);
            float oi = 0.f;
#pragma unroll
            for (int j = 0; j < kCols; ++j) {
                s[j] = fmaf(a, s[j], cc * kf[j]);
                oi = fmaf(s[j], qf[j], oi);
            }
            oi = sum8(oi);
            if ((t % kParts) == 0) O[(size_t)(start + r) * rstride + (size_t)h * kDim + i] = (bf16)oi;
        }
        // Stage st is read by every wave before the next chunk's copies overwrite it.
        if (c + 1 < n_chunks) put_ab(st ^ 1);
        wait_vmem<0>();
        barrier();
    }
    while (len == next_ck) save();
}

hipError_t launch_gdn_scan(const DevPlan& p, int l0, int n_br, int H, const void* q,
                           const void* k, const void* v, const float* alpha,
                           const float* beta, void* o, float* states, hipStream_t s) {
    if (n_br <= 0) return hipSuccess;
    hipLaunchKernelGGL(gdn_scan_kernel, dim3(n_br * H * kSplit), dim3(kThreads), 0, s, p, l0, H,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta, (bf16*)o,
                       states);
    return hipGetLastError();
}

}  // namespace octo
