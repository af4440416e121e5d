// Forward of packed-DAG attention on gfx950.
//
// The Octopus trainer runs one block-sparse attention pass over all branches of a
// tree packed into one unpadded 1-D stream (project page, card "03 · Training";
// ia.com.br article, section "Crédito contrafactual ..."): query i attends to
// Ctx(i) only.  The host planner lists, per 128-row query tile, the 64-key KV tiles
// some row sees (FULL, or PARTIAL with a per-row bit mask); this kernel walks that
// list with an online softmax.
//
// bf16 kernel: one workgroup = one (query tile, query head); four wave64s, each
// owning 32 query rows.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16 so that every lane holds one query column: the row max
// and row sum are in-lane plus one exchange with lane ^ 32, and the probabilities
// come out of the accumulator already laid out as the B operand of O^T = V^T P^T.
// K is staged row-major in LDS (A operand of S^T), V transposed (A operand of O^T);
// the next tile's global loads are issued before the current tile's MFMAs.  The
// G = Hq/Hkv query heads reading one KV head are launched adjacently on one XCD so
// their shared K/V tiles hit the same L2.
#include "device_common.h"
#include "kernels.h"

namespace octo {

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    DevPlan P, int Hq, int Hkv, float scale_log2, const bf16* __restrict__ Q,
    const bf16* __restrict__ K, const bf16* __restrict__ V, bf16* __restrict__ O,
    float* __restrict__ LSE) {
    constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
    constexpr int DB = D / 32;   // 32-row blocks of O^T
    constexpr int KST = D + 8;   // LDS row stride of K (elements), padded
    constexpr int VST = kBk + 8; // LDS row stride of V^T
    constexpr int C8 = D / 8;    // 16-byte chunks per K/V row
    constexpr int NLOAD = (kBk / 4) * C8;  // loader items: 4 rows x 8 columns each
    __shared__ __attribute__((aligned(16))) bf16 Ks[kBk * KST];
    __shared__ __attribute__((aligned(16))) bf16 Vt[D * VST];

    const int G = Hq / Hkv;
    int grp, hh;
    if (!xcd_group(blockIdx.x, G, P.nQT * Hkv, grp, hh)) return;
    const int qt = P.fwd_order[grp / Hkv];
    const int kvh = grp % Hkv;
    const int h = kvh * G + hh;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int T = P.T;
    const int rr = w * 32 + n;       // row inside the query tile
    const int row = qt * kBq + rr;   // packed query row of this lane
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;

    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = row < T ? ld16(Q + row * qstride + (size_t)h * D + 16 * ks + 8 * g) : zero8();

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();
    float m = -1e30f, l = 0.f;

    const bool loader = tid < NLOAD;
    const int c8 = tid % C8, rg = tid / C8;
    bf16x8 kr[4], vr[4];
    auto gload = [&](int kt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = kt * kBk + 4 * rg + j;
            if (loader && key < T) {
                const size_t off = (size_t)key * kvstride + (size_t)kvh * D + 8 * c8;
                kr[j] = ld16(K + off);
                vr[j] = ld16(V + off);
            } else {
                kr[j] = zero8();
                vr[j] = zero8();
            }
        }
    };
    auto lds_put = [&]() {
        if (!loader) return;
#pragma unroll
        for (int j = 0; j < 4; ++j) st16(&Ks[(4 * rg + j) * KST + 8 * c8], kr[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 t;
            t[0] = vr[0][e];
            t[1] = vr[1][e];
            t[2] = vr[2][e];
            t[3] = vr[3][e];
            st8(&Vt[(8 * c8 + e) * VST + 4 * rg], t);
        }
    };

    const int p0 = P.qt_ptr[qt], p1 = P.qt_ptr[qt + 1];
    if (p0 < p1) gload(P.q_pairs[p0].x);
    for (int pi = p0; pi < p1; ++pi) {
        const int2 pr = P.q_pairs[pi];
        __syncthreads();
        lds_put();
        __syncthreads();
        if (pi + 1 < p1) gload(P.q_pairs[pi + 1].x);

        // S^T (64 keys x 32 queries) = K Q^T, two 32-key blocks.
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = ld16(&Ks[(kb * 32 + n) * KST + 16 * ks + 8 * g]);
                s[kb] = mfma_32x32x16(a, qf[ks], s[kb]);
            }
        }
        if (pr.y >= 0) {
            const uint64_t bits = P.mask_rows[(size_t)pr.y * kBq + rr];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int x = kb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
                    if (!((bits >> x) & 1ull)) s[kb][j] = -INFINITY;
                }
        }
        // Online softmax in the log2 domain.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                s[kb][j] *= scale_log2;
                mx = fmaxf(mx, s[kb][j]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        bf16x8 pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float pv = fast_exp2(s[kb][j] - mnew);
                l += pv;
                pf[kb * 2 + (j >> 3)][j & 7] = (bf16)pv;
            }
        // O^T (D x 32 queries) += V^T P^T over 4 k-steps of 16 keys.  The lane's 8 keys
        // of k-step kk are 16kk + 4g + {0..3} and 16kk + 8 + 4g + {0..3}, matching the
        // rows its accumulator holds.
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16* vrow = &Vt[(db * 32 + n) * VST + 16 * kk + 4 * g];
                const bf16x8 a = cat(ld8(vrow), ld8(vrow + 8));
                o[db] = mfma_32x32x16(a, pf[kk], o[db]);
            }
    }

    l += __shfl_xor(l, 32);
    if (row < T) {
        const float inv = 1.f / l;
        bf16* orow = O + row * qstride + (size_t)h * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                bf16x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = (bf16)(o[db][4 * q4 + e] * inv);
                st8(orow + db * 32 + 8 * q4 + 4 * g, t);
            }
        if (g == 0) LSE[(size_t)h * T + row] = (m + log2f(l)) * kLn2;
    }
}

// fp32: one thread per query row, keys streamed through LDS 32 at a time, exact
// float32 arithmetic (used for float32 inputs).
template <int D>
__global__ __launch_bounds__(128) void fwd_fp32_kernel(DevPlan P, int Hq, int Hkv, float scale,
                                                       const float* __restrict__ Q,
                                                       const float* __restrict__ K,
                                                       const float* __restrict__ V,
                                                       float* __restrict__ O,
                                                       float* __restrict__ LSE) {
    constexpr int HALF = 32;
    __shared__ float Ksh[HALF][D];
    __shared__ float Vsh[HALF][D];
    const int qt = P.fwd_order[blockIdx.x / Hq];
    const int h = blockIdx.x % Hq;
    const int kvh = h / (Hq / Hkv);
    const int T = P.T;
    const int rr = threadIdx.x;
    const int row = qt * kBq + rr;
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;
    float q[D], o[D];
    for (int d = 0; d < D; ++d) {
        q[d] = row < T ? Q[row * qstride + (size_t)h * D + d] : 0.f;
        o[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int pi = P.qt_ptr[qt]; pi < P.qt_ptr[qt + 1]; ++pi) {
        const int2 pr = P.q_pairs[pi];
        const uint64_t bits = pr.y >= 0 ? P.mask_rows[(size_t)pr.y * kBq + rr] : ~0ull;
        for (int half = 0; half < 2; ++half) {
            __syncthreads();
            for (int idx = threadIdx.x; idx < HALF * D; idx += blockDim.x) {
                const int kk = idx / D, d = idx % D;
                const int key = pr.x * kBk + half * HALF + kk;
                Ksh[kk][d] = key < T ? K[key * kvstride + (size_t)kvh * D + d] : 0.f;
                Vsh[kk][d] = key < T ? V[key * kvstride + (size_t)kvh * D + d] : 0.f;
            }
            __syncthreads();
            for (int kk = 0; kk < HALF; ++kk) {
                if (!((bits >> (half * HALF + kk)) & 1ull)) continue;
                float sc = 0.f;
                for (int d = 0; d < D; ++d) sc = fmaf(q[d], Ksh[kk][d], sc);
                sc *= scale;
                const float mn = fmaxf(m, sc);
                const float a = expf(m - mn);
                const float pe = expf(sc - mn);
                l = l * a + pe;
                for (int d = 0; d < D; ++d) o[d] = fmaf(pe, Vsh[kk][d], o[d] * a);
                m = mn;
            }
        }
    }
    if (row < T) {
        const float inv = 1.f / l;
        for (int d = 0; d < D; ++d) O[row * qstride + (size_t)h * D + d] = o[d] * inv;
        LSE[(size_t)h * T + row] = m + logf(l);
    }
}

hipError_t launch_fwd_bf16(const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, void* o, float* lse,
                           hipStream_t s) {
    const int G = Hq / Hkv;
    dim3 grid(xcd_grid(p.nQT * Hkv, G)), block(256);
    const float sl2 = scale * kLog2e;
    if (D == 128)
        hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block, 0, s, p, Hq, Hkv, sl2,
                           (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse);
    else
        hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block, 0, s, p, Hq, Hkv, sl2,
                           (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse);
    return hipGetLastError();
}

hipError_t launch_fwd_fp32(const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, void* o, float* lse,
                           hipStream_t s) {
    dim3 grid(p.nQT * Hq), block(kBq);
    if (D == 128)
        hipLaunchKernelGGL(fwd_fp32_kernel<128>, grid, block, 0, s, p, Hq, Hkv, scale,
                           (const float*)q, (const float*)k, (const float*)v, (float*)o, lse);
    else
        hipLaunchKernelGGL(fwd_fp32_kernel<64>, grid, block, 0, s, p, Hq, Hkv, scale,
                           (const float*)q, (const float*)k, (const float*)v, (float*)o, lse);
    return hipGetLastError();
}

}  // namespace octo
