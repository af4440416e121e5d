// dQ pass of the packed-DAG attention backward on gfx950 (the third of the three launches
// described in bwd.hip; Octopus project page, card "03 · Training": the mount edges are
// differentiable, so a reader's dQ sums over its own context, the shared prefix and the
// mounted spans alike).  dQ = scale dS K with dS = P (dO V^T - Delta) and P = exp(S - LSE),
// the scores recomputed from the workspace's LSE2 and Delta rows: one workgroup per
// (query tile, one or two query heads of one KV group), walking the forward's tile lists.
// Kept in a file of its own, so that its code-generation options can differ from the dK/dV
// pass's.
#include "device_common.h"
#include "kernels.h"
#include "kvstage.h"

namespace octo {

// With ROPE, Q and K come rotated and dQ is turned back at the row's position before it
// is stored.
template <int D, int HPW, bool ROPE>
__global__ __launch_bounds__(256 * HPW, 1) void dq_bf16_kernel(
    DevPlan P, int Hq, int Hkv, float scale, float scale_log2, const bf16* __restrict__ Q,
    const bf16* __restrict__ K, const bf16* __restrict__ V, const bf16* __restrict__ dO,
    const float* __restrict__ ws, bf16* __restrict__ dQ, RopeFreq rt) {
    using L = KvLayout<D>;
    constexpr int NTHR = 256 * HPW;
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int PER_STAGE = 2 * (L::MAT / (16 * NTHR)) + 1;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[L::BYTES];

    const int G = Hq / Hkv;
    int grp, hp;
    if (!xcd_group(blockIdx.x, G / HPW, P.nQT * Hkv, grp, hp)) return;
    const int qt = ld_const(P.fwd_order + grp / Hkv);
    const int kvh = grp % Hkv;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = kvh * G + hp * HPW + (w >> 2);
    const int n = lane & 31, g = lane >> 5;
    const int T = P.T, Tp = padded_rows(T);
    const int rr = (w & 3) * 32 + n;
    const int row = qt * kBq + rr;
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;
    const unsigned smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // Q enters the scores pre-multiplied by scale * log2(e) (rounded to bf16), and the
    // row terms as one extra MFMA k-step (this lane's -LSE2 or -Delta in three bf16
    // parts against a row of ones), so the accumulators come out as the exponent of P
    // and as dP - Delta.
    bf16x8 qf[KS], df[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const size_t off = (size_t)row * qstride + (size_t)h * D + 16 * ks + 8 * g;
        const bf16x8 qr = row < T ? ld16(Q + off) : zero8();
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)((float)qr[e] * scale_log2);
        df[ks] = row < T ? ld16(dO + off) : zero8();
    }
    const bf16x8 xl = split3(-ws[(size_t)h * Tp + row], g == 0);
    const bf16x8 xd = split3(-ws[(size_t)Hq * Tp + (size_t)h * Tp + row], g == 0);
    bf16x8 ones = zero8();
    if (g == 0) ones[0] = ones[1] = ones[2] = (bf16)1.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        settle(qf[ks]);
        settle(df[ks]);
    }
    settle(xl);
    settle(xd);

    KvOffsets<D> off;
    off.init(lane);
    int offv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) offv[ks] = off.k[ks] - L::K0 + L::V0;
    TileDma<D, NTHR> dm;
    dm.init(tid, kvstride);

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();

    const int p0 = ld_const(P.qt_ptr + qt), p1 = ld_const(P.qt_ptr + qt + 1);
    const int n_it = p1 - p0;
    // The tile pair of the next iteration to issue (index jn) is loaded at the end of the
    // iteration before (`fetch_pair`), so that no scalar load is waited for right after the
    // barrier.  `partial` keeps, per stage, whether its tile is PARTIAL.
    int jn = 0;
    int2 jpr = n_it > 0 ? ld_const(P.q_pairs + p0) : make_int2(0, -1);
    bool partial[3];
    auto fetch_pair = [&]() {
        asm volatile("" ::: "memory");
        jpr = ld_const(P.q_pairs + p0 + min(jn, n_it - 1));
    };
    auto issue = [&](auto st_c, int it) {
        constexpr int ST = decltype(st_c)::value;
        const int2 pr = jpr;
        asm volatile("" ::"s"(pr.x), "s"(pr.y));
        partial[ST] = pr.y >= 0;
        ++jn;
        issue_kv_stage<D, NTHR, ST>(smem_base, K, V, P.mask_rows, pr.x,
                                    pr.y >= 0 ? pr.y : P.n_partial, T, kvh, kvstride, dm, tid,
                                    w, lane);
    };
    auto step = [&](auto st_c, int it) {
        constexpr int ST = decltype(st_c)::value;
        if (it + 1 < n_it) wait_vmem<PER_STAGE>();
        else wait_vmem<0>();
        barrier();
        if (it + 2 < n_it) issue(ic<(ST + 2) % 3>{}, it + 2);

        // One 32-key block at a time: S and dP, dS, then its two k-steps of
        // dQ^T += K^T dS^T, whose MFMAs overlap the next block's softmax.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 sc = mfma_32x32x16(ones, xl, zero16());
            f32x16 dp = mfma_32x32x16(ones, xd, zero16());
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int imm = ST * L::MAT + kb * 32 * L::ROWB;
                sc = mfma_32x32x16(lds16(smem, off.k[ks], imm), qf[ks], sc);
                dp = mfma_32x32x16(lds16(smem, offv[ks], imm), df[ks], dp);
            }
            bf16x8 sb[2];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                sb[j >> 3][j & 7] = (bf16)(fast_exp2(sc[j]) * dp[j]);
            if (__builtin_expect(partial[ST], 0)) {  // wave-uniform and rare: clear dS where
                asm volatile("");                   // the mask is 0 (a real branch)
                // The row's mask word, addressed from the lane id afresh (the opaque
                // copy keeps the address from being hoisted and held across the loop).
                int lid = __lane_id();
                asm volatile("" : "+v"(lid));
                const int om = L::M0 + ((w & 3) * 32 + (lid & 31)) * 8;
                const uint32_t bw = *reinterpret_cast<const uint32_t*>(
                                        smem + om + ST * L::MASKB + 4 * kb) >> (4 * g);
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (!((bw >> (8 * (j >> 2) + (j & 3))) & 1u)) sb[j >> 3][j & 7] = (bf16)0.f;
            }
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int imm = ST * L::MAT + 16 * (2 * kb + k2) * L::ROWB;
                    const bf16x8 a = cat(lds8_tr(smem, off.kt[db][0], imm),
                                         lds8_tr(smem, off.kt[db][1], imm));
                    dq[db] = mfma_32x32x16(a, sb[k2], dq[db]);
                }
        }
        fetch_pair();
    };

    if (n_it > 0) {
        issue(ic<0>{}, 0);
        fetch_pair();
    }
    if (n_it > 1) {
        issue(ic<1>{}, 1);
        fetch_pair();
    }
    for (int it = 0; it < n_it; it += 3) {
        step(ic<0>{}, it);
        if (it + 1 < n_it) step(ic<1>{}, it + 1);
        if (it + 2 < n_it) step(ic<2>{}, it + 2);
    }

    if (row < T) {
        if constexpr (ROPE) rope_accum(dq, P.pos[row], rt, g, -1.f);
        bf16* out = dQ + (size_t)row * qstride + (size_t)h * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                bf16x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = (bf16)(scale * dq[db][4 * q4 + e]);
                st8(out + db * 32 + 8 * q4 + 4 * g, t);
            }
    }
}

// Exact float32 dQ (for float32 inputs): one thread per query row of a tile and head.
template <int D>
__global__ __launch_bounds__(128) void dq_fp32_kernel(DevPlan P, int Hq, int Hkv, float scale,
                                                      const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      const float* __restrict__ dO,
                                                      const float* __restrict__ ws,
                                                      float* __restrict__ dQ) {
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
    float q[D], d[D], acc[D];
    for (int x = 0; x < D; ++x) {
        q[x] = row < T ? Q[row * qstride + (size_t)h * D + x] : 0.f;
        d[x] = row < T ? dO[row * qstride + (size_t)h * D + x] : 0.f;
        acc[x] = 0.f;
    }
    const int Tp = padded_rows(T);
    const float lse2 = ws[(size_t)h * Tp + row];
    const float dlt = ws[(size_t)Hq * Tp + (size_t)h * Tp + row];
    const float sl2 = scale * kLog2e;
    for (int pi = P.qt_ptr[qt]; pi < P.qt_ptr[qt + 1]; ++pi) {
        const int2 pr = P.q_pairs[pi];
        const uint64_t bits = pr.y >= 0 ? P.mask_rows[(size_t)pr.y * kBq + rr] : ~0ull;
        for (int half = 0; half < 2; ++half) {
            __syncthreads();
            for (int idx = threadIdx.x; idx < HALF * D; idx += blockDim.x) {
                const int kk = idx / D, x = idx % D;
                const int key = pr.x * kBk + half * HALF + kk;
                Ksh[kk][x] = key < T ? K[key * kvstride + (size_t)kvh * D + x] : 0.f;
                Vsh[kk][x] = key < T ? V[key * kvstride + (size_t)kvh * D + x] : 0.f;
            }
            __syncthreads();
            for (int kk = 0; kk < HALF; ++kk) {
                if (!((bits >> (half * HALF + kk)) & 1ull) || row >= T) continue;
                float sc = 0.f, dp = 0.f;
                for (int x = 0; x < D; ++x) {
                    sc = fmaf(q[x], Ksh[kk][x], sc);
                    dp = fmaf(d[x], Vsh[kk][x], dp);
                }
                const float p = exp2f(sc * sl2 - lse2);
                const float ds = p * (dp - dlt);
                for (int x = 0; x < D; ++x) acc[x] = fmaf(ds, Ksh[kk][x], acc[x]);
            }
        }
    }
    if (row < T)
        for (int x = 0; x < D; ++x) dQ[row * qstride + (size_t)h * D + x] = scale * acc[x];
}

// ------------------------------------------------------------------ launchers

template <int D, int HPW>
static hipError_t dq_bf16_launch(const DevPlan& p, int Hq, int Hkv, float scale, const void* q,
                                 const void* k, const void* v, const void* dout, float* ws,
                                 void* dq, const RopeFreq* rope, hipStream_t s) {
    const dim3 grid(xcd_grid(p.nQT * Hkv, Hq / Hkv / HPW)), block(256 * HPW);
    const RopeFreq rt = rope ? *rope : RopeFreq{};
    if (rope)
        hipLaunchKernelGGL((dq_bf16_kernel<D, HPW, true>), grid, block, 0, s, p, Hq, Hkv, scale,
                           scale * kLog2e, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                           (const bf16*)dout, ws, (bf16*)dq, rt);
    else
        hipLaunchKernelGGL((dq_bf16_kernel<D, HPW, false>), grid, block, 0, s, p, Hq, Hkv, scale,
                           scale * kLog2e, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                           (const bf16*)dout, ws, (bf16*)dq, rt);
    return hipGetLastError();
}

template <int D>
static hipError_t dq_launch(bool bf16_, const DevPlan& p, int Hq, int Hkv, float scale,
                            const void* q, const void* k, const void* v, const void* dout,
                            float* ws, void* dq, const RopeFreq* rope, hipStream_t s) {
    if (bf16_) {
        if ((Hq / Hkv) % 2 == 0)
            return dq_bf16_launch<D, 2>(p, Hq, Hkv, scale, q, k, v, dout, ws, dq, rope, s);
        return dq_bf16_launch<D, 1>(p, Hq, Hkv, scale, q, k, v, dout, ws, dq, rope, s);
    }
    hipLaunchKernelGGL(dq_fp32_kernel<D>, dim3(p.nQT * Hq), dim3(kBq), 0, s, p, Hq, Hkv, scale,
                       (const float*)q, (const float*)k, (const float*)v, (const float*)dout,
                       ws, (float*)dq);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(bool bf16_, const DevPlan& p, int Hq, int Hkv, int D, float scale,
                         const void* q, const void* k, const void* v, const void* dout,
                         float* ws, void* dq, const RopeFreq* rope, hipStream_t s) {
    if (D == 128) return dq_launch<128>(bf16_, p, Hq, Hkv, scale, q, k, v, dout, ws, dq, rope, s);
    return dq_launch<64>(bf16_, p, Hq, Hkv, scale, q, k, v, dout, ws, dq, rope, s);
}

}  // namespace octo
