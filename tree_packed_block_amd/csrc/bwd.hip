// Backward of packed-DAG attention on gfx950.
//
// The trainer's mount edges are differentiable end to end: a reader's gradient flows
// through the mounted keys into the producer's tokens, and a shared prefix is owned
// once (Octopus project page, card "03 · Training"; ia.com.br article, section
// "Crédito contrafactual ..."; rit.work blog on the packed pass).  With the packed
// layout this is plain attention backward over the visibility mask:
//     Delta_i = <dO_i, O_i>,  P = exp(S - LSE),  dS = P (dO V^T - Delta)
//     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K
// summed over the query heads of each KV head.
//
// Three launches on the caller's stream:
//   1. Delta (HBM-bound row dot products);
//   2. dK/dV: one workgroup owns one (64-key KV tile, KV head) and walks the list of
//      query tiles that see the tile (the planner's transposed lists: later tiles of
//      the same branch, descendants through the shared prefix, readers through
//      mounts), for every query head of the group.  Each dK/dV row is written by its
//      owner only, so there are no atomics and the result does not depend on the
//      schedule;
//   3. dQ: one workgroup per (query tile, query head), like the forward.
// Scores are recomputed from LSE in both 2 and 3.
#include "device_common.h"
#include "kernels.h"

namespace octo {

// ------------------------------------------------------------------ Delta

template <int D>
__global__ __launch_bounds__(256) void delta_bf16_kernel(int T, int Hq, const bf16* __restrict__ O,
                                                         const bf16* __restrict__ dO,
                                                         float* __restrict__ Delta) {
    constexpr int L = D / 8;  // lanes per (row, head)
    const long long pair = ((long long)blockIdx.x * blockDim.x + threadIdx.x) / L;
    const int sub = threadIdx.x % L;
    const bool valid = pair < (long long)T * Hq;
    float acc = 0.f;
    if (valid) {
        const bf16x8 a = ld16(O + pair * D + 8 * sub);
        const bf16x8 b = ld16(dO + pair * D + 8 * sub);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    }
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, L);
    if (valid && sub == 0) {
        const int row = (int)(pair / Hq), h = (int)(pair % Hq);
        Delta[(size_t)h * T + row] = acc;
    }
}

template <int D>
__global__ __launch_bounds__(256) void delta_fp32_kernel(int T, int Hq, const float* __restrict__ O,
                                                         const float* __restrict__ dO,
                                                         float* __restrict__ Delta) {
    const long long pair = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (pair >= (long long)T * Hq) return;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(O[pair * D + d], dO[pair * D + d], acc);
    const int row = (int)(pair / Hq), h = (int)(pair % Hq);
    Delta[(size_t)h * T + row] = acc;
}

// ------------------------------------------------------------------ dK / dV (bf16)
//
// Workgroup = (KV tile, KV head), 4 wave64s: wave w owns keys 32*(w&1) .. +32 of the
// tile and, for each 64-row chunk of a query tile, query rows 32*(w>>1) .. +32 of
// the chunk.  S = Q K^T is computed with K as the register-resident B operand so a
// lane holds one key column: P and dS then serve directly as B operands of
// dV^T += dO^T P and dK^T += Q^T dS, with Q and dO staged in LDS both row-major (A
// of S and dP) and transposed (A of dV^T and dK^T).  The two waves sharing a key
// half add their partial sums through LDS at the end.

template <int D>
struct DkdvSmem {
    static constexpr int RST = D + 8, TST = 64 + 8;
    bf16 Qs[64 * RST];
    bf16 dOs[64 * RST];
    bf16 Qt[D * TST];
    bf16 dOt[D * TST];
    float Ls[64];
    float Ds[64];
};

template <int D>
__global__ __launch_bounds__(256, 1) void dkdv_bf16_kernel(
    DevPlan P, int Hq, int Hkv, float scale, float scale_log2, const bf16* __restrict__ Q,
    const bf16* __restrict__ K, const bf16* __restrict__ V, const bf16* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, bf16* __restrict__ dK,
    bf16* __restrict__ dV) {
    constexpr int KS = D / 16, DB = D / 32, C8 = D / 8, NLOAD = 16 * C8;
    constexpr int RST = DkdvSmem<D>::RST, TST = DkdvSmem<D>::TST;
    constexpr int M = 4;  // consecutive KV tiles of one KV head placed on one XCD
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[sizeof(DkdvSmem<D>)];
    DkdvSmem<D>& S = *reinterpret_cast<DkdvSmem<D>*>(smem_raw);

    int grp, mm;
    if (!xcd_group(blockIdx.x, M, (P.nKT + M - 1) / M * Hkv, grp, mm)) return;
    const int rank = (grp / Hkv) * M + mm;
    if (rank >= P.nKT) return;
    const int kvh = grp % Hkv;
    const int kt = P.bwd_order[rank];

    const int T = P.T, G = Hq / Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, g = lane >> 5, kh = w & 1, qh = w >> 1;
    const int key = kt * kBk + 32 * kh + n;
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;

    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const size_t off = (size_t)key * kvstride + (size_t)kvh * D + 16 * ks + 8 * g;
        kf[ks] = key < T ? ld16(K + off) : zero8();
        vf[ks] = key < T ? ld16(V + off) : zero8();
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = zero16();
        dv[db] = zero16();
    }

    const int p0 = P.kt_ptr[kt], p1 = P.kt_ptr[kt + 1];
    const int n_it = (p1 - p0) * G * 2;  // (query tile, head, 64-row chunk)

    const bool loader = tid < NLOAD;
    const int c8 = tid % C8, rg = tid / C8;
    bf16x8 qr[4], dr[4];
    float lr = 0.f;
    auto gload = [&](int it) {
        const int pi = p0 + it / (2 * G);
        const int hh = (it >> 1) % G, c = it & 1;
        const int h = kvh * G + hh;
        const int row0 = P.k_pairs[pi].x * kBq + c * 64;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = row0 + 4 * rg + j;
            if (loader && r < T) {
                const size_t off = (size_t)r * qstride + (size_t)h * D + 8 * c8;
                qr[j] = ld16(Q + off);
                dr[j] = ld16(dO + off);
            } else {
                qr[j] = zero8();
                dr[j] = zero8();
            }
        }
        if (tid < 64) {
            const int r = row0 + tid;
            lr = r < T ? LSE[(size_t)h * T + r] * kLog2e : INFINITY;
        } else if (tid < 128) {
            const int r = row0 + tid - 64;
            lr = r < T ? Delta[(size_t)h * T + r] : 0.f;
        }
    };
    auto lds_put = [&]() {
        if (loader) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                st16(&S.Qs[(4 * rg + j) * RST + 8 * c8], qr[j]);
                st16(&S.dOs[(4 * rg + j) * RST + 8 * c8], dr[j]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 a, b;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    a[j] = qr[j][e];
                    b[j] = dr[j][e];
                }
                st8(&S.Qt[(8 * c8 + e) * TST + 4 * rg], a);
                st8(&S.dOt[(8 * c8 + e) * TST + 4 * rg], b);
            }
        }
        if (tid < 64) S.Ls[tid] = lr;
        else if (tid < 128) S.Ds[tid - 64] = lr;
    };

    if (n_it > 0) gload(0);
    for (int it = 0; it < n_it; ++it) {
        const int pi = p0 + it / (2 * G);
        const int c = it & 1;
        const int mask = P.k_pairs[pi].y;
        __syncthreads();
        lds_put();
        __syncthreads();
        if (it + 1 < n_it) gload(it + 1);

        // S and dP for 32 query rows x this wave's 32 keys.
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 aq = ld16(&S.Qs[(32 * qh + n) * RST + 16 * ks + 8 * g]);
            const bf16x8 ad = ld16(&S.dOs[(32 * qh + n) * RST + 16 * ks + 8 * g]);
            s = mfma_32x32x16(aq, kf[ks], s);
            dp = mfma_32x32x16(ad, vf[ks], dp);
        }
        uint64_t bits = ~0ull;
        if (mask >= 0) bits = P.mask_cols[((size_t)mask * kBk + 32 * kh + n) * 2 + c];
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int qrow = 32 * qh + 8 * (j >> 2) + 4 * g + (j & 3);  // row in the chunk
            float p = fast_exp2(s[j] * scale_log2 - S.Ls[qrow]);
            if (!((bits >> qrow) & 1ull)) p = 0.f;
            const float ds = p * (dp[j] - S.Ds[qrow]);
            pb[j >> 3][j & 7] = (bf16)p;
            sb[j >> 3][j & 7] = (bf16)ds;
        }
        // dV^T += dO^T P and dK^T += Q^T dS over 2 k-steps of 16 query rows.
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int off = (db * 32 + n) * TST + 32 * qh + 16 * st + 4 * g;
                const bf16x8 ao = cat(ld8(&S.dOt[off]), ld8(&S.dOt[off + 8]));
                const bf16x8 aq = cat(ld8(&S.Qt[off]), ld8(&S.Qt[off + 8]));
                dv[db] = mfma_32x32x16(ao, pb[st], dv[db]);
                dk[db] = mfma_32x32x16(aq, sb[st], dk[db]);
            }
    }

    // Sum the two query halves: waves with qh = 1 hand their partials to qh = 0.
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem_raw);  // [kh][2][DB*16][64]
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                red[((kh * 2 + 0) * DB * 16 + db * 16 + j) * 64 + lane] = dk[db][j];
                red[((kh * 2 + 1) * DB * 16 + db * 16 + j) * 64 + lane] = dv[db][j];
            }
    }
    __syncthreads();
    if (qh == 0 && key < T) {
        bf16* krow = dK + (size_t)key * kvstride + (size_t)kvh * D;
        bf16* vrow = dV + (size_t)key * kvstride + (size_t)kvh * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                bf16x4 a, b;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * q4 + e;
                    a[e] = (bf16)(scale * (dk[db][j] + red[((kh * 2 + 0) * DB * 16 + db * 16 + j) * 64 + lane]));
                    b[e] = (bf16)(dv[db][j] + red[((kh * 2 + 1) * DB * 16 + db * 16 + j) * 64 + lane]);
                }
                st8(krow + db * 32 + 8 * q4 + 4 * g, a);
                st8(vrow + db * 32 + 8 * q4 + 4 * g, b);
            }
    }
}

// ------------------------------------------------------------------ dQ (bf16)
//
// Workgroup = (query tile, query head), wave w owns 32 query rows; like the forward,
// S^T = K Q^T and dP^T = V dO^T put one query per lane, and dS^T is the B operand of
// dQ^T += K^T dS^T with K staged transposed in LDS.

template <int D>
struct DqSmem {
    static constexpr int RST = D + 8, TST = 64 + 8;
    bf16 Ks[64 * RST];
    bf16 Vs[64 * RST];
    bf16 Kt[D * TST];
};

template <int D>
__global__ __launch_bounds__(256, 1) void dq_bf16_kernel(
    DevPlan P, int Hq, int Hkv, float scale, float scale_log2, const bf16* __restrict__ Q,
    const bf16* __restrict__ K, const bf16* __restrict__ V, const bf16* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, bf16* __restrict__ dQ) {
    constexpr int KS = D / 16, DB = D / 32, C8 = D / 8, NLOAD = 16 * C8;
    constexpr int RST = DqSmem<D>::RST, TST = DqSmem<D>::TST;
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[sizeof(DqSmem<D>)];
    DqSmem<D>& S = *reinterpret_cast<DqSmem<D>*>(smem_raw);

    const int G = Hq / Hkv;
    int grp, hh;
    if (!xcd_group(blockIdx.x, G, P.nQT * Hkv, grp, hh)) return;
    const int qt = P.fwd_order[grp / Hkv];
    const int kvh = grp % Hkv;
    const int h = kvh * G + hh;

    const int T = P.T;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int rr = w * 32 + n;
    const int row = qt * kBq + rr;
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;

    bf16x8 qf[KS], df[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const size_t off = (size_t)row * qstride + (size_t)h * D + 16 * ks + 8 * g;
        qf[ks] = row < T ? ld16(Q + off) : zero8();
        df[ks] = row < T ? ld16(dO + off) : zero8();
    }
    const float lse2 = row < T ? LSE[(size_t)h * T + row] * kLog2e : INFINITY;
    const float dlt = row < T ? Delta[(size_t)h * T + row] : 0.f;
    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();

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
        for (int j = 0; j < 4; ++j) {
            st16(&S.Ks[(4 * rg + j) * RST + 8 * c8], kr[j]);
            st16(&S.Vs[(4 * rg + j) * RST + 8 * c8], vr[j]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 a;
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = kr[j][e];
            st8(&S.Kt[(8 * c8 + e) * TST + 4 * rg], a);
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

        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = zero16();
            dp[kb] = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ak = ld16(&S.Ks[(kb * 32 + n) * RST + 16 * ks + 8 * g]);
                const bf16x8 av = ld16(&S.Vs[(kb * 32 + n) * RST + 16 * ks + 8 * g]);
                s[kb] = mfma_32x32x16(ak, qf[ks], s[kb]);
                dp[kb] = mfma_32x32x16(av, df[ks], dp[kb]);
            }
        }
        const uint64_t bits = pr.y >= 0 ? P.mask_rows[(size_t)pr.y * kBq + rr] : ~0ull;
        bf16x8 sb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int x = kb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
                float p = fast_exp2(s[kb][j] * scale_log2 - lse2);
                if (!((bits >> x) & 1ull)) p = 0.f;
                sb[kb * 2 + (j >> 3)][j & 7] = (bf16)(p * (dp[kb][j] - dlt));
            }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16* krow = &S.Kt[(db * 32 + n) * TST + 16 * kk + 4 * g];
                dq[db] = mfma_32x32x16(cat(ld8(krow), ld8(krow + 8)), sb[kk], dq[db]);
            }
    }

    if (row < T) {
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

// ------------------------------------------------------------------ fp32 (exact float32)

template <int D>
__global__ __launch_bounds__(128) void dq_fp32_kernel(DevPlan P, int Hq, int Hkv, float scale,
                                                      const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      const float* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      const float* __restrict__ Delta,
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
    const float lse = row < T ? LSE[(size_t)h * T + row] : INFINITY;
    const float dlt = row < T ? Delta[(size_t)h * T + row] : 0.f;
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
                const float p = expf(sc * scale - lse);
                const float ds = p * (dp - dlt);
                for (int x = 0; x < D; ++x) acc[x] = fmaf(ds, Ksh[kk][x], acc[x]);
            }
        }
    }
    if (row < T)
        for (int x = 0; x < D; ++x) dQ[row * qstride + (size_t)h * D + x] = scale * acc[x];
}

template <int D>
__global__ __launch_bounds__(64) void dkdv_fp32_kernel(DevPlan P, int Hq, int Hkv, float scale,
                                                       const float* __restrict__ Q,
                                                       const float* __restrict__ K,
                                                       const float* __restrict__ V,
                                                       const float* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       const float* __restrict__ Delta,
                                                       float* __restrict__ dK,
                                                       float* __restrict__ dV) {
    constexpr int CH = 32;
    __shared__ float Qsh[CH][D];
    __shared__ float Dsh[CH][D];
    __shared__ float Lsh[CH], Tsh[CH];
    const int kt = P.bwd_order[blockIdx.x / Hkv];
    const int kvh = blockIdx.x % Hkv;
    const int G = Hq / Hkv;
    const int T = P.T;
    const int kk = threadIdx.x;
    const int key = kt * kBk + kk;
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;
    float k[D], v[D], dk[D], dv[D];
    for (int x = 0; x < D; ++x) {
        k[x] = key < T ? K[key * kvstride + (size_t)kvh * D + x] : 0.f;
        v[x] = key < T ? V[key * kvstride + (size_t)kvh * D + x] : 0.f;
        dk[x] = 0.f;
        dv[x] = 0.f;
    }
    for (int pi = P.kt_ptr[kt]; pi < P.kt_ptr[kt + 1]; ++pi) {
        const int2 pr = P.k_pairs[pi];
        for (int hh = 0; hh < G; ++hh) {
            const int h = kvh * G + hh;
            for (int c = 0; c < kBq / CH; ++c) {
                const int row0 = pr.x * kBq + c * CH;
                __syncthreads();
                for (int idx = threadIdx.x; idx < CH * D; idx += blockDim.x) {
                    const int r = idx / D, x = idx % D;
                    const int row = row0 + r;
                    Qsh[r][x] = row < T ? Q[row * qstride + (size_t)h * D + x] : 0.f;
                    Dsh[r][x] = row < T ? dO[row * qstride + (size_t)h * D + x] : 0.f;
                }
                if (threadIdx.x < CH) {
                    const int row = row0 + threadIdx.x;
                    Lsh[threadIdx.x] = row < T ? LSE[(size_t)h * T + row] : INFINITY;
                    Tsh[threadIdx.x] = row < T ? Delta[(size_t)h * T + row] : 0.f;
                }
                __syncthreads();
                const uint64_t bits =
                    pr.y >= 0 ? P.mask_cols[((size_t)pr.y * kBk + kk) * 2 + (c * CH) / 64] : ~0ull;
                for (int r = 0; r < CH; ++r) {
                    const int qrow = c * CH + r;
                    if (!((bits >> (qrow & 63)) & 1ull) || row0 + r >= T || key >= T) continue;
                    float sc = 0.f, dp = 0.f;
                    for (int x = 0; x < D; ++x) {
                        sc = fmaf(Qsh[r][x], k[x], sc);
                        dp = fmaf(Dsh[r][x], v[x], dp);
                    }
                    const float p = expf(sc * scale - Lsh[r]);
                    const float ds = p * (dp - Tsh[r]);
                    for (int x = 0; x < D; ++x) {
                        dv[x] = fmaf(p, Dsh[r][x], dv[x]);
                        dk[x] = fmaf(ds, Qsh[r][x], dk[x]);
                    }
                }
            }
        }
    }
    if (key < T)
        for (int x = 0; x < D; ++x) {
            dK[key * kvstride + (size_t)kvh * D + x] = scale * dk[x];
            dV[key * kvstride + (size_t)kvh * D + x] = dv[x];
        }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_bwd_delta(bool bf16_, const DevPlan& p, int Hq, int D, const void* o,
                            const void* dout, float* delta, hipStream_t s) {
    const long long pairs = (long long)p.T * Hq;
    if (bf16_) {
        const int per_block = 256 / (D / 8);
        const dim3 grid((unsigned)((pairs + per_block - 1) / per_block));
        if (D == 128)
            hipLaunchKernelGGL(delta_bf16_kernel<128>, grid, dim3(256), 0, s, p.T, Hq,
                               (const bf16*)o, (const bf16*)dout, delta);
        else
            hipLaunchKernelGGL(delta_bf16_kernel<64>, grid, dim3(256), 0, s, p.T, Hq,
                               (const bf16*)o, (const bf16*)dout, delta);
    } else {
        const dim3 grid((unsigned)((pairs + 255) / 256));
        if (D == 128)
            hipLaunchKernelGGL(delta_fp32_kernel<128>, grid, dim3(256), 0, s, p.T, Hq,
                               (const float*)o, (const float*)dout, delta);
        else
            hipLaunchKernelGGL(delta_fp32_kernel<64>, grid, dim3(256), 0, s, p.T, Hq,
                               (const float*)o, (const float*)dout, delta);
    }
    return hipGetLastError();
}

template <int D>
static void dkdv_launch(bool bf16_, const DevPlan& p, int Hq, int Hkv, float scale,
                        const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, const float* delta, void* dk, void* dv, hipStream_t s) {
    if (bf16_)
        hipLaunchKernelGGL(dkdv_bf16_kernel<D>, dim3(xcd_grid((p.nKT + 3) / 4 * Hkv, 4)),
                           dim3(256), 0, s, p, Hq, Hkv, scale, scale * kLog2e, (const bf16*)q,
                           (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse, delta,
                           (bf16*)dk, (bf16*)dv);
    else
        hipLaunchKernelGGL(dkdv_fp32_kernel<D>, dim3(p.nKT * Hkv), dim3(64), 0, s, p, Hq, Hkv,
                           scale, (const float*)q, (const float*)k, (const float*)v,
                           (const float*)dout, lse, delta, (float*)dk, (float*)dv);
}

hipError_t launch_bwd_dkdv(bool bf16_, const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, const float* delta, void* dk, void* dv,
                           hipStream_t s) {
    if (D == 128)
        dkdv_launch<128>(bf16_, p, Hq, Hkv, scale, q, k, v, lse, dout, delta, dk, dv, s);
    else
        dkdv_launch<64>(bf16_, p, Hq, Hkv, scale, q, k, v, lse, dout, delta, dk, dv, s);
    return hipGetLastError();
}

template <int D>
static void dq_launch(bool bf16_, const DevPlan& p, int Hq, int Hkv, float scale, const void* q,
                      const void* k, const void* v, const float* lse, const void* dout,
                      const float* delta, void* dq, hipStream_t s) {
    if (bf16_)
        hipLaunchKernelGGL(dq_bf16_kernel<D>, dim3(xcd_grid(p.nQT * Hkv, Hq / Hkv)), dim3(256), 0,
                           s, p, Hq, Hkv, scale, scale * kLog2e, (const bf16*)q, (const bf16*)k,
                           (const bf16*)v, (const bf16*)dout, lse, delta, (bf16*)dq);
    else
        hipLaunchKernelGGL(dq_fp32_kernel<D>, dim3(p.nQT * Hq), dim3(kBq), 0, s, p, Hq, Hkv,
                           scale, (const float*)q, (const float*)k, (const float*)v,
                           (const float*)dout, lse, delta, (float*)dq);
}

hipError_t launch_bwd_dq(bool bf16_, const DevPlan& p, int Hq, int Hkv, int D, float scale,
                         const void* q, const void* k, const void* v, const float* lse,
                         const void* dout, const float* delta, void* dq, hipStream_t s) {
    if (D == 128)
        dq_launch<128>(bf16_, p, Hq, Hkv, scale, q, k, v, lse, dout, delta, dq, s);
    else
        dq_launch<64>(bf16_, p, Hq, Hkv, scale, q, k, v, lse, dout, delta, dq, s);
    return hipGetLastError();
}

}  // namespace octo
