// Forward of packed-DAG attention on gfx950.
//
// The Octopus trainer runs one block-sparse attention pass over all branches of a
// tree packed into one unpadded 1-D stream (project page, card "03 · Training";
// ia.com.br article, section "Crédito contrafactual ..."): query i attends to
// Ctx(i) only.  The host planner lists, per 128-row query tile, the 64-key KV tiles
// some row sees (FULL, or PARTIAL with a per-row bit mask); this kernel walks that
// list with an online softmax.
//
// bf16 kernel: one workgroup = one query tile for HPW query heads of one KV group
// (HPW = 2 when the group size is even), 4 wave64s per head, each owning 32 query
// rows.  Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 so
// that every lane holds one query column: the row max and row sum are in-lane plus
// one exchange with lane ^ 32, and the probabilities come out of the accumulator
// already laid out as the B operand of O^T = V^T P^T.  K tiles (XOR-swizzled rows) and
// V tiles re-laid by tiles_t_kernel (so every V^T operand is one 16-byte LDS read) are
// copied global -> LDS asynchronously, three stages in flight, together with the query
// tile's row masks.
// Workgroups of one KV group are launched adjacently on one XCD so their shared K/V
// tiles hit the same L2.
#include "device_common.h"
#include "kernels.h"
#include "kvstage.h"

namespace octo {

// Forward.  HPW query heads (of one KV group) per workgroup, 4 waves per head, each
// wave owning 32 query rows.
// One workgroup per (64-key tile, KV head): the tile's 64 x D block of src, read
// row by row, written out in the tiles_t order (see kernels.h).
template <int D>
__global__ __launch_bounds__(256) void tiles_t_kernel(int T, int nKT, int Hkv,
                                                      const bf16* __restrict__ src,
                                                      bf16* __restrict__ dst) {
    constexpr int RS = D + 8;  // padded LDS row, elements
    __shared__ __attribute__((aligned(16))) bf16 tile[64 * RS];
    const int kt = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
    for (int i = threadIdx.x; i < 64 * D / 8; i += 256) {
        const int r = i / (D / 8), c8 = i % (D / 8);
        const int key = kt * kBk + r;
        const bf16x8 v = key < T ? ld16(src + ((size_t)key * Hkv + kvh) * D + 8 * c8) : zero8();
        st16(tile + r * RS + 8 * c8, v);
    }
    __syncthreads();
    bf16* out = dst + ((size_t)kvh * nKT + kt) * (64 * D);
    for (int u = threadIdx.x; u < 8 * D; u += 256) {  // u = chunk * D + row
        const int c = u / D, d = u % D;
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[(16 * (c >> 1) + kperm(8 * (c & 1) + e)) * RS + d];
        st16(out + (size_t)u * 8, v);
    }
}

size_t tiles_t_bytes(int nKT, int Hkv, int D) { return (size_t)Hkv * nKT * 64 * D * 2; }

hipError_t launch_tiles_t(int T, int nKT, int Hkv, int D, const void* src, void* dst,
                          hipStream_t s) {
    if (D == 128)
        hipLaunchKernelGGL(tiles_t_kernel<128>, dim3(nKT * Hkv), dim3(256), 0, s, T, nKT, Hkv,
                           (const bf16*)src, (bf16*)dst);
    else
        hipLaunchKernelGGL(tiles_t_kernel<64>, dim3(nKT * Hkv), dim3(256), 0, s, T, nKT, Hkv,
                           (const bf16*)src, (bf16*)dst);
    return hipGetLastError();
}

// With ROPE, Q is given unrotated and each lane turns its query row's operand in
// registers at the row's plan position (K comes rotated).
template <int D, int HPW, bool ROPE>
__global__ __launch_bounds__(256 * HPW, 1) void fwd_bf16_kernel(
    DevPlan P, int Hq, int Hkv, float scale_log2, const bf16* __restrict__ Q,
    const bf16* __restrict__ K, const bf16* __restrict__ VX, bf16* __restrict__ O,
    float* __restrict__ LSE, RopeFreq rt) {
    using L = KvLayout<D>;
    constexpr int NTHR = 256 * HPW;
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int PER_STAGE = 2 * (L::MAT / (16 * NTHR)) + 1;
    // A row's running max moves only when a tile exceeds it by more than 2^8 (log2
    // units): probabilities stay below 256, and the final division by the running sum
    // makes the result independent of where the max was taken.
    constexpr float kLazy = 8.f;
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
    const int T = P.T;
    const int rr = (w & 3) * 32 + n;  // row inside the query tile
    const int row = qt * kBq + rr;
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;
    const unsigned smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = row < T ? ld16(Q + row * qstride + (size_t)h * D + 16 * ks + 8 * g) : zero8();
    if constexpr (ROPE) {
        if (row < T) rope_operand(qf, P.pos[row], rt, g, 1.f);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);

    KvOffsets<D> off;
    off.init(lane);
    const int off_mask = L::M0 + rr * 8;
    const int ovx = L::V0 + tile_t_lane<D>(lane);  // V^T operands (tiles_t layout)
    TileDma<D, NTHR> dm;
    dm.init(tid, kvstride);

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();
    float m = -1e30f, l = 0.f;

    const int p0 = ld_const(P.qt_ptr + qt), p1 = ld_const(P.qt_ptr + qt + 1);
    const int n_it = p1 - p0;
    // The tile pair of the next iteration to issue (index jn) is loaded at the end of the
    // iteration before (`fetch_pair`), where it is not waited for until the next LDS wait:
    // a scalar load waited for right after the barrier would stall every iteration.
    // `partial` keeps, per stage, whether its tile is PARTIAL.
    int jn = 0;
    int2 jpr = n_it > 0 ? ld_const(P.q_pairs + p0) : make_int2(0, -1);
    bool partial[3];
    auto fetch_pair = [&]() {
        __builtin_amdgcn_sched_barrier(0);  // after everything else of the iteration
        asm volatile("" ::: "memory");
        jpr = ld_const(P.q_pairs + p0 + min(jn, n_it - 1));
    };
    auto issue = [&](auto st_c, int it) {
        constexpr int ST = decltype(st_c)::value;
        const int2 pr = jpr;
        asm volatile("" ::"s"(pr.x), "s"(pr.y));
        partial[ST] = pr.y >= 0;
        ++jn;
        issue_kv_stage<D, NTHR, ST, false>(smem_base, K, nullptr, P.mask_rows, pr.x,
                                           pr.y >= 0 ? pr.y : P.n_partial, T, kvh, kvstride, dm,
                                           tid, w, lane);
        issue_tile_t<D, NTHR>(smem_base, L::V0 + ST * L::MAT, VX, P.nKT, kvh, pr.x, tid, w);
    };

    auto step = [&](auto st_c, int it) {
        constexpr int ST = decltype(st_c)::value;
        if (it + 1 < n_it) wait_vmem<PER_STAGE>();
        else wait_vmem<0>();
        barrier();
        if (it + 2 < n_it) issue(ic<(ST + 2) % 3>{}, it + 2);

        // S^T (64 keys x 32 queries) = K Q^T, two 32-key blocks.
        f32x16 s[2];
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[0] = mfma_32x32x16(lds16(smem, off.k[ks], ST * L::MAT), qf[ks], s[0]);
            s[1] = mfma_32x32x16(lds16(smem, off.k[ks], ST * L::MAT + 32 * L::ROWB), qf[ks], s[1]);
        }
        lead_reads<2 * KS>();
        if (partial[ST]) {
            const uint64_t bits =
                *reinterpret_cast<const uint64_t*>(smem + off_mask + ST * L::MASKB);
            const uint32_t b0 = (uint32_t)(bits >> (4 * g)), b1 = (uint32_t)(bits >> (32 + 4 * g));
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int x = 8 * (j >> 2) + (j & 3);
                if (!((b0 >> x) & 1u)) s[0][j] = -INFINITY;
                if (!((b1 >> x) & 1u)) s[1][j] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(fmaxf(mx, s[0][j]), s[1][j]);  // v_max3
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
        if (__any(mx > m + kLazy)) {
            const float mnew = fmaxf(m, mx);
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        }
        bf16x8 pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                pf[kb * 2 + (j >> 3)][j & 7] = (bf16)fast_exp2(fmaf(s[kb][j], scale_log2, -m));
        // Row sum of the bf16 probabilities that enter O, two per instruction.
#pragma unroll
        for (int i = 0; i < 4; ++i) l = row_sum8(pf[i], l);
        // O^T += V^T P^T over 4 k-steps of 16 keys; the lane's 8 keys in k-step kk are
        // 16kk + 4g + {0..3} and 16kk + 8 + 4g + {0..3}, contiguous in the V tile.
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = mfma_32x32x16(lds16(smem, ovx, ST * L::MAT + tile_t_imm<D>(kk, db)),
                                      pf[kk], o[db]);
        lead_reads<4 * DB>();
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

template <int D, int HPW>
static void fwd_bf16_launch(const DevPlan& p, int Hq, int Hkv, float sl2, const void* q,
                            const void* k, const void* vx, void* o, float* lse,
                            const RopeFreq* rope, hipStream_t s) {
    const int G = Hq / Hkv;
    const dim3 grid(xcd_grid(p.nQT * Hkv, G / HPW)), block(256 * HPW);
    const RopeFreq rt = rope ? *rope : RopeFreq{};
    if (rope)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, HPW, true>), grid, block, 0, s, p, Hq, Hkv, sl2,
                           (const bf16*)q, (const bf16*)k, (const bf16*)vx, (bf16*)o, lse, rt);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, HPW, false>), grid, block, 0, s, p, Hq, Hkv, sl2,
                           (const bf16*)q, (const bf16*)k, (const bf16*)vx, (bf16*)o, lse, rt);
}

hipError_t launch_fwd_bf16(const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* vx, void* o, float* lse,
                           const RopeFreq* rope, hipStream_t s) {
    const float sl2 = scale * kLog2e;
    const bool pair = (Hq / Hkv) % 2 == 0;
    if (D == 128) {
        if (pair) fwd_bf16_launch<128, 2>(p, Hq, Hkv, sl2, q, k, vx, o, lse, rope, s);
        else fwd_bf16_launch<128, 1>(p, Hq, Hkv, sl2, q, k, vx, o, lse, rope, s);
    } else {
        if (pair) fwd_bf16_launch<64, 2>(p, Hq, Hkv, sl2, q, k, vx, o, lse, rope, s);
        else fwd_bf16_launch<64, 1>(p, Hq, Hkv, sl2, q, k, vx, o, lse, rope, s);
    }
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
