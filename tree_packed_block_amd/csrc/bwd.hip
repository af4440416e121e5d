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
//   3. dQ (dq.hip): one workgroup per query tile and pair of query heads, like the
//      forward.
// Scores are recomputed from LSE in both 2 and 3.
#include "device_common.h"
#include "kernels.h"
#include "kvstage.h"

namespace octo {

// ------------------------------------------------------------------ preprocess
//
// Workspace (float32): LSE2[Hq][Tp] = LSE * log2(e) and Delta[Hq][Tp], Tp = T rounded
// up to a multiple of the 128-row query tile.  Rows >= T hold LSE2 = +inf and
// Delta = 0, so a padded row gets P = 0 and dS = 0 with no per-row test, and every
// 64-row run of a query tile is in bounds and 16-byte aligned.


template <int D>
__global__ __launch_bounds__(256) void preprocess_bf16_kernel(int T, int Tp, int Hq,
                                                              const bf16* __restrict__ O,
                                                              const bf16* __restrict__ dO,
                                                              const float* __restrict__ LSE,
                                                              float* __restrict__ ws) {
    constexpr int L = D / 8;  // lanes per (row, head)
    const long long pair = ((long long)blockIdx.x * blockDim.x + threadIdx.x) / L;
    const int sub = threadIdx.x % L;
    const bool valid = pair < (long long)Tp * Hq;
    const int row = (int)(pair / Hq), h = (int)(pair % Hq);
    float acc = 0.f;
    if (valid && row < T) {
        const bf16x8 a = ld16(O + pair * D + 8 * sub);
        const bf16x8 b = ld16(dO + pair * D + 8 * sub);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    }
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, L);
    if (valid && sub == 0) {
        ws[(size_t)h * Tp + row] = row < T ? LSE[(size_t)h * T + row] * kLog2e : INFINITY;
        ws[(size_t)Hq * Tp + (size_t)h * Tp + row] = acc;
    }
}

template <int D>
__global__ __launch_bounds__(256) void preprocess_fp32_kernel(int T, int Tp, int Hq,
                                                              const float* __restrict__ O,
                                                              const float* __restrict__ dO,
                                                              const float* __restrict__ LSE,
                                                              float* __restrict__ ws) {
    const long long pair = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (pair >= (long long)Tp * Hq) return;
    const int row = (int)(pair / Hq), h = (int)(pair % Hq);
    float acc = 0.f;
    if (row < T)
        for (int d = 0; d < D; ++d) acc = fmaf(O[pair * D + d], dO[pair * D + d], acc);
    ws[(size_t)h * Tp + row] = row < T ? LSE[(size_t)h * T + row] * kLog2e : INFINITY;
    ws[(size_t)Hq * Tp + (size_t)h * Tp + row] = acc;
}

// ------------------------------------------------------------------ dK / dV (bf16)
//
// Workgroup = (128-key block = KV tiles 2b and 2b+1, KV head), 4 wave64s in two pairs;
// pair p owns the 64 keys of tile 2b+p, and inside a pair wave 0 accumulates dK and
// wave 1 dV for all 64 keys.  The workgroup walks the block's merged list of query
// tiles; for every entry, every query head of the group and each 64-row half of the
// query tile, the Q and dO rows (and their LSE2/Delta) are copied global -> LDS
// asynchronously (three stages in flight).  In a pair each wave takes 32 of the 64
// rows: S = Q K^T and dP = dO V^T for its rows against the pair's 64 keys (K and V are
// register-resident B operands, so a lane owns one key column per 32-key block), then
// P and dS.  The dK wave hands its P rows to the dV wave and receives the dV wave's dS
// rows through LDS, after which dV^T += dO^T P and dK^T += Q^T dS run over all 64 rows
// with A operands read transposed from the row-major tiles (ds_read_b64_tr_b16).  Each
// A operand read from LDS thus feeds two MFMAs (two 32-key blocks), which halves LDS
// traffic per MFMA against one wave per 32 keys.  The row terms enter the MFMA as one
// extra k-step: a lane's own row value (-LSE2/(scale log2 e) for S, -Delta for dP) is
// split into three bf16 parts that multiply a column of ones, so the accumulators come
// out as S - LSE/scale and dP - Delta without any per-element loads.  Every dK/dV row
// has one writer; there are no atomics.

// LDS layout of the dK/dV stages, stage-major by kind: [Q x 3][dO x 3][LSE2/Delta x 3]
// [key-major mask words x 3], then two sets of 4 KiB hand-over buffers, one per wave.
template <int D>
struct DkdvLayout {
    static constexpr int ROWB = D * 2;               // bytes per row
    static constexpr int MAT = 64 * ROWB;            // one 64-row Q or dO chunk
    static constexpr int NST = 3;                    // stages in flight
    static constexpr int NDMA = MAT / (16 * 256);    // copies per thread per matrix
    static constexpr int Q0 = 0;
    static constexpr int D0 = NST * MAT;
    static constexpr int L0 = 2 * NST * MAT;         // LSE2[64] then Delta[64] per stage
    static constexpr int M0 = L0 + NST * 512;        // 2 tiles x 64 keys x 2 words
    static constexpr int MASKB = 4 * 512;
    static constexpr int X0 = M0 + NST * MASKB;      // hand-over: 4 B operands per wave,
    static constexpr int XB = 4 * 4096;              // two buffers by iteration parity
    static constexpr int BYTES = X0 + 2 * XB;
    static constexpr int PER_STAGE = 2 * NDMA + 2;   // copies per wave per stage
};


// One wave of a dK/dV workgroup.  ROLE 0 accumulates dK (and hands P to its partner),
// ROLE 1 accumulates dV (and hands dS over).  Both roles run the same sequence of
// barriers.
// With ROPE, Q and K come rotated at the plan's positions and the dK wave turns its
// result back at the keys' positions before storing it (the gradient with respect to the
// unrotated K; the rotation is orthogonal).
template <int D, int ROLE, bool ROPE>
__device__ __forceinline__ void dkdv_wave(const DevPlan& P, int Hq, int Hkv, int kb, int kvh,
                                          float scale, float scale_log2,
                                          const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                          const bf16* __restrict__ V, const bf16* __restrict__ dO,
                                          const float* __restrict__ ws, bf16* __restrict__ out,
                                          unsigned char* smem, const RopeFreq& rt) {
    using C = DkdvLayout<D>;
    constexpr int KS = D / 16, DB = D / 32, CPR = D / 8;
    const int T = P.T, G = Hq / Hkv, Tp = padded_rows(T);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int pr = w >> 1;                                    // pair = KV tile 2kb+pr
    const int n = lane & 31, g = lane >> 5;
    const int key0 = kb * 128 + 64 * pr + n;                  // + 32 per key block
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;
    const float* LSE2 = ws;
    const float* DEL = ws + (size_t)Hq * Tp;
    const unsigned smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    const float inv_sl2 = 1.f / scale_log2;

    // K enters the scores pre-multiplied by scale * log2(e) (rounded to bf16), so the
    // S accumulator is directly the exponent of P.
    bf16x8 kf[2][KS], vf[2][KS];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int key = key0 + 32 * kk;
            const size_t off = (size_t)key * kvstride + (size_t)kvh * D + 16 * ks + 8 * g;
            const bf16x8 kr = key < T ? ld16(K + off) : zero8();
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[kk][ks][e] = (bf16)((float)kr[e] * scale_log2);
            vf[kk][ks] = key < T ? ld16(V + off) : zero8();
        }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            settle(kf[kk][ks]);
            park(vf[kk][ks]);
        }
    bf16x8 ones = zero8();
    if (g == 0) ones[0] = ones[1] = ones[2] = (bf16)1.f;

    f32x16 acc[2][DB];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[kk][db] = zero16();

    // Per-lane LDS offsets.  Row-major reads: row n of this wave's 32 rows, chunk 2ks+g
    // (the wave's +32 rows and the stage go into the immediate).  Transposed reads:
    // rows 4g + r/4 (+8) of each 16-row k-step of Q (ROLE 0) or dO (ROLE 1).
    const int r_in = lane & 15, dh = (lane >> 4) & 1;
    int oq[KS], ot[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        oq[ks] = C::Q0 + n * C::ROWB + (((2 * ks + g) ^ swz_key<D>(n)) * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int r = 4 * g + (r_in >> 2) + 8 * hf;
            const int chunk = 4 * db + 2 * dh + ((r_in & 3) >> 1);
            ot[db][hf] = (ROLE == 0 ? C::Q0 : C::D0) + r * C::ROWB +
                         ((chunk ^ swz_key<D>(r)) * 16) + 8 * (r_in & 1);
        }
    const int ol = C::L0 + (32 * ROLE + n) * 4;          // this lane's row: LSE2, +256 Delta
    const int om = C::M0 + pr * 1024 + n * 16 + 4 * ROLE; // + 512 kk + 8 c: 32 mask bits
    const int ox = C::X0 + w * 4096 + lane * 16;          // own hand-over slots
    const int ox_in = C::X0 + (w ^ 1) * 4096 + lane * 16; // partner's

    const int e0 = ld_const(P.blk_ptr + kb), e1 = ld_const(P.blk_ptr + kb + 1);
    const int n_it = (e1 - e0) * G * 2;  // (entry, head, 64-row half)
    if (n_it == 0) return;
    TileDma<D, 256> dm;  // per-lane offsets of the copies
    dm.init(tid, qstride);
    const unsigned off_ld = (unsigned)((4 * ((8 * w + (lane & 7)) & 15)) * 4);
    const unsigned off_mk = (unsigned)((32 * (w & 1) + (lane & 31)) * 16);
    const int n_run = (n_it + 2) / 3 * 3;  // iterations run: whole rounds of 3 stages

    // Copies of iteration `it` into stage ST: the 64 rows of Q and dO, their LSE2 and
    // Delta, and this wave's 32 key-major mask words (the all-ones mask for a FULL tile,
    // the all-zeros one for a tile the query tile does not see and for the padding
    // iterations it >= n_it, which repeat the last entry and so contribute nothing).
    // The entries are walked from the last query tile down: the key blocks of one branch
    // then start on the same query tiles together and share them in L2.
    // The iterations are issued in order; (je, jh, jc) are the next one's entry, head and
    // half, stepped without divisions.  Its entry is loaded at the end of the iteration
    // before (`fetch_entry`), where the wait ahead of the barrier covers it: a scalar load
    // in flight turns every LDS wait into a full one (scalar loads complete out of order),
    // so none is left outstanding in the middle of an iteration.  `masked` keeps, per
    // stage, whether the iteration using it needs its mask (PARTIAL, unseen or padding).
    int je = e1 - 1, jh = 0, jc = 0;
    int4 jent = ld_const(P.blk_entries + je);
    bool masked[3];
    auto fetch_entry = [&]() {
        asm volatile("" ::: "memory");
        jent = ld_const(P.blk_entries + je);
    };
    auto issue = [&](auto st_c, int it) {
        constexpr int ST = decltype(st_c)::value;
        const bool pad = it >= n_it;
        const int h = kvh * G + jh;
        const int4 ent = jent;
        // all four loaded registers stay live until here (otherwise the unused fourth one
        // is reused while the load is in flight, which forces an early wait)
        asm volatile("" ::"s"(ent.x), "s"(ent.y), "s"(ent.z), "s"(ent.w));
        const int row0 = ent.x * kBq + jc * 64;
        if (++jc == 2) {
            jc = 0;
            if (++jh == G) {
                jh = 0;
                je = max(je - 1, e0);
            }
        }
        const int mraw = pr ? ent.z : ent.y;
        masked[ST] = mraw != -1 || pad;
        issue_rows<D, 256>(smem_base, C::Q0 + ST * C::MAT, Q, row0, T, h, qstride, dm, tid, w);
        issue_rows<D, 256>(smem_base, C::D0 + ST * C::MAT, dO, row0, T, h, qstride, dm, tid, w);
        if (lane < 8)  // 32 pieces of 16 bytes, 8 per wave: LSE2 (waves 0, 1), Delta (2, 3)
            dma16_s((w < 2 ? LSE2 : DEL) + (size_t)h * Tp + row0, off_ld,
                    smem_base + C::L0 + ST * 512 + 8 * w * 16);
        if (lane < 32) {
            int mk = pr ? ent.z : ent.y;
            mk = pad || mk == -2 ? P.n_partial + 1 : (mk == -1 ? P.n_partial : mk);
            dma16_s(P.mask_cols + (size_t)mk * kBk * 2, off_mk,
                    smem_base + C::M0 + ST * C::MASKB + w * 512);
        }
    };

    // The wave's MFMAs over the partner's rows of one iteration run in the next one,
    // interleaved with that iteration's softmax: `ap` carries their A operands (read
    // before the barrier that ends the iteration) and the partner's B operands come
    // from the hand-over buffer of that iteration's parity.
    bf16x8 ap[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) ap[db][0] = ap[db][1] = zero8();
#pragma unroll
    for (int i = 0; i < 2 * 4; ++i)  // both hand-over buffers start as zeros
        *reinterpret_cast<bf16x8*>(smem + ox + (i >> 2) * C::XB + (i & 3) * 1024) = zero8();

    auto partner_mfmas = [&](int xoff) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ql = 0; ql < 2; ++ql) {
                const bf16x8 part = lds16(smem, ox_in + xoff, (2 * kk + ql) * 1024);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[kk][db] = mfma_32x32x16(ap[db][ql], part, acc[kk][db]);
            }
    };

    // One iteration: S, dP, P and dS for this wave's 32 rows; the previous iteration's
    // partner rows; the hand-over; dV or dK over this wave's own rows.
    auto step = [&](auto st_c, int it) {
        constexpr int ST = decltype(st_c)::value;
        wait_vmem<C::PER_STAGE>();
        wait_lds();
        barrier();
        issue(ic<(ST + 2) % 3>{}, it + 2);
        const int c = it & 1;
        const int xcur = (it & 1) * C::XB, xprev = C::XB - xcur;

        const float l2 = *reinterpret_cast<const float*>(smem + ol + ST * 512);
        const float dl = *reinterpret_cast<const float*>(smem + ol + ST * 512 + 256);
        const bf16x8 xl = split3(-l2, g == 0);
        const bf16x8 xd = split3(-dl, g == 0);
        // A operands: all eight Q k-steps are read first, the dO k-steps one per pair
        // of S MFMAs, so the reads run ahead of the MFMAs that consume them.
        bf16x8 aq[KS], ad[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            aq[ks] = lds16(smem, oq[ks], ST * C::MAT + ROLE * 32 * C::ROWB);
        f32x16 sc[2], dp[2];
        // S (exponent of P: scale log2e Q K^T - LSE2), then dP - Delta.
        sc[0] = sc[1] = mfma_32x32x16(xl, ones, zero16());
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) sc[kk] = mfma_32x32x16(aq[ks], kf[kk][ks], sc[kk]);
            ad[ks] = lds16(smem, oq[ks] - C::Q0 + C::D0, ST * C::MAT + ROLE * 32 * C::ROWB);
        }
        dp[0] = dp[1] = mfma_32x32x16(xd, ones, zero16());
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) dp[kk] = mfma_32x32x16(ad[ks], vf[kk][ks], dp[kk]);
        __builtin_amdgcn_sched_group_barrier(0x100, KS + 2, 0);  // LSE2, Delta, Q reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        // The previous iteration's partner rows, overlapping the softmax below.
        partner_mfmas(xprev);
        // keep: the B operand this wave uses itself (dS for dK, P for dV); give: the
        // partner's.  Index [kk][ql]: 32-key block, 16-row k-step of this wave's rows;
        // slot e of lane (n, g) is row 16 ql + 4g + e (e < 4) or 16 ql + 8 + 4g + e - 4.
        bf16x8 keep[2][2], give[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float pv = fast_exp2(sc[kk][j]);
                const float dsv = pv * dp[kk][j];
                if constexpr (ROLE == 0) {
                    keep[kk][j >> 3][j & 7] = (bf16)dsv;
                    give[kk][j >> 3][j & 7] = (bf16)pv;
                } else {
                    keep[kk][j >> 3][j & 7] = (bf16)pv;
                    give[kk][j >> 3][j & 7] = (bf16)dsv;
                }
            }
        if (__builtin_expect(masked[ST], 0)) {  // wave-uniform and rare: clear P and dS where
            asm volatile("");                  // the mask is 0 (a real branch, not selects)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint32_t mb = *reinterpret_cast<const uint32_t*>(
                                        smem + om + ST * C::MASKB + 512 * kk + 8 * c) >> (4 * g);
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (!((mb >> (8 * (j >> 2) + (j & 3))) & 1u)) {
                        keep[kk][j >> 3][j & 7] = (bf16)0.f;
                        give[kk][j >> 3][j & 7] = (bf16)0.f;
                    }
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ql = 0; ql < 2; ++ql)
                *reinterpret_cast<bf16x8*>(smem + ox + xcur + (2 * kk + ql) * 1024) = give[kk][ql];
        // A operands of the partner's rows, for the next iteration.
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int ql = 0; ql < 2; ++ql) {
                const int imm = ST * C::MAT + (32 * (1 - ROLE) + 16 * ql) * C::ROWB;
                ap[db][ql] = cat(lds8_tr(smem, ot[db][0], imm), lds8_tr(smem, ot[db][1], imm));
            }
        // This wave's own 32 rows.
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int ql = 0; ql < 2; ++ql) {
                const int imm = ST * C::MAT + (32 * ROLE + 16 * ql) * C::ROWB;
                const bf16x8 a = cat(lds8_tr(smem, ot[db][0], imm), lds8_tr(smem, ot[db][1], imm));
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc[kk][db] = mfma_32x32x16(a, keep[kk][ql], acc[kk][db]);
            }
        fetch_entry();
    };

    issue(ic<0>{}, 0);
    fetch_entry();
    issue(ic<1>{}, 1);
    fetch_entry();
    for (int it = 0; it < n_run; it += 3) {
        step(ic<0>{}, it);
        step(ic<1>{}, it + 1);
        step(ic<2>{}, it + 2);
    }
    wait_lds();
    barrier();
    partner_mfmas(((n_run - 1) & 1) * C::XB);
    wait_vmem<0>();  // the trailing copies land before the workgroup's LDS is released

    const float os = ROLE == 0 ? scale : 1.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int key = key0 + 32 * kk;
        if (key >= T) continue;
        if constexpr (ROPE && ROLE == 0) rope_accum(acc[kk], P.pos[key], rt, g, -1.f);
        bf16* row = out + (size_t)key * kvstride + (size_t)kvh * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                bf16x4 a;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) a[e2] = (bf16)(os * acc[kk][db][4 * q4 + e2]);
                st8(row + db * 32 + 8 * q4 + 4 * g, a);
            }
    }
}

template <int D, bool ROPE>
__global__ __launch_bounds__(256, 1) void dkdv_bf16_kernel(
    DevPlan P, int Hq, int Hkv, float scale, float scale_log2, const bf16* __restrict__ Q,
    const bf16* __restrict__ K, const bf16* __restrict__ V, const bf16* __restrict__ dO,
    const float* __restrict__ ws, bf16* __restrict__ dK, bf16* __restrict__ dV, RopeFreq rt) {
    constexpr int M = 4;  // consecutive blocks of one KV head dealt to one XCD
    __shared__ __attribute__((aligned(1024))) unsigned char smem[DkdvLayout<D>::BYTES];
    int grp, mm;
    if (!xcd_group(blockIdx.x, M, (P.nKB + M - 1) / M * Hkv, grp, mm)) return;
    const int rank = (grp / Hkv) * M + mm;
    if (rank >= P.nKB) return;
    const int kvh = grp % Hkv;
    const int kb = ld_const(P.blk_order + rank);
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1)
        dkdv_wave<D, 1, ROPE>(P, Hq, Hkv, kb, kvh, scale, scale_log2, Q, K, V, dO, ws, dV, smem,
                              rt);
    else
        dkdv_wave<D, 0, ROPE>(P, Hq, Hkv, kb, kvh, scale, scale_log2, Q, K, V, dO, ws, dK, smem,
                              rt);
}

// ------------------------------------------------------------------ fp32 (exact float32)

template <int D>
__global__ __launch_bounds__(64) void dkdv_fp32_kernel(DevPlan P, int Hq, int Hkv, float scale,
                                                       const float* __restrict__ Q,
                                                       const float* __restrict__ K,
                                                       const float* __restrict__ V,
                                                       const float* __restrict__ dO,
                                                       const float* __restrict__ ws,
                                                       float* __restrict__ dK,
                                                       float* __restrict__ dV) {
    constexpr int CH = 32;
    __shared__ float Qsh[CH][D];
    __shared__ float Dsh[CH][D];
    __shared__ float Lsh[CH], Tsh[CH];
    const int kt = P.bwd_order[blockIdx.x / Hkv];
    const int kvh = blockIdx.x % Hkv;
    const int G = Hq / Hkv;
    const int T = P.T, Tp = padded_rows(T);
    const float sl2 = scale * kLog2e;
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
                    Lsh[threadIdx.x] = ws[(size_t)h * Tp + row];
                    Tsh[threadIdx.x] = ws[(size_t)Hq * Tp + (size_t)h * Tp + row];
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
                    const float p = exp2f(sc * sl2 - Lsh[r]);
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

size_t bwd_workspace_floats(int T, int Hq) { return (size_t)2 * Hq * padded_rows(T); }


hipError_t launch_bwd_preprocess(bool bf16_, const DevPlan& p, int Hq, int D, const void* o,
                                 const void* dout, const float* lse, float* ws, hipStream_t s) {
    const int Tp = padded_rows(p.T);
    const long long pairs = (long long)Tp * Hq;
    if (bf16_) {
        const int per_block = 256 / (D / 8);
        const dim3 grid((unsigned)((pairs + per_block - 1) / per_block));
        if (D == 128)
            hipLaunchKernelGGL(preprocess_bf16_kernel<128>, grid, dim3(256), 0, s, p.T, Tp, Hq,
                               (const bf16*)o, (const bf16*)dout, lse, ws);
        else
            hipLaunchKernelGGL(preprocess_bf16_kernel<64>, grid, dim3(256), 0, s, p.T, Tp, Hq,
                               (const bf16*)o, (const bf16*)dout, lse, ws);
    } else {
        const dim3 grid((unsigned)((pairs + 255) / 256));
        if (D == 128)
            hipLaunchKernelGGL(preprocess_fp32_kernel<128>, grid, dim3(256), 0, s, p.T, Tp, Hq,
                               (const float*)o, (const float*)dout, lse, ws);
        else
            hipLaunchKernelGGL(preprocess_fp32_kernel<64>, grid, dim3(256), 0, s, p.T, Tp, Hq,
                               (const float*)o, (const float*)dout, lse, ws);
    }
    return hipGetLastError();
}

template <int D>
static void dkdv_launch(bool bf16_, const DevPlan& p, int Hq, int Hkv, float scale,
                        const void* q, const void* k, const void* v, const void* dout,
                        const float* ws, void* dk, void* dv, const RopeFreq* rope,
                        hipStream_t s) {
    const dim3 grid(xcd_grid((p.nKB + 3) / 4 * Hkv, 4));
    const RopeFreq rt = rope ? *rope : RopeFreq{};
    if (bf16_ && rope)
        hipLaunchKernelGGL((dkdv_bf16_kernel<D, true>), grid, dim3(256), 0, s, p, Hq, Hkv, scale,
                           scale * kLog2e, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                           (const bf16*)dout, ws, (bf16*)dk, (bf16*)dv, rt);
    else if (bf16_)
        hipLaunchKernelGGL((dkdv_bf16_kernel<D, false>), grid, dim3(256), 0, s, p, Hq, Hkv, scale,
                           scale * kLog2e, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                           (const bf16*)dout, ws, (bf16*)dk, (bf16*)dv, rt);
    else
        hipLaunchKernelGGL(dkdv_fp32_kernel<D>, dim3(p.nKT * Hkv), dim3(64), 0, s, p, Hq, Hkv,
                           scale, (const float*)q, (const float*)k, (const float*)v,
                           (const float*)dout, ws, (float*)dk, (float*)dv);
}

hipError_t launch_bwd_dkdv(bool bf16_, const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, const void* dout,
                           const float* ws, void* dk, void* dv, const RopeFreq* rope,
                           hipStream_t s) {
    if (D == 128) dkdv_launch<128>(bf16_, p, Hq, Hkv, scale, q, k, v, dout, ws, dk, dv, rope, s);
    else dkdv_launch<64>(bf16_, p, Hq, Hkv, scale, q, k, v, dout, ws, dk, dv, rope, s);
    return hipGetLastError();
}

}  // namespace octo
