// Chunked branch-aware gated delta-rule scan on gfx950 (matrix cores).
//
// The recurrence of the hybrid backbone's Gated DeltaNet layers (Octopus project page,
// primitives table: `fork` clones the parent's recurrent checkpoint, mounted spans
// bypass the recurrent layers), per head with state S (Dv x Dk):
//     S_t = alpha_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
// is applied 32 tokens at a time.  Within a chunk starting from S_0, with
// gamma_t = alpha_1 ... alpha_t, the state is
//     S_t = gamma_t S_0 + sum_{i<=t} (gamma_t / gamma_i) w_i k_i^T
// where the rows w_t solve the unit lower-triangular system
//     w_t + beta_t sum_{i<t} (gamma_t / gamma_i) (k_t . k_i) w_i = beta_t (v_t - gamma_t S_0 k_t),
// so that, as matrices over the chunk (rows = tokens),
//     W = solve(I + diag(beta) (K K^T o Gamma_strict), diag(beta) (V - diag(gamma) K S_0^T))
//     O = diag(gamma) Q S_0^T + (Q K^T o Gamma_incl) W
//     S_C = gamma_C S_0 + W^T diag(gamma_C / gamma) K.
// (Gamma[t][i] = gamma_t / gamma_i <= 1: every factor is bounded.)  These are the
// chunk-wise products of the published gated delta rule (Yang, Kautz and Hatamizadeh,
// 2024), restated for this kernel's layout.
//
// One workgroup per (branch, head) walks the branch's chunks in order; chunk boundaries
// fall every 32 own tokens and at every offset where a child forks (its checkpoint is the
// state there).  Value rows evolve independently, so wave w owns value rows
// [32 w, 32 w + 32) of the state, held transposed in MFMA accumulators (S^T: 4 tiles of
// 32 keys x 32 values, lane = value row), and needs no other wave's data: the chunk's
// K, Q, V, alpha, beta are staged once in LDS for all four waves.  Products whose operands
// are bf16 inputs (K K^T, Q K^T) are exact on v_mfma_f32_32x32x16_bf16; operands held in
// float32 (the state, W, the gated score matrix) enter as a bf16 high part plus a bf16
// low part (relative error below 2^-16 per operand).  The 32-row triangular solve runs
// on the vector unit, each lane holding 16 rows of one value column and exchanging
// partial sums with its partner lane.
#include "device_common.h"
#include "kernels.h"

namespace octo {

namespace {

constexpr int kD = 128;         // Dk = Dv
constexpr int kC = 32;          // tokens per chunk
constexpr int kWaves = kD / 32; // one wave per 32 value rows
constexpr int kThr = 64 * kWaves;
constexpr int kRowB = kD * 2;   // bytes of one bf16 row

// Element e of hi and lo take x as hi + lo, both bf16 (|x - hi - lo| <= 2^-16 |x|).
__device__ __forceinline__ void split2(float x, bf16x8& hi, bf16x8& lo, int e) {
    const bf16 h = (bf16)x;
    hi[e] = h;
    lo[e] = (bf16)(x - (float)h);
}

// x plus the value of the lane 32 away (the other half of the wave).
__device__ __forceinline__ float pair_sum(float x) { return x + __shfl_xor(x, 32); }

// Row r of the chunk's lane layout: accumulator element j of lane half g holds row
// 8 (j / 4) + 4 g + j % 4.
__device__ __forceinline__ constexpr int acc_row(int j, int g) { return 8 * (j >> 2) + 4 * g + (j & 3); }

// Forward substitution w_t -= sum_{i<t} c_t L[t][i] w_i over the 32 rows of this lane's
// value column (rows acc_row(j, g); the other 16 rows are in the lane 32 away).  L is
// [t][i] row-major with zeros on and above the diagonal; c_t = beta[t] if beta is given,
// else 1.  Rows go in 8 blocks of 4 consecutive rows, each held by one half of the wave:
// both halves sum their finished rows for the block's rows, exchanges (independent of
// one another, so their latencies overlap) add the halves, and the owner finishes the
// block's rows in order.
__device__ __forceinline__ void fwd_solve(float (&wv)[16], const float* L, const float* beta,
                                          int g) {
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
        const int q = blk >> 1, gb = blk & 1;
        float tot[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 8 * q + 4 * gb + r;
            float part = 0.f;
#pragma unroll
            for (int q4 = 0; q4 <= q; ++q4) {
                // the owner's own run q is the block itself (done below)
                if (q4 == q && g == gb) continue;
                const float4 l4 = *reinterpret_cast<const float4*>(L + t * 32 + 8 * q4 + 4 * g);
                part = fmaf(l4.x, wv[4 * q4], part);
                part = fmaf(l4.y, wv[4 * q4 + 1], part);
                part = fmaf(l4.z, wv[4 * q4 + 2], part);
                part = fmaf(l4.w, wv[4 * q4 + 3], part);
            }
            tot[r] = pair_sum(part);
        }
        if (g == gb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 8 * q + 4 * gb + r;
                float acc = tot[r];
#pragma unroll
                for (int r2 = 0; r2 < r; ++r2) acc = fmaf(L[t * 32 + 8 * q + 4 * gb + r2], wv[4 * q + r2], acc);
                wv[4 * q + r] -= beta ? beta[t] * acc : acc;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Back substitution d_t -= sum_{s>t} beta_s LT[t][s] d_s (LT[t][s] = L[s][t], zero for
// s <= t), the transposed system of fwd_solve, blocks in reverse order.
__device__ __forceinline__ void bwd_solve(float (&dr)[16], const float* LT, const float* beta,
                                          int g) {
#pragma unroll
    for (int blk = 7; blk >= 0; --blk) {
        const int q = blk >> 1, gb = blk & 1;
        float tot[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 8 * q + 4 * gb + r;
            float part = 0.f;
#pragma unroll
            for (int q4 = q; q4 < 4; ++q4) {
                if (q4 == q && g == gb) continue;
                const float4 l4 = *reinterpret_cast<const float4*>(LT + t * 32 + 8 * q4 + 4 * g);
                const float4 b4 = *reinterpret_cast<const float4*>(beta + 8 * q4 + 4 * g);
                part = fmaf(l4.x * b4.x, dr[4 * q4], part);
                part = fmaf(l4.y * b4.y, dr[4 * q4 + 1], part);
                part = fmaf(l4.z * b4.z, dr[4 * q4 + 2], part);
                part = fmaf(l4.w * b4.w, dr[4 * q4 + 3], part);
            }
            tot[r] = pair_sum(part);
        }
        if (g == gb) {
#pragma unroll
            for (int r = 3; r >= 0; --r) {
                const int t = 8 * q + 4 * gb + r;
                float acc = tot[r];
#pragma unroll
                for (int r2 = r + 1; r2 < 4; ++r2) {
                    const int s2 = 8 * q + 4 * gb + r2;
                    acc = fmaf(LT[t * 32 + s2] * beta[s2], dr[4 * q + r2], acc);
                }
                dr[4 * q + r] -= acc;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

struct ChunkSmem {
    unsigned char K[kC * kRowB];   // swizzled rows (tile_off)
    unsigned char Q[kC * kRowB];
    unsigned char V[kC * kRowB];
    float alpha[kC], beta[kC];
    // per wave: beta-scaled gated K K^T (strict lower, [t][i]) and gated Q K^T
    // (lower with diagonal, [t][i]), gamma and log2 gamma of the chunk's tokens
    float L[kWaves][kC * kC];
    float M[kWaves][kC * kC];
    float gam[kWaves][kC], lg[kWaves][kC];
};

}  // namespace

// states: checkpoint slots [n_slots][H][Dv][Dk] float32 (row = value index).
// chunk_states (may be NULL): the state at the start of every chunk of every branch,
// [P.sc_chunk_base[b] + c][H][Dv][Dk] float32, for the backward.  Og may be NULL (the
// backward's recomputation needs the states only).
__global__ __launch_bounds__(kThr, 1) void gdn_chunk_fwd_kernel(
    DevPlan P, int l0, int H, const bf16* __restrict__ Qg, const bf16* __restrict__ Kg,
    const bf16* __restrict__ Vg, const float* __restrict__ Ag, const float* __restrict__ Bg,
    bf16* __restrict__ Og, float* __restrict__ states, float* __restrict__ chunk_states) {
    __shared__ __attribute__((aligned(1024))) ChunkSmem S;
    const int b = ld_const(P.sc_level_br + l0 + blockIdx.x / H);
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int dv = 32 * w + n;  // this lane's value row (accumulator column)
    const int start = ld_const(P.sc_start + b), len = ld_const(P.sc_len + b);
    const int init = ld_const(P.sc_init + b);
    const size_t rs = (size_t)H * kD;  // elements per token in q, k, v, o

    // S^T tiles: St[bk][j] = S[dv][32 bk + acc_row(j, g)].
    f32x16 St[4];
    if (init >= 0) {
        const float* src = states + (((size_t)init * H + h) * kD + dv) * kD;
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 x = *reinterpret_cast<const float4*>(src + 32 * bk + 8 * q4 + 4 * g);
                St[bk][4 * q4] = x.x;
                St[bk][4 * q4 + 1] = x.y;
                St[bk][4 * q4 + 2] = x.z;
                St[bk][4 * q4 + 3] = x.w;
            }
    } else {
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) St[bk] = zero16();
    }
    auto store_state = [&](float* dst_base) {
        float* dst = dst_base + ((size_t)h * kD + dv) * kD;
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4*>(dst + 32 * bk + 8 * q4 + 4 * g) =
                    make_float4(St[bk][4 * q4], St[bk][4 * q4 + 1], St[bk][4 * q4 + 2],
                                St[bk][4 * q4 + 3]);
    };
    int ck = ld_const(P.sc_ck_ptr + b);
    const int ck_end = ld_const(P.sc_ck_ptr + b + 1);
    auto save_due = [&](int r) {  // checkpoints at own offset r (children forking there)
        while (ck < ck_end && ld_const(P.sc_ck_off + ck) == r) {
            store_state(states + (size_t)ld_const(P.sc_ck_slot + ck) * H * kD * kD);
            ++ck;
        }
    };
    const int cbase = chunk_states ? ld_const(P.sc_chunk_base + b) : 0;

    // Per-lane LDS offsets of the operands.  Row reads (A operand: row n, k values
    // 16 ks + 8 g .. + 8) and the permuted pairs of 4 (k values 16 kh + 4 g .. + 4 and
    // 16 kh + 8 + 4 g .. + 4, matching the accumulator rows a lane holds); transposed
    // reads of K for the A operand of the state update (rows 4g + r/4 (+8) of each 16-row
    // k-step, as the forward kernel's V^T reads).
    int tr_[4][2];
    {
        const int r_in = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = 4 * g + (r_in >> 2) + 8 * hf;
                const int chunk = 4 * db + 2 * dh + ((r_in & 3) >> 1);
                tr_[db][hf] = row * kRowB + swz<kD>(row, chunk) * 16 + 8 * (r_in & 1);
            }
    }
    // 8-byte read of k values [k0, k0 + 4) of row `row` of a swizzled tile.
    auto rd4 = [&](const unsigned char* base, int row, int k0) {
        return *reinterpret_cast<const bf16x4*>(base + row * kRowB + swz<kD>(row, k0 >> 3) * 16 +
                                                (k0 & 7) * 2);
    };
    auto rd8 = [&](const unsigned char* base, int row, int k0) {
        return *reinterpret_cast<const bf16x8*>(base + row * kRowB + swz<kD>(row, k0 >> 3) * 16);
    };

    // Chunk loads: thread tid copies 16-byte pieces p = tid and tid + 256 of K, Q and V
    // (row p / 16, columns 8 (p % 16) ..), zeros past the chunk's length; lanes below 64
    // of wave 0 fetch alpha (t < 32) or beta.  Loaded into registers one chunk ahead.
    bf16x8 pk[2], pq[2], pv[2];
    float pab = 0.f;
    auto fetch = [&](int r0, int nt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = u * kThr + tid, t = p >> 4;
            const size_t off = (size_t)(start + r0 + t) * rs + (size_t)h * kD + 8 * (p & 15);
            const bool in = t < nt;
            pk[u] = in ? ld16(Kg + off) : zero8();
            pq[u] = in ? ld16(Qg + off) : zero8();
            pv[u] = in ? ld16(Vg + off) : zero8();
        }
        if (tid < 2 * kC) {
            const int t = tid & (kC - 1);
            const size_t off = (size_t)(start + r0 + t) * H + h;
            pab = t < nt ? (tid < kC ? Ag : Bg)[off] : (tid < kC ? 1.f : 0.f);
        }
    };
    auto put = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = u * kThr + tid;
            const int off = tile_off<kD>(p >> 4, p & 15);
            *reinterpret_cast<bf16x8*>(S.K + off) = pk[u];
            *reinterpret_cast<bf16x8*>(S.Q + off) = pq[u];
            *reinterpret_cast<bf16x8*>(S.V + off) = pv[u];
        }
        if (tid < 2 * kC) (tid < kC ? S.alpha : S.beta)[tid & (kC - 1)] = pab;
    };
    // next chunk end after own offset r: every 32 tokens and at every checkpoint offset
    auto chunk_end = [&](int r, int ckp) {
        int e = min(len, (r / kC + 1) * kC);
        if (ckp < ck_end) e = min(e, max(ld_const(P.sc_ck_off + ckp), r + 1));
        return e;
    };

    save_due(0);
    int r0 = 0;
    int e0 = chunk_end(0, ck);
    bf16 ostash[16];
    int o_row0 = 0, o_nt = 0;
    fetch(0, e0);
    float* Lw = S.L[w];
    float* Mw = S.M[w];
    float* gam = S.gam[w];
    float* lg = S.lg[w];
    for (int ci = 0; r0 < len; ++ci) {
        const int nt = e0 - r0;  // tokens in this chunk (1..32)
        barrier();               // every wave is done with the previous chunk's LDS
        put();
        wait_lds();
        barrier();
        // The previous chunk's outputs, stored now: issued before this chunk's loads, they
        // have a whole chunk to complete before the next wait on those loads.
        if (Og != nullptr && o_nt > 0) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int t = acc_row(j, g);
                if (t < o_nt) Og[(size_t)(start + o_row0 + t) * rs + (size_t)h * kD + dv] = ostash[j];
            }
        }
        if (chunk_states) store_state(chunk_states + (size_t)(cbase + ci) * H * kD * kD);
        const int r1 = e0;
        int ck_next = ck;
        while (ck_next < ck_end && ld_const(P.sc_ck_off + ck_next) <= r1) ++ck_next;
        const int e1 = r1 < len ? chunk_end(r1, ck_next) : r1;
        if (r1 < len) fetch(r1, e1 - r1);  // in flight while this chunk is computed

        // gamma_t (inclusive products of alpha over the chunk), in log2 and linear form
        {
            // (alpha is clamped at 2^-100: a zero gate still empties the state, and every
            // ratio of gammas stays a finite difference of logarithms)
            float la = lane < kC ? __log2f(fmaxf(S.alpha[lane], 7.8886e-31f)) : 0.f;
#pragma unroll
            for (int d = 1; d < kC; d <<= 1) {
                const float y = __shfl_up(la, d, 64);
                if ((lane & (kC - 1)) >= d) la += y;
            }
            if (lane < kC) {
                lg[lane] = la;
                gam[lane] = exp2f(la);
            }
        }
        // K K^T and Q K^T (exact bf16 products), gated and masked into L and M.
        f32x16 akk = zero16(), aqk = zero16();
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
            const bf16x8 kb = rd8(S.K, n, 16 * ks + 8 * g);  // B: K row n (= key i)
            akk = mfma_32x32x16(rd8(S.K, n, 16 * ks + 8 * g), kb, akk);
            aqk = mfma_32x32x16(rd8(S.Q, n, 16 * ks + 8 * g), kb, aqk);
        }
        wait_lds();  // gam, lg written by this wave's lanes
        __builtin_amdgcn_wave_barrier();
        {
            // accumulator: column i = n, rows t = acc_row(j, g)
            const int i = n;
            const float lgi = lg[i];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int t = acc_row(j, g);
                const float gt = exp2f(lg[t] - lgi);
                Lw[t * kC + i] = i < t ? S.beta[t] * akk[j] * gt : 0.f;
                Mw[t * kC + i] = i <= t ? aqk[j] * gt : 0.f;
            }
        }
        // X = K S_0^T and Y = Q S_0^T for this wave's value rows: A = K (Q) rows with the
        // k values in the accumulator's row order, B = the state's hi and lo parts.
        // (high and low parts into separate accumulators: four independent MFMA chains)
        f32x16 X = zero16(), Y = zero16(), X2 = zero16(), Y2 = zero16();
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                bf16x8 shi, slo;
#pragma unroll
                for (int e = 0; e < 8; ++e) split2(St[bk][8 * kh + e], shi, slo, e);
                const int k0 = 32 * bk + 16 * kh + 4 * g;
                const bf16x8 ak = cat(rd4(S.K, n, k0), rd4(S.K, n, k0 + 8));
                const bf16x8 aq = cat(rd4(S.Q, n, k0), rd4(S.Q, n, k0 + 8));
                X = mfma_32x32x16(ak, shi, X);
                X2 = mfma_32x32x16(ak, slo, X2);
                Y = mfma_32x32x16(aq, shi, Y);
                Y2 = mfma_32x32x16(aq, slo, Y2);
            }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            X[j] += X2[j];
            Y[j] += Y2[j];
        }
        wait_lds();
        __builtin_amdgcn_wave_barrier();
        // R = diag(beta) (V - diag(gamma) X), then the triangular solve for W in place.
        float wv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = acc_row(j, g);
            const float vt = (float)*reinterpret_cast<const bf16*>(
                S.V + t * kRowB + swz<kD>(t, dv >> 3) * 16 + (dv & 7) * 2);
            wv[j] = S.beta[t] * (vt - gam[t] * X[j]);
        }
        fwd_solve(wv, Lw, nullptr, g);
        // O = diag(gamma) Y + M W (M: A operand in the accumulator's row order).
        bf16x8 whi[2], wlo[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) split2(wv[8 * kk + e], whi[kk], wlo[kk], e);
        f32x16 MW = zero16();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float4 m0 = *reinterpret_cast<const float4*>(Mw + n * kC + 16 * kk + 4 * g);
            const float4 m1 = *reinterpret_cast<const float4*>(Mw + n * kC + 16 * kk + 8 + 4 * g);
            const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            bf16x8 mhi, mlo;
#pragma unroll
            for (int e = 0; e < 8; ++e) split2(mv[e], mhi, mlo, e);
            MW = mfma_32x32x16(mhi, whi[kk], MW);
            MW = mfma_32x32x16(mhi, wlo[kk], MW);
            MW = mfma_32x32x16(mlo, whi[kk], MW);
        }
        // (stored at the start of the next chunk)
#pragma unroll
        for (int j = 0; j < 16; ++j) ostash[j] = (bf16)(gam[acc_row(j, g)] * Y[j] + MW[j]);
        o_row0 = r0;
        o_nt = nt;
        // S^T <- gamma_C S^T + K^T (diag(gamma_C / gamma) W): A = K^T (transposed reads),
        // B = the scaled W rows of this lane's value column.
        const float gC = gam[nt - 1];
        bf16x8 uhi[2], ulo[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = acc_row(8 * kk + e, g);
                split2(wv[8 * kk + e] * (gC / gam[t]), uhi[kk], ulo[kk], e);
            }
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
#pragma unroll
            for (int j = 0; j < 16; ++j) St[bk][j] *= gC;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 ak = cat(lds8_tr(S.K, tr_[bk][0], 16 * kk * kRowB),
                                      lds8_tr(S.K, tr_[bk][1], 16 * kk * kRowB));
                St[bk] = mfma_32x32x16(ak, uhi[kk], St[bk]);
                St[bk] = mfma_32x32x16(ak, ulo[kk], St[bk]);
            }
        }
        r0 = r1;
        e0 = e1;
        save_due(r0);
    }
    if (Og != nullptr) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = acc_row(j, g);
            if (t < o_nt) Og[(size_t)(start + o_row0 + t) * rs + (size_t)h * kD + dv] = ostash[j];
        }
    }
}

// ---------------------------------------------------------------- backward
//
// Gradients of L = sum_t <dO_t, o_t> chunk by chunk in reverse, from the state at the
// start of every chunk (saved by a forward pass) and the gradient dS_C of the state at
// the chunk's end (carried from the chunk after it).  With R = diag(beta) (V - diag(gamma)
// X), X = K S_0^T, Y = Q S_0^T, N = I + diag(beta) LG (LG = K K^T o Gamma_strict),
// M = Q K^T o Gamma_incl, W = N^{-1} R:
//     dW   = M^T dO + diag(gamma_C / gamma) K dS_C^T
//     dR   = N^{-T} dW                 (back substitution)
//     d(diag(beta) LG) = -dR W^T       (strict lower part)
//     dV   = diag(beta) dR,  dX = -diag(beta gamma) dR,  dY = diag(gamma) dO
//     dM   = dO W^T                    (lower part with diagonal)
//     dQ   = dY S_0 + (dM o Gamma) K
//     dK   = dX S_0 + diag(gamma_C / gamma) W dS_C + (dA + dA^T) K + (dM o Gamma)^T Q,
//            dA = diag(beta) d(diag(beta) LG) o Gamma
//     dS_0 = gamma_C dS_C + K^T dX + Q^T dY
// and the gates through log gamma (natural log; every factor gamma_t / gamma_i and every
// gamma_t, gamma_C contributes its own term), summed from the end of the chunk to give
// d log alpha.  A child's initial-state gradient is added to its parent's at the fork
// offset (atomically: siblings forked at one offset share a slot).
//
// Wave w owns value rows [32 w, 32 w + 32) for everything that evolves row by row (the
// state, dS, W, dR, dV) and key columns [32 w, 32 w + 32) of the chunk's dQ and dK; the
// sums over value rows (dQ, dK partials, dR W^T, dO W^T, the gate and beta terms) are
// gathered in LDS.
struct ChunkBwdSmem {
    unsigned char K[kC * kRowB];
    unsigned char Q[kC * kRowB];
    unsigned char V[kC * kRowB];
    unsigned char dO[kC * kRowB];
    float alpha[kC], beta[kC], gam[kC], lg[kC];
    float LG[kC * kC];   // gated K K^T, strict lower, [t][i]
    float LGT[kC * kC];  // its transpose
    float M[kC * kC];    // gated Q K^T, lower with diagonal, [t][i]
    float MT[kC * kC];   // its transpose
    float P[kC * kC];    // sum over value rows of dR_t . W_i, then dA
    float dM[kC * kC];   // sum over value rows of dO_t . W_i, then dM o Gamma
    float dQa[kC * kD];  // sums over value rows of the state products, [t][dk]
    float dKa[kC * kD];
    float dg[kC];        // d L / d (natural log gamma_t)
    float db[kC];        // d L / d beta_t
    float W[kWaves][kC * 32];   // per wave: W [t][value row]
    float dR[kWaves][kC * 32];  // dR [t][value row]
    float S0[kWaves][32 * 32];  // one key tile of S_0: [key][value row]
    float dS[kWaves][32 * 32];  // the same tile of dS_C
};

// Sum of v[j] over the 32 lanes of this lane's half (lanes with the same g).
__device__ __forceinline__ void half_sum16(float (&v)[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) v[j] += __shfl_xor(v[j], off);
}

__global__ __launch_bounds__(kThr, 1) void gdn_chunk_bwd_kernel(
    DevPlan P, int l0, int H, const bf16* __restrict__ Qg, const bf16* __restrict__ Kg,
    const bf16* __restrict__ Vg, const float* __restrict__ Ag, const float* __restrict__ Bg,
    const bf16* __restrict__ dOg, const float* __restrict__ chunk_states,
    float* __restrict__ dstates, bf16* __restrict__ dQg, bf16* __restrict__ dKg,
    bf16* __restrict__ dVg, float* __restrict__ dAg, float* __restrict__ dBg) {
    __shared__ __attribute__((aligned(1024))) ChunkBwdSmem S;
    const int b = ld_const(P.sc_level_br + l0 + blockIdx.x / H);
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int dv = 32 * w + n;
    const int start = ld_const(P.sc_start + b), len = ld_const(P.sc_len + b);
    const int init = ld_const(P.sc_init + b);
    const size_t rs = (size_t)H * kD;
    const int ck_lo = ld_const(P.sc_ck_ptr + b);
    int ckr = ld_const(P.sc_ck_ptr + b + 1) - 1;
    const int cbase = ld_const(P.sc_chunk_base + b);
    const int nch = ld_const(P.sc_chunk_base + b + 1) - cbase;
    float* Wl = S.W[w];
    float* dRl = S.dR[w];
    float* S0l = S.S0[w];
    float* dSl = S.dS[w];

    int tr_[4][2];
    {
        const int r_in = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = 4 * g + (r_in >> 2) + 8 * hf;
                const int chunk = 4 * db + 2 * dh + ((r_in & 3) >> 1);
                tr_[db][hf] = row * kRowB + swz<kD>(row, chunk) * 16 + 8 * (r_in & 1);
            }
    }
    auto rd4 = [&](const unsigned char* base, int row, int k0) {
        return *reinterpret_cast<const bf16x4*>(base + row * kRowB + swz<kD>(row, k0 >> 3) * 16 +
                                                (k0 & 7) * 2);
    };
    auto rd8 = [&](const unsigned char* base, int row, int k0) {
        return *reinterpret_cast<const bf16x8*>(base + row * kRowB + swz<kD>(row, k0 >> 3) * 16);
    };
    // 8 floats at p[0..3] and p[off..off+3], split into bf16 high and low parts
    auto ld_split = [&](const float* p, int off, bf16x8& hi, bf16x8& lo, float scale) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 c = *reinterpret_cast<const float4*>(p + off);
        const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) split2(v[e] * scale, hi, lo, e);
    };

    // dS^T tiles (rows: keys, lane: value row), the gradient of the state at the current
    // boundary; starts with what children forked at the branch's end handed over.
    f32x16 dSt[4];
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) dSt[bk] = zero16();
    auto add_handed = [&](int r) {
        while (ckr >= ck_lo && ld_const(P.sc_ck_off + ckr) == r) {
            const float* src =
                dstates + (((size_t)ld_const(P.sc_ck_slot + ckr) * H + h) * kD + dv) * kD;
#pragma unroll
            for (int bk = 0; bk < 4; ++bk)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 x = *reinterpret_cast<const float4*>(src + 32 * bk + 8 * q4 + 4 * g);
                    dSt[bk][4 * q4] += x.x;
                    dSt[bk][4 * q4 + 1] += x.y;
                    dSt[bk][4 * q4 + 2] += x.z;
                    dSt[bk][4 * q4 + 3] += x.w;
                }
            --ckr;
        }
    };
    add_handed(len);

    int r1 = len;
    for (int j = nch - 1; j >= 0; --j) {
        int r0 = ((r1 - 1) / kC) * kC;
        if (ckr >= ck_lo) r0 = max(r0, ld_const(P.sc_ck_off + ckr));
        const int nt = r1 - r0;

        barrier();  // the previous chunk is done with every shared array
        // ---- loads: chunk inputs (zeros past nt; alpha 1, beta 0), cleared sums, S_0
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = u * kThr + tid, t = p >> 4;
            const size_t off = (size_t)(start + r0 + t) * rs + (size_t)h * kD + 8 * (p & 15);
            const bool in = t < nt;
            const int lo = tile_off<kD>(t, p & 15);
            *reinterpret_cast<bf16x8*>(S.K + lo) = in ? ld16(Kg + off) : zero8();
            *reinterpret_cast<bf16x8*>(S.Q + lo) = in ? ld16(Qg + off) : zero8();
            *reinterpret_cast<bf16x8*>(S.V + lo) = in ? ld16(Vg + off) : zero8();
            *reinterpret_cast<bf16x8*>(S.dO + lo) = in ? ld16(dOg + off) : zero8();
        }
        if (tid < 2 * kC) {
            const int t = tid & (kC - 1);
            const size_t off = (size_t)(start + r0 + t) * H + h;
            (tid < kC ? S.alpha : S.beta)[t] = t < nt ? (tid < kC ? Ag : Bg)[off] : (tid < kC ? 1.f : 0.f);
            (tid < kC ? S.dg : S.db)[t] = 0.f;
        }
        {
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < kC * kD / 4 / kThr; ++u) {
                reinterpret_cast<float4*>(S.dQa)[u * kThr + tid] = z;
                reinterpret_cast<float4*>(S.dKa)[u * kThr + tid] = z;
            }
            reinterpret_cast<float4*>(S.P)[tid] = z;
            reinterpret_cast<float4*>(S.dM)[tid] = z;
        }
        f32x16 St[4];
        {
            const float* src = chunk_states + (((size_t)(cbase + j) * H + h) * kD + dv) * kD;
#pragma unroll
            for (int bk = 0; bk < 4; ++bk)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 x = *reinterpret_cast<const float4*>(src + 32 * bk + 8 * q4 + 4 * g);
                    St[bk][4 * q4] = x.x;
                    St[bk][4 * q4 + 1] = x.y;
                    St[bk][4 * q4 + 2] = x.z;
                    St[bk][4 * q4 + 3] = x.w;
                }
        }
        wait_lds();
        barrier();

        // ---- gammas and the gated score matrices (wave 0); X, Y (every wave)
        if (w == 0) {
            float la = lane < kC ? __log2f(fmaxf(S.alpha[lane], 7.8886e-31f)) : 0.f;
#pragma unroll
            for (int d = 1; d < kC; d <<= 1) {
                const float y = __shfl_up(la, d, 64);
                if ((lane & (kC - 1)) >= d) la += y;
            }
            if (lane < kC) {
                S.lg[lane] = la;
                S.gam[lane] = exp2f(la);
            }
            f32x16 akk = zero16(), aqk = zero16();
#pragma unroll
            for (int ks = 0; ks < kD / 16; ++ks) {
                const bf16x8 kb = rd8(S.K, n, 16 * ks + 8 * g);
                akk = mfma_32x32x16(rd8(S.K, n, 16 * ks + 8 * g), kb, akk);
                aqk = mfma_32x32x16(rd8(S.Q, n, 16 * ks + 8 * g), kb, aqk);
            }
            wait_lds();
            __builtin_amdgcn_wave_barrier();
            const int i = n;
            const float lgi = S.lg[i];
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int t = acc_row(jj, g);
                const float gt = exp2f(S.lg[t] - lgi);
                const float lgv = i < t ? akk[jj] * gt : 0.f;
                const float mv = i <= t ? aqk[jj] * gt : 0.f;
                S.LG[t * kC + i] = lgv;
                S.LGT[i * kC + t] = lgv;
                S.M[t * kC + i] = mv;
                S.MT[i * kC + t] = mv;
            }
        }
        f32x16 X = zero16(), Y = zero16();
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                bf16x8 shi, slo;
#pragma unroll
                for (int e = 0; e < 8; ++e) split2(St[bk][8 * kh + e], shi, slo, e);
                const int k0 = 32 * bk + 16 * kh + 4 * g;
                const bf16x8 ak = cat(rd4(S.K, n, k0), rd4(S.K, n, k0 + 8));
                const bf16x8 aq = cat(rd4(S.Q, n, k0), rd4(S.Q, n, k0 + 8));
                X = mfma_32x32x16(ak, shi, X);
                X = mfma_32x32x16(ak, slo, X);
                Y = mfma_32x32x16(aq, shi, Y);
                Y = mfma_32x32x16(aq, slo, Y);
            }
        wait_lds();
        barrier();

        const float gC = S.gam[nt - 1];
        // per row t of this lane (accumulator order): V and dO of this lane's value column
        auto vat = [&](const unsigned char* base, int t) {
            return (float)*reinterpret_cast<const bf16*>(base + t * kRowB +
                                                         swz<kD>(t, dv >> 3) * 16 + (dv & 7) * 2);
        };
        // gate term of O = diag(gamma) Y + ...: gamma_t <dO_t, Y_t>, summed over value rows
        {
            float r[16];
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int t = acc_row(jj, g);
                r[jj] = S.gam[t] * vat(S.dO, t) * Y[jj];
            }
            half_sum16(r);
            if (n == 0) {
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) atomicAdd(&S.dg[acc_row(jj, g)], r[jj]);
            }
        }
        // ---- forward: R and the solve for W (as in the forward kernel); vx = V - gamma X
        float wv[16], vx[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int t = acc_row(jj, g);
            vx[jj] = vat(S.V, t) - S.gam[t] * X[jj];
            wv[jj] = S.beta[t] * vx[jj];
        }
        fwd_solve(wv, S.LG, S.beta, g);
        // ---- dW = M^T dO + diag(gamma_C / gamma) K dS_C^T
        f32x16 tA = zero16(), tB = zero16();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 mhi, mlo;
            ld_split(S.MT + n * kC + 16 * kk + 4 * g, 8, mhi, mlo, 1.f);
            const bf16x8 bo = cat(lds8_tr(S.dO, tr_[w][0], 16 * kk * kRowB),
                                  lds8_tr(S.dO, tr_[w][1], 16 * kk * kRowB));
            tA = mfma_32x32x16(mhi, bo, tA);
            tA = mfma_32x32x16(mlo, bo, tA);
        }
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                bf16x8 shi, slo;
#pragma unroll
                for (int e = 0; e < 8; ++e) split2(dSt[bk][8 * kh + e], shi, slo, e);
                const int k0 = 32 * bk + 16 * kh + 4 * g;
                const bf16x8 ak = cat(rd4(S.K, n, k0), rd4(S.K, n, k0 + 8));
                tB = mfma_32x32x16(ak, shi, tB);
                tB = mfma_32x32x16(ak, slo, tB);
            }
        float dr[16], tb[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            tb[jj] = tB[jj] * (gC / S.gam[acc_row(jj, g)]);
            dr[jj] = tA[jj] + tb[jj];
        }
        // ---- dR = N^{-T} dW: back substitution, N^T[t][s] = beta_s LG[s][t] (s > t)
        bwd_solve(dr, S.LGT, S.beta, g);
        // ---- W and dR to LDS ([t][value row]); dV; the beta and gate terms per row
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int t = acc_row(jj, g);
            Wl[t * 32 + n] = wv[jj];
            dRl[t * 32 + n] = dr[jj];
            if (t < nt)
                dVg[(size_t)(start + r0 + t) * rs + (size_t)h * kD + dv] =
                    (bf16)(S.beta[t] * dr[jj]);
        }
        {
            float rdb[16], rdg[16];
            float sx = 0.f;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int t = acc_row(jj, g);
                rdb[jj] = dr[jj] * vx[jj];
                const float x = wv[jj] * tb[jj];
                sx += x;
                // -beta_t gamma_t <dR_t, X_t> - x_t, with gamma_t X_t = V_t - vx_t
                rdg[jj] = -S.beta[t] * dr[jj] * (vat(S.V, t) - vx[jj]) - x;
            }
            // gamma_C <dS_C, S_0> over this lane's elements
#pragma unroll
            for (int bk = 0; bk < 4; ++bk)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) sx += gC * dSt[bk][jj] * St[bk][jj];
            half_sum16(rdb);
            half_sum16(rdg);
            sx += __shfl_xor(sx, 32);
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) sx += __shfl_xor(sx, off);
            if (n == 0) {
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const int t = acc_row(jj, g);
                    atomicAdd(&S.db[t], rdb[jj]);
                    atomicAdd(&S.dg[t], rdg[jj]);
                }
            }
            if (lane == 0) atomicAdd(&S.dg[nt - 1], sx);
        }
        wait_lds();
        __builtin_amdgcn_wave_barrier();
        // ---- sums over this wave's value rows: dR W^T and dO W^T (C x C)
        {
            f32x16 pp = zero16(), pm = zero16();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 ah, al, bh, bl;
                ld_split(dRl + n * 32 + 16 * ks + 8 * g, 4, ah, al, 1.f);
                ld_split(Wl + n * 32 + 16 * ks + 8 * g, 4, bh, bl, 1.f);
                pp = mfma_32x32x16(ah, bh, pp);
                pp = mfma_32x32x16(ah, bl, pp);
                pp = mfma_32x32x16(al, bh, pp);
                const bf16x8 ao = rd8(S.dO, n, 32 * w + 16 * ks + 8 * g);
                pm = mfma_32x32x16(ao, bh, pm);
                pm = mfma_32x32x16(ao, bl, pm);
            }
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int t = acc_row(jj, g);
                atomicAdd(&S.P[t * kC + n], pp[jj]);
                atomicAdd(&S.dM[t * kC + n], pm[jj]);
            }
        }
        // ---- dQ, dK partials over this wave's value rows, one key tile at a time
        float gmn = S.gam[n], btn = S.beta[n];  // the A operands' rows are t = n
        const float xs = -btn * gmn, ws_ = gC / gmn;
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int kr = acc_row(jj, g);
                S0l[kr * 32 + n] = St[bk][jj];
                dSl[kr * 32 + n] = dSt[bk][jj];
            }
            wait_lds();
            __builtin_amdgcn_wave_barrier();
            f32x16 pk = zero16(), pq = zero16();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 xh, xl, wh, wl, sh, sl, dh, dl, yh, yl;
                ld_split(dRl + n * 32 + 16 * ks + 8 * g, 4, xh, xl, xs);
                ld_split(Wl + n * 32 + 16 * ks + 8 * g, 4, wh, wl, ws_);
                ld_split(S0l + n * 32 + 16 * ks + 8 * g, 4, sh, sl, 1.f);
                ld_split(dSl + n * 32 + 16 * ks + 8 * g, 4, dh, dl, 1.f);
                {
                    const bf16x8 o8 = rd8(S.dO, n, 32 * w + 16 * ks + 8 * g);
#pragma unroll
                    for (int e = 0; e < 8; ++e) split2((float)o8[e] * gmn, yh, yl, e);
                }
                pk = mfma_32x32x16(xh, sh, pk);
                pk = mfma_32x32x16(xh, sl, pk);
                pk = mfma_32x32x16(xl, sh, pk);
                pk = mfma_32x32x16(wh, dh, pk);
                pk = mfma_32x32x16(wh, dl, pk);
                pk = mfma_32x32x16(wl, dh, pk);
                pq = mfma_32x32x16(yh, sh, pq);
                pq = mfma_32x32x16(yh, sl, pq);
                pq = mfma_32x32x16(yl, sh, pq);
            }
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int t = acc_row(jj, g);
                atomicAdd(&S.dKa[t * kD + 32 * bk + n], pk[jj]);
                atomicAdd(&S.dQa[t * kD + 32 * bk + n], pq[jj]);
            }
            wait_lds();
            __builtin_amdgcn_wave_barrier();
        }
        // ---- dS_0 = gamma_C dS_C + K^T dX + Q^T dY (the new carry)
        {
            bf16x8 xh[2], xl[2], yh[2], yl[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 o8 = cat(lds8_tr(S.dO, tr_[w][0], 16 * kk * kRowB),
                                      lds8_tr(S.dO, tr_[w][1], 16 * kk * kRowB));
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int jj = 8 * kk + e, t = acc_row(jj, g);
                    const float gt = S.gam[t];
                    split2(-S.beta[t] * gt * dr[jj], xh[kk], xl[kk], e);
                    split2(gt * (float)o8[e], yh[kk], yl[kk], e);
                }
            }
#pragma unroll
            for (int bk = 0; bk < 4; ++bk) {
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) dSt[bk][jj] *= gC;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 ak = cat(lds8_tr(S.K, tr_[bk][0], 16 * kk * kRowB),
                                          lds8_tr(S.K, tr_[bk][1], 16 * kk * kRowB));
                    const bf16x8 aq = cat(lds8_tr(S.Q, tr_[bk][0], 16 * kk * kRowB),
                                          lds8_tr(S.Q, tr_[bk][1], 16 * kk * kRowB));
                    dSt[bk] = mfma_32x32x16(ak, xh[kk], dSt[bk]);
                    dSt[bk] = mfma_32x32x16(ak, xl[kk], dSt[bk]);
                    dSt[bk] = mfma_32x32x16(aq, yh[kk], dSt[bk]);
                    dSt[bk] = mfma_32x32x16(aq, yl[kk], dSt[bk]);
                }
            }
        }
        wait_lds();
        barrier();

        // ---- C x C terms (every thread: row t, columns 4q .. 4q + 3)
        {
            const int t = tid >> 3, q = tid & 7;
            const float lgt = S.lg[t], btt = S.beta[t];
            float erow = 0.f, brow = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * q + e;
                const float gt = i <= t ? exp2f(lgt - S.lg[i]) : 0.f;
                const float dbl = i < t ? -S.P[t * kC + i] : 0.f;  // d(diag(beta) LG)
                const float lgv = S.LG[t * kC + i];
                const float dmv = i <= t ? S.dM[t * kC + i] : 0.f;
                // (the diagonal ratio gamma_t / gamma_t is 1: no gate term)
                const float ek = btt * dbl * lgv, eq = i < t ? dmv * S.M[t * kC + i] : 0.f;
                brow += dbl * lgv;
                erow += ek + eq;
                if (i < t) atomicAdd(&S.dg[i], -(ek + eq));
                S.P[t * kC + i] = btt * dbl * gt;  // dA (strict lower)
                S.dM[t * kC + i] = dmv * gt;       // dM o Gamma (lower with diagonal)
            }
#pragma unroll
            for (int off = 4; off >= 1; off >>= 1) {
                erow += __shfl_xor(erow, off);
                brow += __shfl_xor(brow, off);
            }
            if (q == 0) {
                atomicAdd(&S.dg[t], erow);
                atomicAdd(&S.db[t], brow);
            }
        }
        wait_lds();
        barrier();

        // ---- dQ and dK of key columns [32 w, 32 w + 32)
        {
            f32x16 fq, fk;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int t = acc_row(jj, g);
                fq[jj] = S.dQa[t * kD + dv];
                fk[jj] = S.dKa[t * kD + dv];
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 bkv = cat(lds8_tr(S.K, tr_[w][0], 16 * kk * kRowB),
                                       lds8_tr(S.K, tr_[w][1], 16 * kk * kRowB));
                const bf16x8 bqv = cat(lds8_tr(S.Q, tr_[w][0], 16 * kk * kRowB),
                                       lds8_tr(S.Q, tr_[w][1], 16 * kk * kRowB));
                // rows i of this k-step in the accumulator order
                bf16x8 qh, ql, ah, al, th, tl;
                ld_split(S.dM + n * kC + 16 * kk + 4 * g, 8, qh, ql, 1.f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = 16 * kk + 8 * (e >> 2) + 4 * g + (e & 3);
                    split2(S.P[n * kC + i] + S.P[i * kC + n], ah, al, e);
                    split2(S.dM[i * kC + n], th, tl, e);
                }
                fq = mfma_32x32x16(qh, bkv, fq);
                fq = mfma_32x32x16(ql, bkv, fq);
                fk = mfma_32x32x16(ah, bkv, fk);
                fk = mfma_32x32x16(al, bkv, fk);
                fk = mfma_32x32x16(th, bqv, fk);
                fk = mfma_32x32x16(tl, bqv, fk);
            }
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int t = acc_row(jj, g);
                if (t < nt) {
                    const size_t o = (size_t)(start + r0 + t) * rs + (size_t)h * kD + dv;
                    dQg[o] = (bf16)fq[jj];
                    dKg[o] = (bf16)fk[jj];
                }
            }
        }
        // ---- d alpha (suffix sums of d log gamma) and d beta
        if (w == 0 && lane < kC) {
            float v = lane < nt ? S.dg[lane] : 0.f;
#pragma unroll
            for (int d = 1; d < kC; d <<= 1) {
                const float y = __shfl_down(v, d, 64);
                if (lane + d < kC) v += y;
            }
            if (lane < nt) {
                const size_t o = (size_t)(start + r0 + lane) * H + h;
                dAg[o] = v / S.alpha[lane];
                dBg[o] = S.db[lane];
            }
        }
        add_handed(r0);
        r1 = r0;
    }
    // the gradient of this branch's initial state goes to its parent's fork slot
    if (init >= 0) {
        float* dst = dstates + (((size_t)init * H + h) * kD + dv) * kD;
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
                atomicAdd(dst + 32 * bk + acc_row(jj, g), dSt[bk][jj]);
    }
}

__global__ void fill_zero_kernel(float4* p, size_t n4) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_gdn_chunk_bwd(const DevPlan& p, int l0, int n_br, int H, const void* q,
                                const void* k, const void* v, const float* alpha,
                                const float* beta, const void* dout, const float* chunk_states,
                                float* dstates, void* dq, void* dk, void* dv, float* dalpha,
                                float* dbeta, hipStream_t s) {
    if (n_br <= 0) return hipSuccess;
    hipLaunchKernelGGL(gdn_chunk_bwd_kernel, dim3(n_br * H), dim3(kThr), 0, s, p, l0, H,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta,
                       (const bf16*)dout, chunk_states, dstates, (bf16*)dq, (bf16*)dk, (bf16*)dv,
                       dalpha, dbeta);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n_floats, hipStream_t s) {
    const size_t n4 = n_floats / 4;
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<float4*>(p), n4);
    return hipGetLastError();
}

hipError_t launch_gdn_chunk_fwd(const DevPlan& p, int l0, int n_br, int H, const void* q,
                                const void* k, const void* v, const float* alpha,
                                const float* beta, void* o, float* states, float* chunk_states,
                                hipStream_t s) {
    if (n_br <= 0) return hipSuccess;
    hipLaunchKernelGGL(gdn_chunk_fwd_kernel, dim3(n_br * H), dim3(kThr), 0, s, p, l0, H,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta, (bf16*)o,
                       states, chunk_states);
    return hipGetLastError();
}

}  // namespace octo
