// Paged mounted extend (prefill of several new tokens per cursor) on gfx950.
//
// Serving side of the episode DAG (Octopus project page, primitives table: `fork`
// shares the parent's radix KV pages, `read_thread` mounts another branch's span
// c_A[s_A:e_A) in place; ia.com.br article, section on the O(|Δm|) deltas: a
// continuation sends only the new tokens of a turn).  Cursor c appends its branch's last
// m_c own tokens, whose K/V are already in its pages; new token j (own offset r) attends
// to Ctx of its packed index: everything the branch inherits, the spans it mounted at
// offsets <= r, and its own tokens up to r.
//
// The host lists the pages of the context of the cursor's last token as segments
// (page, slot_lo, slot_hi) with a threshold: a new token at own offset r sees the
// segment's slot x iff r >= thr (+ x - slot_lo for the cursor's own pages, which are
// causal).  Segments are sorted by threshold, so a tile of new tokens needs a prefix of
// the list.  One workgroup (4 waves per query head, HPW heads of one KV head) takes a tile
// of 128 new tokens; per segment the page-head blocks of K and V (16 KiB each, the
// pool's contiguous [64][D] block) are copied to LDS asynchronously, three stages in
// flight, rows XOR-swizzled; S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (a lane owns a
// query column), visibility from the thresholds (only tiles not wholly visible are
// masked), online softmax with a lazy running max, and O^T += V^T P^T with V^T from
// transposed LDS reads.
#include "device_common.h"
#include "kernels.h"
#include "kvstage.h"

namespace octo {

namespace {

constexpr int kSlots = 64;  // page size = KV tile

template <int D>
struct ExtLayout {
    static constexpr int ROWB = D * 2;
    static constexpr int MAT = kSlots * ROWB;  // one page-head block
    static constexpr int NST = 3;
    static constexpr int K0 = 0;
    static constexpr int V0 = NST * MAT;
    static constexpr int BYTES = 2 * NST * MAT;
};

}  // namespace

template <int D, int HPW>
__global__ __launch_bounds__(256 * HPW, 1) void extend_bf16_kernel(
    int B, int Hq, int Hkv, int n_qt, float scale_log2, const bf16* __restrict__ Q,
    const bf16* __restrict__ Kp, const bf16* __restrict__ Vp, int n_pages,
    const int32_t* __restrict__ q_ptr, const int32_t* __restrict__ first_off,
    const int32_t* __restrict__ seg_ptr, const int32_t* __restrict__ seg_page,
    const int32_t* __restrict__ seg_lo, const int32_t* __restrict__ seg_hi,
    const int32_t* __restrict__ seg_thr, const int32_t* __restrict__ seg_causal,
    bf16* __restrict__ O, float* __restrict__ LSE) {
    using L = ExtLayout<D>;
    constexpr int NTHR = 256 * HPW;
    constexpr int KS = D / 16, DB = D / 32, CPR = D / 8, ROWB = L::ROWB;
    constexpr int NDMA = L::MAT / (16 * NTHR);
    constexpr int PER_STAGE = 2 * NDMA;
    constexpr float kLazy = 8.f;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[L::BYTES];

    const int G = Hq / Hkv;
    int grp, hp;
    if (!xcd_group(blockIdx.x, G / HPW, B * n_qt * Hkv, grp, hp)) return;
    const int kvh = grp % Hkv;
    const int qt = (grp / Hkv) % n_qt;
    const int c = grp / (Hkv * n_qt);
    const int row0 = ld_const(q_ptr + c);
    const int m_c = ld_const(q_ptr + c + 1) - row0;
    if (qt * kBq >= m_c) return;  // the whole workgroup leaves before any barrier

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = kvh * G + hp * HPW + (w >> 2);
    const int n = lane & 31, g = lane >> 5;
    const int jrow = qt * kBq + (w & 3) * 32 + n;  // this lane's new token (column)
    const bool valid = jrow < m_c;
    const int f0 = ld_const(first_off + c);
    const int r_own = f0 + jrow;
    const int r_min = f0 + qt * kBq;                          // wave-uniform
    const int r_max = f0 + min(m_c, qt * kBq + kBq) - 1;      // wave-uniform
    const size_t qstride = (size_t)Hq * D;
    const unsigned smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // The tile needs the segments with thr <= r_max: a prefix of the sorted list.
    const int s0 = ld_const(seg_ptr + c), s1 = ld_const(seg_ptr + c + 1);
    int lo_s = s0, hi_s = s1;
    while (lo_s < hi_s) {
        const int mid = (lo_s + hi_s) >> 1;
        if (ld_const(seg_thr + mid) <= r_max) lo_s = mid + 1; else hi_s = mid;
    }
    const int n_it = lo_s - s0;

    bf16x8 qf[KS];
    const bf16* qrow = Q + (size_t)(row0 + (valid ? jrow : 0)) * qstride + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = valid ? ld16(qrow + 16 * ks + 8 * g) : zero8();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);

    // LDS operand offsets: K rows for S^T (row n, chunk 2ks + g; +32 rows per key
    // block) and transposed V reads (rows 4g + r/4 (+8) of each 16-slot k-step).
    int ok_[KS], ov_[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ok_[ks] = L::K0 + n * ROWB + swz<D>(n, 2 * ks + g) * 16;
    {
        const int r_in = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = 4 * g + (r_in >> 2) + 8 * hf;
                const int chunk = 4 * db + 2 * dh + ((r_in & 3) >> 1);
                ov_[db][hf] = L::V0 + row * ROWB + swz<D>(row, chunk) * 16 + 8 * (r_in & 1);
            }
    }
    TileDma<D, NTHR> dm;  // full-page copy offsets (row stride D in the pool)
    dm.init(tid, (size_t)D);

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();
    float m = -1e30f, l = 0.f;

    // Copies of segment s0 + it into stage ST.  A page outside the pool or a malformed
    // slot range copies page 0 and is masked out entirely.  For a partial page, rows
    // outside [lo, hi) are filled from row lo, so every V row the MFMAs read is finite
    // (those rows get probability 0).
    // The segment of the next iteration to issue (jn) is loaded at the end of the iteration
    // before (`fetch_seg`), so that no scalar load is waited for right after the barrier;
    // the fields the step needs are kept per stage.
    int jn = 0;
    int jpg = 0, jlo = 0, jhi = 0, jthr = 0, jcau = 0;
    auto fetch_seg = [&]() {
        __builtin_amdgcn_sched_barrier(0);  // after everything else of the iteration
        asm volatile("" ::: "memory");
        const int sg = s0 + min(jn, n_it - 1);
        jpg = ld_const(seg_page + sg);
        jlo = ld_const(seg_lo + sg);
        jhi = ld_const(seg_hi + sg);
        jthr = ld_const(seg_thr + sg);
        jcau = ld_const(seg_causal + sg);
    };
    int st_lo[3], st_hi[3], st_thr[3];
    bool st_ok[3], st_cau[3];
    auto issue = [&](auto st_c, int it) {
        constexpr int ST = decltype(st_c)::value;
        const int pg = jpg, lo = jlo, hi = jhi;
        asm volatile("" ::"s"(jpg), "s"(jlo), "s"(jhi), "s"(jthr), "s"(jcau));
        const bool ok = pg >= 0 && pg < n_pages && lo >= 0 && lo < hi && hi <= kSlots;
        st_lo[ST] = lo;
        st_hi[ST] = hi;
        st_thr[ST] = jthr;
        st_cau[ST] = jcau != 0;
        st_ok[ST] = ok;
        ++jn;
        const size_t blk = ((size_t)(ok ? pg : 0) * Hkv + kvh) * kSlots * D;
        const bf16* kb = Kp + blk;
        const bf16* vb = Vp + blk;
        const unsigned kdst = smem_base + L::K0 + ST * L::MAT, vdst = smem_base + L::V0 + ST * L::MAT;
        if (ok && lo == 0 && hi == kSlots) {
#pragma unroll
            for (int i = 0; i < NDMA; ++i) {
                dma16_s(kb, dm.off[i], kdst + (i * NTHR + w * 64) * 16);
                dma16_s(vb, dm.off[i], vdst + (i * NTHR + w * 64) * 16);
            }
        } else {
            const int lo_c = ok ? lo : 0, hi_c = ok ? hi : 1;
#pragma unroll
            for (int i = 0; i < NDMA; ++i) {
                const int li = i * NTHR + tid;
                const int rho = li / CPR, slot = li % CPR;
                const int src = min(max(rho, lo_c), hi_c - 1);
                const unsigned off = (unsigned)((src * D + 8 * swz<D>(rho, slot)) * 2);
                dma16_s(kb, off, kdst + (i * NTHR + w * 64) * 16);
                dma16_s(vb, off, vdst + (i * NTHR + w * 64) * 16);
            }
        }
    };

    auto step = [&](auto st_c, int it) {
        constexpr int ST = decltype(st_c)::value;
        if (it + 1 < n_it) wait_vmem<PER_STAGE>();
        else wait_vmem<0>();
        barrier();
        if (it + 2 < n_it) issue(ic<(ST + 2) % 3>{}, it + 2);
        const int lo = st_lo[ST], hi = st_hi[ST], thr = st_thr[ST];
        const bool ok = st_ok[ST], causal = st_cau[ST];

        f32x16 s[2];
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[0] = mfma_32x32x16(lds16(smem, ok_[ks], ST * L::MAT), qf[ks], s[0]);
            s[1] = mfma_32x32x16(lds16(smem, ok_[ks], ST * L::MAT + 32 * ROWB), qf[ks], s[1]);
        }
        lead_reads<2 * KS>();
        // Every new token of the tile sees the whole page unless it is partial or its
        // threshold reaches past the tile's first token.
        const bool whole = ok && lo == 0 && hi == kSlots && r_min >= thr + (causal ? kSlots - 1 : 0);
        if (__builtin_expect(!whole, 0)) {
            asm volatile("");
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int x = kb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
                    const bool vis = ok && x >= lo && x < hi && r_own >= thr + (causal ? x - lo : 0);
                    if (!vis) s[kb][j] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(fmaxf(mx, s[0][j]), s[1][j]);
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
#pragma unroll
        for (int i = 0; i < 4; ++i) l = row_sum8(pf[i], l);
        // O^T += V^T P^T over 4 k-steps of 16 slots; the lane's 8 slots in k-step kk are
        // 16kk + 4g + {0..3} and 16kk + 8 + 4g + {0..3}.
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 va = cat(lds8_tr(smem, ov_[db][0], ST * L::MAT + 16 * kk * ROWB),
                                      lds8_tr(smem, ov_[db][1], ST * L::MAT + 16 * kk * ROWB));
                o[db] = mfma_32x32x16(va, pf[kk], o[db]);
            }
        // Two transposed reads per MFMA operand: keep six operands' reads ahead.
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
        for (int i = 0; i < 4 * DB - 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        fetch_seg();
    };

    if (n_it > 0) {
        fetch_seg();
        issue(ic<0>{}, 0);
        fetch_seg();
    }
    if (n_it > 1) {
        issue(ic<1>{}, 1);
        fetch_seg();
    }
    for (int it = 0; it < n_it; it += 3) {
        step(ic<0>{}, it);
        if (it + 1 < n_it) step(ic<1>{}, it + 1);
        if (it + 2 < n_it) step(ic<2>{}, it + 2);
    }

    l += __shfl_xor(l, 32);
    if (valid) {
        const float inv = 1.f / l;
        bf16* orow = O + (size_t)(row0 + jrow) * qstride + (size_t)h * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                bf16x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = (bf16)(o[db][4 * q4 + e] * inv);
                st8(orow + db * 32 + 8 * q4 + 4 * g, t);
            }
        if (g == 0) LSE[(size_t)(row0 + jrow) * Hq + h] = (m + log2f(l)) * kLn2;
    }
}

// ------------------------------------------------------------------ float32
//
// Exact float32 extend (for float32 pools): one wave64 per (cursor, new token j <
// max_new, KV head), tokens past the cursor's count leaving at once; each
// lane owning one slot of a page.  Per segment the wave stages the page-head blocks of K
// and V in LDS, scores its slot for the G query heads with the visibility rule of the
// thresholds, and keeps a running max and sum per head (wave-uniform) and the
// accumulator split across the lanes by feature.  Segments are sorted by threshold, so
// the walk stops at the first one the token's offset does not reach.
template <int D>
__global__ __launch_bounds__(64) void extend_fp32_kernel(
    int Hq, int Hkv, int max_new, float scale_log2, const float* __restrict__ Q,
    const float* __restrict__ Kp, const float* __restrict__ Vp, int n_pages,
    const int32_t* __restrict__ q_ptr, const int32_t* __restrict__ first_off,
    const int32_t* __restrict__ seg_ptr, const int32_t* __restrict__ seg_page,
    const int32_t* __restrict__ seg_lo, const int32_t* __restrict__ seg_hi,
    const int32_t* __restrict__ seg_thr, const int32_t* __restrict__ seg_causal,
    float* __restrict__ O, float* __restrict__ LSE) {
    constexpr int E = D / 64;
    constexpr int GMAX = 16;
    __shared__ float ks[kSlots][D + 1];
    __shared__ float vs[kSlots][D + 1];
    __shared__ float qs[GMAX][D];
    __shared__ float ps[GMAX][kSlots];
    const int lane = threadIdx.x;
    const int kvh = blockIdx.x % Hkv;
    const int j = (blockIdx.x / Hkv) % max_new;  // new token j of cursor c
    const int c = blockIdx.x / (Hkv * max_new);
    const int G = Hq / Hkv;
    if (j >= q_ptr[c + 1] - q_ptr[c]) return;
    const int row = q_ptr[c] + j;
    const int r_own = first_off[c] + j;
    const size_t qrow = ((size_t)row * Hq + kvh * G) * D;
    for (int i = lane; i < G * D; i += 64) qs[i / D][i % D] = Q[qrow + i];

    float m[GMAX], l[GMAX], o[GMAX][E];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] = 0.f;
    }
    for (int sg = seg_ptr[c]; sg < seg_ptr[c + 1]; ++sg) {
        const int thr = seg_thr[sg];
        if (thr > r_own) break;  // sorted by threshold: no later segment is seen
        const int pg = seg_page[sg], lo = seg_lo[sg], hi = seg_hi[sg];
        const bool causal = seg_causal[sg] != 0;
        if (!(pg >= 0 && pg < n_pages && lo >= 0 && lo < hi && hi <= kSlots)) continue;
        const size_t blk = ((size_t)pg * Hkv + kvh) * kSlots * D;
        __syncthreads();
        for (int i = lane; i < kSlots * D; i += 64) {
            const int r = i / D, d = i % D;
            const bool in = r >= lo && r < hi;
            ks[r][d] = in ? Kp[blk + i] : 0.f;
            vs[r][d] = in ? Vp[blk + i] : 0.f;
        }
        __syncthreads();
        const bool vis = lane >= lo && lane < hi && r_own >= thr + (causal ? lane - lo : 0);
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h >= G) break;
            float sc = 0.f;
            for (int d = 0; d < D; ++d) sc = fmaf(qs[h][d], ks[lane][d], sc);
            const float t = vis ? sc * scale_log2 : -INFINITY;
            float mx = t;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float mnew = fmaxf(m[h], mx);
            const float alpha = m[h] == -INFINITY ? 0.f : exp2f(m[h] - mnew);
            const float pv = t == -INFINITY ? 0.f : exp2f(t - mnew);
            float sum = pv;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
            l[h] = l[h] * alpha + sum;
            m[h] = mnew;
#pragma unroll
            for (int e = 0; e < E; ++e) o[h][e] *= alpha;
            ps[h][lane] = pv;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h >= G) break;
            for (int j = lo; j < hi; ++j) {
                const float pj = ps[h][j];
#pragma unroll
                for (int e = 0; e < E; ++e) o[h][e] = fmaf(pj, vs[j][lane + 64 * e], o[h][e]);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        if (h >= G) break;
        const float inv = 1.f / l[h];
#pragma unroll
        for (int e = 0; e < E; ++e) O[qrow + (size_t)h * D + lane + 64 * e] = o[h][e] * inv;
        if (lane == 0) LSE[(size_t)row * Hq + kvh * G + h] = (m[h] + log2f(l[h])) * kLn2;
    }
}

template <int D, int HPW>
static void extend_launch(int B, int Hq, int Hkv, int n_qt, float sl2, const void* q,
                          const void* k_pool, const void* v_pool, int n_pages,
                          const int32_t* q_ptr, const int32_t* first_off, const int32_t* seg_ptr,
                          const int32_t* seg_page, const int32_t* seg_lo, const int32_t* seg_hi,
                          const int32_t* seg_thr, const int32_t* seg_causal, void* o, float* lse,
                          hipStream_t s) {
    const int G = Hq / Hkv;
    hipLaunchKernelGGL((extend_bf16_kernel<D, HPW>), dim3(xcd_grid(B * n_qt * Hkv, G / HPW)),
                       dim3(256 * HPW), 0, s, B, Hq, Hkv, n_qt, sl2, (const bf16*)q,
                       (const bf16*)k_pool, (const bf16*)v_pool, n_pages, q_ptr, first_off,
                       seg_ptr, seg_page, seg_lo, seg_hi, seg_thr, seg_causal, (bf16*)o, lse);
}

template <int D>
static void extend_dispatch(bool b16, int B, int Hq, int Hkv, int max_new, int n_qt, float sl2,
                            const void* q, const void* k_pool, const void* v_pool, int n_pages,
                            const int32_t* q_ptr, const int32_t* first_off,
                            const int32_t* seg_ptr, const int32_t* seg_page,
                            const int32_t* seg_lo, const int32_t* seg_hi, const int32_t* seg_thr,
                            const int32_t* seg_causal, void* o, float* lse, hipStream_t s) {
    if (!b16) {
        hipLaunchKernelGGL(extend_fp32_kernel<D>, dim3(B * max_new * Hkv), dim3(64), 0, s, Hq,
                           Hkv, max_new, sl2, (const float*)q, (const float*)k_pool,
                           (const float*)v_pool, n_pages, q_ptr, first_off, seg_ptr, seg_page,
                           seg_lo, seg_hi, seg_thr, seg_causal, (float*)o, lse);
    } else if ((Hq / Hkv) % 2 == 0) {
        extend_launch<D, 2>(B, Hq, Hkv, n_qt, sl2, q, k_pool, v_pool, n_pages, q_ptr, first_off,
                            seg_ptr, seg_page, seg_lo, seg_hi, seg_thr, seg_causal, o, lse, s);
    } else {
        extend_launch<D, 1>(B, Hq, Hkv, n_qt, sl2, q, k_pool, v_pool, n_pages, q_ptr, first_off,
                            seg_ptr, seg_page, seg_lo, seg_hi, seg_thr, seg_causal, o, lse, s);
    }
}

hipError_t launch_extend(bool b16, int B, int Hq, int Hkv, int D, float scale, const void* q,
                         const void* k_pool, const void* v_pool, int n_pages,
                         const int32_t* q_ptr, int max_new, const int32_t* first_off,
                         const int32_t* seg_ptr, const int32_t* seg_page,
                         const int32_t* seg_lo, const int32_t* seg_hi,
                         const int32_t* seg_thr, const int32_t* seg_causal, void* o,
                         float* lse, hipStream_t s) {
    const int n_qt = (max_new + kBq - 1) / kBq;
    const float sl2 = scale * kLog2e;
    if (D == 128)
        extend_dispatch<128>(b16, B, Hq, Hkv, max_new, n_qt, sl2, q, k_pool, v_pool, n_pages,
                             q_ptr, first_off, seg_ptr, seg_page, seg_lo, seg_hi, seg_thr,
                             seg_causal, o, lse, s);
    else
        extend_dispatch<64>(b16, B, Hq, Hkv, max_new, n_qt, sl2, q, k_pool, v_pool, n_pages,
                            q_ptr, first_off, seg_ptr, seg_page, seg_lo, seg_hi, seg_thr,
                            seg_causal, o, lse, s);
    return hipGetLastError();
}

}  // namespace octo
