// Paged mounted decode on gfx950.
//
// Serving side of the episode DAG (Octopus project page, primitives table: `fork`
// shares the parent's radix KV pages, `read_thread` mounts another branch's pages
// c_A[s_A:e_A) zero-copy, `done` pins finished pages for mounts; card
// "02 · Memory": a mount allocates no KV pages).  A cursor's current token attends to
// its ancestor prefix, its own branch and its mounted spans, each read in place from
// the page of the branch that owns it.  The host turns that context into segments
// (page, slot_lo, slot_hi); this kernel streams them.
//
// Split kernel: every wave64 owns one (cursor, KV head, split) work item, a
// contiguous run of the cursor's segments, and keeps a partial softmax state.  Per
// 64-slot page the next page's K and V (2 x 16 KiB contiguous blocks of the pool) are
// loaded into registers while the current one is computed.  Scores use the forward
// kernel's transposed form S^T = K q^T (v_mfma_f32_32x32x16_bf16): the G query heads
// of the KV head are the B operand's columns, so lane l holds head l % 32's scores
// over 16 slots and the probabilities feed O^T += V^T P^T directly.  K and V are
// staged row-major in the wave's own LDS region, 16-byte chunks XOR-swizzled per row
// so that the row writes, the row reads of K and the transposed reads of V
// (ds_read_b64_tr_b16, giving the V^T operand) all hit distinct banks.  Slots outside
// the segment are zero-filled and masked.  The combine kernel merges the splits of
// each (cursor, head) by LSE.
#include "device_common.h"
#include "kernels.h"

namespace octo {

namespace {

constexpr int kPage = 64;
constexpr int kWaves = 4;
// Word 3 of a raw buffer resource on gfx9-family chips (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;

// A segment is read only if its page is in the pool and its slot range is well formed.
__device__ __forceinline__ bool seg_ok(int page, int lo, int hi, int n_pages) {
    return page >= 0 && page < n_pages && lo >= 0 && lo < hi && hi <= kPage;
}

template <int D>
struct DecodeSmem {
    static constexpr int MAT = kPage * D * 2;  // bytes of one page-head block
    unsigned char Ks[MAT];
    unsigned char Vs[MAT];
};

}  // namespace

// Work items (one wave each).  Own items: (cursor c, KV head, split) over c's own
// segment list c; the 4 waves of a workgroup take consecutive splits of one (cursor,
// head), which keeps their lengths alike.  Group items (with n_groups > 0, after the
// own items in the same grid):
// (position p in grp_cur, KV head, split) over the shared list B + gi of the group gi
// that holds p; only positions at the start of a block of 32 / G cursors of the group
// work, and the MFMA's 32 query columns are those cursors' G heads, so the group's pages
// are read once per block of cursors.  Split `split` writes partial state slot `split`
// (own lists) or n_split + split (shared lists) of each of its columns' (cursor, head).
template <int D>
__global__ __launch_bounds__(256, 1) void decode_split_kernel(
    int B, int Hq, int Hkv, int n_split, int n_slots, float scale_log2,
    const bf16* __restrict__ Qd, const bf16* __restrict__ Kp, const bf16* __restrict__ Vp,
    int n_pages, const int32_t* __restrict__ seg_ptr, const int32_t* __restrict__ seg_page,
    const int32_t* __restrict__ seg_lo, const int32_t* __restrict__ seg_hi, int n_groups,
    const int32_t* __restrict__ grp_ptr, const int32_t* __restrict__ grp_cur,
    float* __restrict__ partial) {
    constexpr int KS = D / 16, DB = D / 32, C8 = D / 8, ROWB = D * 2;
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kWaves * sizeof(DecodeSmem<D>)];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int per = B * Hkv * n_split;  // items of each kind
    int item = blockIdx.x * kWaves + w;
    if (item >= (n_groups > 0 ? 2 * per : per)) return;  // whole wave leaves; no block barriers below
    const bool grp = n_groups > 0 && item >= per;  // wave-uniform
    if (grp) item -= per;
    DecodeSmem<D>& S = reinterpret_cast<DecodeSmem<D>*>(smem_raw)[w];
    const int split = item % n_split;
    const int kvh = (item / n_split) % Hkv;
    const int c = item / (n_split * Hkv);
    const int G = Hq / Hkv;
    const int n = lane & 31, g = lane >> 5;
    int list = c, cursor = c, head = kvh * G + n;
    bool col_ok = n < G;
    if (grp) {
        int lo_g = 0, hi_g = n_groups;  // the group gi with grp_ptr[gi] <= c < grp_ptr[gi+1]
        while (hi_g - lo_g > 1) {
            const int mid = (lo_g + hi_g) >> 1;
            if (grp_ptr[mid] <= c) lo_g = mid; else hi_g = mid;
        }
        const int g0 = grp_ptr[lo_g], g1 = grp_ptr[lo_g + 1];
        const int cpb = 32 / G;  // cursors per block of columns
        if ((c - g0) % cpb != 0) return;
        list = B + lo_g;
        const int pos = c + n / G;
        col_ok = n < cpb * G && pos < g1 && pos < B;
        cursor = col_ok ? grp_cur[pos] : 0;
        if (cursor < 0 || cursor >= B) {  // not a cursor: the column stays empty
            col_ok = false;
            cursor = 0;
        }
        head = kvh * G + n % G;
    }
    // Per-lane LDS byte offsets: K rows (A operand of S^T: row n, chunk 2ks + g; + 32
    // rows for the second key block) and transposed V reads (rows 4g + r/4 (+8) of
    // each 16-slot k-step, columns 32db + 16(l/16 % 2) + 4(r % 4), r = l % 16).
    int ok_[KS], ov_[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ok_[ks] = n * ROWB + swz<D>(n, 2 * ks + g) * 16;
    {
        const int r_in = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = 4 * g + (r_in >> 2) + 8 * hf;
                const int chunk = 4 * db + 2 * dh + ((r_in & 3) >> 1);
                ov_[db][hf] = row * ROWB + swz<D>(row, chunk) * 16 + 8 * (r_in & 1);
            }
    }

    const int s0 = seg_ptr[list], s1 = seg_ptr[list + 1];
    const long long ns = s1 - s0;
    const int a = s0 + (int)((ns * split) / n_split);
    const int b = s0 + (int)((ns * (split + 1)) / n_split);

    // B operand: column n is query (cursor, head) (zero where col_ok is false).
    bf16x8 qf[KS];
    const bf16* qrow = Qd + ((size_t)cursor * Hq + (col_ok ? head : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = col_ok ? ld16(qrow + 16 * ks + 8 * g) : zero8();

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();
    float m = -1e30f, l = 0.f;

    // Loader: lane covers column chunk c8 = lane % C8 of 4-row groups rg.
    constexpr int RGS = kPage / 4;        // 16 row groups
    constexpr int LPR = 64 / C8;          // lanes per column pass
    constexpr int ITEMS = RGS / LPR;      // row groups per lane
    const int c8 = lane % C8, rg0 = lane / C8;
    bf16x8 kr[ITEMS][4], vr[ITEMS][4];
    // Byte offset (within a page-head block) of the first row this lane copies in pass
    // `it`; its rows are 4 (rg0 + LPR it) + j, j = 0..3, chunk c8.
    unsigned loff[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) loff[it] = (unsigned)(4 * (rg0 + LPR * it) * ROWB + 16 * c8);
    // Raw buffer loads through a resource that spans exactly slots [lo, hi) of the
    // page-head block: slots outside it read as zero with no branch, and nothing outside
    // the block is ever read (a segment that is not valid gets an empty resource).
    // Offsets are relative to slot lo; below it they wrap to huge values, which are out
    // of range too.
    auto gload = [&](int sg) {
        const int page = seg_page[sg], lo = seg_lo[sg], hi = seg_hi[sg];
        const bool ok = seg_ok(page, lo, hi, n_pages);
        const size_t blk = (((size_t)(ok ? page : 0) * Hkv + kvh) * kPage + (ok ? lo : 0)) * ROWB;
        const int bytes = ok ? (hi - lo) * ROWB : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(reinterpret_cast<const unsigned char*>(Kp) + blk), 0, bytes,
            kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(reinterpret_cast<const unsigned char*>(Vp) + blk), 0, bytes,
            kBufferWord3);
        const unsigned sub = (unsigned)((ok ? lo : 0) * ROWB);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int off = (int)(loff[it] + (unsigned)(j * ROWB) - sub);
                kr[it][j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
                vr[it][j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
            }
    };
    auto lds_put = [&]() {
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int rg = rg0 + LPR * it;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int off = tile_off<D>(4 * rg + j, c8);
                *reinterpret_cast<bf16x8*>(S.Ks + off) = kr[it][j];
                *reinterpret_cast<bf16x8*>(S.Vs + off) = vr[it][j];
            }
        }
    };

    if (a < b) gload(a);
    for (int sg = a; sg < b; ++sg) {
        const int lo = seg_lo[sg], hi = seg_hi[sg];
        const bool ok = seg_ok(seg_page[sg], lo, hi, n_pages);
        // The wave's previous reads of its LDS region come before these writes, and
        // these writes before the reads below: one wave's LDS operations stay in order.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        lds_put();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (sg + 1 < b) gload(sg + 1);

        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[kb] = mfma_32x32x16(lds16(S.Ks, ok_[ks], kb * 32 * ROWB), qf[ks], s[kb]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int x = kb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
                const float t = (ok && x >= lo && x < hi) ? s[kb][j] * scale_log2 : -INFINITY;
                s[kb][j] = t;
                mx = fmaxf(mx, t);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // The running max moves only when a page exceeds it by more than 2^8 (log2
        // units); the final division by the running sum makes the result independent
        // of where it was taken.
        if (__any(mx > m + 8.f)) {
            const float mnew = fmaxf(m, mx);
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        }
        const float mnew = m;
        bf16x8 pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float pv = fast_exp2(s[kb][j] - mnew);
                l += pv;
                pf[kb * 2 + (j >> 3)][j & 7] = (bf16)pv;
            }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 a = cat(lds8_tr(S.Vs, ov_[db][0], 16 * kk * ROWB),
                                     lds8_tr(S.Vs, ov_[db][1], 16 * kk * ROWB));
                o[db] = mfma_32x32x16(a, pf[kk], o[db]);
            }
    }

    l += __shfl_xor(l, 32);
    if (col_ok) {
        const int slot = grp ? n_split + split : split;
        float* out = partial + (((size_t)cursor * n_slots + slot) * Hq + head) * (D + 4);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float4 t = make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2],
                                       o[db][4 * q4 + 3]);
                *reinterpret_cast<float4*>(out + db * 32 + 8 * q4 + 4 * g) = t;
            }
        if (g == 0) {
            out[D] = (a < b && l > 0.f) ? m : -INFINITY;
            out[D + 1] = l;
        }
    }
}

// Merge the n_slots partial states of every (cursor, query head): one wave each.
// A partial state is D accumulator floats, the running max (log2 units), the running
// sum, and 2 floats of padding so every state starts 16-byte aligned.  Every slot is
// written by the split pass (an empty one as max -inf, sum 0, zero accumulator), so
// the lanes read 64 slots' maxima at once and the accumulation needs no branch.
template <int D, typename OT>
__global__ __launch_bounds__(64) void decode_combine_kernel(int B, int Hq, int n_slots,
                                                            const float* __restrict__ partial,
                                                            OT* __restrict__ O,
                                                            float* __restrict__ LSE) {
    const int c = blockIdx.x / Hq, h = blockIdx.x % Hq;
    const int lane = threadIdx.x;
    const size_t sstride = (size_t)Hq * (D + 4);  // floats between consecutive slots
    const float* base = partial + ((size_t)c * n_slots * Hq + h) * (D + 4);
    float M = -INFINITY;
    for (int j = lane; j < n_slots; j += 64) M = fmaxf(M, base[j * sstride + D]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
    float acc[D / 64];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
    for (int j0 = 0; j0 < n_slots; j0 += 64) {
        const int j = j0 + lane;
        float wj = 0.f;
        if (j < n_slots) {
            const float mj = base[j * sstride + D];
            wj = mj == -INFINITY ? 0.f : fast_exp2(mj - M);
            L += wj * base[j * sstride + D + 1];
        }
        const int nj = min(64, n_slots - j0);
        int t = 0;
        for (; t + 8 <= nj; t += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float w = __shfl(wj, t + u);
                const float* p = base + (size_t)(j0 + t + u) * sstride;
#pragma unroll
                for (int e = 0; e < D / 64; ++e) acc[e] += w * p[lane + 64 * e];
            }
        }
        for (; t < nj; ++t) {
            const float w = __shfl(wj, t);
            const float* p = base + (size_t)(j0 + t) * sstride;
#pragma unroll
            for (int e = 0; e < D / 64; ++e) acc[e] += w * p[lane + 64 * e];
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < D / 64; ++e)
        O[((size_t)c * Hq + h) * D + lane + 64 * e] = (OT)(acc[e] * inv);
    if (LSE != nullptr && lane == 0) LSE[(size_t)c * Hq + h] = (M + log2f(L)) * kLn2;
}

// ------------------------------------------------------------------ float32
//
// Exact float32 decode (for float32 pools): one wave64 per work item as above, each lane
// owning one slot of the page.  Per page the K and V blocks are staged in LDS (rows padded
// by one float so the per-slot row reads spread over the banks), every lane scores its
// slot for the G query heads, the running max and sum per head are wave-uniform, and the
// accumulator is split across the lanes by feature (lane l holds features l + 64e).  A
// group item serves one cursor of its group (the inherited context is read once per
// cursor: this variant is for exactness, not bandwidth).  It writes the same partial
// states as the bf16 kernel, which the combine kernel merges.
template <int D>
__global__ __launch_bounds__(64) void decode_split_fp32_kernel(
    int B, int Hq, int Hkv, int n_split, int n_slots, float scale_log2,
    const float* __restrict__ Qd, const float* __restrict__ Kp, const float* __restrict__ Vp,
    int n_pages, const int32_t* __restrict__ seg_ptr, const int32_t* __restrict__ seg_page,
    const int32_t* __restrict__ seg_lo, const int32_t* __restrict__ seg_hi, int n_groups,
    const int32_t* __restrict__ grp_ptr, const int32_t* __restrict__ grp_cur,
    float* __restrict__ partial) {
    constexpr int E = D / 64;   // features per lane
    constexpr int GMAX = 8;     // query heads per KV head
    __shared__ float ks[kPage][D + 1];
    __shared__ float vs[kPage][D + 1];
    __shared__ float qs[GMAX][D];
    __shared__ float ps[GMAX][kPage];
    const int lane = threadIdx.x;
    const int per = B * Hkv * n_split;
    int item = blockIdx.x;
    const bool grp = n_groups > 0 && item >= per;
    if (grp) item -= per;
    const int split = item % n_split;
    const int kvh = (item / n_split) % Hkv;
    const int c = item / (n_split * Hkv);
    const int G = Hq / Hkv;
    int list = c, cursor = c;
    if (grp) {
        int lo_g = 0, hi_g = n_groups;
        while (hi_g - lo_g > 1) {
            const int mid = (lo_g + hi_g) >> 1;
            if (grp_ptr[mid] <= c) lo_g = mid; else hi_g = mid;
        }
        if (c < grp_ptr[lo_g] || c >= grp_ptr[lo_g + 1]) return;
        list = B + lo_g;
        cursor = grp_cur[c];
        if (cursor < 0 || cursor >= B) return;  // not a cursor: nothing to write
    }
    for (int i = lane; i < G * D; i += 64)
        qs[i / D][i % D] = Qd[((size_t)cursor * Hq + kvh * G) * D + i];

    const int s0 = seg_ptr[list], s1 = seg_ptr[list + 1];
    const long long ns = s1 - s0;
    const int a = s0 + (int)((ns * split) / n_split);
    const int b = s0 + (int)((ns * (split + 1)) / n_split);

    float m[GMAX], l[GMAX], o[GMAX][E];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] = 0.f;
    }
    for (int sg = a; sg < b; ++sg) {
        const int page = seg_page[sg], lo = seg_lo[sg], hi = seg_hi[sg];
        if (!seg_ok(page, lo, hi, n_pages)) continue;  // wave-uniform
        const size_t blk = ((size_t)page * Hkv + kvh) * kPage * D;
        __syncthreads();  // the previous page's LDS reads are done
        for (int i = lane; i < kPage * D; i += 64) {
            const int r = i / D, d = i % D;
            const bool in = r >= lo && r < hi;
            ks[r][d] = in ? Kp[blk + i] : 0.f;
            vs[r][d] = in ? Vp[blk + i] : 0.f;
        }
        __syncthreads();
        const bool vis = lane >= lo && lane < hi;
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
            float ps_sum = pv;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ps_sum += __shfl_xor(ps_sum, off);
            l[h] = l[h] * alpha + ps_sum;
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
    const int slot = grp ? n_split + split : split;
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        if (h >= G) break;
        float* out = partial + (((size_t)cursor * n_slots + slot) * Hq + kvh * G + h) * (D + 4);
#pragma unroll
        for (int e = 0; e < E; ++e) out[lane + 64 * e] = o[h][e];
        if (lane == 0) {
            out[D] = (a < b && l[h] > 0.f) ? m[h] : -INFINITY;
            out[D + 1] = l[h];
        }
    }
}

template <int D>
static void decode_launch(bool b16, int B, int Hq, int Hkv, float scale, const void* q,
                          const void* k_pool, const void* v_pool, int n_pages,
                          const int32_t* seg_ptr, const int32_t* seg_page, const int32_t* seg_lo,
                          const int32_t* seg_hi, int n_groups, const int32_t* grp_ptr,
                          const int32_t* grp_cur, int n_split, void* o, float* lse,
                          float* partial, hipStream_t s) {
    const int n_slots = n_groups > 0 ? 2 * n_split : n_split;
    const int items = (n_groups > 0 ? 2 : 1) * B * Hkv * n_split;
    if (b16) {
        hipLaunchKernelGGL(decode_split_kernel<D>, dim3((items + kWaves - 1) / kWaves),
                           dim3(64 * kWaves), 0, s, B, Hq, Hkv, n_split, n_slots,
                           scale * kLog2e, (const bf16*)q, (const bf16*)k_pool,
                           (const bf16*)v_pool, n_pages, seg_ptr, seg_page, seg_lo, seg_hi,
                           n_groups, grp_ptr, grp_cur, partial);
        hipLaunchKernelGGL((decode_combine_kernel<D, bf16>), dim3(B * Hq), dim3(64), 0, s, B,
                           Hq, n_slots, partial, (bf16*)o, lse);
    } else {
        hipLaunchKernelGGL(decode_split_fp32_kernel<D>, dim3(items), dim3(64), 0, s, B, Hq,
                           Hkv, n_split, n_slots, scale * kLog2e, (const float*)q,
                           (const float*)k_pool, (const float*)v_pool, n_pages, seg_ptr,
                           seg_page, seg_lo, seg_hi, n_groups, grp_ptr, grp_cur, partial);
        hipLaunchKernelGGL((decode_combine_kernel<D, float>), dim3(B * Hq), dim3(64), 0, s, B,
                           Hq, n_slots, partial, (float*)o, lse);
    }
}

hipError_t launch_decode(bool b16, int B, int Hq, int Hkv, int D, int page_size, float scale,
                         const void* q, const void* k_pool, const void* v_pool, int n_pages,
                         const int32_t* seg_ptr, const int32_t* seg_page,
                         const int32_t* seg_lo, const int32_t* seg_hi, int n_groups,
                         const int32_t* grp_ptr, const int32_t* grp_cur, int n_split, void* o,
                         float* lse, float* partial, hipStream_t s) {
    (void)page_size;  // checked by the caller: page_size == 64
    if (D == 128)
        decode_launch<128>(b16, B, Hq, Hkv, scale, q, k_pool, v_pool, n_pages, seg_ptr,
                           seg_page, seg_lo, seg_hi, n_groups, grp_ptr, grp_cur, n_split, o,
                           lse, partial, s);
    else
        decode_launch<64>(b16, B, Hq, Hkv, scale, q, k_pool, v_pool, n_pages, seg_ptr,
                          seg_page, seg_lo, seg_hi, n_groups, grp_ptr, grp_cur, n_split, o,
                          lse, partial, s);
    return hipGetLastError();
}

}  // namespace octo
