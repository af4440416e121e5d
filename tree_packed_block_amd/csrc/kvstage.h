// K/V tile staging shared by the forward and dQ kernels (internal).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace octo {

// LDS layout of the three stages, stage-major by kind so that every offset a lane
// reads is a per-lane register plus a compile-time immediate below 64 KiB:
// [K tile x 3][V tile x 3][row-mask words x 3].
template <int D>
struct KvLayout {
    static constexpr int ROWB = D * 2;         // bytes per row
    static constexpr int MAT = 64 * ROWB;      // one 64-key tile
    static constexpr int NST = 3;              // stages in flight
    static constexpr int K0 = 0;
    static constexpr int V0 = NST * MAT;
    static constexpr int M0 = 2 * NST * MAT;
    static constexpr int MASKB = kBq * 8;      // 128 row words
    static constexpr int BYTES = M0 + NST * MASKB;
};

template <int V>
using ic = std::integral_constant<int, V>;

// Position p of a 16-key group in the tiles_t layout holds key kperm(p) (an
// involution): lane half g of an MFMA holds keys 4g..4g+3 and 8+4g..8+4g+3 of each
// 16-key step, which become the contiguous positions 8g..8g+7.
__host__ __device__ constexpr int kperm(int p) { return (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1); }

// Copy tile `kt` of a tiles_t array (one contiguous block of 64 * D bf16) into the LDS
// region at byte `lds_off`, NDMA copies of 16 bytes per thread, in order.
template <int D, int NTHR>
__device__ __forceinline__ void issue_tile_t(unsigned smem_base, unsigned lds_off,
                                             const bf16* X, int nKT, int kvh, int kt, int tid,
                                             int w) {
    constexpr int NDMA = 64 * D * 2 / (16 * NTHR);
    const bf16* src = X + ((size_t)kvh * nKT + kt) * (64 * D);
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
        dma16_s(src, (unsigned)((i * NTHR + tid) * 16),
                smem_base + lds_off + (i * NTHR + w * 64) * 16);
}

// Per-lane byte offset, inside a tiles_t tile in LDS, of the A operand that covers
// rows d = 32 db + n (lane n = l % 32) and k-step kk (16 keys): chunk 2kk + g, so
// lane base n * 16 + g * D * 16 plus the immediate tile_t_imm(kk, db).
template <int D>
__device__ __forceinline__ int tile_t_lane(int lane) {
    return (lane & 31) * 16 + (lane >> 5) * D * 16;
}
template <int D>
__host__ __device__ constexpr int tile_t_imm(int kk, int db) {
    return kk * 2 * D * 16 + db * 32 * 16;
}

// Order the N LDS reads and N MFMAs of one basic block so that the reads run AHEAD
// operands in front of the MFMAs that consume them (left alone, the scheduler keeps
// only two in flight and each MFMA pair waits out a full LDS latency).
template <int N, int AHEAD = 6>
__device__ __forceinline__ void lead_reads() {
    constexpr int A = N < AHEAD ? N : AHEAD;
    __builtin_amdgcn_sched_group_barrier(0x100, A, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < N - A; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}

// Copy K/V tile `kt` and the row masks of mask `m` into stage ST: 64 rows of K and V
// (XOR-swizzled) and 1 KiB of mask words.  Every wave issues the same number of
// copies: 2 * (64 * D * 2 / 16 / NTHR) + 1 per thread.
// Per-lane byte offsets of the copies of one 64-row tile of a [rows][heads][D] tensor
// (row stride `stride` elements), relative to the tile's first row and head: copy i of
// thread t moves row (i * NTHR + t) / (D / 8), XOR-swizzled chunk, into LDS position
// i * NTHR + t.
template <int D, int NTHR>
struct TileDma {
    static constexpr int NDMA = 64 * D * 2 / (16 * NTHR);
    unsigned off[NDMA];
    __device__ __forceinline__ void init(int tid, size_t stride) {
        constexpr int CPR = D / 8;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int li = i * NTHR + tid;
            const int rho = li / CPR, slot = li % CPR;
            off[i] = (unsigned)(((size_t)rho * stride + 8 * swz<D>(rho, slot)) * 2);
        }
    }
};

// Copy rows row0 .. row0 + 63 (head `head`) of X into the LDS region at byte `lds_off`:
// from a scalar base when the whole tile lies below T, else row by row with the rows
// clamped to T - 1 (they are masked out by the caller).
template <int D, int NTHR>
__device__ __forceinline__ void issue_rows(unsigned smem_base, unsigned lds_off, const bf16* X,
                                           int row0, int T, int head, size_t stride,
                                           const TileDma<D, NTHR>& dm, int tid, int w) {
    constexpr int CPR = D / 8;
    if (row0 + 64 <= T) {
        const bf16* base = X + (size_t)row0 * stride + (size_t)head * D;
#pragma unroll
        for (int i = 0; i < dm.NDMA; ++i)
            dma16_s(base, dm.off[i], smem_base + lds_off + (i * NTHR + w * 64) * 16);
    } else {
#pragma unroll
        for (int i = 0; i < dm.NDMA; ++i) {
            const int li = i * NTHR + tid;
            const int rho = li / CPR, slot = li % CPR;
            const int r = min(row0 + rho, T - 1);
            dma16(X + (size_t)r * stride + (size_t)head * D + 8 * swz<D>(rho, slot),
                  smem_base + lds_off + (i * NTHR + w * 64) * 16);
        }
    }
}

template <int D, int NTHR, int ST, bool WITH_V = true, typename L = KvLayout<D>>
__device__ __forceinline__ void issue_kv_stage(unsigned smem_base, const bf16* K, const bf16* V,
                                               const uint64_t* mask_rows, int kt, int m, int T,
                                               int kvh, size_t kvstride,
                                               const TileDma<D, NTHR>& dm, int tid, int w,
                                               int lane) {
    issue_rows<D, NTHR>(smem_base, L::K0 + ST * L::MAT, K, kt * kBk, T, kvh, kvstride, dm, tid, w);
    if constexpr (WITH_V)
        issue_rows<D, NTHR>(smem_base, L::V0 + ST * L::MAT, V, kt * kBk, T, kvh, kvstride, dm, tid,
                            w);
    constexpr int LANES = 64 / (NTHR / 64);  // 16-byte pieces per wave for 1 KiB
    if (lane < LANES)
        dma16_s(mask_rows + (size_t)m * kBq, (unsigned)((w * LANES + lane) * 16),
                smem_base + L::M0 + ST * L::MASKB + w * LANES * 16);
}

// Per-lane byte offsets (relative to the LDS base) of the operands a wave reads from
// one stage, for query rows owned as S^T = K Q^T columns (lane n = l % 32, g = l / 32).
template <int D>
struct KvOffsets {
    static constexpr int KS = D / 16, DB = D / 32;
    int k[KS];      // A operand of S^T (row n, chunk 2ks+g); +32 rows: + 32 * ROWB
    int kt[DB][2];  // transposed A operand from the K tile; +16 rows per k-step
    __device__ __forceinline__ void init(int lane) {
        using L = KvLayout<D>;
        const int n = lane & 31, g = lane >> 5, r_in = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            k[ks] = L::K0 + n * L::ROWB + (((2 * ks + g) ^ swz_key<D>(n)) * 16);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = 4 * g + (r_in >> 2) + 8 * hf;
                const int chunk = 4 * db + 2 * dh + ((r_in & 3) >> 1);
                const int off = row * L::ROWB + ((chunk ^ swz_key<D>(row)) * 16) + 8 * (r_in & 1);
                kt[db][hf] = L::K0 + off;
            }
    }
};


}  // namespace octo
