// K/V tile staging shared by the forward and dQ kernels (internal).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace octo {

// Stage layout shared by the forward and dQ kernels: one 64-key K tile, the V tile,
// and the 128 row-mask words of the query tile (the all-ones mask when FULL).
template <int D>
struct KvStage {
    static constexpr int MAT = 64 * D * 2;
    static constexpr int MASK_OFF = 2 * MAT;
    static constexpr int BYTES = MASK_OFF + 128 * 8;
    static constexpr int NST = 3;
};

// Copy K/V tile `kt` and the mask of pair `m` into the stage at LDS byte address
// `base`: 64 rows of K and V (16 KiB each at D = 128, XOR-swizzled rows) and 1 KiB of
// mask words.  Every wave issues the same number of copies: per thread
// 2 * (64 * D * 2 / 16 / threads) + 1.
template <int D, int NTHR>
__device__ __forceinline__ void issue_kv_stage(unsigned base, const bf16* K, const bf16* V,
                                               const uint64_t* mask_rows, int kt, int m, int T,
                                               int kvh, size_t kvstride, int tid, int w,
                                               int lane) {
    constexpr int CPR = D / 8;
    constexpr int NDMA = KvStage<D>::MAT / (16 * NTHR);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int L = i * NTHR + tid;
        const int rho = L / CPR, slot = L % CPR;
        const int chunk = swz<D>(rho, slot);
        const int key = min(kt * kBk + rho, T - 1);
        const size_t off = (size_t)key * kvstride + (size_t)kvh * D + 8 * chunk;
        dma16(K + off, base + (i * NTHR + w * 64) * 16);
        dma16(V + off, base + KvStage<D>::MAT + (i * NTHR + w * 64) * 16);
    }
    constexpr int LANES = 64 / (NTHR / 64);  // 16-byte pieces per wave for 1 KiB
    if (lane < LANES)
        dma16(mask_rows + (size_t)m * kBq + 2 * (w * LANES + lane),
              base + KvStage<D>::MASK_OFF + w * LANES * 16);
}

}  // namespace octo
