// Device-side interface shared by the C ABI and the HIP kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace octo {

// Device view of an uploaded plan (see plan.h for how the host builds it).
struct DevPlan {
    int32_t T, nQT, nKT, n_partial;
    const int32_t* fwd_order;   // [nQT] query tiles, longest list first
    const int32_t* qt_ptr;      // [nQT+1]
    const int2* q_pairs;        // [n_pairs] {kv_tile, mask (-1 = FULL)}
    const int32_t* bwd_order;   // [nKT] KV tiles, longest list first
    const int32_t* kt_ptr;      // [nKT+1]
    const int2* k_pairs;        // [n_pairs] {q_tile, mask}
    const uint64_t* mask_rows;  // [n_partial][128]   bit x of row r: row sees key x
    const uint64_t* mask_cols;  // [n_partial][64][2] bit r of key x: row r sees key x
};

constexpr int kBq = 128;  // query rows per tile
constexpr int kBk = 64;   // keys per KV tile

hipError_t launch_fwd_bf16(const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, void* o, float* lse,
                           hipStream_t s);
hipError_t launch_fwd_fp32(const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, void* o, float* lse,
                           hipStream_t s);
// Backward phases.  `bf16` selects the MFMA kernels, otherwise float32.
hipError_t launch_bwd_delta(bool bf16, const DevPlan& p, int Hq, int D, const void* o,
                            const void* dout, float* delta, hipStream_t s);
hipError_t launch_bwd_dkdv(bool bf16, const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, const float* delta, void* dk, void* dv,
                           hipStream_t s);
hipError_t launch_bwd_dq(bool bf16, const DevPlan& p, int Hq, int Hkv, int D, float scale,
                         const void* q, const void* k, const void* v, const float* lse,
                         const void* dout, const float* delta, void* dq, hipStream_t s);
hipError_t launch_decode_bf16(int B, int Hq, int Hkv, int D, int page_size, float scale,
                              const void* q, const void* k_pool, const void* v_pool,
                              int n_pages, const int32_t* seg_ptr, const int32_t* seg_page,
                              const int32_t* seg_lo, const int32_t* seg_hi, int n_split,
                              void* o, float* lse, float* partial, hipStream_t s);

}  // namespace octo
