// C ABI of the packed-DAG attention library (see include/octopus_dag.h).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "octopus_dag.h"
#include "plan.h"

struct octopus_plan {
    octo::Plan p;
};

namespace {

thread_local std::string g_err;

int fail(int code, std::string msg) {
    g_err = std::move(msg);
    return code;
}

int ok() {
    g_err.clear();
    return OCTOPUS_OK;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(OCTOPUS_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

octo::DevPlan dev_view(const octo::Plan& p) {
    const unsigned char* base = static_cast<const unsigned char*>(p.dev);
    octo::DevPlan d;
    d.T = p.T;
    d.nQT = p.nQT;
    d.nKT = p.nKT;
    d.n_partial = (int32_t)p.n_partial;
    d.fwd_order = reinterpret_cast<const int32_t*>(base + p.layout.fwd_order);
    d.qt_ptr = reinterpret_cast<const int32_t*>(base + p.layout.qt_ptr);
    d.q_pairs = reinterpret_cast<const int2*>(base + p.layout.q_pairs);
    d.bwd_order = reinterpret_cast<const int32_t*>(base + p.layout.bwd_order);
    d.kt_ptr = reinterpret_cast<const int32_t*>(base + p.layout.kt_ptr);
    d.k_pairs = reinterpret_cast<const int2*>(base + p.layout.k_pairs);
    d.mask_rows = reinterpret_cast<const uint64_t*>(base + p.layout.mask_rows);
    d.mask_cols = reinterpret_cast<const uint64_t*>(base + p.layout.mask_cols);
    d.nKB = p.nKB;
    d.pad = 0;
    d.blk_order = reinterpret_cast<const int32_t*>(base + p.layout.blk_order);
    d.blk_ptr = reinterpret_cast<const int32_t*>(base + p.layout.blk_ptr);
    d.blk_entries = reinterpret_cast<const int4*>(base + p.layout.blk_entries);
    d.pos = reinterpret_cast<const int32_t*>(base + p.layout.pos);
    d.sc_start = reinterpret_cast<const int32_t*>(base + p.layout.sc_start);
    d.sc_len = reinterpret_cast<const int32_t*>(base + p.layout.sc_len);
    d.sc_init = reinterpret_cast<const int32_t*>(base + p.layout.sc_init);
    d.sc_ck_ptr = reinterpret_cast<const int32_t*>(base + p.layout.sc_ck_ptr);
    d.sc_ck_off = reinterpret_cast<const int32_t*>(base + p.layout.sc_ck_off);
    d.sc_ck_slot = reinterpret_cast<const int32_t*>(base + p.layout.sc_ck_slot);
    d.sc_level_br = reinterpret_cast<const int32_t*>(base + p.layout.sc_level_br);
    d.sc_chunk_base = reinterpret_cast<const int32_t*>(base + p.layout.sc_chunk_base);
    d.sc_chunk_tok = reinterpret_cast<const int32_t*>(base + p.layout.sc_chunk_tok);
    d.sc_chunk_nt = reinterpret_cast<const int32_t*>(base + p.layout.sc_chunk_nt);
    d.sc_ck_kid_ptr = reinterpret_cast<const int32_t*>(base + p.layout.sc_ck_kid_ptr);
    d.sc_ck_kid = reinterpret_cast<const int32_t*>(base + p.layout.sc_ck_kid);
    return d;
}

// Checks shared by the forward and the backward.
int check_attn(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq, int32_t Hkv,
               int32_t D, std::initializer_list<const void*> ptrs) {
    if (plan == nullptr) return fail(OCTOPUS_EINVAL, "plan is NULL");
    if (plan->p.dev == nullptr) return fail(OCTOPUS_ESTATE, "plan not uploaded");
    if (dtype != OCTOPUS_BF16 && dtype != OCTOPUS_FP32)
        return fail(OCTOPUS_EUNSUPPORTED, "dtype must be bf16 or fp32");
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(OCTOPUS_EINVAL, "Hq and Hkv must be positive with Hq % Hkv == 0");
    if (Hq / Hkv > 16) return fail(OCTOPUS_EUNSUPPORTED, "Hq / Hkv must be <= 16");
    if (D != 64 && D != 128) return fail(OCTOPUS_EUNSUPPORTED, "head_dim must be 64 or 128");
    for (const void* p : ptrs) {
        if (p == nullptr) return fail(OCTOPUS_EINVAL, "a tensor pointer is NULL");
        if (!aligned(p, 16)) return fail(OCTOPUS_EINVAL, "tensors must be 16-byte aligned");
    }
    return OCTOPUS_OK;
}

}  // namespace

extern "C" {

const char* octopus_last_error(void) { return g_err.c_str(); }

const char* octopus_version(void) { return "octopus_dag 0.1 (gfx950)"; }

int octopus_dag_plan(const octopus_branch* branches, int32_t n_branches,
                     const octopus_mount* mounts, int32_t n_mounts, int32_t total_tokens,
                     int32_t kv_tile, octopus_plan** out) {
    if (out == nullptr) return fail(OCTOPUS_EINVAL, "out is NULL");
    *out = nullptr;
    try {
        std::unique_ptr<octopus_plan> h(new octopus_plan());  // freed on every error path
        std::string err;
        const int rc = octo::build_plan(branches, n_branches, mounts, n_mounts, total_tokens,
                                        kv_tile, h->p, err);
        if (rc != OCTOPUS_OK) return fail(rc, err);
        *out = h.release();
        return ok();
    } catch (const std::bad_alloc&) {
        return fail(OCTOPUS_ENOMEM, "host allocation failed while planning");
    }
}

int octopus_plan_positions(const octopus_plan* plan, int32_t* pos_out) {
    if (plan == nullptr || pos_out == nullptr) return fail(OCTOPUS_EINVAL, "NULL argument");
    for (int32_t i = 0; i < plan->p.T; ++i) pos_out[i] = (int32_t)plan->p.dag.pos[i];
    return ok();
}

int octopus_plan_stats_get(const octopus_plan* plan, octopus_plan_stats* out) {
    if (plan == nullptr || out == nullptr) return fail(OCTOPUS_EINVAL, "NULL argument");
    const octo::Plan& p = plan->p;
    out->nnz = p.nnz;
    out->n_pairs = (int64_t)p.q_pairs.size();
    out->n_partial = p.n_partial;
    out->total_tokens = p.T;
    out->q_tile = p.Bq;
    out->kv_tile = p.Bk;
    out->n_q_tiles = p.nQT;
    out->n_kv_tiles = p.nKT;
    out->max_q_list = p.max_q_list;
    out->max_kv_list = p.max_kv_list;
    out->reserved = 0;
    return ok();
}

size_t octopus_plan_device_bytes(const octopus_plan* plan) {
    return plan ? plan->p.layout.total : 0;
}

int octopus_plan_upload(octopus_plan* plan, void* dev_buf, size_t bytes, void* stream) {
    if (plan == nullptr || dev_buf == nullptr) return fail(OCTOPUS_EINVAL, "NULL argument");
    if (!aligned(dev_buf, 256)) return fail(OCTOPUS_EINVAL, "plan buffer must be 256-byte aligned");
    if (bytes < plan->p.layout.total)
        return fail(OCTOPUS_EWORKSPACE, "plan buffer smaller than octopus_plan_device_bytes");
    // Stage through page-locked memory owned by the plan so the copy is truly
    // asynchronous (no implicit wait for earlier work on the stream).
    if (plan->p.pinned == nullptr) {
        void* h = nullptr;
        const hipError_t ea = hipHostMalloc(&h, plan->p.layout.total, hipHostMallocDefault);
        if (ea != hipSuccess) return hip_fail(ea, "plan upload (page-locked staging)");
        octo::write_device_image(plan->p, static_cast<unsigned char*>(h));
        plan->p.pinned = h;
    }
    const hipError_t e = hipMemcpyAsync(dev_buf, plan->p.pinned, plan->p.layout.total,
                                        hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "plan upload");
    plan->p.dev = dev_buf;
    return ok();
}

int octopus_plan_export_mask(const octopus_plan* plan, int32_t row_lo, int32_t row_hi,
                             uint8_t* bits_out) {
    if (plan == nullptr || bits_out == nullptr) return fail(OCTOPUS_EINVAL, "NULL argument");
    if (row_lo < 0 || row_hi > plan->p.T || row_lo > row_hi)
        return fail(OCTOPUS_EINVAL, "row range outside [0, T)");
    octo::export_mask(plan->p, row_lo, row_hi, bits_out);
    return ok();
}

int octopus_plan_export_tiles(const octopus_plan* plan, int32_t* qt_ptr_out,
                              int32_t* kv_tile_out, int32_t* mask_out, uint64_t* rows_out) {
    if (plan == nullptr || !qt_ptr_out || !kv_tile_out || !mask_out)
        return fail(OCTOPUS_EINVAL, "NULL argument");
    const octo::Plan& p = plan->p;
    std::copy(p.qt_ptr.begin(), p.qt_ptr.end(), qt_ptr_out);
    for (size_t i = 0; i < p.q_pairs.size(); ++i) {
        kv_tile_out[i] = p.q_pairs[i].tile;
        mask_out[i] = p.q_pairs[i].mask;
    }
    if (rows_out)
        std::copy(p.mask_rows.begin(), p.mask_rows.begin() + p.n_partial * p.Bq * p.row_words,
                  rows_out);
    return ok();
}

void octopus_plan_destroy(octopus_plan* plan) {
    if (plan == nullptr) return;
    if (plan->p.pinned != nullptr) (void)hipHostFree(plan->p.pinned);
    delete plan;
}

size_t octopus_fwd_workspace_bytes(const octopus_plan* plan, octopus_dtype dtype, int32_t,
                                   int32_t Hkv, int32_t D) {
    if (plan == nullptr || dtype != OCTOPUS_BF16 || Hkv < 1 || (D != 64 && D != 128)) return 0;
    return octo::tiles_t_bytes(plan->p.nKT, Hkv, D);
}

int octopus_dag_attn_fwd(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                         int32_t Hkv, int32_t D, float scale, const void* q, const void* k,
                         const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
    int rc = check_attn(plan, dtype, Hq, Hkv, D, {q, k, v, o, lse});
    if (rc != OCTOPUS_OK) return rc;
    const size_t need = octopus_fwd_workspace_bytes(plan, dtype, Hq, Hkv, D);
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 16)))
        return fail(OCTOPUS_EWORKSPACE, "forward workspace needs " + std::to_string(need) +
                                            " bytes, 16-byte aligned");
    if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
    const octo::DevPlan dp = dev_view(plan->p);
    hipError_t e;
    if (dtype == OCTOPUS_BF16) {
        e = octo::launch_tiles_t(dp.T, dp.nKT, Hkv, D, v, ws, (hipStream_t)stream);
        if (e == hipSuccess)
            e = octo::launch_fwd_bf16(dp, Hq, Hkv, D, scale, q, k, ws, o, lse, nullptr,
                                      (hipStream_t)stream);
    } else {
        e = octo::launch_fwd_fp32(dp, Hq, Hkv, D, scale, q, k, v, o, lse, (hipStream_t)stream);
    }
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    return ok();
}

namespace {

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Rotated copies of Q and K at the front of a RoPE workspace.
size_t rope_part(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq, int32_t Hkv,
                 int32_t D) {
    const size_t es = dtype == OCTOPUS_BF16 ? 2 : 4;
    const size_t T = (size_t)plan->p.T;
    return round256(T * Hq * D * es) + round256(T * Hkv * D * es);
}

}  // namespace

size_t octopus_rope_workspace_bytes(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                                    int32_t Hkv, int32_t D) {
    if (plan == nullptr || Hq < 1 || Hkv < 1 || (D != 64 && D != 128) ||
        (dtype != OCTOPUS_BF16 && dtype != OCTOPUS_FP32))
        return 0;
    return rope_part(plan, dtype, Hq, Hkv, D);
}

int octopus_dag_attn_fwd_rope(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                              int32_t Hkv, int32_t D, float scale, float rope_base,
                              const void* q, const void* k, const void* v, void* o, float* lse,
                              void* ws, size_t ws_bytes, void* stream) {
    int rc = check_attn(plan, dtype, Hq, Hkv, D, {q, k, v, o, lse});
    if (rc != OCTOPUS_OK) return rc;
    if (!(rope_base > 1.f)) return fail(OCTOPUS_EINVAL, "rope_base must be > 1");
    const bool b16 = dtype == OCTOPUS_BF16;
    const size_t es = b16 ? 2 : 4;
    const size_t T = (size_t)plan->p.T;
    // bf16: only K is rotated by a pass (the forward turns each query row in registers);
    // fp32: rotated copies of Q and K.
    const size_t head = b16 ? round256(T * Hkv * D * es) : rope_part(plan, dtype, Hq, Hkv, D);
    const size_t need = head + octopus_fwd_workspace_bytes(plan, dtype, Hq, Hkv, D);
    if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
        return fail(OCTOPUS_EWORKSPACE, "forward (rope) workspace needs " +
                                            std::to_string(need) + " bytes, 256-byte aligned");
    unsigned char* w = static_cast<unsigned char*>(ws);
    const octo::DevPlan dp = dev_view(plan->p);
    hipStream_t st = (hipStream_t)stream;
    if (b16) {
        void* kr = w;
        hipError_t e = octo::launch_rope(true, dp.T, Hkv, D, rope_base, false, dp.pos, k, kr, st);
        if (e == hipSuccess) e = octo::launch_tiles_t(dp.T, dp.nKT, Hkv, D, v, w + head, st);
        if (e == hipSuccess) {
            if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
            const octo::RopeFreq rt = octo::rope_freq(D, rope_base);
            e = octo::launch_fwd_bf16(dp, Hq, Hkv, D, scale, q, kr, w + head, o, lse, &rt, st);
        }
        if (e != hipSuccess) return hip_fail(e, "forward (rope) launch");
        return ok();
    }
    void* qr = w;
    void* kr = w + round256(T * Hq * D * es);
    const hipError_t e = octo::launch_rope2(false, dp.T, D, rope_base, false, dp.pos, Hq, q, qr,
                                            Hkv, k, kr, st);
    if (e != hipSuccess) return hip_fail(e, "rope launch");
    return octopus_dag_attn_fwd(plan, dtype, Hq, Hkv, D, scale, qr, kr, v, o, lse, w + head,
                                ws_bytes - head, stream);
}

size_t octopus_bwd_workspace_bytes(const octopus_plan* plan, octopus_dtype, int32_t Hq,
                                   int32_t, int32_t) {
    if (plan == nullptr || Hq < 1) return 0;
    return octo::bwd_workspace_floats(plan->p.T, Hq) * sizeof(float);
}

namespace {

int check_bwd_ws(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq, int32_t Hkv,
                 int32_t D, void* ws, size_t ws_bytes) {
    const size_t need = octopus_bwd_workspace_bytes(plan, dtype, Hq, Hkv, D);
    if (ws == nullptr || ws_bytes < need || !aligned(ws, 16))
        return fail(OCTOPUS_EWORKSPACE, "backward workspace needs " + std::to_string(need) +
                                            " bytes, 16-byte aligned");
    return OCTOPUS_OK;
}

}  // namespace

int octopus_dag_attn_bwd_preprocess(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                                    int32_t Hkv, int32_t D, const void* o, const float* lse,
                                    const void* dout, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_attn(plan, dtype, Hq, Hkv, D, {o, lse, dout});
    if (rc == OCTOPUS_OK) rc = check_bwd_ws(plan, dtype, Hq, Hkv, D, ws, ws_bytes);
    if (rc != OCTOPUS_OK) return rc;
    const hipError_t e =
        octo::launch_bwd_preprocess(dtype == OCTOPUS_BF16, dev_view(plan->p), Hq, D, o, dout, lse,
                                    static_cast<float*>(ws), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "backward preprocess launch");
    return ok();
}

int octopus_dag_attn_bwd_dkdv(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                              int32_t Hkv, int32_t D, float scale, const void* q, const void* k,
                              const void* v, const void* dout, void* dk, void* dv,
                              const void* ws, size_t ws_bytes, void* stream) {
    int rc = check_attn(plan, dtype, Hq, Hkv, D, {q, k, v, dout, dk, dv});
    if (rc == OCTOPUS_OK)
        rc = check_bwd_ws(plan, dtype, Hq, Hkv, D, const_cast<void*>(ws), ws_bytes);
    if (rc != OCTOPUS_OK) return rc;
    if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
    const hipError_t e = octo::launch_bwd_dkdv(dtype == OCTOPUS_BF16, dev_view(plan->p), Hq, Hkv,
                                               D, scale, q, k, v, dout,
                                               static_cast<const float*>(ws), dk, dv, nullptr,
                                               (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "backward dK/dV launch");
    return ok();
}

int octopus_dag_attn_bwd_dq(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                            int32_t Hkv, int32_t D, float scale, const void* q, const void* k,
                            const void* v, const void* dout, void* dq, const void* ws,
                            size_t ws_bytes, void* stream) {
    int rc = check_attn(plan, dtype, Hq, Hkv, D, {q, k, v, dout, dq});
    if (rc == OCTOPUS_OK)
        rc = check_bwd_ws(plan, dtype, Hq, Hkv, D, const_cast<void*>(ws), ws_bytes);
    if (rc != OCTOPUS_OK) return rc;
    if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
    const hipError_t e = octo::launch_bwd_dq(dtype == OCTOPUS_BF16, dev_view(plan->p), Hq, Hkv, D,
                                             scale, q, k, v, dout,
                                             static_cast<float*>(const_cast<void*>(ws)), dq,
                                             nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "backward dQ launch");
    return ok();
}

int octopus_dag_attn_bwd(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                         int32_t Hkv, int32_t D, float scale, const void* q, const void* k,
                         const void* v, const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                         void* stream) {
    int rc = check_attn(plan, dtype, Hq, Hkv, D, {q, k, v, o, lse, dout, dq, dk, dv});
    if (rc == OCTOPUS_OK) rc = check_bwd_ws(plan, dtype, Hq, Hkv, D, ws, ws_bytes);
    if (rc != OCTOPUS_OK) return rc;
    rc = octopus_dag_attn_bwd_preprocess(plan, dtype, Hq, Hkv, D, o, lse, dout, ws, ws_bytes,
                                         stream);
    if (rc == OCTOPUS_OK)
        rc = octopus_dag_attn_bwd_dkdv(plan, dtype, Hq, Hkv, D, scale, q, k, v, dout, dk, dv, ws,
                                       ws_bytes, stream);
    if (rc == OCTOPUS_OK)
        rc = octopus_dag_attn_bwd_dq(plan, dtype, Hq, Hkv, D, scale, q, k, v, dout, dq, ws,
                                     ws_bytes, stream);
    return rc;
}

int octopus_dag_attn_bwd_rope(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                              int32_t Hkv, int32_t D, float scale, float rope_base,
                              const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              void* ws, size_t ws_bytes, void* stream) {
    int rc = check_attn(plan, dtype, Hq, Hkv, D, {q, k, v, o, lse, dout, dq, dk, dv});
    if (rc != OCTOPUS_OK) return rc;
    if (!(rope_base > 1.f)) return fail(OCTOPUS_EINVAL, "rope_base must be > 1");
    const size_t head = rope_part(plan, dtype, Hq, Hkv, D);
    const size_t need = head + octopus_bwd_workspace_bytes(plan, dtype, Hq, Hkv, D);
    if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
        return fail(OCTOPUS_EWORKSPACE, "backward (rope) workspace needs " +
                                            std::to_string(need) + " bytes, 256-byte aligned");
    unsigned char* w = static_cast<unsigned char*>(ws);
    const size_t es = dtype == OCTOPUS_BF16 ? 2 : 4;
    void* qr = w;
    void* kr = w + round256((size_t)plan->p.T * Hq * D * es);
    const octo::DevPlan dp = dev_view(plan->p);
    const bool b16 = dtype == OCTOPUS_BF16;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = octo::launch_rope2(b16, dp.T, D, rope_base, false, dp.pos, Hq, q, qr, Hkv, k,
                                      kr, st);
    if (e != hipSuccess) return hip_fail(e, "rope launch");
    if (b16) {
        // Gradients with respect to the rotated Q and K, each turned back in registers by
        // the kernel that produces it (the rotation is orthogonal).
        void* bws = w + head;
        const size_t bws_bytes = ws_bytes - head;
        if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
        const octo::RopeFreq rt = octo::rope_freq(D, rope_base);
        rc = octopus_dag_attn_bwd_preprocess(plan, dtype, Hq, Hkv, D, o, lse, dout, bws,
                                             bws_bytes, stream);
        if (rc != OCTOPUS_OK) return rc;
        e = octo::launch_bwd_dkdv(true, dp, Hq, Hkv, D, scale, qr, kr, v, dout,
                                  static_cast<const float*>(bws), dk, dv, &rt, st);
        if (e == hipSuccess)
            e = octo::launch_bwd_dq(true, dp, Hq, Hkv, D, scale, qr, kr, v, dout,
                                    static_cast<float*>(bws), dq, &rt, st);
        if (e != hipSuccess) return hip_fail(e, "backward (rope) launch");
        return ok();
    }
    // fp32: gradients with respect to the rotated Q and K, then turned back in place.
    rc = octopus_dag_attn_bwd(plan, dtype, Hq, Hkv, D, scale, qr, kr, v, o, lse, dout, dq, dk,
                              dv, w + head, ws_bytes - head, stream);
    if (rc != OCTOPUS_OK) return rc;
    e = octo::launch_rope2(b16, dp.T, D, rope_base, true, dp.pos, Hq, dq, dq, Hkv, dk, dk, st);
    if (e != hipSuccess) return hip_fail(e, "rope launch");
    return ok();
}

int octopus_decode_segments(const octopus_branch* branches, int32_t n_branches,
                            const octopus_mount* mounts, int32_t n_mounts,
                            const int32_t* page_ptr, const int32_t* pages, int32_t page_size,
                            int32_t n_pages, const int32_t* cursors, int32_t n_cursors,
                            int32_t share, int32_t* seg_ptr_out, int32_t* seg_page_out,
                            int32_t* seg_lo_out, int32_t* seg_hi_out, int32_t seg_capacity,
                            int32_t* n_seg_out, int32_t* grp_ptr_out, int32_t* grp_cur_out,
                            int32_t* n_groups_out) {
    if (n_seg_out == nullptr) return fail(OCTOPUS_EINVAL, "n_seg_out is NULL");
    if (share && n_groups_out == nullptr) return fail(OCTOPUS_EINVAL, "n_groups_out is NULL");
    try {
        if (n_branches < 1 || branches == nullptr) return fail(OCTOPUS_EINVAL, "no branches");
        int64_t T = 0;
        for (int32_t b = 0; b < n_branches; ++b) T += branches[b].len > 0 ? branches[b].len : 0;
        if (T < 1 || T > octo::kMaxTokens) return fail(OCTOPUS_EINVAL, "total tokens out of range");
        octo::DagInfo dag;
        std::string err;
        int rc = octo::load_dag(branches, n_branches, mounts, n_mounts, (int32_t)T, dag, err,
                                false);
        if (rc != OCTOPUS_OK) return fail(rc, err);
        std::vector<int32_t> sp, pg, lo, hi, gp, gc;
        rc = octo::build_segments(dag, page_ptr, pages, page_size, n_pages, cursors, n_cursors,
                                  share != 0, sp, pg, lo, hi, gp, gc, err);
        if (rc != OCTOPUS_OK) return fail(rc, err);
        if (pg.size() > (size_t)INT32_MAX) return fail(OCTOPUS_EINVAL, "too many segments");
        *n_seg_out = (int32_t)pg.size();
        if (share) *n_groups_out = (int32_t)gp.size() - 1;
        if (seg_capacity < (int64_t)pg.size())
            return fail(OCTOPUS_EWORKSPACE, "segment capacity too small; need " +
                                                std::to_string(pg.size()));
        if (!seg_ptr_out || !seg_page_out || !seg_lo_out || !seg_hi_out)
            return fail(OCTOPUS_EINVAL, "NULL output array");
        if (share && (!grp_ptr_out || !grp_cur_out))
            return fail(OCTOPUS_EINVAL, "NULL group output array");
        std::copy(sp.begin(), sp.end(), seg_ptr_out);
        std::copy(pg.begin(), pg.end(), seg_page_out);
        std::copy(lo.begin(), lo.end(), seg_lo_out);
        std::copy(hi.begin(), hi.end(), seg_hi_out);
        if (share) {
            std::copy(gp.begin(), gp.end(), grp_ptr_out);
            std::copy(gc.begin(), gc.end(), grp_cur_out);
        }
        return ok();
    } catch (const std::bad_alloc&) {
        return fail(OCTOPUS_ENOMEM, "host allocation failed while building segments");
    }
}

int octopus_dag_positions(const octopus_branch* branches, int32_t n_branches,
                          const octopus_mount* mounts, int32_t n_mounts, int32_t total_tokens,
                          int32_t* pos_out) {
    if (pos_out == nullptr) return fail(OCTOPUS_EINVAL, "pos_out is NULL");
    try {
        octo::DagInfo dag;
        std::string err;
        const int rc = octo::load_dag(branches, n_branches, mounts, n_mounts, total_tokens, dag,
                                      err);
        if (rc != OCTOPUS_OK) return fail(rc, err);
        for (int32_t i = 0; i < total_tokens; ++i) pos_out[i] = (int32_t)dag.pos[i];
        return ok();
    } catch (const std::bad_alloc&) {
        return fail(OCTOPUS_ENOMEM, "host allocation failed while computing positions");
    }
}

int octopus_rope(octopus_dtype dtype, int32_t rows, int32_t H, int32_t D, float rope_base,
                 int32_t inverse, const int32_t* pos, const void* x, void* out, void* stream) {
    if (dtype != OCTOPUS_BF16 && dtype != OCTOPUS_FP32)
        return fail(OCTOPUS_EUNSUPPORTED, "dtype must be bf16 or fp32");
    if (D != 64 && D != 128) return fail(OCTOPUS_EUNSUPPORTED, "head_dim must be 64 or 128");
    if (rows < 0 || H < 1) return fail(OCTOPUS_EINVAL, "rows must be >= 0 and H >= 1");
    if (!(rope_base > 1.f)) return fail(OCTOPUS_EINVAL, "rope_base must be > 1");
    if (rows > 0 && (!pos || !x || !out)) return fail(OCTOPUS_EINVAL, "NULL pointer");
    const hipError_t e = octo::launch_rope(dtype == OCTOPUS_BF16, rows, H, D, rope_base,
                                           inverse != 0, pos, x, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "rope launch");
    return ok();
}

namespace {
// Bytes of one float32 H x 128 x 128 state set (a checkpoint slot, or one chunk's).
size_t gdn_state_bytes(int32_t H) { return (size_t)H * 128 * 128 * sizeof(float); }
size_t gdn_prep_bytes(const octopus_plan* plan, int32_t H) {
    return octo::gdn_prep_floats(plan->p.n_chunks, H) * sizeof(float);
}

// A second stream of the current device (default priority) with three events, created on
// first use and kept for the life of the process.  The scan runs independent launches on
// it next to the caller's stream: a fork event recorded on the caller's stream, work on
// the side stream (with an optional mark the caller's stream may wait for), a join event
// the caller's stream waits for.  g_side_mu is held from the fork to the join so that
// concurrent calls do not re-record the events in between.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr, mid = nullptr;
};
std::mutex g_side_mu;
std::map<int, SideStream> g_side;
hipError_t side_stream(SideStream& out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    auto it = g_side.find(dev);
    if (it == g_side.end()) {
        SideStream sd;
        e = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&sd.join, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&sd.mid, hipEventDisableTiming);
        if (e != hipSuccess) {
            if (sd.mid) (void)hipEventDestroy(sd.mid);
            if (sd.join) (void)hipEventDestroy(sd.join);
            if (sd.fork) (void)hipEventDestroy(sd.fork);
            if (sd.s) (void)hipStreamDestroy(sd.s);
            return e;
        }
        it = g_side.emplace(dev, sd).first;
    }
    out = it->second;
    return hipSuccess;
}
// Forks work off `st` onto the side stream and joins it back: fork() records the fork
// event and makes the side stream wait for it; mark() records a point of the side stream
// that wait_mark() makes `st` wait for; join() (also run by the destructor, so every
// return path joins) records the join event and makes `st` wait for it.
class SideFork {
  public:
    explicit SideFork(hipStream_t st) : st_(st) {}
    hipError_t fork(hipStream_t& side) {
        lock_ = std::unique_lock<std::mutex>(g_side_mu);
        hipError_t e = side_stream(sd_);
        if (e == hipSuccess) e = hipEventRecord(sd_.fork, st_);
        if (e == hipSuccess) e = hipStreamWaitEvent(sd_.s, sd_.fork, 0);
        if (e != hipSuccess) {
            lock_.unlock();
            return e;
        }
        forked_ = true;
        side = sd_.s;
        return hipSuccess;
    }
    hipError_t mark() { return forked_ ? hipEventRecord(sd_.mid, sd_.s) : hipSuccess; }
    hipError_t wait_mark() { return forked_ ? hipStreamWaitEvent(st_, sd_.mid, 0) : hipSuccess; }
    hipError_t join() {
        if (!forked_) return hipSuccess;
        forked_ = false;
        hipError_t e = hipEventRecord(sd_.join, sd_.s);
        if (e == hipSuccess) e = hipStreamWaitEvent(st_, sd_.join, 0);
        if (e != hipSuccess) (void)hipStreamSynchronize(sd_.s);  // cannot order st after it
        lock_.unlock();
        return e;
    }
    ~SideFork() { (void)join(); }

  private:
    hipStream_t st_;
    SideStream sd_;
    bool forked_ = false;
    std::unique_lock<std::mutex> lock_;
};

// The scan forward: the records of every chunk, then the branches level by level.  The
// first level's branches need only their own chunks' records, and one workgroup per
// (branch, head) leaves most compute units idle, so the deeper levels' records are
// prepared on the side stream while the first level runs.  chunk_states may be NULL.
int gdn_forward_run(const octopus_plan* plan, int32_t H, const void* q, const void* k,
                    const void* v, const float* alpha, const float* beta, void* o, float* slots,
                    float* chunk_states, float* prep, hipStream_t st) {
    const octo::DevPlan dp = dev_view(plan->p);
    const std::vector<int32_t>& lp = plan->p.level_ptr;
    const std::vector<int32_t>& lc = plan->p.level_chunk;
    const int32_t first = lc[1];
    const int64_t rest = plan->p.n_chunks - first;
    // Order of the launches: the first level's records, then the fork, the first level's
    // forward, and only then the side stream's records.  The forward's workgroups each need
    // a whole compute unit, so they must be dispatched before the side stream's many small
    // workgroups fill every unit (they become ready together when the first records land).
    // (the transposed record blocks only when a backward follows: chunk_states kept)
    const bool with_t = chunk_states != nullptr;
    hipError_t e = octo::launch_gdn_chunk_prep(dp, 0, first, H, with_t, q, k, alpha, beta,
                                               prep, st);
    if (e != hipSuccess) return hip_fail(e, "scan prep launch");
    SideFork side(st);
    hipStream_t s2 = nullptr;
    if (rest > 0) {
        e = side.fork(s2);
        if (e != hipSuccess) return hip_fail(e, "scan side stream");
    }
    e = octo::launch_gdn_chunk_fwd(dp, lp[0], lp[1] - lp[0], H, q, k, v, prep, o, slots,
                                   chunk_states, st);
    if (e != hipSuccess) return hip_fail(e, "scan forward launch");
    if (rest > 0) {
        e = octo::launch_gdn_chunk_prep(dp, first, rest, H, with_t, q, k, alpha, beta, prep,
                                        s2);
        if (e != hipSuccess) return hip_fail(e, "scan prep launch");
    }
    e = side.join();
    if (e != hipSuccess) return hip_fail(e, "scan side stream");
    for (size_t l = 1; l + 1 < lp.size(); ++l) {
        e = octo::launch_gdn_chunk_fwd(dp, lp[l], lp[l + 1] - lp[l], H, q, k, v, prep, o,
                                       slots, chunk_states, st);
        if (e != hipSuccess) return hip_fail(e, "scan forward launch");
    }
    return OCTOPUS_OK;
}
// Arguments shared by the scan's forward and backward.
int check_gdn(const octopus_plan* plan, octopus_dtype dtype, int32_t H, int32_t Dk, int32_t Dv,
              std::initializer_list<const void*> tensors) {
    if (plan == nullptr) return fail(OCTOPUS_EINVAL, "plan is NULL");
    if (plan->p.dev == nullptr) return fail(OCTOPUS_ESTATE, "plan not uploaded");
    if (dtype != OCTOPUS_BF16) return fail(OCTOPUS_EUNSUPPORTED, "the scan supports bf16 only");
    if (Dk != 128 || Dv != 128) return fail(OCTOPUS_EUNSUPPORTED, "the scan supports Dk = Dv = 128");
    if (H < 1) return fail(OCTOPUS_EINVAL, "H must be >= 1");
    if ((int64_t)plan->p.n_chunks * H > INT32_MAX)
        return fail(OCTOPUS_EUNSUPPORTED, "too many (chunk, head) pairs for one launch");
    for (const void* p : tensors) {
        if (p == nullptr) return fail(OCTOPUS_EINVAL, "a tensor pointer is NULL");
        if (!aligned(p, 16)) return fail(OCTOPUS_EINVAL, "tensors must be 16-byte aligned");
    }
    return OCTOPUS_OK;
}
}  // namespace

size_t octopus_gdn_workspace_bytes(const octopus_plan* plan, int32_t H, int32_t Dk,
                                   int32_t Dv) {
    if (plan == nullptr || H < 1 || Dk != 128 || Dv != 128) return 0;
    return (size_t)std::max(plan->p.n_slots, 1) * gdn_state_bytes(H) + gdn_prep_bytes(plan, H);
}

int octopus_gated_delta_scan(const octopus_plan* plan, octopus_dtype dtype, int32_t H,
                             int32_t Dk, int32_t Dv, const void* q, const void* k,
                             const void* v, const float* alpha, const float* beta, void* o,
                             void* ws, size_t ws_bytes, void* stream) {
    const int rc = check_gdn(plan, dtype, H, Dk, Dv,
                             {q, k, v, (const void*)alpha, (const void*)beta, (const void*)o});
    if (rc != OCTOPUS_OK) return rc;
    const size_t need = octopus_gdn_workspace_bytes(plan, H, Dk, Dv);
    if (ws == nullptr || ws_bytes < need || !aligned(ws, 16))
        return fail(OCTOPUS_EWORKSPACE, "scan workspace needs " + std::to_string(need) +
                                            " bytes, 16-byte aligned");
    float* slots = static_cast<float*>(ws);
    float* prep = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                           (size_t)std::max(plan->p.n_slots, 1) *
                                               gdn_state_bytes(H));
    const int r = gdn_forward_run(plan, H, q, k, v, alpha, beta, o, slots, nullptr, prep,
                                  (hipStream_t)stream);
    return r == OCTOPUS_OK ? ok() : r;
}

size_t octopus_gdn_bwd_workspace_bytes(const octopus_plan* plan, int32_t H, int32_t Dk,
                                       int32_t Dv) {
    if (plan == nullptr || H < 1 || Dk != 128 || Dv != 128) return 0;
    return ((size_t)std::max(plan->p.n_slots, 1) + plan->p.sc_init.size() +
            (size_t)2 * plan->p.n_chunks) * gdn_state_bytes(H) +
           gdn_prep_bytes(plan, H);
}

namespace {
// The scan backward's workspace, in order: checkpoint slots [n_slots][H][128][128], every
// branch's initial-state gradient [nb][H][128][128], the state at every chunk start and the
// state gradient at every chunk end [n_chunks][H][128][128] (key-major), the per-chunk
// records.
struct GdnBwdWs {
    float *slots, *dkids, *chunks, *dsc, *prep;
};
GdnBwdWs gdn_bwd_ws(const octopus_plan* plan, int32_t H, void* ws) {
    const size_t n_slots = (size_t)std::max(plan->p.n_slots, 1);
    const size_t per = gdn_state_bytes(H) / sizeof(float);  // floats per state set
    const size_t nc = (size_t)plan->p.n_chunks;
    GdnBwdWs w;
    w.slots = static_cast<float*>(ws);
    w.dkids = w.slots + per * n_slots;
    w.chunks = w.dkids + per * plan->p.sc_init.size();
    w.dsc = w.chunks + per * nc;
    w.prep = w.dsc + per * nc;
    return w;
}
int check_gdn_bwd_ws(const octopus_plan* plan, int32_t H, int32_t Dk, int32_t Dv, void* ws,
                     size_t ws_bytes) {
    const size_t need = octopus_gdn_bwd_workspace_bytes(plan, H, Dk, Dv);
    if (ws == nullptr || ws_bytes < need || !aligned(ws, 16))
        return fail(OCTOPUS_EWORKSPACE, "scan backward workspace needs " + std::to_string(need) +
                                            " bytes, 16-byte aligned");
    return OCTOPUS_OK;
}
// The forward, keeping in the backward's workspace what the backward reads: the records
// and the state at every chunk start (o may be NULL).
int gdn_forward_keep(const octopus_plan* plan, int32_t H, const void* q, const void* k,
                     const void* v, const float* alpha, const float* beta, void* o, void* ws,
                     hipStream_t st) {
    const GdnBwdWs w = gdn_bwd_ws(plan, H, ws);
    return gdn_forward_run(plan, H, q, k, v, alpha, beta, o, w.slots, w.chunks, w.prep, st);
}
// The backward proper, from what gdn_forward_keep left in the workspace.
int gdn_backward_kept(const octopus_plan* plan, int32_t H, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta, const void* dout,
                      void* dq, void* dk, void* dv, float* dalpha, float* dbeta, void* ws,
                      hipStream_t st) {
    const octo::DevPlan dp = dev_view(plan->p);
    const std::vector<int32_t>& lp = plan->p.level_ptr;
    const std::vector<int32_t>& lc = plan->p.level_chunk;
    const GdnBwdWs w = gdn_bwd_ws(plan, H, ws);
    hipError_t e = hipSuccess;
    // state gradients, deepest level first: a child's initial-state gradient is written
    // before its parent runs
    for (size_t l = lp.size() - 1; l-- > 1;) {
        e = octo::launch_gdn_chunk_dstate(dp, lp[l], lp[l + 1] - lp[l], H, q, k, dout, w.prep,
                                          w.dsc, w.dkids, st);
        if (e != hipSuccess) return hip_fail(e, "scan backward (state gradient) launch");
    }
    // The deeper levels' chunks have their state gradients now: their gradients run on the
    // side stream while the first level's state gradient (few workgroups) runs here.
    const int32_t first = lc[1];
    const int64_t rest = plan->p.n_chunks - first;
    // (the first level's state gradient is enqueued first, so that its workgroups, which
    // each need a whole compute unit, are dispatched before the side stream's)
    SideFork side(st);
    hipStream_t s2 = nullptr;
    if (rest > 0) {
        e = side.fork(s2);
        if (e != hipSuccess) return hip_fail(e, "scan side stream");
    }
    e = octo::launch_gdn_chunk_dstate(dp, lp[0], lp[1] - lp[0], H, q, k, dout, w.prep, w.dsc,
                                      w.dkids, st);
    if (e != hipSuccess) return hip_fail(e, "scan backward (state gradient) launch");
    if (rest > 0) {
        e = octo::launch_gdn_chunk_grad(dp, first, rest, H, q, k, v, alpha, beta, dout, w.prep,
                                        w.chunks, w.dsc, dq, dk, dv, dalpha, dbeta, s2);
        if (e != hipSuccess) return hip_fail(e, "scan backward launch");
    }
    e = octo::launch_gdn_chunk_grad(dp, 0, first, H, q, k, v, alpha, beta, dout, w.prep,
                                    w.chunks, w.dsc, dq, dk, dv, dalpha, dbeta, st);
    if (e != hipSuccess) return hip_fail(e, "scan backward launch");
    e = side.join();
    if (e != hipSuccess) return hip_fail(e, "scan side stream");
    return OCTOPUS_OK;
}
}  // namespace

namespace {
// The backward with its forward replay.  The state gradient needs only q, k, dout and the
// records, not the forward's states, so the whole state-gradient chain (deepest level first)
// runs on the side stream while this stream replays the forward's levels; the gradients
// follow once both are done.  (The first level's records come first, then the fork, the
// first level's forward and the deeper levels' records on the side stream, as in the
// forward.)
int gdn_backward_full(const octopus_plan* plan, int32_t H, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta, const void* dout,
                      void* dq, void* dk, void* dv, float* dalpha, float* dbeta, void* ws,
                      hipStream_t st) {
    const octo::DevPlan dp = dev_view(plan->p);
    const std::vector<int32_t>& lp = plan->p.level_ptr;
    const std::vector<int32_t>& lc = plan->p.level_chunk;
    const GdnBwdWs w = gdn_bwd_ws(plan, H, ws);
    const int32_t first = lc[1];
    const int64_t rest = plan->p.n_chunks - first;
    hipError_t e = octo::launch_gdn_chunk_prep(dp, 0, first, H, true, q, k, alpha, beta,
                                               w.prep, st);
    if (e != hipSuccess) return hip_fail(e, "scan prep launch");
    SideFork side(st);
    hipStream_t s2 = nullptr;
    e = side.fork(s2);
    if (e != hipSuccess) return hip_fail(e, "scan side stream");
    e = octo::launch_gdn_chunk_fwd(dp, lp[0], lp[1] - lp[0], H, q, k, v, w.prep, nullptr,
                                   w.slots, w.chunks, st);
    if (e != hipSuccess) return hip_fail(e, "scan forward launch");
    e = octo::launch_gdn_chunk_prep(dp, first, rest, H, true, q, k, alpha, beta, w.prep, s2);
    if (e == hipSuccess) e = side.mark();
    if (e != hipSuccess) return hip_fail(e, "scan prep launch");
    for (size_t l = lp.size() - 1; l-- > 0;) {
        e = octo::launch_gdn_chunk_dstate(dp, lp[l], lp[l + 1] - lp[l], H, q, k, dout, w.prep,
                                          w.dsc, w.dkids, s2);
        if (e != hipSuccess) return hip_fail(e, "scan backward (state gradient) launch");
    }
    e = side.wait_mark();
    if (e != hipSuccess) return hip_fail(e, "scan side stream");
    for (size_t l = 1; l + 1 < lp.size(); ++l) {
        e = octo::launch_gdn_chunk_fwd(dp, lp[l], lp[l + 1] - lp[l], H, q, k, v, w.prep, nullptr,
                                       w.slots, w.chunks, st);
        if (e != hipSuccess) return hip_fail(e, "scan forward launch");
    }
    e = side.join();
    if (e != hipSuccess) return hip_fail(e, "scan side stream");
    e = octo::launch_gdn_chunk_grad(dp, 0, plan->p.n_chunks, H, q, k, v, alpha, beta, dout,
                                    w.prep, w.chunks, w.dsc, dq, dk, dv, dalpha, dbeta, st);
    if (e != hipSuccess) return hip_fail(e, "scan backward launch");
    return OCTOPUS_OK;
}
}  // namespace

int octopus_gated_delta_scan_bwd(const octopus_plan* plan, octopus_dtype dtype, int32_t H,
                                 int32_t Dk, int32_t Dv, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const void* dout, void* dq, void* dk, void* dv, float* dalpha,
                                 float* dbeta, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_gdn(plan, dtype, H, Dk, Dv,
                       {q, k, v, (const void*)alpha, (const void*)beta, dout, (const void*)dq,
                        (const void*)dk, (const void*)dv, (const void*)dalpha,
                        (const void*)dbeta});
    if (rc == OCTOPUS_OK) rc = check_gdn_bwd_ws(plan, H, Dk, Dv, ws, ws_bytes);
    if (rc != OCTOPUS_OK) return rc;
    // the forward again (keeping the state at the start of every chunk) beside the state
    // gradient, then the gradients
    rc = gdn_backward_full(plan, H, q, k, v, alpha, beta, dout, dq, dk, dv, dalpha, dbeta, ws,
                           (hipStream_t)stream);
    return rc == OCTOPUS_OK ? ok() : rc;
}

int octopus_gated_delta_scan_save(const octopus_plan* plan, octopus_dtype dtype, int32_t H,
                                  int32_t Dk, int32_t Dv, const void* q, const void* k,
                                  const void* v, const float* alpha, const float* beta, void* o,
                                  void* ws, size_t ws_bytes, void* stream) {
    int rc = check_gdn(plan, dtype, H, Dk, Dv,
                       {q, k, v, (const void*)alpha, (const void*)beta, (const void*)o});
    if (rc == OCTOPUS_OK) rc = check_gdn_bwd_ws(plan, H, Dk, Dv, ws, ws_bytes);
    if (rc != OCTOPUS_OK) return rc;
    rc = gdn_forward_keep(plan, H, q, k, v, alpha, beta, o, ws, (hipStream_t)stream);
    return rc == OCTOPUS_OK ? ok() : rc;
}

int octopus_gated_delta_scan_bwd_saved(const octopus_plan* plan, octopus_dtype dtype,
                                       int32_t H, int32_t Dk, int32_t Dv, const void* q,
                                       const void* k, const void* v, const float* alpha,
                                       const float* beta, const void* dout, void* dq, void* dk,
                                       void* dv, float* dalpha, float* dbeta, void* ws,
                                       size_t ws_bytes, void* stream) {
    int rc = check_gdn(plan, dtype, H, Dk, Dv,
                       {q, k, v, (const void*)alpha, (const void*)beta, dout, (const void*)dq,
                        (const void*)dk, (const void*)dv, (const void*)dalpha,
                        (const void*)dbeta});
    if (rc == OCTOPUS_OK) rc = check_gdn_bwd_ws(plan, H, Dk, Dv, ws, ws_bytes);
    if (rc != OCTOPUS_OK) return rc;
    rc = gdn_backward_kept(plan, H, q, k, v, alpha, beta, dout, dq, dk, dv, dalpha, dbeta, ws,
                           (hipStream_t)stream);
    return rc == OCTOPUS_OK ? ok() : rc;
}

int octopus_extend_segments(const octopus_branch* branches, int32_t n_branches,
                            const octopus_mount* mounts, int32_t n_mounts,
                            const int32_t* page_ptr, const int32_t* pages, int32_t page_size,
                            int32_t n_pages, const int32_t* cursors, int32_t n_cursors,
                            const int32_t* n_new, int32_t* seg_ptr_out, int32_t* seg_page_out,
                            int32_t* seg_lo_out, int32_t* seg_hi_out, int32_t* seg_thr_out,
                            int32_t* seg_causal_out, int32_t seg_capacity, int32_t* n_seg_out,
                            int32_t* first_off_out) {
    if (n_seg_out == nullptr) return fail(OCTOPUS_EINVAL, "n_seg_out is NULL");
    try {
        if (n_branches < 1 || branches == nullptr) return fail(OCTOPUS_EINVAL, "no branches");
        int64_t T = 0;
        for (int32_t b = 0; b < n_branches; ++b) T += branches[b].len > 0 ? branches[b].len : 0;
        if (T < 1 || T > octo::kMaxTokens) return fail(OCTOPUS_EINVAL, "total tokens out of range");
        octo::DagInfo dag;
        std::string err;
        int rc = octo::load_dag(branches, n_branches, mounts, n_mounts, (int32_t)T, dag, err,
                                false);
        if (rc != OCTOPUS_OK) return fail(rc, err);
        std::vector<int32_t> sp, pg, lo, hi, th, ca, fo;
        rc = octo::build_extend_segments(dag, page_ptr, pages, page_size, n_pages, cursors,
                                         n_cursors, n_new, sp, pg, lo, hi, th, ca, fo, err);
        if (rc != OCTOPUS_OK) return fail(rc, err);
        if (pg.size() > (size_t)INT32_MAX) return fail(OCTOPUS_EINVAL, "too many segments");
        *n_seg_out = (int32_t)pg.size();
        if (seg_capacity < (int64_t)pg.size())
            return fail(OCTOPUS_EWORKSPACE, "segment capacity too small; need " +
                                                std::to_string(pg.size()));
        if (!seg_ptr_out || !seg_page_out || !seg_lo_out || !seg_hi_out || !seg_thr_out ||
            !seg_causal_out || !first_off_out)
            return fail(OCTOPUS_EINVAL, "NULL output array");
        std::copy(sp.begin(), sp.end(), seg_ptr_out);
        std::copy(pg.begin(), pg.end(), seg_page_out);
        std::copy(lo.begin(), lo.end(), seg_lo_out);
        std::copy(hi.begin(), hi.end(), seg_hi_out);
        std::copy(th.begin(), th.end(), seg_thr_out);
        std::copy(ca.begin(), ca.end(), seg_causal_out);
        std::copy(fo.begin(), fo.end(), first_off_out);
        return ok();
    } catch (const std::bad_alloc&) {
        return fail(OCTOPUS_ENOMEM, "host allocation failed while building segments");
    }
}

int octopus_paged_mount_extend(octopus_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t page_size, float scale, const void* q,
                               const void* k_pool, const void* v_pool, int32_t n_pages,
                               const int32_t* q_ptr, int32_t max_new, const int32_t* first_off,
                               const int32_t* seg_ptr, const int32_t* seg_page,
                               const int32_t* seg_lo, const int32_t* seg_hi,
                               const int32_t* seg_thr, const int32_t* seg_causal, void* o,
                               float* lse, void* stream) {
    if (dtype != OCTOPUS_BF16 && dtype != OCTOPUS_FP32)
        return fail(OCTOPUS_EUNSUPPORTED, "dtype must be bf16 or fp32");
    if (D != 64 && D != 128) return fail(OCTOPUS_EUNSUPPORTED, "head_dim must be 64 or 128");
    if (page_size != 64) return fail(OCTOPUS_EUNSUPPORTED, "extend supports page_size 64 only");
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(OCTOPUS_EINVAL, "B, Hq, Hkv must be positive with Hq % Hkv == 0");
    if (Hq / Hkv > 16) return fail(OCTOPUS_EUNSUPPORTED, "Hq / Hkv must be <= 16");
    if (max_new < 1) return fail(OCTOPUS_EINVAL, "max_new must be >= 1");
    if (n_pages < 1) return fail(OCTOPUS_EINVAL, "n_pages must be >= 1");
    for (const void* p : {q, k_pool, v_pool, (const void*)o, (const void*)lse}) {
        if (p == nullptr) return fail(OCTOPUS_EINVAL, "a tensor pointer is NULL");
        if (!aligned(p, 16)) return fail(OCTOPUS_EINVAL, "tensors must be 16-byte aligned");
    }
    if (!q_ptr || !first_off || !seg_ptr || !seg_page || !seg_lo || !seg_hi || !seg_thr ||
        !seg_causal)
        return fail(OCTOPUS_EINVAL, "index arrays must not be NULL");
    if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
    hipError_t e = octo::launch_extend(dtype == OCTOPUS_BF16, B, Hq, Hkv, D, scale, q, k_pool,
                                       v_pool, n_pages, q_ptr, max_new, first_off, seg_ptr,
                                       seg_page, seg_lo, seg_hi, seg_thr, seg_causal, o, lse,
                                       (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "extend launch");
    return ok();
}

size_t octopus_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t n_split) {
    if (B < 1 || Hq < 1 || D < 1 || n_split < 1) return 0;
    return (size_t)B * 2 * n_split * Hq * (D + 4) * sizeof(float);
}

namespace {

// Argument checks shared by the two decode entry points (nothing is enqueued on error).
int check_decode(octopus_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                 int32_t page_size, const void* q, const void* k_pool, const void* v_pool,
                 int32_t n_pages, const int32_t* seg_ptr, const int32_t* seg_page,
                 const int32_t* seg_lo, const int32_t* seg_hi, int32_t n_groups,
                 const int32_t* grp_ptr, const int32_t* grp_cur, int32_t n_split, void* o) {
    if (dtype != OCTOPUS_BF16 && dtype != OCTOPUS_FP32)
        return fail(OCTOPUS_EUNSUPPORTED, "dtype must be bf16 or fp32");
    if (D != 64 && D != 128) return fail(OCTOPUS_EUNSUPPORTED, "head_dim must be 64 or 128");
    if (page_size != 64) return fail(OCTOPUS_EUNSUPPORTED, "decode supports page_size 64 only");
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(OCTOPUS_EINVAL, "B, Hq, Hkv must be positive with Hq % Hkv == 0");
    if (Hq / Hkv > 8) return fail(OCTOPUS_EUNSUPPORTED, "Hq / Hkv must be <= 8");
    if (n_split < 1 || n_split > 256) return fail(OCTOPUS_EINVAL, "n_split must be in [1, 256]");
    if (n_pages < 0) return fail(OCTOPUS_EINVAL, "n_pages < 0");
    for (const void* p : {q, k_pool, v_pool, (const void*)o}) {
        if (p == nullptr) return fail(OCTOPUS_EINVAL, "a tensor pointer is NULL");
        if (!aligned(p, 16)) return fail(OCTOPUS_EINVAL, "tensors must be 16-byte aligned");
    }
    if (!seg_ptr || !seg_page || !seg_lo || !seg_hi)
        return fail(OCTOPUS_EINVAL, "segment arrays must not be NULL");
    if (n_groups < 0 || n_groups > B) return fail(OCTOPUS_EINVAL, "n_groups must be in [0, B]");
    if (n_groups > 0 && (!grp_ptr || !grp_cur))
        return fail(OCTOPUS_EINVAL, "group arrays must not be NULL");
    return OCTOPUS_OK;
}

}  // namespace

int octopus_paged_mount_decode(octopus_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t page_size, float scale, const void* q,
                               const void* k_pool, const void* v_pool, int32_t n_pages,
                               const int32_t* seg_ptr, const int32_t* seg_page,
                               const int32_t* seg_lo, const int32_t* seg_hi, int32_t n_groups,
                               const int32_t* grp_ptr, const int32_t* grp_cur, int32_t n_split,
                               void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
    const int rc = check_decode(dtype, B, Hq, Hkv, D, page_size, q, k_pool, v_pool, n_pages,
                                seg_ptr, seg_page, seg_lo, seg_hi, n_groups, grp_ptr, grp_cur,
                                n_split, o);
    if (rc != OCTOPUS_OK) return rc;
    const size_t need = octopus_decode_workspace_bytes(B, Hq, D, n_split);
    if (ws == nullptr || ws_bytes < need || !aligned(ws, 16))
        return fail(OCTOPUS_EWORKSPACE, "decode workspace needs " + std::to_string(need) +
                                            " bytes, 16-byte aligned");
    if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
    hipError_t e = octo::launch_decode(dtype == OCTOPUS_BF16, B, Hq, Hkv, D, page_size, scale,
                                       q, k_pool, v_pool, n_pages, seg_ptr, seg_page, seg_lo,
                                       seg_hi, n_groups, grp_ptr, grp_cur, n_split, o, lse,
                                       static_cast<float*>(ws), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
}

int octopus_paged_mount_decode_noalloc(octopus_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t D, int32_t page_size, float scale, const void* q,
                                       const void* k_pool, const void* v_pool, int32_t n_pages,
                                       const int32_t* seg_ptr, const int32_t* seg_page,
                                       const int32_t* seg_lo, const int32_t* seg_hi,
                                       int32_t n_groups, const int32_t* grp_ptr,
                                       const int32_t* grp_cur, int32_t n_split, void* o,
                                       float* lse, void* stream) {
    const int rc = check_decode(dtype, B, Hq, Hkv, D, page_size, q, k_pool, v_pool, n_pages,
                                seg_ptr, seg_page, seg_lo, seg_hi, n_groups, grp_ptr, grp_cur,
                                n_split, o);
    if (rc != OCTOPUS_OK) return rc;
    const size_t need = octopus_decode_workspace_bytes(B, Hq, D, n_split);
    if (need > (size_t)OCTOPUS_DECODE_SCRATCH_BYTES)
        return fail(OCTOPUS_EWORKSPACE,
                    "decode partial states need " + std::to_string(need) +
                        " bytes; the no-allocation entry point holds at most " +
                        std::to_string((size_t)OCTOPUS_DECODE_SCRATCH_BYTES) +
                        " (fewer splits or cursors per call)");
    void* scratch = nullptr;
    hipError_t e = octo::decode_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "decode scratch lookup");
    if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
    e = octo::launch_decode(dtype == OCTOPUS_BF16, B, Hq, Hkv, D, page_size, scale, q, k_pool,
                            v_pool, n_pages, seg_ptr, seg_page, seg_lo, seg_hi, n_groups, grp_ptr,
                            grp_cur, n_split, o, lse, static_cast<float*>(scratch),
                            (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
}

}  // extern "C"
