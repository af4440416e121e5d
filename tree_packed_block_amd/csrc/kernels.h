// Device-side interface shared by the C ABI and the HIP kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace octo {

// Device view of an uploaded plan (see plan.h for how the host builds it).
struct DevPlan {
    int32_t T, nQT, nKT, n_partial;  // mask index n_partial is all ones (FULL)
    const int32_t* fwd_order;   // [nQT] query tiles, longest list first
    const int32_t* qt_ptr;      // [nQT+1]
    const int2* q_pairs;        // [n_pairs] {kv_tile, mask (-1 = FULL)}
    const int32_t* bwd_order;   // [nKT] KV tiles, longest list first
    const int32_t* kt_ptr;      // [nKT+1]
    const int2* k_pairs;        // [n_pairs] {q_tile, mask}
    const uint64_t* mask_rows;  // [n_partial + 1][128] bit x of row r: row sees key x
                                // (n_partial: all ones)
    const uint64_t* mask_cols;  // [n_partial + 2][64][2] bit r of key x: row r sees key x
                                // (n_partial: all ones, n_partial + 1: all zeros)
    int32_t nKB, pad;           // 128-key blocks
    const int32_t* blk_order;   // [nKB] blocks, longest list first
    const int32_t* blk_ptr;     // [nKB+1]
    const int4* blk_entries;    // {q_tile, mask of tile 2b, mask of tile 2b+1, 0};
                                // mask -1 FULL, -2 not seen, else PARTIAL index
    const int32_t* pos;         // [T] position of every packed token
    // Recurrent scan (per branch): own tokens [start, start + len), initial checkpoint
    // slot (-1: zero state), checkpoints to save (CSR over branches: own offset, slot),
    // branches grouped by depth.
    const int32_t *sc_start, *sc_len, *sc_init, *sc_ck_ptr, *sc_ck_off, *sc_ck_slot,
        *sc_level_br;
    // Chunked scan: first chunk of every branch [nb+1]; first packed token and length of
    // every chunk [n_chunks].
    const int32_t *sc_chunk_base, *sc_chunk_tok, *sc_chunk_nt;
    // The children forking at every checkpoint (CSR over the checkpoint entries, ascending).
    const int32_t *sc_ck_kid_ptr, *sc_ck_kid;
};

// Rotary-embedding frequencies of rotate-half pairs (x_i, x_{i+D/2}): pair i turns by
// pos * theta_i radians, theta_i = base^(-2i/D), i.e. pos * turn0 * ratio^i full turns with
// turn0 = 1 / (2 pi) and ratio = base^(-2/D).  Float64: pos * theta_0 reaches 2^24
// radians, which only float64 reduces to a fraction of a turn without losing the angle.
struct RopeFreq {
    double turn0, ratio;
};
RopeFreq rope_freq(int D, float base);

constexpr int kBq = 128;  // query rows per tile
// Rows of the backward's LSE2 and Delta workspace per head: T rounded up to whole query
// tiles (the padded rows hold LSE2 = +inf and Delta = 0).
__host__ __device__ inline int padded_rows(int T) { return (T + kBq - 1) / kBq * kBq; }
constexpr int kBk = 64;   // keys per KV tile

// V re-laid per 64-key tile so that the forward's MFMA operands which contract over
// keys (V^T) are plain 16-byte LDS reads: bf16
// [Hkv][nKT][8 chunks][D][8].  Element e of chunk c of tile t, row d, is key
// 64 t + 16 (c / 2) + kperm(8 (c % 2) + e) of row d (zero past T); kperm swaps bits 2
// and 3 of a key's index in its 16-key group, matching the key order of the
// probabilities held by an MFMA lane.
size_t tiles_t_bytes(int nKT, int Hkv, int D);
hipError_t launch_tiles_t(int T, int nKT, int Hkv, int D, const void* src, void* dst,
                          hipStream_t s);

// The bf16 forward reads V through `vx` (tiles_t layout, filled by the caller).
// With `rope` (not NULL), q is unrotated and turned in registers at the plan positions;
// k must come rotated.
hipError_t launch_fwd_bf16(const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* vx, void* o, float* lse,
                           const RopeFreq* rope, hipStream_t s);
hipError_t launch_fwd_fp32(const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, void* o, float* lse,
                           hipStream_t s);
// Backward phases.  `bf16` selects the MFMA kernels, otherwise float32.  The
// workspace holds LSE * log2(e) and Delta, float32 [2][Hq][Tp], Tp = T rounded up to
// a multiple of 128 (padding rows: +inf and 0).
size_t bwd_workspace_floats(int T, int Hq);
hipError_t launch_bwd_preprocess(bool bf16, const DevPlan& p, int Hq, int D, const void* o,
                                 const void* dout, const float* lse, float* ws, hipStream_t s);
// With `rope` (bf16 only), q and k come rotated at the plan positions and dk (dq) is
// turned back in registers before it is stored.
hipError_t launch_bwd_dkdv(bool bf16, const DevPlan& p, int Hq, int Hkv, int D, float scale,
                           const void* q, const void* k, const void* v, const void* dout,
                           const float* ws, void* dk, void* dv, const RopeFreq* rope,
                           hipStream_t s);
hipError_t launch_bwd_dq(bool bf16, const DevPlan& p, int Hq, int Hkv, int D, float scale,
                         const void* q, const void* k, const void* v, const void* dout,
                         float* ws, void* dq, const RopeFreq* rope, hipStream_t s);
// Decode: per-cursor segment lists 0..B-1, then (n_groups > 0) one shared list per group
// of cursors (grp_ptr / grp_cur).  partial: float32 [B][2 n_split][Hq][D + 4].  `bf16`
// selects the MFMA kernel, otherwise float32 pools and outputs.  D in {64, 128}.
hipError_t launch_decode(bool bf16, int B, int Hq, int Hkv, int D, int page_size, float scale,
                         const void* q, const void* k_pool, const void* v_pool, int n_pages,
                         const int32_t* seg_ptr, const int32_t* seg_page,
                         const int32_t* seg_lo, const int32_t* seg_hi, int n_groups,
                         const int32_t* grp_ptr, const int32_t* grp_cur, int n_split, void* o,
                         float* lse, float* partial, hipStream_t s);

// Address of this device's scratch array of OCTOPUS_DECODE_SCRATCH_BYTES bytes (the
// current device; looked up once per device and kept).  Used by the decode entry point
// that allocates nothing.
hipError_t decode_scratch(void** ptr);

// Rotary embedding in place or out of place: x is [rows][H][D] (bf16 if `bf16`, else
// float32); row r turns by pos[r] * base^(-2i/D) on pairs (i, i + D/2), by the opposite
// angle if `inverse`.  out may equal x.
hipError_t launch_rope(bool bf16, int rows, int H, int D, float base, bool inverse,
                       const int32_t* pos, const void* x, void* out, hipStream_t s);
// The same for two tensors sharing the rows' positions in one pass (x2/out2 with H2
// heads; x2 may be NULL).
hipError_t launch_rope2(bool bf16, int rows, int D, float base, bool inverse,
                        const int32_t* pos, int H, const void* x, void* out, int H2,
                        const void* x2, void* out2, hipStream_t s);

// Chunked gated delta-rule scan (matrix cores, 32-token chunks as listed by the plan):
// q, k, v, dout [T][H][128] bf16, alpha, beta float32 [T][H].  The prep kernel writes a
// record of gdn_prep_floats / (n_chunks H) floats per (chunk, head) into `prep` for the
// n_chunks chunks from chunk c0 on (with_t: also the transposed blocks that only the backward
// reads); the forward walks the branches level_br[l0 .. l0 + n_br)
// (one workgroup per (branch, head)) from their checkpoint slots `states`
// [n_slots][H][128][128] float32 (row = value index), writing o [T][H][128] bf16 (may be
// NULL) and, with chunk_states (may be NULL), the state at the start of every chunk
// [c][H][128][128].
size_t gdn_prep_floats(int64_t n_chunks, int H);
hipError_t launch_gdn_chunk_prep(const DevPlan& p, int c0, int64_t n_chunks, int H, bool with_t,
                                 const void* q, const void* k, const float* alpha,
                                 const float* beta, float* prep, hipStream_t s);
hipError_t launch_gdn_chunk_fwd(const DevPlan& p, int l0, int n_br, int H, const void* q,
                                const void* k, const void* v, const float* prep, void* o,
                                float* states, float* chunk_states, hipStream_t s);
// Backward: the state gradient of the branches level_br[l0 .. l0 + n_br) in reverse
// (levels deepest first), written at every chunk's end into dsc [c][H][128][128]
// (key-major); dkids [nb][H][128][128] float32: every child's initial-state gradient,
// written by the child and added by its parent.  Then, over the n_chunks chunks from c0 on,
// the gradients dq, dk, dv [T][H][128] bf16 and dalpha, dbeta [T][H] float32 of their
// tokens.
hipError_t launch_gdn_chunk_dstate(const DevPlan& p, int l0, int n_br, int H, const void* q,
                                   const void* k, const void* dout, const float* prep,
                                   float* dsc, float* dkids, hipStream_t s);
hipError_t launch_gdn_chunk_grad(const DevPlan& p, int c0, int64_t n_chunks, int H,
                                 const void* q, const void* k, const void* v, const float* alpha,
                                 const float* beta, const void* dout, const float* prep,
                                 const float* chunk_states, const float* dsc, void* dq, void* dk,
                                 void* dv, float* dalpha, float* dbeta, hipStream_t s);

// Extend: rows q_ptr[c] .. q_ptr[c+1]-1 of q are cursor c's new tokens (own offsets
// first_off[c] + j); segments as built by build_extend_segments.  max_new >= every m_c.
// `bf16` selects the MFMA kernel, otherwise float32.  D in {64, 128}.
hipError_t launch_extend(bool bf16, int B, int Hq, int Hkv, int D, float scale, const void* q,
                         const void* k_pool, const void* v_pool, int n_pages,
                         const int32_t* q_ptr, int max_new, const int32_t* first_off,
                         const int32_t* seg_ptr, const int32_t* seg_page,
                         const int32_t* seg_lo, const int32_t* seg_hi,
                         const int32_t* seg_thr, const int32_t* seg_causal, void* o,
                         float* lse, hipStream_t s);

}  // namespace octo
