/*
 * octopus_dag.h -- C ABI of the packed-DAG attention library for AMD Instinct MI355X
 * (gfx950).
 *
 * What it computes.  An episode of branching agents is a DAG of branches (Octopus
 * project page, section "Architecture & Co-Design": a cursor-addressed DAG
 * G = (V, E_tree, E_mount)).  A branch is created by `fork` and shares its parent's
 * prefix; `read_thread` mounts a span c_A[s_A:e_A) of another branch into the
 * reader's attention layers without copying it (primitives table, rows "fork" and
 * "read_thread").  The trainer packs every branch of a tree into one unpadded 1-D
 * token stream and runs one block-sparse attention pass over it, forward and
 * backward, with a shared prefix owned once and reader gradients routed into the
 * producer's tokens (card "03 · Training"; ia.com.br article, section "Crédito
 * contrafactual ...").  The serving side decodes cursors whose context is an
 * ancestor prefix, their own branch and mounted spans, read in place from a page
 * pool (primitives table; card "02 · Memory": mounts allocate no KV pages).
 *
 * Visibility.  For branch b and own offset r, with g(b,r) = start_b + r:
 *     A(b,r) = H(b) ∪ {g(b,r') : r' < r}
 *              ∪ {g(p_m,t) : s_m <= t < e_m, for mounts m with reader b, rpos_m <= r}
 *     H(root) = {} for every root,  H(b) = A(parent_b, fork_b)
 * and packed token i = g(b,r) attends to Ctx(i) = A(b,r) ∪ {i}, each key once.
 * Attention is ordinary softmax attention restricted to Ctx(i):
 *     S = scale * Q K^T,  LSE = log sum exp S,  P = exp(S - LSE),  O = P V
 * with query head h reading KV head h / (Hq / Hkv).
 *
 * Positions.  Keys keep the position they were written at; after a mount a reader's
 * next position is max(p_B, e_A + 1) (card "02 · Memory"; ia.com.br, section
 * "Memória associativa versus memória de trabalho"), e_A being the span's exclusive
 * end in positions.  The attention entry points take Q and K already rotated at
 * these positions; octopus_plan_positions returns them.
 *
 * Conventions.
 *   - Device tensors are row-major and contiguous.  "THD" means [T][H][D].
 *   - bf16 is IEEE bfloat16 storage with float32 accumulation; outputs are rounded to
 *     nearest even.  fp32 tensors are float32 throughout.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream) of the current
 *     device.  Device work is enqueued asynchronously on it; no entry point synchronises
 *     it.  (The gated delta-rule scan also runs part of its work on a second stream of
 *     the device, ordered into `stream`; see there.)
 *   - The caller owns every device buffer (tensors, plan buffer, workspaces).  The
 *     library never allocates or frees device memory.  A plan owns host memory only.
 *   - Return value: OCTOPUS_OK (0) or a negative error code.  On an argument error
 *     (EINVAL, ESTATE, EUNSUPPORTED, EWORKSPACE, ECYCLE) nothing has been enqueued and
 *     outputs are untouched; EHIP (a failed launch) may follow launches of the same call
 *     that were enqueued.  octopus_last_error() returns a thread-local message naming the
 *     offending row or argument.
 */
#ifndef OCTOPUS_DAG_H
#define OCTOPUS_DAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One branch (one `fork`): parent index, or -1 for a root (fork 0; row 0 is always a
 * root; every other row's parent has a lower index), fork = offset into the parent's
 * own tokens at which the child forked (0 <= fork <= parent len), start = where the
 * branch's own tokens sit in the packed stream, len >= 1 own tokens.  The branch
 * spans must tile [0, total_tokens) exactly, in any order.  Several roots make a
 * forest: independent episode trees packed into one stream and one plan, no token
 * seeing another tree (the trainer's step batches several trees; card "03 ·
 * Training"); each tree's positions start at 0. */
typedef struct {
    int32_t parent, fork, start, len;
} octopus_branch;

/* One mount (one `read_thread`): the reader, when its own length was rpos
 * (0 <= rpos <= reader len), mounted the producer's own tokens [s, e)
 * (0 <= s < e <= producer len, producer != reader, both in the same tree).  Reader
 * tokens at own offsets >= rpos see the span. */
typedef struct {
    int32_t reader, rpos, producer, s, e;
} octopus_mount;

typedef enum { OCTOPUS_BF16 = 0, OCTOPUS_FP32 = 1 } octopus_dtype;

enum {
    OCTOPUS_OK = 0,
    OCTOPUS_EINVAL = -1,       /* malformed table or argument */
    OCTOPUS_ECYCLE = -2,       /* a token's position depends on itself */
    OCTOPUS_EUNSUPPORTED = -3, /* dtype, head_dim, tile size or GQA ratio not built */
    OCTOPUS_ENOMEM = -4,       /* host allocation failed */
    OCTOPUS_EWORKSPACE = -5,   /* caller buffer too small */
    OCTOPUS_EHIP = -6,         /* a HIP runtime or launch error (message kept) */
    OCTOPUS_ESTATE = -7        /* plan not uploaded */
};

typedef struct octopus_plan octopus_plan;

typedef struct {
    int64_t nnz;          /* visible (query, key) pairs, each key once per query */
    int64_t n_pairs;      /* listed (query tile, KV tile) pairs */
    int64_t n_partial;    /* of which carry a bit mask */
    int32_t total_tokens; /* T */
    int32_t q_tile;       /* rows per query tile (128) */
    int32_t kv_tile;      /* keys per KV tile */
    int32_t n_q_tiles;
    int32_t n_kv_tiles;
    int32_t max_q_list;   /* longest KV-tile list of a query tile */
    int32_t max_kv_list;  /* longest query-tile list of a KV tile */
    int32_t reserved;
} octopus_plan_stats;

/* ---------------------------------------------------------------- planning (host) */

/* Plans one packed tree (Octopus project page, card "03 · Training": every branch of a
 * tree packed into one unpadded 1-D pass, compiled once per tree; the branch and mount
 * rows are the `fork` and `read_thread` rows of the primitives table).
 * Validate the tables, compute positions, and build the tile plan: for every
 * 128-row query tile the ordered list of KV tiles holding a key some row of the
 * tile sees, each FULL (every row sees every key) or PARTIAL (a per-row bit mask),
 * the transposed lists (for every KV tile, the query tiles that see it), and
 * longest-first launch orders.  kv_tile must be 64.  total_tokens must be in
 * [1, 2^24].  Synchronous and re-entrant; touches no device.  The per-tile lists and
 * the mask transposes of plans with many query tiles run on up to 16 host threads that the
 * call starts and joins; the plan does not depend on how many.
 * Errors: EINVAL (table rules above), ECYCLE, EUNSUPPORTED, ENOMEM.
 * On success *out owns the plan; free it with octopus_plan_destroy. */
int octopus_dag_plan(const octopus_branch* branches, int32_t n_branches,
                     const octopus_mount* mounts, int32_t n_mounts,
                     int32_t total_tokens, int32_t kv_tile, octopus_plan** out);

/* Positions of the T packed tokens (host int32[T]). */
int octopus_plan_positions(const octopus_plan* plan, int32_t* pos_out);

int octopus_plan_stats_get(const octopus_plan* plan, octopus_plan_stats* out);

/* Bytes of the device copy of the plan. */
size_t octopus_plan_device_bytes(const octopus_plan* plan);

/* Enqueue an asynchronous host-to-device copy of the plan into dev_buf
 * (caller-owned, >= octopus_plan_device_bytes, 256-byte aligned) on `stream`, and
 * remember dev_buf for the attention calls.  The first upload copies the plan into
 * page-locked host memory owned by the plan (so the copy does not wait for earlier
 * work on the stream); destroy the plan only after the stream has finished the copy
 * and every attention call that uses it.
 * Errors: EINVAL (NULL or misaligned buffer), EWORKSPACE (too small), EHIP. */
int octopus_plan_upload(octopus_plan* plan, void* dev_buf, size_t bytes, void* stream);

/* Dense visibility bits of rows [row_lo, row_hi), expanded from the tile lists and
 * masks alone (not from the tables): bits_out is host uint8[(row_hi-row_lo)]
 * [ceil(T/8)], bit (j % 8) of byte j / 8 of a row set iff the row sees key j. */
int octopus_plan_export_mask(const octopus_plan* plan, int32_t row_lo, int32_t row_hi,
                             uint8_t* bits_out);

/* The forward tile lists as the kernels see them: qt_ptr_out int32[n_q_tiles+1],
 * kv_tile_out and mask_out int32[n_pairs] (mask -1 = FULL, else the PARTIAL mask
 * index), and, if rows_out is not NULL, the PARTIAL masks as uint64[n_partial][128]
 * (bit x of row r: row r of the query tile sees key x of the KV tile).  For
 * inspection and tests. */
int octopus_plan_export_tiles(const octopus_plan* plan, int32_t* qt_ptr_out,
                              int32_t* kv_tile_out, int32_t* mask_out, uint64_t* rows_out);

void octopus_plan_destroy(octopus_plan* plan);

/* ---------------------------------------------------------------- attention (device) */

/* Workspace bytes the forward needs: for bf16, a copy of V re-laid per 64-key tile
 * (bf16 [Hkv][n_kv_tiles][8][D][8], keys transposed so that every V^T operand of the
 * MFMAs is one contiguous 16-byte read), written by the forward itself; 0 for fp32
 * (callers may then pass NULL/0).  Caller-owned device memory, 16-byte aligned; its
 * contents need not survive between calls. */
size_t octopus_fwd_workspace_bytes(const octopus_plan* plan, octopus_dtype dtype,
                                   int32_t Hq, int32_t Hkv, int32_t D);

/* Forward of packed-DAG attention over the uploaded plan: the block-sparse pass
 * structured as a prefix tree (ia.com.br article, section "Crédito contrafactual ...";
 * project page, card "03 · Training"), row i attending to Ctx(i) above.
 *   q   THD [T][Hq][D], k, v THD [T][Hkv][D]  (dtype; rotated at the plan's positions)
 *   o   THD [T][Hq][D] (dtype), lse float32 [Hq][T] (natural log) -- both written
 * Supported: bf16 with D in {64, 128}; fp32 with D in {64, 128}; Hq % Hkv == 0,
 * Hq / Hkv <= 16.  scale <= 0 selects 1/sqrt(D).
 * Errors: ESTATE (plan not uploaded), EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP. */
int octopus_dag_attn_fwd(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                         int32_t Hkv, int32_t D, float scale, const void* q,
                         const void* k, const void* v, void* o, float* lse, void* ws,
                         size_t ws_bytes, void* stream);

/* Workspace bytes the backward needs: float32 [2][Hq][Tp] (LSE * log2(e) and Delta),
 * Tp = T rounded up to a multiple of 128. */
size_t octopus_bwd_workspace_bytes(const octopus_plan* plan, octopus_dtype dtype,
                                   int32_t Hq, int32_t Hkv, int32_t D);

/* Backward of L = sum <dO, O> given the forward's o and lse (project page, card
 * "03 · Training": a shared prefix owned once, reader gradients routed into the
 * producer's KV; ia.com.br article, section "Crédito contrafactual ...": mount edges
 * differentiable end to end):
 *   dq THD [T][Hq][D]; dk, dv THD [T][Hkv][D]  (dtype) -- written, not accumulated.
 * Every dK/dV row is produced by exactly one work unit (the owner of its KV tile),
 * summing the queries of every branch that sees it (descendants through the shared
 * prefix, readers through mounts), so no atomics are used and results do not
 * depend on scheduling.  Same support and errors as the forward. */
int octopus_dag_attn_bwd(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                         int32_t Hkv, int32_t D, float scale, const void* q,
                         const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, void* ws,
                         size_t ws_bytes, void* stream);

/* The same backward as three launches, for callers that time or overlap them.  The
 * workspace carries LSE and Delta from the preprocess to the other two, which are
 * independent of each other (they may run on two streams once the preprocess has
 * completed).
 *   preprocess: Delta = rowsum(dO * O), and LSE * log2(e), into ws;
 *   dkdv:       dk, dv from q, k, v, dout and ws (atomics-free owner pass);
 *   dq:         dq from q, k, v, dout and ws.
 * Same support and errors as octopus_dag_attn_bwd. */
int octopus_dag_attn_bwd_preprocess(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                                    int32_t Hkv, int32_t D, const void* o, const float* lse,
                                    const void* dout, void* ws, size_t ws_bytes, void* stream);
int octopus_dag_attn_bwd_dkdv(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                              int32_t Hkv, int32_t D, float scale, const void* q, const void* k,
                              const void* v, const void* dout, void* dk, void* dv,
                              const void* ws, size_t ws_bytes, void* stream);
int octopus_dag_attn_bwd_dq(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                            int32_t Hkv, int32_t D, float scale, const void* q, const void* k,
                            const void* v, const void* dout, void* dq, const void* ws,
                            size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- rotary positions */

/* Positions only (host): int32[total_tokens] as octopus_plan_positions returns them, with
 * no tile plan built (for serving, where queries are rotated at their cursor's
 * positions).  Errors: EINVAL, ECYCLE, ENOMEM. */
int octopus_dag_positions(const octopus_branch* branches, int32_t n_branches,
                          const octopus_mount* mounts, int32_t n_mounts, int32_t total_tokens,
                          int32_t* pos_out);

/* Rotary embedding on the device (rotate-half): row r of x [rows][H][D] has its pairs
 * (x_i, x_{i+D/2}) turned by pos[r] * rope_base^(-2i/D) (by the opposite angle if
 * inverse), written to out (may equal x).  pos: device int32[rows].  Mounted keys keep
 * the position they were written at, so paged keys are stored rotated once, at their
 * producer's positions (card "02 · Memory": rotation-free mounts).  Angles are reduced in
 * float64 (pos * theta reaches 2^24 radians).
 * Supported: bf16 and fp32, D in {64, 128}.  Errors: EINVAL, EUNSUPPORTED, EHIP. */
int octopus_rope(octopus_dtype dtype, int32_t rows, int32_t H, int32_t D, float rope_base,
                 int32_t inverse, const int32_t* pos, const void* x, void* out, void* stream);

/* Extra workspace bytes of the RoPE variants below: rotated copies of Q and K (the bf16
 * forward uses only the part for K). */
size_t octopus_rope_workspace_bytes(const octopus_plan* plan, octopus_dtype dtype,
                                    int32_t Hq, int32_t Hkv, int32_t D);

/* octopus_dag_attn_fwd with Q and K given unrotated, turned at the plan's positions
 * (card "02 · Memory": keys keep the rotation of the position they were written at; a
 * reader's positions jump after a mount).  bf16: K is turned by one pass into the front
 * of the workspace and every query row is turned in the forward kernel's registers; fp32:
 * Q and K are turned into copies first.  ws: 256-byte aligned, octopus_rope_workspace_bytes
 * + octopus_fwd_workspace_bytes bytes suffice (the rotated copies first).  Errors as
 * octopus_dag_attn_fwd. */
int octopus_dag_attn_fwd_rope(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                              int32_t Hkv, int32_t D, float scale, float rope_base,
                              const void* q, const void* k, const void* v, void* o, float* lse,
                              void* ws, size_t ws_bytes, void* stream);

/* octopus_dag_attn_bwd with Q and K given unrotated: Q and K are turned by one pass into
 * the front of the workspace, gradients are taken with respect to the rotated copies and
 * dQ, dK are turned back (the rotation is orthogonal), so they are the gradients with
 * respect to the unrotated inputs.  bf16: the dQ and dK/dV kernels turn their results back
 * in registers before storing them; fp32: a pass turns them back in place.  ws: 256-byte
 * aligned, octopus_rope_workspace_bytes + octopus_bwd_workspace_bytes bytes, the rotated
 * copies first.  Errors as octopus_dag_attn_bwd. */
int octopus_dag_attn_bwd_rope(const octopus_plan* plan, octopus_dtype dtype, int32_t Hq,
                              int32_t Hkv, int32_t D, float scale, float rope_base,
                              const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- recurrent scan */

/* Workspace bytes of octopus_gated_delta_scan: float32 fork checkpoints
 * [n_slots][H][Dv][Dk], one slot per distinct (parent, fork offset) of the plan, then one
 * 21,504-byte record per (chunk, head) (the chunk's gated score matrices, the inverse of
 * its triangular system and its gates): 2.8 GB at 262,144 tokens and H = 16. */
size_t octopus_gdn_workspace_bytes(const octopus_plan* plan, int32_t H, int32_t Dk,
                                   int32_t Dv);

/* Branch-aware gated delta-rule scan (the recurrent layers of a hybrid backbone, Gated
 * DeltaNet; Octopus project page, primitives table: `fork` clones the parent's recurrent
 * checkpoint, mounted spans bypass the recurrent layers).  Per head, state S (Dv x Dk):
 *     S_t = alpha_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * over each branch's own tokens in order, a root from S = 0, a child from its parent's
 * state just before the parent's own token `fork`; mounts are ignored.
 * q, k [T][H][Dk], v, o [T][H][Dv] (dtype); alpha, beta float32 [T][H] (device).
 * alpha in (0, 1] (values below 2^-100 act as 2^-100), beta in [0, 1].
 * The plan must be uploaded.  Every branch is taken 32 tokens at a time on the matrix
 * cores (chunks also end at every fork offset): the chunks' records are prepared in
 * parallel, then the levels of the tree run one launch each, in order, one workgroup per
 * (branch, head).  The deeper levels' records are prepared on a second stream of the
 * current device while the first level runs (the scan entry points create that stream and
 * two events per device on first use and keep them until the process ends); the second
 * stream starts after the work already on `stream` and `stream` waits for it before the
 * next level, so the call is ordered on `stream` like a plain launch sequence.  Calls from
 * several host threads are serialised around the second stream.
 * Supported: bf16, Dk = Dv = 128.  Errors: EINVAL, ESTATE, EUNSUPPORTED, EWORKSPACE,
 * EHIP. */
int octopus_gated_delta_scan(const octopus_plan* plan, octopus_dtype dtype, int32_t H,
                             int32_t Dk, int32_t Dv, const void* q, const void* k,
                             const void* v, const float* alpha, const float* beta, void* o,
                             void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of octopus_gated_delta_scan_bwd: float32 checkpoint slots, one
 * initial-state gradient per branch, the state at the start and the state gradient at the
 * end of every chunk of the plan (32-token chunks, split at fork offsets), each
 * H x Dv x Dk, and the per-chunk records of the forward (20.0 GB at 262,144 tokens and
 * H = 16). */
size_t octopus_gdn_bwd_workspace_bytes(const octopus_plan* plan, int32_t H, int32_t Dk,
                                       int32_t Dv);

/* Backward of octopus_gated_delta_scan: gradients of L = sum_t <dout_t, o_t> with respect
 * to q, k, v (written, [T][H][D] bf16) and to alpha, beta (written, [T][H] float32).  The
 * gradient of a child's initial state (its parent's state at the fork) flows into the
 * parent's earlier tokens; mounted spans receive nothing (the recurrent layers skip them;
 * project page, primitives table).  Recomputes the forward (the states at chunk starts go
 * to the workspace) and, beside it on the second stream (see octopus_gated_delta_scan),
 * walks every branch's chunks in reverse carrying only the state gradient (deepest
 * branches first); then computes every chunk's gradients in parallel.
 * Deterministic: the children forking at one offset hand their initial-state gradients
 * to the parent in ascending branch order (no atomics), so repeated calls give the same
 * bits.  Same support and errors as octopus_gated_delta_scan. */
int octopus_gated_delta_scan_bwd(const octopus_plan* plan, octopus_dtype dtype, int32_t H,
                                 int32_t Dk, int32_t Dv, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const void* dout, void* dq, void* dk, void* dv, float* dalpha,
                                 float* dbeta, void* ws, size_t ws_bytes, void* stream);

/* Training pair: octopus_gated_delta_scan_save is octopus_gated_delta_scan (o written)
 * that also leaves in ws (octopus_gdn_bwd_workspace_bytes bytes) the per-chunk records and
 * the state at every chunk start; octopus_gated_delta_scan_bwd_saved is
 * octopus_gated_delta_scan_bwd without its recomputation of the forward, reading them
 * from that ws.  The caller passes the same plan and the same q, k, v, alpha, beta to both
 * and leaves ws untouched in between (results are undefined otherwise: nothing checks
 * it).  The backward leaves the saved part in place, so it may run again on the same ws
 * (with another dout); it runs the deeper levels' gradients on the second stream while the
 * first level's state gradient runs.  Same support and errors as
 * octopus_gated_delta_scan_bwd. */
int octopus_gated_delta_scan_save(const octopus_plan* plan, octopus_dtype dtype, int32_t H,
                                  int32_t Dk, int32_t Dv, const void* q, const void* k,
                                  const void* v, const float* alpha, const float* beta, void* o,
                                  void* ws, size_t ws_bytes, void* stream);
int octopus_gated_delta_scan_bwd_saved(const octopus_plan* plan, octopus_dtype dtype,
                                       int32_t H, int32_t Dk, int32_t Dv, const void* q,
                                       const void* k, const void* v, const float* alpha,
                                       const float* beta, const void* dout, void* dq, void* dk,
                                       void* dv, float* dalpha, float* dbeta, void* ws,
                                       size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- paged decode */

/* Host helper: turn a DAG of branches held in a page pool into per-cursor segment
 * lists.  page_ptr (int32[n_branches+1]) / pages (int32[page_ptr[n_branches]]) is
 * the page table: branch b's own token r lives in page pages[page_ptr[b] + r /
 * page_size], slot r % page_size.  cursors (int32[n_cursors]) are branch ids whose
 * last own token is the current query.  Segments are (page, slot_lo, slot_hi) runs;
 * mounted keys are read from the producer's own pages; no page is created.
 *
 * share = 0: list c (c < n_cursors) covers exactly Ctx of cursor c's token (ancestor
 * prefix, own branch, mounted spans, each key once), in packed-key order; n_groups is
 * not written and the group arrays may be NULL.
 * share != 0: the cursors are grouped by the (parent, fork) of their branches; all
 * cursors of a group inherit the same context H (the shared radix prefix; primitives
 * table, `fork`).  List c then covers Ctx minus H, and list n_cursors + g the H of group
 * g; grp_ptr_out (int32[n_groups+1]) / grp_cur_out (int32[n_cursors]) list the cursors
 * of every group, each cursor in exactly one group (a group with an empty H has an
 * empty list).  The decode reads a shared list once per block of cursors instead of
 * once per cursor.
 *
 * Two calls: with seg_capacity < needed (e.g. 0) only *n_seg_out (and *n_groups_out)
 * are set and the call returns EWORKSPACE; then with room for *n_seg_out segments it
 * fills seg_ptr_out (int32[n_cursors + n_groups + 1]; size it 2 n_cursors + 1 when
 * sharing), seg_page/lo/hi_out (int32[n_seg]) and the group arrays.
 * Errors: EINVAL (tables, page ids outside [0, n_pages), short page table, NULL
 * outputs), ECYCLE, EWORKSPACE. */
int octopus_decode_segments(const octopus_branch* branches, int32_t n_branches,
                            const octopus_mount* mounts, int32_t n_mounts,
                            const int32_t* page_ptr, const int32_t* pages,
                            int32_t page_size, int32_t n_pages, const int32_t* cursors,
                            int32_t n_cursors, int32_t share, int32_t* seg_ptr_out,
                            int32_t* seg_page_out, int32_t* seg_lo_out,
                            int32_t* seg_hi_out, int32_t seg_capacity,
                            int32_t* n_seg_out, int32_t* grp_ptr_out, int32_t* grp_cur_out,
                            int32_t* n_groups_out);

/* Workspace bytes for octopus_paged_mount_decode: float32 partial states
 * [B][2 n_split][Hq][D + 4] (own and shared lists). */
size_t octopus_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t n_split);

/* One-token attention of B cursors over their segments, read in place from the
 * pools (project page, primitives table, rows "fork" and "read_thread": shared radix
 * pages and mounted spans read zero-copy; card "01 · Runtime": paged serving of the
 * branch cursors).  q [B][Hq][D]; k_pool, v_pool [n_pages][Hkv][page_size][D] (dtype);
 * seg_* and, with n_groups > 0, grp_ptr / grp_cur as produced by
 * octopus_decode_segments (n_groups = 0: share = 0 lists, group arrays ignored), on
 * the device.  Every list is split into n_split contiguous chunks (1 <= n_split <=
 * 256); the partial softmax states of a cursor's own chunks and of its group's shared
 * chunks are merged by LSE.  Writes o [B][Hq][D] (dtype) and, if lse is not NULL,
 * float32 [B][Hq].  Segments naming a page outside [0, n_pages) are skipped; group
 * entries naming no cursor in [0, B) are ignored.  Supported: bf16 (matrix cores) and
 * fp32 (exact float32 arithmetic), D in {64, 128}, page_size = 64, Hq / Hkv <= 8.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP. */
int octopus_paged_mount_decode(octopus_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t page_size, float scale, const void* q,
                               const void* k_pool, const void* v_pool, int32_t n_pages,
                               const int32_t* seg_ptr, const int32_t* seg_page,
                               const int32_t* seg_lo, const int32_t* seg_hi,
                               int32_t n_groups, const int32_t* grp_ptr,
                               const int32_t* grp_cur, int32_t n_split, void* o, float* lse,
                               void* ws, size_t ws_bytes, void* stream);

/* Bytes of device scratch octopus_paged_mount_decode_noalloc holds per GPU (48 MiB). */
#define OCTOPUS_DECODE_SCRATCH_BYTES (48u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): octopus_paged_mount_decode with the
 * partial softmax states kept in a device array of OCTOPUS_DECODE_SCRATCH_BYTES bytes
 * that the library holds on every GPU it runs on until the process ends, instead of a
 * caller workspace.  The array of the current device is used (the stream must belong to
 * it); its address is looked up on the first call on each device.  The call allocates
 * and frees nothing.  Calls on one GPU share its array: calls whose work overlaps on
 * that GPU (several streams, or several host threads) race and give undefined results.
 * The array keeps the last call's contents; nothing in it needs clearing, since every
 * partial state a call reads was written by the same call.  Arguments, support and
 * results as octopus_paged_mount_decode.
 * Errors: as octopus_paged_mount_decode, EWORKSPACE when the partial states
 * (octopus_decode_workspace_bytes) exceed OCTOPUS_DECODE_SCRATCH_BYTES (nothing is
 * enqueued), EHIP if the array's address cannot be looked up. */
int octopus_paged_mount_decode_noalloc(octopus_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t D, int32_t page_size, float scale, const void* q,
                                       const void* k_pool, const void* v_pool, int32_t n_pages,
                                       const int32_t* seg_ptr, const int32_t* seg_page,
                                       const int32_t* seg_lo, const int32_t* seg_hi,
                                       int32_t n_groups, const int32_t* grp_ptr,
                                       const int32_t* grp_cur, int32_t n_split, void* o,
                                       float* lse, void* stream);

/* ---------------------------------------------------------------- paged extend */

/* Host helper for extend (prefill of several new tokens per cursor: a continuation
 * sends only its new tokens, ia.com.br article, section on O(|Δm|) deltas).  Cursor c's
 * new tokens are the last n_new[c] own tokens of branch cursors[c] (1 <= n_new[c] <=
 * branch length), already written to its pages.  The segments of cursor c cover the
 * context of its last token, each (page, slot_lo, slot_hi) with a threshold thr: a new
 * token at own offset r sees slot x of the segment iff r >= thr (inherited keys: 0; a
 * mounted span: the mount's rpos) or, where causal is 1 (the cursor's own pages), iff
 * r >= thr + x - slot_lo.  A key reachable in several ways gets the smallest threshold,
 * and each key appears once.  Segments are sorted by thr within a cursor.
 * first_off_out (int32[n_cursors]) receives each cursor's first new token's own offset.
 * Two calls as for octopus_decode_segments: seg_ptr_out int32[n_cursors+1],
 * seg_page/lo/hi/thr/causal_out int32[n_seg].
 * Errors: EINVAL (tables, page table, n_new out of range), ECYCLE, EWORKSPACE. */
int octopus_extend_segments(const octopus_branch* branches, int32_t n_branches,
                            const octopus_mount* mounts, int32_t n_mounts,
                            const int32_t* page_ptr, const int32_t* pages, int32_t page_size,
                            int32_t n_pages, const int32_t* cursors, int32_t n_cursors,
                            const int32_t* n_new, int32_t* seg_ptr_out, int32_t* seg_page_out,
                            int32_t* seg_lo_out, int32_t* seg_hi_out, int32_t* seg_thr_out,
                            int32_t* seg_causal_out, int32_t seg_capacity, int32_t* n_seg_out,
                            int32_t* first_off_out);

/* Attention of every cursor's new tokens over their context, read in place from the
 * pools: q [n_rows][Hq][D] (dtype) with q_ptr (int32[B+1], device) delimiting cursor c's
 * rows q_ptr[c] .. q_ptr[c+1]-1 (its new tokens in order, at most max_new of them);
 * first_off and seg_* as produced by octopus_extend_segments, on the device; k_pool,
 * v_pool [n_pages][Hkv][page_size][D].  Writes o [n_rows][Hq][D] (dtype) and lse
 * float32 [n_rows][Hq].  Needs no workspace.  Index arrays that do not come from
 * octopus_extend_segments give undefined values (never a read outside the pools: a
 * segment naming a page outside [0, n_pages) reads page 0 and is masked).
 * Supported: bf16 (matrix cores) and fp32 (exact float32 arithmetic), D in {64, 128},
 * page_size = 64, Hq / Hkv <= 16.
 * Errors: EINVAL, EUNSUPPORTED, EHIP. */
int octopus_paged_mount_extend(octopus_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t page_size, float scale, const void* q,
                               const void* k_pool, const void* v_pool, int32_t n_pages,
                               const int32_t* q_ptr, int32_t max_new, const int32_t* first_off,
                               const int32_t* seg_ptr, const int32_t* seg_page,
                               const int32_t* seg_lo, const int32_t* seg_hi,
                               const int32_t* seg_thr, const int32_t* seg_causal, void* o,
                               float* lse, void* stream);

/* ---------------------------------------------------------------- misc */

/* Message of the last error on this thread ("" if none). */
const char* octopus_last_error(void);

/* Library version string. */
const char* octopus_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OCTOPUS_DAG_H */
