// Host-side planner for packed-DAG attention (internal interface).
//
// Builds, from the branch and mount tables, everything the device kernels need:
// per 128-row query tile the KV tiles some row sees (FULL or PARTIAL with a per-row
// bit mask), the transposed lists for the backward's KV-tile owners, and
// longest-first launch orders.  Visibility follows the fork / read_thread rules of
// the Octopus project page (primitives table) and positions follow the monotonic
// jump rule of its card "02 · Memory".
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "octopus_dag.h"

namespace octo {

constexpr int kQTile = 128;
constexpr int kMaxTokens = 1 << 24;

struct Interval {
    int64_t lo, hi;  // [lo, hi) in packed indices
};

// A listed (query tile, KV tile) pair as the kernels read it: 8 bytes.
struct TilePair {
    int32_t tile;  // KV tile (forward lists) or query tile (transposed lists)
    int32_t mask;  // -1 for FULL, else the index of the PARTIAL bit mask
};

// Validated tables plus the derived per-branch data the planner and the decode
// segment builder share.
struct DagInfo {
    int32_t T = 0;
    std::vector<octopus_branch> br;
    std::vector<octopus_mount> mt;
    std::vector<std::vector<int32_t>> mounts_of;  // per reader: mount ids sorted by rpos
    std::vector<std::vector<Interval>> inherited;  // H(b), merged
    std::vector<int32_t> order_by_start;           // branches sorted by start
    std::vector<int32_t> tree;                     // root row of every branch's tree
    std::vector<int64_t> pos;                      // position of every packed token

    // Ctx(g(b, r)) as sorted, disjoint, non-adjacent intervals (the query included).
    void row_context(int32_t b, int32_t r, std::vector<Interval>& out,
                     std::vector<Interval>& scratch) const;
    // Owning branch of a packed index.
    int32_t owner(int64_t j) const;
};

// Returns OCTOPUS_OK or an error code with `err` set.  Positions are always computed
// (their dependency cycles are errors); with_positions = false leaves `pos` empty for
// callers that need only visibility (the decode and extend segment builders).
int load_dag(const octopus_branch* br, int32_t nb, const octopus_mount* mt, int32_t nm,
             int32_t T, DagInfo& out, std::string& err, bool with_positions = true);

// One entry of a 128-key block's list: a query tile and, for each of the block's two
// 64-key tiles, -1 (FULL), -2 (the tile is not seen by this query tile) or the
// index of its PARTIAL mask.
struct BlockEntry {
    int32_t qt, mask0, mask1, pad;
};

struct DevLayout {
    size_t fwd_order = 0, qt_ptr = 0, q_pairs = 0, bwd_order = 0, kt_ptr = 0,
           k_pairs = 0, mask_rows = 0, mask_cols = 0, blk_order = 0, blk_ptr = 0,
           blk_entries = 0, pos = 0, sc_start = 0, sc_len = 0, sc_init = 0, sc_ck_ptr = 0,
           sc_ck_off = 0, sc_ck_slot = 0, sc_level_br = 0, sc_chunk_base = 0, sc_chunk_tok = 0,
           sc_chunk_nt = 0, sc_ck_kid_ptr = 0, sc_ck_kid = 0, total = 0;
};

struct Plan {
    DagInfo dag;
    int32_t T = 0, Bq = kQTile, Bk = 64, nQT = 0, nKT = 0;
    int32_t row_words = 1;  // uint64 words per row of a PARTIAL mask   (Bk / 64)
    int32_t col_words = 2;  // uint64 words per key of a PARTIAL mask   (Bq / 64)
    std::vector<int32_t> fwd_order, qt_ptr;
    std::vector<TilePair> q_pairs;
    std::vector<int32_t> bwd_order, kt_ptr;
    std::vector<TilePair> k_pairs;
    int32_t nKB = 0;                      // 128-key blocks (pairs of KV tiles)
    std::vector<int32_t> blk_order, blk_ptr;
    std::vector<BlockEntry> blk_entries;  // merged transposed lists of each block
    std::vector<uint64_t> mask_rows;  // [n_partial][Bq][row_words]
    std::vector<uint64_t> mask_cols;  // [n_partial][Bk][col_words]
    int64_t nnz = 0, n_partial = 0;
    int32_t max_q_list = 0, max_kv_list = 0;
    // Recurrent scan: branches grouped by depth (level_ptr over level_br); a branch
    // starts from checkpoint slot sc_init (-1: zero state) and saves its state before own
    // token sc_ck_off[j] into slot sc_ck_slot[j] (its children's fork points).
    std::vector<int32_t> sc_init, sc_ck_ptr, sc_ck_off, sc_ck_slot, level_ptr, level_br;
    // The children forking at checkpoint j: sc_ck_kid[sc_ck_kid_ptr[j] .. [j+1]), ascending.
    std::vector<int32_t> sc_ck_kid_ptr, sc_ck_kid;
    int32_t n_slots = 0;
    // Chunked scan: branch b's chunks (own tokens split every kScanChunk tokens and at
    // every checkpoint offset) are numbered sc_chunk_base[2b] .. sc_chunk_base[2b+1]-1;
    // chunk c covers packed tokens sc_chunk_tok[c] .. sc_chunk_tok[c] + sc_chunk_nt[c] - 1.
    // Chunks are numbered level by level (in level_br order), so the chunks of level l are
    // level_chunk[l] .. level_chunk[l+1]-1 (host only: launch ranges).
    std::vector<int32_t> sc_chunk_base, sc_chunk_tok, sc_chunk_nt, level_chunk;
    int64_t n_chunks = 0;
    DevLayout layout;
    void* dev = nullptr;     // caller-owned device copy after upload
    void* pinned = nullptr;  // page-locked image of the device copy (write_device_image)
};

// Tokens per chunk of the chunked recurrent scan.
constexpr int32_t kScanChunk = 32;

int build_plan(const octopus_branch* br, int32_t nb, const octopus_mount* mt, int32_t nm,
               int32_t T, int32_t kv_tile, Plan& out, std::string& err);
// The device image of a plan (layout.total bytes, every array at its layout offset, the
// padding between them zero) written into dst, e.g. page-locked staging for an upload.
void write_device_image(const Plan& p, unsigned char* dst);

// Dense bits of rows [lo, hi) from the tile lists only (see octopus_plan_export_mask).
void export_mask(const Plan& p, int32_t lo, int32_t hi, uint8_t* bits);

// Decode segments of every cursor (see octopus_decode_segments).  With `share`, each
// cursor's list holds only what it does not inherit, and the inherited context of every
// group of cursors forked from the same (parent, fork) follows as one list per group;
// grp_ptr / grp_cur list the cursors of each group.
int build_segments(const DagInfo& dag, const int32_t* page_ptr, const int32_t* pages,
                   int32_t page_size, int32_t n_pages, const int32_t* cursors,
                   int32_t n_cursors, bool share, std::vector<int32_t>& seg_ptr,
                   std::vector<int32_t>& seg_page, std::vector<int32_t>& seg_lo,
                   std::vector<int32_t>& seg_hi, std::vector<int32_t>& grp_ptr,
                   std::vector<int32_t>& grp_cur, std::string& err);

// Extend segments (see octopus_extend_segments): for cursor c, the segments of the
// context of its last token, each with the smallest own offset of a new token that sees
// it (thr; for own-token segments, `causal`: slot x needs offset thr + x - lo), sorted by
// that threshold; first_off[c] is the own offset of c's first new token.
int build_extend_segments(const DagInfo& dag, const int32_t* page_ptr, const int32_t* pages,
                          int32_t page_size, int32_t n_pages, const int32_t* cursors,
                          int32_t n_cursors, const int32_t* n_new, std::vector<int32_t>& seg_ptr,
                          std::vector<int32_t>& seg_page, std::vector<int32_t>& seg_lo,
                          std::vector<int32_t>& seg_hi, std::vector<int32_t>& seg_thr,
                          std::vector<int32_t>& seg_causal, std::vector<int32_t>& first_off,
                          std::string& err);

}  // namespace octo
