// Host-side planner for packed-DAG attention.  See plan.h.
#include "plan.h"

#include <algorithm>
#include <atomic>
#include <exception>
#include <thread>
#include <map>
#include <climits>
#include <cstring>
#include <numeric>

namespace octo {

namespace {

std::string row_msg(const char* what, long long idx, const char* detail) {
    return std::string(what) + " " + std::to_string(idx) + ": " + detail;
}

// Set bits [a, e) of a little-endian bit string held in 64-bit words.
void set_bits(uint64_t* w, int64_t a, int64_t e) {
    while (a < e) {
        const int64_t wi = a >> 6, b0 = a & 63;
        const int64_t b1 = std::min<int64_t>(64, b0 + (e - a));
        const uint64_t hi = b1 == 64 ? ~0ull : ((1ull << b1) - 1);
        w[wi] |= hi & ~((1ull << b0) - 1);
        a += b1 - b0;
    }
}

// In place: word c gets bit r = bit c of word r (a 64 x 64 bit matrix, bit c of word r
// being entry (r, c)), by swapping ever smaller off-diagonal blocks.
void transpose64(uint64_t a[64]) {
    uint64_t m = 0x00000000FFFFFFFFull;
    for (int j = 32; j != 0; j >>= 1, m ^= (m << j)) {
        for (int k = 0; k < 64; k = ((k | j) + 1) & ~j) {
            const uint64_t t = ((a[k] >> j) ^ a[k | j]) & m;
            a[k] ^= t << j;
            a[k | j] ^= t;
        }
    }
}

// Sort and merge intervals in place (adjacent ones are joined).
void merge(std::vector<Interval>& v) {
    if (v.empty()) return;
    std::sort(v.begin(), v.end(),
              [](const Interval& a, const Interval& b) { return a.lo < b.lo; });
    size_t w = 0;
    for (size_t i = 1; i < v.size(); ++i) {
        if (v[i].lo <= v[w].hi) {
            v[w].hi = std::max(v[w].hi, v[i].hi);
        } else {
            v[++w] = v[i];
        }
    }
    v.resize(w + 1);
}

// fn(i) for every i in [0, n), spread over up to `threads` host threads that take the
// items in turn (the caller's results must not depend on which thread runs an item).  An
// exception thrown by fn is rethrown here after every thread has stopped.
template <class F>
void parallel_for(int32_t n, int32_t threads, const F& fn) {
    threads = std::max<int32_t>(1, std::min(threads, n));
    if (threads == 1) {
        for (int32_t i = 0; i < n; ++i) fn(i);
        return;
    }
    std::atomic<int32_t> next{0};
    std::vector<std::exception_ptr> fault(threads);
    std::vector<std::thread> pool;
    pool.reserve(threads);
    for (int32_t w = 0; w < threads; ++w)
        pool.emplace_back([&, w]() {
            try {
                for (int32_t i = next++; i < n; i = next++) fn(i);
            } catch (...) {
                fault[w] = std::current_exception();
                next = n;
            }
        });
    for (std::thread& t : pool) t.join();
    for (const std::exception_ptr& e : fault)
        if (e) std::rethrow_exception(e);
}

// Host threads for the planner's parallel phases.
int32_t plan_threads() {
    const int32_t hw = (int32_t)std::thread::hardware_concurrency();
    return std::max<int32_t>(1, std::min<int32_t>(hw, 16));
}

int validate(const octopus_branch* br, int32_t nb, const octopus_mount* mt, int32_t nm,
             int32_t T, std::string& err) {
    if (nb < 1 || br == nullptr) { err = "no branches"; return OCTOPUS_EINVAL; }
    if (nm < 0 || (nm > 0 && mt == nullptr)) { err = "bad mount table"; return OCTOPUS_EINVAL; }
    if (T < 1 || T > kMaxTokens) {
        err = "total_tokens must be in [1, 2^24]";
        return OCTOPUS_EINVAL;
    }
    // tree[b]: the root row of b's tree.  Every row with parent -1 starts a tree of
    // its own (a forest packs several episodes into one stream); row 0 is one.
    std::vector<int32_t> tree(nb);
    for (int32_t b = 0; b < nb; ++b) {
        const octopus_branch& x = br[b];
        if (x.len < 1) { err = row_msg("branch", b, "len < 1"); return OCTOPUS_EINVAL; }
        if (x.parent == -1) {
            if (x.fork != 0) {
                err = row_msg("branch", b, "a root must have fork 0");
                return OCTOPUS_EINVAL;
            }
            tree[b] = b;
        } else {
            if (x.parent < 0 || x.parent >= b) {
                err = row_msg("branch", b, "parent must be -1 or a lower index");
                return OCTOPUS_EINVAL;
            }
            if (x.fork < 0 || x.fork > br[x.parent].len) {
                err = row_msg("branch", b, "fork outside the parent");
                return OCTOPUS_EINVAL;
            }
            tree[b] = tree[x.parent];
        }
        if (x.start < 0 || (int64_t)x.start + x.len > T) {
            err = row_msg("branch", b, "span outside [0, T)");
            return OCTOPUS_EINVAL;
        }
    }
    // The spans must tile [0, T): sorted by start they are back to back.
    std::vector<int32_t> ord(nb);
    std::iota(ord.begin(), ord.end(), 0);
    std::sort(ord.begin(), ord.end(), [&](int a, int b) { return br[a].start < br[b].start; });
    int64_t at = 0;
    for (int32_t b : ord) {
        if (br[b].start != at) {
            err = row_msg("branch", b, "branch spans do not tile [0, T) exactly");
            return OCTOPUS_EINVAL;
        }
        at += br[b].len;
    }
    if (at != T) { err = "branch spans do not tile [0, T) exactly"; return OCTOPUS_EINVAL; }
    for (int32_t i = 0; i < nm; ++i) {
        const octopus_mount& m = mt[i];
        if (m.reader < 0 || m.reader >= nb || m.producer < 0 || m.producer >= nb) {
            err = row_msg("mount", i, "branch index out of range");
            return OCTOPUS_EINVAL;
        }
        if (m.reader == m.producer) {
            err = row_msg("mount", i, "reader == producer");
            return OCTOPUS_EINVAL;
        }
        if (m.rpos < 0 || m.rpos > br[m.reader].len) {
            err = row_msg("mount", i, "rpos outside the reader");
            return OCTOPUS_EINVAL;
        }
        if (!(0 <= m.s && m.s < m.e && m.e <= br[m.producer].len)) {
            err = row_msg("mount", i, "span outside the producer");
            return OCTOPUS_EINVAL;
        }
        if (tree[m.reader] != tree[m.producer]) {
            err = row_msg("mount", i, "producer belongs to another tree");
            return OCTOPUS_EINVAL;
        }
    }
    return OCTOPUS_OK;
}

// Positions by an explicit worklist over (branch, offset) requests.  A branch is
// "open" while it sits on the stack; asking an open branch for an offset it has
// not reached yet is a dependency cycle.  Along a branch a position only moves by
// one per token except at a mount offset, so each branch's positions are kept as runs
// (first offset, its position) and computed run by run: the cost follows the branches
// and mounts, not the tokens (the dense positions are written only when asked for).
int compute_positions(DagInfo& d, bool fill, std::string& err) {
    const int32_t nb = (int32_t)d.br.size();
    struct Run { int32_t k; int64_t v; };
    std::vector<std::vector<Run>> runs(nb);
    std::vector<int32_t> done(nb, 0);  // offsets 0 .. done - 1 are known
    // Position of branch b's offset k (k < done[b]).
    auto at = [&](int32_t b, int32_t k) -> int64_t {
        const std::vector<Run>& rs = runs[b];
        size_t lo = 0, hi = rs.size();
        while (hi - lo > 1) {
            const size_t mid = (lo + hi) / 2;
            if (rs[mid].k <= k) lo = mid; else hi = mid;
        }
        return rs[lo].v + (k - rs[lo].k);
    };
    std::vector<size_t> next_mount(nb, 0);
    std::vector<char> open(nb, 0);
    struct Req { int32_t b, r; };
    std::vector<Req> stack;
    stack.reserve(nb);
    for (int32_t b0 = 0; b0 < nb; ++b0) {
        stack.push_back({b0, d.br[b0].len});
        open[b0] = 1;
        while (!stack.empty()) {
            Req& top = stack.back();
            const int32_t b = top.b;
            if (done[b] > top.r) {
                open[b] = 0;
                stack.pop_back();
                continue;
            }
            const int32_t k = done[b];
            const octopus_branch& B = d.br[b];
            // Dependencies of x_b(k): the parent's position at the fork (k = 0), and the
            // last mounted key of every mount issued at offset k.
            Req need{-1, -1};
            if (k == 0 && B.parent >= 0 && done[B.parent] <= B.fork) {
                need = {B.parent, B.fork};
            } else {
                const auto& ms = d.mounts_of[b];
                for (size_t i = next_mount[b]; i < ms.size() && d.mt[ms[i]].rpos == k; ++i) {
                    const octopus_mount& m = d.mt[ms[i]];
                    if (done[m.producer] <= m.e - 1) {
                        need = {m.producer, m.e - 1};
                        break;
                    }
                }
            }
            if (need.b >= 0) {
                if (open[need.b]) {
                    err = "position of branch " + std::to_string(need.b) + " offset " +
                          std::to_string(need.r) + " depends on itself";
                    return OCTOPUS_ECYCLE;
                }
                open[need.b] = 1;
                stack.push_back(need);
                continue;
            }
            int64_t v = (k == 0) ? (B.parent < 0 ? 0 : at(B.parent, B.fork)) : at(b, k - 1) + 1;
            const auto& ms = d.mounts_of[b];
            while (next_mount[b] < ms.size() && d.mt[ms[next_mount[b]]].rpos == k) {
                const octopus_mount& m = d.mt[ms[next_mount[b]]];
                // e_A = position of the last mounted key + 1; next = max(p_B, e_A + 1).
                v = std::max(v, at(m.producer, m.e - 1) + 2);
                ++next_mount[b];
            }
            if (k == 0 || v != at(b, k - 1) + 1) runs[b].push_back({k, v});
            // Up to the branch's next mount offset nothing else moves a position: the
            // run continues by one per token (and depends on nothing).
            done[b] = (next_mount[b] < ms.size() ? d.mt[ms[next_mount[b]]].rpos - 1 : B.len) + 1;
        }
    }
    for (int32_t b = 0; b < nb; ++b) {  // positions increase along a branch
        if (d.br[b].len > 0 && at(b, d.br[b].len - 1) > INT32_MAX) {
            err = "position exceeds int32";
            return OCTOPUS_EINVAL;
        }
    }
    if (!fill) return OCTOPUS_OK;
    d.pos.assign(d.T, 0);
    for (int32_t b = 0; b < nb; ++b) {
        const std::vector<Run>& rs = runs[b];
        for (size_t j = 0; j < rs.size(); ++j) {
            const int32_t k1 = j + 1 < rs.size() ? rs[j + 1].k : d.br[b].len;
            for (int32_t k = rs[j].k; k < std::min(k1, d.br[b].len); ++k)
                d.pos[(size_t)d.br[b].start + k] = rs[j].v + (k - rs[j].k);
        }
    }
    return OCTOPUS_OK;
}

}  // namespace

void DagInfo::row_context(int32_t b, int32_t r, std::vector<Interval>& out,
                          std::vector<Interval>& scratch) const {
    scratch.assign(inherited[b].begin(), inherited[b].end());
    const octopus_branch& B = br[b];
    scratch.push_back({B.start, (int64_t)B.start + r + 1});
    for (int32_t id : mounts_of[b]) {
        const octopus_mount& m = mt[id];
        if (m.rpos > r) break;
        const int64_t ps = br[m.producer].start;
        scratch.push_back({ps + m.s, ps + m.e});
    }
    merge(scratch);
    out.swap(scratch);
}

int32_t DagInfo::owner(int64_t j) const {
    // order_by_start sorted by start: the last branch whose start <= j.
    size_t lo = 0, hi = order_by_start.size();
    while (hi - lo > 1) {
        size_t mid = (lo + hi) / 2;
        if (br[order_by_start[mid]].start <= j) lo = mid; else hi = mid;
    }
    return order_by_start[lo];
}

int load_dag(const octopus_branch* br, int32_t nb, const octopus_mount* mt, int32_t nm,
             int32_t T, DagInfo& d, std::string& err, bool with_positions) {
    int rc = validate(br, nb, mt, nm, T, err);
    if (rc != OCTOPUS_OK) return rc;
    d.T = T;
    d.br.assign(br, br + nb);
    d.mt.assign(mt, mt + nm);
    d.mounts_of.assign(nb, {});
    for (int32_t i = 0; i < nm; ++i) d.mounts_of[mt[i].reader].push_back(i);
    for (auto& v : d.mounts_of) {
        std::stable_sort(v.begin(), v.end(),
                         [&](int32_t a, int32_t b) { return d.mt[a].rpos < d.mt[b].rpos; });
    }
    d.tree.resize(nb);
    for (int32_t b = 0; b < nb; ++b) d.tree[b] = br[b].parent < 0 ? b : d.tree[br[b].parent];
    // H(b) = H(parent) ∪ parent's own [0, fork) ∪ parent's mounts issued at rpos <= fork.
    d.inherited.assign(nb, {});
    for (int32_t b = 1; b < nb; ++b) {
        const octopus_branch& B = d.br[b];
        if (B.parent < 0) continue;  // the root of another tree: H = {}
        const octopus_branch& P = d.br[B.parent];
        std::vector<Interval> h = d.inherited[B.parent];
        if (B.fork > 0) h.push_back({P.start, (int64_t)P.start + B.fork});
        for (int32_t id : d.mounts_of[B.parent]) {
            const octopus_mount& m = d.mt[id];
            if (m.rpos > B.fork) break;
            const int64_t ps = d.br[m.producer].start;
            h.push_back({ps + m.s, ps + m.e});
        }
        merge(h);
        d.inherited[b].swap(h);
    }
    d.order_by_start.resize(nb);
    std::iota(d.order_by_start.begin(), d.order_by_start.end(), 0);
    std::sort(d.order_by_start.begin(), d.order_by_start.end(),
              [&](int a, int b) { return d.br[a].start < d.br[b].start; });
    return compute_positions(d, with_positions, err);
}

int build_plan(const octopus_branch* br, int32_t nb, const octopus_mount* mt, int32_t nm,
               int32_t T, int32_t kv_tile, Plan& p, std::string& err) {
    if (kv_tile != 64) {
        err = "kv_tile must be 64";
        return OCTOPUS_EUNSUPPORTED;
    }
    int rc = load_dag(br, nb, mt, nm, T, p.dag, err);
    if (rc != OCTOPUS_OK) return rc;
    const DagInfo& d = p.dag;
    const int32_t Bq = kQTile, Bk = kv_tile;
    p.T = T;
    p.Bq = Bq;
    p.Bk = Bk;
    p.row_words = Bk / 64;
    p.col_words = Bq / 64;
    p.nQT = (T + Bq - 1) / Bq;
    p.nKT = (T + Bk - 1) / Bk;
    const int32_t nQT = p.nQT, nKT = p.nKT;

    std::vector<int32_t> row_branch(T);
    for (int32_t b = 0; b < nb; ++b)
        for (int32_t r = 0; r < d.br[b].len; ++r) row_branch[d.br[b].start + r] = b;

    // The query tiles' lists, planned in blocks of consecutive tiles that host threads take
    // in turn; the blocks are joined in tile order (mask indices offset by the masks of the
    // blocks before), so the plan does not depend on the threads.
    struct TileBlock {
        std::vector<TilePair> pairs;   // mask: index among this block's partial masks
        std::vector<uint64_t> masks;
        std::vector<int32_t> count;    // pairs per query tile
        int64_t nnz = 0;
    };
    auto plan_tiles = [&](int32_t qt_lo, int32_t qt_hi, TileBlock& out) {
        std::vector<std::vector<Interval>> rows(Bq);
        std::vector<Interval> scratch;
        // Difference arrays over KV tiles, cleared entry by entry after each query tile;
        // only the tile ranges some row touches are swept, so planning costs O(rows x
        // intervals + listed pairs) rather than O(query tiles x KV tiles) (a forest of many
        // trees would otherwise sweep every tile of every tree for every query tile).
        std::vector<int32_t> full_diff(nKT + 1, 0), touch_diff(nKT + 1, 0);
        std::vector<std::pair<int64_t, int64_t>> spans;  // touched tile ranges [t0, t1)
        std::vector<std::pair<int64_t, int64_t>> row_sp, prev_sp;  // one row's ranges
        std::vector<size_t> cursor(Bq);
        std::vector<uint64_t> words(Bq * p.row_words);
        out.count.assign(qt_hi - qt_lo, 0);
        for (int32_t qt = qt_lo; qt < qt_hi; ++qt) {
            const size_t n_before = out.pairs.size();
            const int32_t r0 = qt * Bq;
            const int32_t nv = std::min(Bq, T - r0);
            spans.clear();
            prev_sp.clear();
            for (int32_t rr = 0; rr < nv; ++rr) {
                const int32_t i = r0 + rr;
                const int32_t b = row_branch[i];
                const int32_t r = i - d.br[b].start;
                // Ctx(b, r) = Ctx(b, r - 1) + the own token i (never already in it: a branch
                // does not mount itself) + the spans mounted at rpos = r.  Without such a
                // mount the previous row's intervals are copied and the one ending at i
                // grows by one key (joining the next interval if that starts at i + 1).
                bool inc = rr > 0 && r > 0 && row_branch[i - 1] == b;
                if (inc)
                    for (int32_t id : d.mounts_of[b])
                        if (d.mt[id].rpos == r) { inc = false; break; }
                if (inc) {
                    std::vector<Interval>& cur = rows[rr];
                    cur = rows[rr - 1];
                    for (size_t j = 0; j < cur.size(); ++j) {
                        if (cur[j].hi != i) continue;
                        cur[j].hi = (int64_t)i + 1;
                        if (j + 1 < cur.size() && cur[j + 1].lo == (int64_t)i + 1) {
                            cur[j].hi = cur[j + 1].hi;
                            cur.erase(cur.begin() + (j + 1));
                        }
                        break;
                    }
                } else {
                    d.row_context(b, r, rows[rr], scratch);
                }
                row_sp.clear();
                for (const Interval& iv : rows[rr]) {
                    out.nnz += iv.hi - iv.lo;
                    const int64_t t0 = iv.lo / Bk, t1 = (iv.hi + Bk - 1) / Bk;
                    touch_diff[t0] += 1;
                    touch_diff[t1] -= 1;
                    // Neighbouring rows mostly repeat their ranges; keep each range once.
                    row_sp.push_back({t0, t1});
                    if (std::find(prev_sp.begin(), prev_sp.end(), row_sp.back()) == prev_sp.end())
                        spans.push_back({t0, t1});
                    const int64_t f0 = (iv.lo + Bk - 1) / Bk, f1 = iv.hi / Bk;
                    if (f0 < f1) {
                        full_diff[f0] += 1;
                        full_diff[f1] -= 1;
                    }
                }
                cursor[rr] = 0;
                prev_sp.swap(row_sp);
            }
            // Merge the touched ranges; every interval starts and ends inside one merged
            // range, so the running sums are 0 at the start of each.
            std::sort(spans.begin(), spans.end());
            size_t n_sp = 0;
            for (size_t j = 0; j < spans.size(); ++j) {
                if (n_sp > 0 && spans[j].first <= spans[n_sp - 1].second)
                    spans[n_sp - 1].second = std::max(spans[n_sp - 1].second, spans[j].second);
                else
                    spans[n_sp++] = spans[j];
            }
            for (size_t sp = 0; sp < n_sp; ++sp) {
                int32_t touch = 0, full = 0;
                for (int32_t t = (int32_t)spans[sp].first; t < (int32_t)spans[sp].second; ++t) {
                    touch += touch_diff[t];
                    full += full_diff[t];
                    if (touch == 0) continue;
                    if (full == nv) {
                        out.pairs.push_back({t, -1});
                        continue;
                    }
                    // PARTIAL: per-row bits of keys [t*Bk, t*Bk + Bk) that the row sees.
                    const int64_t k0 = (int64_t)t * Bk, k1 = k0 + Bk;
                    std::fill(words.begin(), words.end(), 0);
                    for (int32_t rr = 0; rr < nv; ++rr) {
                        const auto& iv = rows[rr];
                        size_t c = cursor[rr];
                        while (c < iv.size() && iv[c].hi <= k0) ++c;
                        cursor[rr] = c;
                        for (size_t j = c; j < iv.size() && iv[j].lo < k1; ++j) {
                            const int64_t a = std::max(iv[j].lo, k0) - k0;
                            const int64_t e = std::min(iv[j].hi, k1) - k0;
                            set_bits(&words[rr * p.row_words], a, e);
                        }
                    }
                    const int32_t idx = (int32_t)(out.masks.size() / (Bq * p.row_words));
                    out.masks.insert(out.masks.end(), words.begin(), words.end());
                    out.pairs.push_back({t, idx});
                }
            }
            // Clear the entries this query tile set.
            for (int32_t rr = 0; rr < nv; ++rr) {
                for (const Interval& iv : rows[rr]) {
                    touch_diff[iv.lo / Bk] = 0;
                    touch_diff[(iv.hi + Bk - 1) / Bk] = 0;
                    full_diff[(iv.lo + Bk - 1) / Bk] = 0;
                    full_diff[iv.hi / Bk] = 0;
                }
            }
            out.count[qt - qt_lo] = (int32_t)(out.pairs.size() - n_before);
        }
    };
    const int32_t n_blocks = std::max<int32_t>(1, std::min<int32_t>(nQT / 8, 256));
    std::vector<TileBlock> blocks(n_blocks);
    auto block_lo = [&](int32_t i) { return (int32_t)((int64_t)nQT * i / n_blocks); };
    const int32_t n_threads = std::min(plan_threads(), std::max<int32_t>(1, n_blocks / 2));
    parallel_for(n_blocks, n_threads,
                 [&](int32_t i) { plan_tiles(block_lo(i), block_lo(i + 1), blocks[i]); });
    // Join the blocks in tile order: each block's pairs and masks go to their offsets (mask
    // indices shifted by the masks of the blocks before).
    const size_t mask_words = (size_t)Bq * p.row_words;
    std::vector<size_t> pair_at(n_blocks + 1, 0), mask_at(n_blocks + 1, 0);
    p.qt_ptr.assign(nQT + 1, 0);
    p.nnz = 0;
    for (int32_t i = 0; i < n_blocks; ++i) {
        pair_at[i + 1] = pair_at[i] + blocks[i].pairs.size();
        mask_at[i + 1] = mask_at[i] + blocks[i].masks.size() / mask_words;
        for (int32_t qt = block_lo(i); qt < block_lo(i + 1); ++qt)
            p.qt_ptr[qt + 1] = p.qt_ptr[qt] + blocks[i].count[qt - block_lo(i)];
        p.nnz += blocks[i].nnz;
    }
    p.q_pairs.resize(pair_at[n_blocks]);
    // (room for the all-ones mask appended below)
    p.mask_rows.reserve((mask_at[n_blocks] + 1) * mask_words);
    p.mask_rows.resize(mask_at[n_blocks] * mask_words);
    parallel_for(n_blocks, n_threads, [&](int32_t i) {
        TileBlock& b = blocks[i];
        const int32_t base = (int32_t)mask_at[i];
        TilePair* dst = p.q_pairs.data() + pair_at[i];
        for (size_t j = 0; j < b.pairs.size(); ++j) {
            const TilePair& tp = b.pairs[j];
            dst[j] = {tp.tile, tp.mask < 0 ? tp.mask : base + tp.mask};
        }
        std::copy(b.masks.begin(), b.masks.end(), p.mask_rows.begin() + mask_at[i] * mask_words);
        TileBlock().pairs.swap(b.pairs);  // free as we go
        TileBlock().masks.swap(b.masks);
    });
    p.n_partial = (int64_t)(p.mask_rows.size() / (Bq * p.row_words));

    // One extra all-ones mask (index n_partial) that kernels may use for FULL tiles.
    p.mask_rows.insert(p.mask_rows.end(), (size_t)Bq * p.row_words, ~0ull);

    // Key-major copy of every PARTIAL mask, for the KV-tile owners of the backward, then
    // an all-ones mask (index n_partial, FULL) and an all-zeros one (n_partial + 1, a
    // tile that the query tile does not see).
    p.mask_cols.assign((p.n_partial + 2) * Bk * p.col_words, 0);
    std::fill(p.mask_cols.begin() + p.n_partial * Bk * p.col_words,
              p.mask_cols.begin() + (p.n_partial + 1) * Bk * p.col_words, ~0ull);
    const int32_t n_mc = (int32_t)std::min<int64_t>(p.n_partial, 256);  // mask groups
    parallel_for(n_mc, p.n_partial >= 512 ? plan_threads() : 1, [&](int32_t grp) {
        const int64_t m0 = p.n_partial * grp / n_mc, m1 = p.n_partial * (grp + 1) / n_mc;
        for (int64_t m = m0; m < m1; ++m) {
            const uint64_t* wr = &p.mask_rows[m * Bq * p.row_words];
            uint64_t* wc = &p.mask_cols[m * Bk * p.col_words];
            if (Bk == 64) {  // one word per row: transpose 64-row blocks as bit matrices
                for (int32_t hf = 0; hf < Bq / 64; ++hf) {
                    uint64_t blk[64];
                    std::copy(wr + 64 * hf, wr + 64 * hf + 64, blk);
                    transpose64(blk);
                    for (int32_t kk = 0; kk < 64; ++kk) wc[kk * p.col_words + hf] = blk[kk];
                }
                continue;
            }
            for (int32_t rr = 0; rr < Bq; ++rr)
                for (int32_t kk = 0; kk < Bk; ++kk)
                    if ((wr[rr * p.row_words + (kk >> 6)] >> (kk & 63)) & 1)
                        wc[kk * p.col_words + (rr >> 6)] |= 1ull << (rr & 63);
        }
    });

    // Transposed lists: for every KV tile, the query tiles that see it, ascending.
    p.kt_ptr.assign(nKT + 1, 0);
    for (const TilePair& tp : p.q_pairs) p.kt_ptr[tp.tile + 1] += 1;
    for (int32_t t = 0; t < nKT; ++t) p.kt_ptr[t + 1] += p.kt_ptr[t];
    p.k_pairs.assign(p.q_pairs.size(), {0, 0});
    {
        std::vector<int32_t> fill(p.kt_ptr.begin(), p.kt_ptr.end() - 1);
        for (int32_t qt = 0; qt < nQT; ++qt)
            for (int32_t i = p.qt_ptr[qt]; i < p.qt_ptr[qt + 1]; ++i)
                p.k_pairs[fill[p.q_pairs[i].tile]++] = {qt, p.q_pairs[i].mask};
    }

    // Launch orders: tree by tree (in the order of their root rows), longest list first
    // inside a tree, ties by index.  A tile belongs to the tree of its first token.  One
    // tree at a time keeps the K/V and Q/dO that concurrently running workgroups read
    // as small as for a single tree; only the last tree's shortest tiles form the tail.
    auto tree_of = [&](int64_t j) { return d.tree[row_branch[j]]; };
    auto order = [&](std::vector<int32_t>& ord, int32_t n, const std::vector<int32_t>& ptr,
                     int32_t rows_per) {
        std::vector<int32_t> tr(n);
        for (int32_t i = 0; i < n; ++i) tr[i] = tree_of((int64_t)i * rows_per);
        ord.resize(n);
        std::iota(ord.begin(), ord.end(), 0);
        std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) {
            if (tr[a] != tr[b]) return tr[a] < tr[b];
            return ptr[a + 1] - ptr[a] > ptr[b + 1] - ptr[b];
        });
    };
    order(p.fwd_order, nQT, p.qt_ptr, Bq);
    order(p.bwd_order, nKT, p.kt_ptr, Bk);
    // 128-key blocks: merge the transposed lists of tiles 2b and 2b+1.
    p.nKB = (nKT + 1) / 2;
    p.blk_ptr.assign(p.nKB + 1, 0);
    p.blk_entries.clear();
    p.blk_entries.reserve(p.k_pairs.size());  // at most one entry per listed pair
    for (int32_t b = 0; b < p.nKB; ++b) {
        const int32_t t0 = 2 * b, t1 = 2 * b + 1;
        int32_t i0 = p.kt_ptr[t0], e0 = p.kt_ptr[t0 + 1];
        int32_t i1 = t1 < nKT ? p.kt_ptr[t1] : 0, e1 = t1 < nKT ? p.kt_ptr[t1 + 1] : 0;
        while (i0 < e0 || i1 < e1) {
            const int32_t q0 = i0 < e0 ? p.k_pairs[i0].tile : INT32_MAX;
            const int32_t q1 = i1 < e1 ? p.k_pairs[i1].tile : INT32_MAX;
            const int32_t qt = std::min(q0, q1);
            BlockEntry be{qt, -2, -2, 0};
            if (q0 == qt) be.mask0 = p.k_pairs[i0++].mask;
            if (q1 == qt) be.mask1 = p.k_pairs[i1++].mask;
            p.blk_entries.push_back(be);
        }
        p.blk_ptr[b + 1] = (int32_t)p.blk_entries.size();
    }
    order(p.blk_order, p.nKB, p.blk_ptr, 2 * Bk);

    p.max_q_list = 0;
    for (int32_t qt = 0; qt < nQT; ++qt)
        p.max_q_list = std::max(p.max_q_list, p.qt_ptr[qt + 1] - p.qt_ptr[qt]);
    p.max_kv_list = 0;
    for (int32_t t = 0; t < nKT; ++t)
        p.max_kv_list = std::max(p.max_kv_list, p.kt_ptr[t + 1] - p.kt_ptr[t]);

    // Recurrent scan metadata: one checkpoint slot per distinct (parent, fork offset);
    // levels by depth so that a level's branches start from states the previous levels
    // saved.
    {
        std::map<std::pair<int32_t, int32_t>, int32_t> slot;
        p.sc_init.assign(nb, -1);
        std::vector<std::vector<std::pair<int32_t, int32_t>>> cks(nb);
        for (int32_t b = 0; b < nb; ++b) {
            const octopus_branch& B = d.br[b];
            if (B.parent < 0) continue;
            const auto key = std::make_pair(B.parent, B.fork);
            auto it = slot.find(key);
            if (it == slot.end()) {
                it = slot.emplace(key, (int32_t)slot.size()).first;
                cks[B.parent].push_back({B.fork, it->second});
            }
            p.sc_init[b] = it->second;
        }
        p.n_slots = (int32_t)slot.size();
        p.sc_ck_ptr.assign(1, 0);
        p.sc_ck_off.clear();
        p.sc_ck_slot.clear();
        for (int32_t b = 0; b < nb; ++b) {
            std::sort(cks[b].begin(), cks[b].end());
            for (const auto& c : cks[b]) {
                p.sc_ck_off.push_back(c.first);
                p.sc_ck_slot.push_back(c.second);
            }
            p.sc_ck_ptr.push_back((int32_t)p.sc_ck_off.size());
        }
        // The children forking at every checkpoint, in ascending branch order (the
        // backward adds their initial-state gradients in this fixed order).
        {
            std::vector<int32_t> ck_of_slot(p.n_slots, -1);
            for (size_t c = 0; c < p.sc_ck_slot.size(); ++c) ck_of_slot[p.sc_ck_slot[c]] = (int32_t)c;
            std::vector<int32_t> count(p.sc_ck_slot.size() + 1, 0);
            for (int32_t b = 0; b < nb; ++b)
                if (p.sc_init[b] >= 0) ++count[ck_of_slot[p.sc_init[b]] + 1];
            p.sc_ck_kid_ptr.assign(p.sc_ck_slot.size() + 1, 0);
            for (size_t c = 0; c < p.sc_ck_slot.size(); ++c)
                p.sc_ck_kid_ptr[c + 1] = p.sc_ck_kid_ptr[c] + count[c + 1];
            p.sc_ck_kid.assign(p.sc_ck_kid_ptr.back(), 0);
            std::vector<int32_t> fill(p.sc_ck_kid_ptr.begin(), p.sc_ck_kid_ptr.end() - 1);
            for (int32_t b = 0; b < nb; ++b)  // ascending b: each list comes out sorted
                if (p.sc_init[b] >= 0) p.sc_ck_kid[fill[ck_of_slot[p.sc_init[b]]]++] = b;
        }
        // Branches by depth (a branch's parent has a smaller index, so one pass suffices).
        std::vector<int32_t> depth(nb, 0);
        int32_t max_depth = 0;
        for (int32_t b = 0; b < nb; ++b) {
            if (d.br[b].parent >= 0) depth[b] = depth[d.br[b].parent] + 1;
            max_depth = std::max(max_depth, depth[b]);
        }
        p.level_ptr.assign(max_depth + 2, 0);
        for (int32_t b = 0; b < nb; ++b) p.level_ptr[depth[b] + 1] += 1;
        for (int32_t l = 0; l <= max_depth; ++l) p.level_ptr[l + 1] += p.level_ptr[l];
        p.level_br.assign(nb, 0);
        std::vector<int32_t> fill(p.level_ptr.begin(), p.level_ptr.end() - 1);
        for (int32_t b = 0; b < nb; ++b) p.level_br[fill[depth[b]]++] = b;
        // Chunks of the chunked scan: boundaries every kScanChunk own tokens and at every
        // checkpoint offset inside the branch (the kernel walks the same rule), numbered
        // level by level so that every level's chunks form one range.
        p.sc_chunk_base.assign(2 * (size_t)nb, 0);
        p.sc_chunk_tok.clear();
        p.sc_chunk_nt.clear();
        p.level_chunk.assign(1, 0);
        for (int32_t l = 0; l <= max_depth; ++l) {
            for (int32_t i = p.level_ptr[l]; i < p.level_ptr[l + 1]; ++i) {
                const int32_t b = p.level_br[i];
                const int32_t len = d.br[b].len;
                p.sc_chunk_base[2 * b] = (int32_t)p.sc_chunk_tok.size();
                int32_t c = p.sc_ck_ptr[b];
                int32_t r = 0;
                while (c < p.sc_ck_ptr[b + 1] && p.sc_ck_off[c] <= r) ++c;
                while (r < len) {
                    int32_t e = std::min(len, (r / kScanChunk + 1) * kScanChunk);
                    if (c < p.sc_ck_ptr[b + 1]) e = std::min(e, p.sc_ck_off[c]);
                    p.sc_chunk_tok.push_back(d.br[b].start + r);
                    p.sc_chunk_nt.push_back(e - r);
                    r = e;
                    while (c < p.sc_ck_ptr[b + 1] && p.sc_ck_off[c] <= r) ++c;
                }
                p.sc_chunk_base[2 * b + 1] = (int32_t)p.sc_chunk_tok.size();
            }
            p.level_chunk.push_back((int32_t)p.sc_chunk_tok.size());
        }
        p.n_chunks = (int64_t)p.sc_chunk_tok.size();
    }

    // Device image: every array 256-byte aligned.
    DevLayout& L = p.layout;
    size_t at = 0;
    auto place = [&](size_t bytes) {
        size_t off = at;
        at = (at + bytes + 255) & ~size_t(255);
        return off;
    };
    L.fwd_order = place(p.fwd_order.size() * 4);
    L.qt_ptr = place(p.qt_ptr.size() * 4);
    L.q_pairs = place(p.q_pairs.size() * sizeof(TilePair));
    L.bwd_order = place(p.bwd_order.size() * 4);
    L.kt_ptr = place(p.kt_ptr.size() * 4);
    L.k_pairs = place(p.k_pairs.size() * sizeof(TilePair));
    L.mask_rows = place(p.mask_rows.size() * 8);
    L.mask_cols = place(p.mask_cols.size() * 8);
    L.blk_order = place(p.blk_order.size() * 4);
    L.blk_ptr = place(p.blk_ptr.size() * 4);
    L.blk_entries = place(p.blk_entries.size() * sizeof(BlockEntry));
    L.pos = place((size_t)T * 4);
    L.sc_start = place((size_t)nb * 4);
    L.sc_len = place((size_t)nb * 4);
    L.sc_init = place((size_t)nb * 4);
    L.sc_ck_ptr = place(p.sc_ck_ptr.size() * 4);
    L.sc_ck_off = place(std::max<size_t>(p.sc_ck_off.size(), 1) * 4);
    L.sc_ck_slot = place(std::max<size_t>(p.sc_ck_slot.size(), 1) * 4);
    L.sc_ck_kid_ptr = place(p.sc_ck_kid_ptr.size() * 4);
    L.sc_ck_kid = place(std::max<size_t>(p.sc_ck_kid.size(), 1) * 4);
    L.sc_level_br = place((size_t)nb * 4);
    L.sc_chunk_base = place(std::max<size_t>(p.sc_chunk_base.size(), 1) * 4);
    L.sc_chunk_tok = place(std::max<size_t>(p.sc_chunk_tok.size(), 1) * 4);
    L.sc_chunk_nt = place(std::max<size_t>(p.sc_chunk_nt.size(), 1) * 4);
    L.total = std::max<size_t>(at, 256);
    return OCTOPUS_OK;
}

void write_device_image(const Plan& p, unsigned char* dst) {
    const DevLayout& L = p.layout;
    const DagInfo& d = p.dag;
    const int32_t nb = (int32_t)d.br.size();
    size_t end = 0;  // end of the last array written; the gaps before each are zeroed
    auto put = [&](size_t off, const void* src, size_t bytes) {
        std::memset(dst + end, 0, off - end);
        if (bytes) std::memcpy(dst + off, src, bytes);
        end = off + bytes;
    };
    put(L.fwd_order, p.fwd_order.data(), p.fwd_order.size() * 4);
    put(L.qt_ptr, p.qt_ptr.data(), p.qt_ptr.size() * 4);
    put(L.q_pairs, p.q_pairs.data(), p.q_pairs.size() * sizeof(TilePair));
    put(L.bwd_order, p.bwd_order.data(), p.bwd_order.size() * 4);
    put(L.kt_ptr, p.kt_ptr.data(), p.kt_ptr.size() * 4);
    put(L.k_pairs, p.k_pairs.data(), p.k_pairs.size() * sizeof(TilePair));
    put(L.mask_rows, p.mask_rows.data(), p.mask_rows.size() * 8);
    put(L.mask_cols, p.mask_cols.data(), p.mask_cols.size() * 8);
    put(L.blk_order, p.blk_order.data(), p.blk_order.size() * 4);
    put(L.blk_ptr, p.blk_ptr.data(), p.blk_ptr.size() * 4);
    put(L.blk_entries, p.blk_entries.data(), p.blk_entries.size() * sizeof(BlockEntry));
    {
        put(L.pos, nullptr, 0);
        int32_t* pos = reinterpret_cast<int32_t*>(dst + L.pos);
        for (int32_t i = 0; i < p.T; ++i) pos[i] = (int32_t)d.pos[i];
        end = L.pos + (size_t)p.T * 4;
        put(L.sc_start, nullptr, 0);
        int32_t* st = reinterpret_cast<int32_t*>(dst + L.sc_start);
        for (int32_t b = 0; b < nb; ++b) st[b] = d.br[b].start;
        end = L.sc_start + (size_t)nb * 4;
        put(L.sc_len, nullptr, 0);
        int32_t* ln = reinterpret_cast<int32_t*>(dst + L.sc_len);
        for (int32_t b = 0; b < nb; ++b) ln[b] = d.br[b].len;
        end = L.sc_len + (size_t)nb * 4;
    }
    put(L.sc_init, p.sc_init.data(), p.sc_init.size() * 4);
    put(L.sc_ck_ptr, p.sc_ck_ptr.data(), p.sc_ck_ptr.size() * 4);
    put(L.sc_ck_off, p.sc_ck_off.data(), p.sc_ck_off.size() * 4);
    put(L.sc_ck_slot, p.sc_ck_slot.data(), p.sc_ck_slot.size() * 4);
    put(L.sc_ck_kid_ptr, p.sc_ck_kid_ptr.data(), p.sc_ck_kid_ptr.size() * 4);
    put(L.sc_ck_kid, p.sc_ck_kid.data(), p.sc_ck_kid.size() * 4);
    put(L.sc_level_br, p.level_br.data(), p.level_br.size() * 4);
    put(L.sc_chunk_base, p.sc_chunk_base.data(), p.sc_chunk_base.size() * 4);
    put(L.sc_chunk_tok, p.sc_chunk_tok.data(), p.sc_chunk_tok.size() * 4);
    put(L.sc_chunk_nt, p.sc_chunk_nt.data(), p.sc_chunk_nt.size() * 4);
    std::memset(dst + end, 0, L.total - end);
}

void export_mask(const Plan& p, int32_t lo, int32_t hi, uint8_t* bits) {
    const size_t row_bytes = (size_t)(p.T + 7) / 8;
    std::memset(bits, 0, row_bytes * (size_t)(hi - lo));
    for (int32_t i = lo; i < hi; ++i) {
        uint8_t* out = bits + (size_t)(i - lo) * row_bytes;
        const int32_t qt = i / p.Bq, rr = i % p.Bq;
        for (int32_t k = p.qt_ptr[qt]; k < p.qt_ptr[qt + 1]; ++k) {
            const TilePair& tp = p.q_pairs[k];
            const int64_t k0 = (int64_t)tp.tile * p.Bk;
            for (int32_t x = 0; x < p.Bk; ++x) {
                const int64_t j = k0 + x;
                if (j >= p.T) break;
                bool on;
                if (tp.mask < 0) {
                    on = true;
                } else {
                    const uint64_t w =
                        p.mask_rows[((size_t)tp.mask * p.Bq + rr) * p.row_words + (x >> 6)];
                    on = (w >> (x & 63)) & 1;
                }
                if (on) out[j >> 3] |= (uint8_t)(1u << (j & 7));
            }
        }
    }
}

// Shared checks of the page table and the cursor list.
static int check_pages(const DagInfo& d, const int32_t* page_ptr, const int32_t* pages,
                       int32_t page_size, int32_t n_pages, const int32_t* cursors,
                       int32_t n_cursors, std::string& err) {
    const int32_t nb = (int32_t)d.br.size();
    if (page_size < 1 || n_pages < 0 || n_cursors < 0 || page_ptr == nullptr ||
        (n_cursors > 0 && cursors == nullptr)) {
        err = "bad page table or cursor arguments";
        return OCTOPUS_EINVAL;
    }
    if (page_ptr[0] != 0) { err = "page_ptr[0] must be 0"; return OCTOPUS_EINVAL; }
    for (int32_t b = 0; b < nb; ++b) {
        const int64_t need = ((int64_t)d.br[b].len + page_size - 1) / page_size;
        if (page_ptr[b + 1] - page_ptr[b] < need) {
            err = row_msg("branch", b, "page table shorter than the branch");
            return OCTOPUS_EINVAL;
        }
        for (int32_t k = page_ptr[b]; k < page_ptr[b] + need; ++k) {
            if (pages == nullptr || pages[k] < 0 || pages[k] >= n_pages) {
                err = row_msg("branch", b, "page id outside [0, n_pages)");
                return OCTOPUS_EINVAL;
            }
        }
    }
    for (int32_t c = 0; c < n_cursors; ++c) {
        if (cursors[c] < 0 || cursors[c] >= nb) {
            err = row_msg("cursor", c, "branch id out of range");
            return OCTOPUS_EINVAL;
        }
    }
    return OCTOPUS_OK;
}

int build_segments(const DagInfo& d, const int32_t* page_ptr, const int32_t* pages,
                   int32_t page_size, int32_t n_pages, const int32_t* cursors,
                   int32_t n_cursors, bool share, std::vector<int32_t>& seg_ptr,
                   std::vector<int32_t>& seg_page, std::vector<int32_t>& seg_lo,
                   std::vector<int32_t>& seg_hi, std::vector<int32_t>& grp_ptr,
                   std::vector<int32_t>& grp_cur, std::string& err) {
    const int rc = check_pages(d, page_ptr, pages, page_size, n_pages, cursors, n_cursors, err);
    if (rc != OCTOPUS_OK) return rc;
    seg_ptr.assign(1, 0);
    seg_page.clear();
    seg_lo.clear();
    seg_hi.clear();
    grp_ptr.clear();
    grp_cur.clear();
    // One segment per (owning branch, page) run of the intervals, in order.
    auto emit = [&](const std::vector<Interval>& ivs) {
        for (const Interval& iv : ivs) {
            int64_t j = iv.lo;
            while (j < iv.hi) {
                const int32_t o = d.owner(j);
                const int64_t ostart = d.br[o].start;
                const int64_t stop = std::min<int64_t>(iv.hi, ostart + d.br[o].len);
                int64_t r = j - ostart;
                const int64_t rend = stop - ostart;
                while (r < rend) {
                    const int64_t pi = r / page_size;
                    const int64_t slot0 = r - pi * page_size;
                    const int64_t slot1 = std::min<int64_t>(page_size, rend - pi * page_size);
                    seg_page.push_back(pages[page_ptr[o] + pi]);
                    seg_lo.push_back((int32_t)slot0);
                    seg_hi.push_back((int32_t)slot1);
                    r = (pi + 1) * page_size;
                }
                j = stop;
            }
        }
        seg_ptr.push_back((int32_t)seg_page.size());
    };
    std::vector<Interval> ctx, scratch, rest;
    for (int32_t c = 0; c < n_cursors; ++c) {
        const int32_t b = cursors[c];
        d.row_context(b, d.br[b].len - 1, ctx, scratch);
        if (!share) {
            emit(ctx);
            continue;
        }
        // ctx minus H(b): both sorted and disjoint, and H(b) lies inside ctx.
        const std::vector<Interval>& h = d.inherited[b];
        rest.clear();
        size_t k = 0;
        for (const Interval& iv : ctx) {
            int64_t lo = iv.lo;
            while (k < h.size() && h[k].hi <= lo) ++k;
            size_t t = k;
            while (lo < iv.hi) {
                if (t < h.size() && h[t].lo < iv.hi) {
                    if (h[t].lo > lo) rest.push_back({lo, h[t].lo});
                    lo = std::max(lo, (int64_t)h[t].hi);
                    ++t;
                } else {
                    rest.push_back({lo, iv.hi});
                    lo = iv.hi;
                }
            }
        }
        emit(rest);
    }
    if (share) {
        // Groups: cursors forked from the same (parent, fork) inherit the same context.
        std::map<std::pair<int32_t, int32_t>, int32_t> gid;
        std::vector<std::vector<int32_t>> members;
        for (int32_t c = 0; c < n_cursors; ++c) {
            const octopus_branch& B = d.br[cursors[c]];
            const auto key = std::make_pair(B.parent, B.parent < 0 ? 0 : B.fork);
            auto it = gid.find(key);
            if (it == gid.end()) {
                it = gid.emplace(key, (int32_t)members.size()).first;
                members.emplace_back();
            }
            members[it->second].push_back(c);
        }
        grp_ptr.assign(1, 0);
        for (const auto& m : members) {
            emit(d.inherited[cursors[m[0]]]);
            grp_cur.insert(grp_cur.end(), m.begin(), m.end());
            grp_ptr.push_back((int32_t)grp_cur.size());
        }
    }
    return OCTOPUS_OK;
}

int build_extend_segments(const DagInfo& d, const int32_t* page_ptr, const int32_t* pages,
                          int32_t page_size, int32_t n_pages, const int32_t* cursors,
                          int32_t n_cursors, const int32_t* n_new, std::vector<int32_t>& seg_ptr,
                          std::vector<int32_t>& seg_page, std::vector<int32_t>& seg_lo,
                          std::vector<int32_t>& seg_hi, std::vector<int32_t>& seg_thr,
                          std::vector<int32_t>& seg_causal, std::vector<int32_t>& first_off,
                          std::string& err) {
    int rc = check_pages(d, page_ptr, pages, page_size, n_pages, cursors, n_cursors, err);
    if (rc != OCTOPUS_OK) return rc;
    if (n_cursors > 0 && n_new == nullptr) { err = "n_new is NULL"; return OCTOPUS_EINVAL; }
    for (int32_t c = 0; c < n_cursors; ++c) {
        if (n_new[c] < 1 || n_new[c] > d.br[cursors[c]].len) {
            err = row_msg("cursor", c, "new-token count outside [1, branch length]");
            return OCTOPUS_EINVAL;
        }
    }
    seg_ptr.assign(1, 0);
    seg_page.clear();
    seg_lo.clear();
    seg_hi.clear();
    seg_thr.clear();
    seg_causal.clear();
    first_off.assign(n_cursors, 0);
    struct Seg { int32_t page, lo, hi, thr, causal; };
    std::vector<Seg> segs;
    struct Piece { int64_t lo, hi; int32_t thr; };
    std::vector<Piece> pieces, resolved;
    std::vector<int64_t> cuts;
    for (int32_t c = 0; c < n_cursors; ++c) {
        const int32_t b = cursors[c];
        const octopus_branch& B = d.br[b];
        const int32_t L = B.len;
        first_off[c] = L - n_new[c];
        // Keys that are not b's own tokens, each with the smallest own offset from which
        // b sees it: 0 for what b inherits, rpos for a mounted span (mounts issued after
        // b's last token are seen by none of its tokens).
        pieces.clear();
        for (const Interval& iv : d.inherited[b]) pieces.push_back({iv.lo, iv.hi, 0});
        for (int32_t id : d.mounts_of[b]) {
            const octopus_mount& m = d.mt[id];
            if (m.rpos > L - 1) continue;
            const int64_t ps = d.br[m.producer].start;
            pieces.push_back({ps + m.s, ps + m.e, m.rpos});
        }
        cuts.clear();
        for (const Piece& p : pieces) {
            cuts.push_back(p.lo);
            cuts.push_back(p.hi);
        }
        std::sort(cuts.begin(), cuts.end());
        cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
        resolved.clear();
        for (size_t k = 0; k + 1 < cuts.size(); ++k) {
            int32_t thr = INT32_MAX;
            for (const Piece& p : pieces)
                if (p.lo <= cuts[k] && cuts[k + 1] <= p.hi) thr = std::min(thr, p.thr);
            if (thr == INT32_MAX) continue;
            if (!resolved.empty() && resolved.back().hi == cuts[k] && resolved.back().thr == thr)
                resolved.back().hi = cuts[k + 1];
            else
                resolved.push_back({cuts[k], cuts[k + 1], thr});
        }
        segs.clear();
        for (const Piece& p : resolved) {
            int64_t j = p.lo;
            while (j < p.hi) {
                const int32_t o = d.owner(j);
                const int64_t ostart = d.br[o].start;
                const int64_t stop = std::min<int64_t>(p.hi, ostart + d.br[o].len);
                int64_t r = j - ostart;
                const int64_t rend = stop - ostart;
                while (r < rend) {
                    const int64_t pi = r / page_size;
                    const int64_t slot0 = r - pi * page_size;
                    const int64_t slot1 = std::min<int64_t>(page_size, rend - pi * page_size);
                    segs.push_back({pages[page_ptr[o] + pi], (int32_t)slot0, (int32_t)slot1,
                                    p.thr, 0});
                    r = (pi + 1) * page_size;
                }
                j = stop;
            }
        }
        // b's own tokens: own offset t is seen by new tokens at offsets >= t.
        for (int64_t pi = 0; pi * page_size < L; ++pi) {
            const int32_t hi = (int32_t)std::min<int64_t>(page_size, L - pi * page_size);
            segs.push_back({pages[page_ptr[b] + pi], 0, hi, (int32_t)(pi * page_size), 1});
        }
        std::stable_sort(segs.begin(), segs.end(),
                         [](const Seg& x, const Seg& y) { return x.thr < y.thr; });
        for (const Seg& sg : segs) {
            seg_page.push_back(sg.page);
            seg_lo.push_back(sg.lo);
            seg_hi.push_back(sg.hi);
            seg_thr.push_back(sg.thr);
            seg_causal.push_back(sg.causal);
        }
        seg_ptr.push_back((int32_t)seg_page.size());
    }
    return OCTOPUS_OK;
}

}  // namespace octo
