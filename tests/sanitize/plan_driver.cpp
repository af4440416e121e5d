// Host planner driver for the AddressSanitizer / UndefinedBehaviorSanitizer test.
//
// Built with g++ and the sanitizers together with the planner's own source (no GPU code
// and no HIP runtime calls are involved).  Reads cases from stdin, one after another:
//
//   T nb nm
//   nb lines: parent fork start len
//   nm lines: reader rpos producer s e
//   page_size n_pages
//   nb + 1 values: page_ptr
//   page_ptr[nb] values: pages
//   n_cursors, then n_cursors cursor branch ids, then n_cursors new-token counts
//
// and runs on each the tile planner (all rows of the mask expanded from the tile
// lists), the decode segment builder with and without shared lists, and the extend
// segment builder.  Prints one line per case: the planner's return code, its nnz and
// the popcount of the expanded mask (equal when the plan is valid), and the segment
// builders' return codes.  Errors in the tables are expected (they come back as return
// codes); the sanitizers abort the process on any memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "plan.h"

namespace {

bool read_ints(std::vector<int32_t>& v, size_t n) {
    v.assign(n, 0);
    for (size_t i = 0; i < n; ++i)
        if (std::scanf("%d", &v[i]) != 1) return false;
    return true;
}

}  // namespace

int main() {
    int T, nb, nm;
    int n_case = 0;
    while (std::scanf("%d %d %d", &T, &nb, &nm) == 3) {
        std::vector<int32_t> b, m, pp, pg, cur, nnew;
        if (nb < 0 || nm < 0 || !read_ints(b, 4 * (size_t)nb) || !read_ints(m, 5 * (size_t)nm))
            return 2;
        int page_size, n_pages, n_cur;
        if (std::scanf("%d %d", &page_size, &n_pages) != 2) return 2;
        if (!read_ints(pp, (size_t)nb + 1)) return 2;
        if (pp[nb] < 0 || !read_ints(pg, (size_t)pp[nb])) return 2;
        if (std::scanf("%d", &n_cur) != 1 || n_cur < 0) return 2;
        if (!read_ints(cur, (size_t)n_cur) || !read_ints(nnew, (size_t)n_cur)) return 2;

        std::vector<octopus_branch> br((size_t)nb);
        for (int i = 0; i < nb; ++i) br[i] = {b[4 * i], b[4 * i + 1], b[4 * i + 2], b[4 * i + 3]};
        std::vector<octopus_mount> mt((size_t)nm);
        for (int i = 0; i < nm; ++i)
            mt[i] = {m[5 * i], m[5 * i + 1], m[5 * i + 2], m[5 * i + 3], m[5 * i + 4]};

        octo::Plan plan;
        std::string err;
        const int rc = octo::build_plan(br.data(), nb, mt.data(), nm, T, 64, plan, err);
        long long pop = 0;
        if (rc == OCTOPUS_OK) {
            const int words = (T + 7) / 8;
            std::vector<uint8_t> bits;
            for (int lo = 0; lo < T; lo += 256) {
                const int hi = lo + 256 < T ? lo + 256 : T;
                bits.assign((size_t)(hi - lo) * words, 0);
                octo::export_mask(plan, lo, hi, bits.data());
                for (uint8_t x : bits) pop += __builtin_popcount(x);
            }
        }
        int rs0 = 0, rs1 = 0, rx = 0;
        if (rc == OCTOPUS_OK) {
            std::vector<int32_t> sp, spg, slo, shi, gp, gc, thr, causal, first;
            rs0 = octo::build_segments(plan.dag, pp.data(), pg.data(), page_size, n_pages,
                                       cur.data(), n_cur, false, sp, spg, slo, shi, gp, gc, err);
            rs1 = octo::build_segments(plan.dag, pp.data(), pg.data(), page_size, n_pages,
                                       cur.data(), n_cur, true, sp, spg, slo, shi, gp, gc, err);
            rx = octo::build_extend_segments(plan.dag, pp.data(), pg.data(), page_size, n_pages,
                                             cur.data(), n_cur, nnew.data(), sp, spg, slo, shi,
                                             thr, causal, first, err);
        }
        // The device image, written into a buffer of exactly its size: its tile lists and
        // positions must equal the plan's own.
        int img = 0;
        if (rc == OCTOPUS_OK) {
            std::vector<unsigned char> im(plan.layout.total);
            octo::write_device_image(plan, im.data());
            const size_t qb = plan.q_pairs.size() * sizeof(octo::TilePair);
            bool same = qb == 0 || std::memcmp(im.data() + plan.layout.q_pairs,
                                               plan.q_pairs.data(), qb) == 0;
            const int32_t* pos = reinterpret_cast<const int32_t*>(im.data() + plan.layout.pos);
            for (int i = 0; i < T && same; ++i) same = pos[i] == (int32_t)plan.dag.pos[i];
            img = same ? 1 : 2;
        }
        std::printf("case %d rc %d nnz %lld pop %lld seg %d %d ext %d img %d\n", n_case, rc,
                    (long long)plan.nnz, pop, rs0, rs1, rx, img);
        ++n_case;
    }
    return 0;
}
