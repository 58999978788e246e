// Host-side check of the graph build (loops and repeats dropped, one self-loop
// per node, rows sorted, CSC the exact transpose, degree order) against
// adjacency sets, built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_host_sanitizers.py.  Host code only: no GPU call is made.
#include <cstdio>
#include <random>
#include <set>
#include "internal.h"
namespace gnnmp {
gnn_status_t fail(gnn_status_t s, const std::string& msg) { std::fprintf(stderr, "fail: %s\n", msg.c_str()); return s; }
}
using namespace gnnmp;
int main() {
    std::mt19937 rng(1);
    int bad = 0;
    for (int trial = 0; trial < 120; ++trial) {
        int64_t n = trial < 5 ? trial : 1 + rng() % (trial < 117 ? 300 : 150000);
        int64_t m = n ? rng() % (8 * n + 1) : 0;
        bool sym = trial & 1, csc = trial & 2;
        std::vector<int32_t> s(m), d(m);
        for (int64_t i = 0; i < m; ++i) {
            // skewed ids, loops and repeats
            s[i] = int32_t(rng() % n); d[i] = int32_t((rng() % 4 == 0) ? s[i] : (rng() % 3 == 0 ? 0 : rng() % n));
        }
        HostGraph hg;
        if (build_host_graph(n, m, s.data(), d.data(), sym, csc, hg) != GNN_OK) { ++bad; continue; }
        // check against sets
        std::vector<std::set<int32_t>> adj(n);
        for (int64_t i = 0; i < m; ++i) if (s[i] != d[i]) { adj[d[i]].insert(s[i]); if (sym) adj[s[i]].insert(d[i]); }
        for (int64_t v = 0; v < n; ++v) adj[v].insert(int32_t(v));
        for (int64_t v = 0; v < n; ++v) {
            std::vector<int32_t> row(hg.col.begin() + hg.row_ptr[v], hg.col.begin() + hg.row_ptr[v + 1]);
            if (std::vector<int32_t>(adj[v].begin(), adj[v].end()) != row) { ++bad; break; }
        }
        if (csc) {
            for (int64_t u = 0; u < n; ++u)
                for (int64_t p = hg.col_ptr[u]; p < hg.col_ptr[u + 1]; ++p)
                    if (hg.col[hg.csc_eid[p]] != u) ++bad;
        }
        std::vector<int32_t> order;
        degree_order(hg.row_ptr, order);
        for (int64_t i = 1; i < n; ++i) {
            int64_t a = hg.row_ptr[order[i - 1] + 1] - hg.row_ptr[order[i - 1]], b = hg.row_ptr[order[i] + 1] - hg.row_ptr[order[i]];
            if (a < b || (a == b && order[i - 1] > order[i])) { ++bad; break; }
        }
    }
    // out-of-range ids are refused
    int32_t s2[2] = {0, 5}, d2[2] = {1, 0};
    HostGraph hg2;
    if (build_host_graph(3, 2, s2, d2, false, false, hg2) != GNN_ERR_INVALID_ARG) ++bad;
    int32_t s3[1] = {-1}, d3[1] = {0};
    if (build_host_graph(3, 1, s3, d3, true, true, hg2) != GNN_ERR_INVALID_ARG) ++bad;
    std::printf("bad=%d\n", bad);
    return bad != 0;
}
