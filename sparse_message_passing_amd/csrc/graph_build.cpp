// graph_build.cpp -- host construction of the graph views.
//
// Sancus (IJCAI'23 extended abstract), Sec. 2 Preliminaries: Abar = A + I and
// Dbar = D + I, so every node carries one self-connection that its degree
// counts; Tango (SC'23), datasets paragraph: reverse edges and self-loops are
// added so the aggregation reaches every node.  Input self-loops and repeated
// edges are dropped before one self-loop per node is added.
//
// Counting sort by destination, then a sort + unique inside each row (rows
// are independent, so they are processed by a pool of host threads).

#include <algorithm>
#include <cmath>
#include <thread>

#include "internal.h"

namespace gnnmp {

namespace {

template <typename F>
void parallel_rows(int64_t n, F&& f) {
    unsigned hw = std::max(1u, std::min(32u, std::thread::hardware_concurrency()));
    if (n < 65536 || hw == 1) {
        f(0, n);
        return;
    }
    std::vector<std::thread> pool;
    int64_t step = (n + hw - 1) / hw;
    for (unsigned t = 0; t < hw; ++t) {
        int64_t b = t * step, e = std::min(n, b + step);
        if (b >= e) break;
        pool.emplace_back([&f, b, e] { f(b, e); });
    }
    for (auto& th : pool) th.join();
}

}  // namespace

gnn_status_t build_host_graph(int64_t n, int64_t m, const int32_t* src, const int32_t* dst, bool symmetrize,
                              bool csc, HostGraph& out) {
    out.n = n;
    // 1. in-degree of the directed edge list (loops dropped, reverse edges added)
    std::vector<int64_t> cnt(n + 1, 0);
    for (int64_t i = 0; i < m; ++i) {
        int32_t u = src[i], v = dst[i];
        if (u < 0 || u >= n || v < 0 || v >= n) return fail(GNN_ERR_INVALID_ARG, "gnn_graph_create: node id out of range");
        if (u == v) continue;
        cnt[v + 1]++;
        if (symmetrize) cnt[u + 1]++;
    }
    for (int64_t v = 0; v < n; ++v) cnt[v + 1] += cnt[v];
    const int64_t raw = cnt[n];
    // 2. scatter sources into their destination's bucket
    std::vector<int32_t> buf(static_cast<size_t>(raw));
    {
        std::vector<int64_t> cur(cnt.begin(), cnt.end() - 1);
        for (int64_t i = 0; i < m; ++i) {
            int32_t u = src[i], v = dst[i];
            if (u == v) continue;
            buf[cur[v]++] = u;
            if (symmetrize) buf[cur[u]++] = v;
        }
    }
    // 3. per row: sort, unique, count the self-loop
    std::vector<int64_t> len(n);
    parallel_rows(n, [&](int64_t b, int64_t e) {
        for (int64_t v = b; v < e; ++v) {
            auto first = buf.begin() + cnt[v], last = buf.begin() + cnt[v + 1];
            std::sort(first, last);
            auto uend = std::unique(first, last);
            len[v] = (uend - first) + 1;  // + self-loop (input loops were dropped)
        }
    });
    out.row_ptr.assign(n + 1, 0);
    for (int64_t v = 0; v < n; ++v) out.row_ptr[v + 1] = out.row_ptr[v] + len[v];
    const int64_t nnz = out.row_ptr[n];
    if (nnz >= (int64_t(1) << 31)) return fail(GNN_ERR_UNSUPPORTED, "gnn_graph_create: nnz must stay below 2^31");
    out.col.resize(static_cast<size_t>(nnz));
    parallel_rows(n, [&](int64_t b, int64_t e) {
        for (int64_t v = b; v < e; ++v) {
            const int32_t* s = buf.data() + cnt[v];
            int64_t k = len[v] - 1;  // distinct non-loop sources, sorted
            int32_t* o = out.col.data() + out.row_ptr[v];
            int64_t i = 0;
            while (i < k && s[i] < v) *o++ = s[i++];
            *o++ = static_cast<int32_t>(v);
            while (i < k) *o++ = s[i++];
        }
    });
    buf.clear();
    buf.shrink_to_fit();
    // 4. dinv = 1/sqrt(row length), binary32, correctly rounded
    out.dinv.resize(n);
    for (int64_t v = 0; v < n; ++v) {
        float dbar = static_cast<float>(out.row_ptr[v + 1] - out.row_ptr[v]);
        out.dinv[v] = 1.0f / std::sqrt(dbar);
    }
    // 5. transposed view: column u lists destinations ascending, eid = CSR slot
    if (csc) {
        out.col_ptr.assign(n + 1, 0);
        for (int64_t e = 0; e < nnz; ++e) out.col_ptr[out.col[e] + 1]++;
        for (int64_t u = 0; u < n; ++u) out.col_ptr[u + 1] += out.col_ptr[u];
        out.csc_row.resize(nnz);
        out.csc_eid.resize(nnz);
        std::vector<int64_t> cur(out.col_ptr.begin(), out.col_ptr.end() - 1);
        for (int64_t v = 0; v < n; ++v)
            for (int64_t e = out.row_ptr[v]; e < out.row_ptr[v + 1]; ++e) {
                int64_t p = cur[out.col[e]]++;
                out.csc_row[p] = static_cast<int32_t>(v);
                out.csc_eid[p] = static_cast<int32_t>(e);
            }
    }
    return GNN_OK;
}

// Rows by degree descending, ties by id ascending (a stable counting sort).
void degree_order(const std::vector<int64_t>& ptr, std::vector<int32_t>& order) {
    const int64_t n = static_cast<int64_t>(ptr.size()) - 1;
    order.resize(n);
    int64_t maxd = 0;
    for (int64_t v = 0; v < n; ++v) maxd = std::max(maxd, ptr[v + 1] - ptr[v]);
    std::vector<int64_t> start(maxd + 2, 0);
    for (int64_t v = 0; v < n; ++v) start[maxd - (ptr[v + 1] - ptr[v]) + 1]++;
    for (int64_t i = 0; i <= maxd; ++i) start[i + 1] += start[i];
    for (int64_t v = 0; v < n; ++v) order[start[maxd - (ptr[v + 1] - ptr[v])]++] = static_cast<int32_t>(v);
}

}  // namespace gnnmp
