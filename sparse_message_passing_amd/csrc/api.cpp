// api.cpp -- the C ABI: errors, graph handles, argument checks and dispatch
// of the primitives.  Every check runs before anything is launched.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "internal.h"

namespace gnnmp {

namespace {
thread_local std::string g_last_error = "no error";
}

const char* last_error_cstr() { return g_last_error.c_str(); }

void set_error(const std::string& msg) { g_last_error = msg; }

gnn_status_t fail(gnn_status_t s, const std::string& msg) {
    set_error(msg);
    return s;
}

gnn_status_t hip_fail(hipError_t e, const char* what) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return e == hipErrorOutOfMemory ? GNN_ERR_OUT_OF_MEMORY : GNN_ERR_HIP;
}

gnn_status_t launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, what);
    return GNN_OK;
}

AggView csr_view(const Graph& g) { return AggView{g.n, g.row_ptr, g.col, nullptr, &g.plan[0], g.wgcn, g.dmean}; }
AggView csc_view(const Graph& g) {
    return AggView{g.n, g.col_ptr, g.csc_row, g.csc_eid, &g.plan[1], nullptr, g.dmean};
}

namespace {

template <typename T>
gnn_status_t upload(Graph& g, const std::vector<T>& h, T** out) {
    *out = nullptr;
    if (h.empty()) return GNN_OK;
    // the slot exists before the allocation, so a failed push_back cannot
    // leak device memory (free_graph frees every recorded slot; null is fine)
    g.allocations.push_back(nullptr);
    void*& p = g.allocations.back();
    GNN_HIP(hipMalloc(&p, h.size() * sizeof(T)));
    GNN_HIP(hipMemcpy(p, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    *out = static_cast<T*>(p);
    return GNN_OK;
}

gnn_status_t make_plan(Graph& g, const std::vector<int64_t>& ptr, RowPlan& p, std::vector<int32_t>* order_out,
                       int64_t chunk) {
    std::vector<int32_t> order;
    degree_order(ptr, order);
    const int64_t n = static_cast<int64_t>(order.size());
    auto deg = [&](int64_t v) { return ptr[v + 1] - ptr[v]; };
    p.max_degree = n ? deg(order[0]) : 0;
    p.chunk = chunk;
    p.n_heavy = 0;
    while (p.n_heavy < n && deg(order[p.n_heavy]) > chunk) ++p.n_heavy;
    p.n_block = 0;
    while (p.n_block < n && deg(order[p.n_block]) > kBlockRow) ++p.n_block;
    std::vector<int32_t> chunk_first(p.n_heavy + 1, 0), chunk_row;
    for (int64_t i = 0; i < p.n_heavy; ++i) {
        const int64_t c = (deg(order[i]) + chunk - 1) / chunk;
        chunk_first[i + 1] = chunk_first[i] + static_cast<int32_t>(c);
        for (int64_t j = 0; j < c; ++j) chunk_row.push_back(static_cast<int32_t>(i));
    }
    p.n_chunks = static_cast<int64_t>(chunk_row.size());
    GNN_TRY(upload(g, order, &p.order));
    GNN_TRY(upload(g, chunk_first, &p.chunk_first));
    GNN_TRY(upload(g, chunk_row, &p.chunk_row));
    if (order_out) *order_out = std::move(order);
    return GNN_OK;
}

// Offsets of the degree buckets in the degree-ordered row list: rows of
// degree > kBlockRow, then > the view's chunk length, then the rest:
// {0, n_block, n_heavy, n}.
void bucket_offsets(const RowPlan& p, int64_t n, int64_t* off) {
    off[0] = 0;
    off[1] = p.n_block;
    off[2] = p.n_heavy;
    off[3] = n;
}

void free_graph(Graph& g) {
    for (void* p : g.allocations) (void)hipFree(p);
    g.allocations.clear();
}

bool bad_dt(gnn_dtype_t t) { return t != GNN_F32 && t != GNN_BF16; }

gnn_status_t check_graph(const gnn_graph* g, const char* what) {
    if (!g) return fail(GNN_ERR_INVALID_ARG, std::string(what) + ": graph handle is NULL");
    return GNN_OK;
}

}  // namespace
}  // namespace gnnmp

using namespace gnnmp;

extern "C" {

const char* gnn_status_string(gnn_status_t s) {
    switch (s) {
        case GNN_OK: return "ok";
        case GNN_ERR_INVALID_ARG: return "invalid argument";
        case GNN_ERR_UNSUPPORTED: return "unsupported";
        case GNN_ERR_OUT_OF_MEMORY: return "out of memory";
        case GNN_ERR_HIP: return "HIP error";
        case GNN_ERR_GRAPH: return "graph lacks the required view";
        case GNN_ERR_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

const char* gnn_last_error(void) { return last_error_cstr(); }

// ---------------------------------------------------------------------------
// graph
// ---------------------------------------------------------------------------
gnn_status_t gnn_graph_create(int64_t n, int64_t m, const int32_t* src, const int32_t* dst, uint32_t flags,
                              gnn_graph_t* out) {
    GNN_REQUIRE(out, "gnn_graph_create: out is NULL");
    *out = nullptr;
    GNN_REQUIRE(n >= 0 && n < (int64_t(1) << 31), "gnn_graph_create: n must be in [0, 2^31)");
    GNN_REQUIRE(m >= 0, "gnn_graph_create: m must be >= 0");
    GNN_REQUIRE(m == 0 || (src && dst), "gnn_graph_create: src/dst are NULL");
    GNN_REQUIRE((flags & ~(GNN_GRAPH_SYMMETRIZE | GNN_GRAPH_CSC)) == 0, "gnn_graph_create: unknown flag bits");
    gnn_graph* h = new (std::nothrow) gnn_graph();
    if (!h) return fail(GNN_ERR_OUT_OF_MEMORY, "gnn_graph_create: host allocation failed");
    Graph& g = h->g;
    gnn_status_t s = GNN_OK;
    try {
        HostGraph hg;
        s = build_host_graph(n, m, src, dst, (flags & GNN_GRAPH_SYMMETRIZE) != 0, (flags & GNN_GRAPH_CSC) != 0, hg);
        if (s == GNN_OK) {
            g.n = n;
            g.nnz = n ? hg.row_ptr[n] : 0;
            g.has_csc = (flags & GNN_GRAPH_CSC) != 0;
            g.symmetric = (flags & GNN_GRAPH_SYMMETRIZE) != 0;
            s = upload(g, hg.row_ptr, &g.row_ptr);
            if (s == GNN_OK) s = upload(g, hg.col, &g.col);
            if (s == GNN_OK) s = upload(g, hg.dinv, &g.dinv);
            if (s == GNN_OK) {
                // GCN edge weights dinv[src] * dinv[dst] (binary32 product), CSR order
                std::vector<float> w(static_cast<size_t>(g.nnz));
                for (int64_t v = 0; v < n; ++v)
                    for (int64_t e = hg.row_ptr[v]; e < hg.row_ptr[v + 1]; ++e) w[e] = hg.dinv[hg.col[e]] * hg.dinv[v];
                s = upload(g, w, &g.wgcn);
            }
            if (s == GNN_OK) {
                std::vector<float> dm(static_cast<size_t>(n));
                for (int64_t v = 0; v < n; ++v)
                    dm[v] = 1.0f / static_cast<float>(hg.row_ptr[v + 1] - hg.row_ptr[v]);
                s = upload(g, dm, &g.dmean);
            }
            if (s == GNN_OK) s = make_plan(g, hg.row_ptr, g.plan[0], nullptr, kChunkCsr);
            if (s == GNN_OK && g.has_csc) {
                s = upload(g, hg.col_ptr, &g.col_ptr);
                if (s == GNN_OK) s = upload(g, hg.csc_row, &g.csc_row);
                if (s == GNN_OK) s = upload(g, hg.csc_eid, &g.csc_eid);
                if (s == GNN_OK) {
                    std::vector<int32_t> cpos(hg.csc_eid.size());
                    for (size_t j = 0; j < cpos.size(); ++j) cpos[hg.csc_eid[j]] = static_cast<int32_t>(j);
                    s = upload(g, cpos, &g.csr_cpos);
                }
                if (s == GNN_OK) s = make_plan(g, hg.col_ptr, g.plan[1], nullptr, kChunkCsc);
            }
        }
    } catch (const std::bad_alloc&) {
        s = fail(GNN_ERR_OUT_OF_MEMORY, "gnn_graph_create: host allocation failed");
    }
    if (s != GNN_OK) {
        free_graph(g);
        delete h;
        return s;
    }
    *out = h;
    return GNN_OK;
}

gnn_status_t gnn_graph_split(gnn_graph_t h, const uint8_t* marginal, gnn_graph_t* local, gnn_graph_t* remote) {
    GNN_TRY(check_graph(h, "gnn_graph_split"));
    GNN_REQUIRE(local && remote, "gnn_graph_split: local or remote is NULL");
    *local = *remote = nullptr;
    const Graph& g = h->g;
    GNN_REQUIRE(g.n == 0 || marginal, "gnn_graph_split: marginal is NULL");
    const size_t n = static_cast<size_t>(g.n), e = static_cast<size_t>(g.nnz);
    gnn_graph* parts[2] = {nullptr, nullptr};
    gnn_status_t s = GNN_OK;
    try {
        std::vector<int64_t> rp(n + 1, 0);
        std::vector<int32_t> col(e);
        std::vector<float> dinv(n), dmean(n), w(e);
        if (n) GNN_HIP(hipMemcpy(rp.data(), g.row_ptr, (n + 1) * 8, hipMemcpyDeviceToHost));
        if (e) {
            GNN_HIP(hipMemcpy(col.data(), g.col, e * 4, hipMemcpyDeviceToHost));
            GNN_HIP(hipMemcpy(w.data(), g.wgcn, e * 4, hipMemcpyDeviceToHost));
        }
        if (n) GNN_HIP(hipMemcpy(dinv.data(), g.dinv, n * 4, hipMemcpyDeviceToHost));
        if (n) GNN_HIP(hipMemcpy(dmean.data(), g.dmean, n * 4, hipMemcpyDeviceToHost));
        for (int k = 0; k < 2 && s == GNN_OK; ++k) {
            // k = 0: in-edges from sources that are not marginal; k = 1: from marginal ones.
            // Each row keeps its edges in CSR order and each edge its weight in g.
            std::vector<int64_t> prp(n + 1, 0);
            std::vector<int32_t> pcol;
            std::vector<float> pw;
            for (size_t v = 0; v < n; ++v) {
                for (int64_t i = rp[v]; i < rp[v + 1]; ++i) {
                    const bool m = marginal[col[i]] != 0;
                    if (m == (k == 1)) {
                        pcol.push_back(col[i]);
                        pw.push_back(w[i]);
                    }
                }
                prp[v + 1] = static_cast<int64_t>(pcol.size());
            }
            gnn_graph* ph = new (std::nothrow) gnn_graph();
            if (!ph) {
                s = fail(GNN_ERR_OUT_OF_MEMORY, "gnn_graph_split: host allocation failed");
                break;
            }
            parts[k] = ph;
            Graph& pg = ph->g;
            pg.n = g.n;
            pg.nnz = static_cast<int64_t>(pcol.size());
            pg.has_csc = false;
            s = upload(pg, prp, &pg.row_ptr);
            if (s == GNN_OK) s = upload(pg, pcol, &pg.col);
            if (s == GNN_OK) s = upload(pg, dinv, &pg.dinv);
            if (s == GNN_OK) s = upload(pg, pw, &pg.wgcn);
            if (s == GNN_OK) s = upload(pg, dmean, &pg.dmean);
            if (s == GNN_OK) s = make_plan(pg, prp, pg.plan[0], nullptr, kChunkCsr);
        }
    } catch (const std::bad_alloc&) {
        s = fail(GNN_ERR_OUT_OF_MEMORY, "gnn_graph_split: host allocation failed");
    }
    if (s != GNN_OK) {
        for (gnn_graph* ph : parts)
            if (ph) {
                free_graph(ph->g);
                delete ph;
            }
        return s;
    }
    *local = parts[0];
    *remote = parts[1];
    return GNN_OK;
}

gnn_status_t gnn_graph_destroy(gnn_graph_t h) {
    if (!h) return GNN_OK;
    free_graph(h->g);
    delete h;
    return GNN_OK;
}

gnn_status_t gnn_graph_info(gnn_graph_t h, gnn_graph_info_t* out) {
    GNN_TRY(check_graph(h, "gnn_graph_info"));
    GNN_REQUIRE(out, "gnn_graph_info: out is NULL");
    const Graph& g = h->g;
    std::memset(out, 0, sizeof(*out));
    out->n = g.n;
    out->nnz = g.nnz;
    out->max_in_degree = g.plan[0].max_degree;
    out->max_out_degree = g.has_csc ? g.plan[1].max_degree : 0;
    out->has_csc = g.has_csc;
    out->row_ptr = g.row_ptr;
    out->col = g.col;
    out->dinv = g.dinv;
    out->perm = g.plan[0].order;
    out->col_ptr = g.col_ptr;
    out->csc_row = g.csc_row;
    out->csc_eid = g.csc_eid;
    out->perm_t = g.plan[1].order;
    out->symmetric = g.symmetric;
    out->bucket_threshold[0] = kBlockRow;
    out->bucket_threshold[1] = g.plan[0].chunk;
    out->bucket_threshold_t[0] = g.has_csc ? kBlockRow : 0;
    out->bucket_threshold_t[1] = g.has_csc ? g.plan[1].chunk : 0;
    bucket_offsets(g.plan[0], g.n, out->bucket_off);
    if (g.has_csc) bucket_offsets(g.plan[1], g.n, out->bucket_off_t);
    return GNN_OK;
}

gnn_status_t gnn_graph_export(gnn_graph_t h, int64_t* row_ptr, int32_t* col, float* dinv, float* w, int32_t* perm,
                              int64_t* bucket_off, int64_t* col_ptr, int32_t* csc_row, int32_t* csc_eid,
                              int32_t* perm_t, int64_t* bucket_off_t) {
    GNN_TRY(check_graph(h, "gnn_graph_export"));
    const Graph& g = h->g;
    if (!g.has_csc && (col_ptr || csc_row || csc_eid || perm_t || bucket_off_t))
        return fail(GNN_ERR_GRAPH, "gnn_graph_export: the graph has no CSC view");
    if (bucket_off) bucket_offsets(g.plan[0], g.n, bucket_off);
    if (bucket_off_t) bucket_offsets(g.plan[1], g.n, bucket_off_t);
    const size_t n1 = static_cast<size_t>(g.n + 1), n = static_cast<size_t>(g.n), e = static_cast<size_t>(g.nnz);
    if (row_ptr && g.row_ptr) GNN_HIP(hipMemcpy(row_ptr, g.row_ptr, n1 * 8, hipMemcpyDeviceToHost));
    if (col && e) GNN_HIP(hipMemcpy(col, g.col, e * 4, hipMemcpyDeviceToHost));
    if (dinv && n) GNN_HIP(hipMemcpy(dinv, g.dinv, n * 4, hipMemcpyDeviceToHost));
    if (perm && n) GNN_HIP(hipMemcpy(perm, g.plan[0].order, n * 4, hipMemcpyDeviceToHost));
    if (col_ptr && g.col_ptr) GNN_HIP(hipMemcpy(col_ptr, g.col_ptr, n1 * 8, hipMemcpyDeviceToHost));
    if (csc_row && e) GNN_HIP(hipMemcpy(csc_row, g.csc_row, e * 4, hipMemcpyDeviceToHost));
    if (csc_eid && e) GNN_HIP(hipMemcpy(csc_eid, g.csc_eid, e * 4, hipMemcpyDeviceToHost));
    if (perm_t && n) GNN_HIP(hipMemcpy(perm_t, g.plan[1].order, n * 4, hipMemcpyDeviceToHost));
    if (w && e) {
        std::vector<int64_t> rp(n1);
        std::vector<int32_t> c(e);
        std::vector<float> di(n);
        GNN_HIP(hipMemcpy(rp.data(), g.row_ptr, n1 * 8, hipMemcpyDeviceToHost));
        GNN_HIP(hipMemcpy(c.data(), g.col, e * 4, hipMemcpyDeviceToHost));
        GNN_HIP(hipMemcpy(di.data(), g.dinv, n * 4, hipMemcpyDeviceToHost));
        for (size_t v = 0; v < n; ++v)
            for (int64_t k = rp[v]; k < rp[v + 1]; ++k) w[k] = di[c[k]] * di[v];
    }
    return GNN_OK;
}

// ---------------------------------------------------------------------------
// primitives
// ---------------------------------------------------------------------------
size_t gnn_spmm_workspace_size(gnn_graph_t h, int transpose, int64_t d) {
    if (!h || d <= 0) return 0;
    const Graph& g = h->g;
    if (transpose && !g.has_csc) return 0;
    return spmm_partial_bytes(g.plan[transpose ? 1 : 0], d);
}

gnn_status_t gnn_spmm(gnn_graph_t h, int transpose, gnn_weights_t wmode, const float* edge_w, int heads,
                      const void* X, gnn_dtype_t x_dt, int64_t ldx, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                      int64_t d, int relu, void* ws, size_t ws_bytes, void* stream) {
    GNN_TRY(check_graph(h, "gnn_spmm"));
    const Graph& g = h->g;
    GNN_REQUIRE(d >= 1, "gnn_spmm: d must be >= 1");
    GNN_REQUIRE(ldx >= d && ldy >= d, "gnn_spmm: leading dimensions must be >= d");
    GNN_REQUIRE(heads >= 1 && d % heads == 0, "gnn_spmm: heads must divide d");
    GNN_REQUIRE(!bad_dt(x_dt) && !bad_dt(y_dt), "gnn_spmm: unknown dtype");
    GNN_REQUIRE(wmode == GNN_W_GCN || wmode == GNN_W_ONES || wmode == GNN_W_EDGE || wmode == GNN_W_MEAN,
                "gnn_spmm: unknown weight mode");
    GNN_REQUIRE((wmode != GNN_W_GCN && wmode != GNN_W_MEAN) || heads == 1,
                "gnn_spmm: GCN and mean weights need heads == 1");
    GNN_REQUIRE(wmode != GNN_W_EDGE || edge_w, "gnn_spmm: edge_w is NULL");
    GNN_REQUIRE(relu == 0 || relu == 1, "gnn_spmm: relu must be 0 or 1");
    GNN_REQUIRE(g.n == 0 || (X && Y), "gnn_spmm: X or Y is NULL");
    GNN_REQUIRE(g.n == 0 || X != Y, "gnn_spmm: X and Y must not overlap");
    if (transpose && !g.has_csc) return fail(GNN_ERR_GRAPH, "gnn_spmm: transpose needs the CSC view");
    const RowPlan& p = g.plan[transpose ? 1 : 0];
    const size_t need = spmm_partial_bytes(p, d);
    if (need && (!ws || ws_bytes < need)) return fail(GNN_ERR_WORKSPACE, "gnn_spmm: workspace too small");
    return launch_spmm(transpose ? csc_view(g) : csr_view(g), g.dinv, wmode, edge_w, heads, X, x_dt, ldx, Y, y_dt,
                       ldy, d, relu, Rank1Epilogue{}, static_cast<float*>(ws), static_cast<hipStream_t>(stream));
}

size_t gnn_spmm_noalloc_max_scratch(void) { return kSpmmScratchBytes; }

gnn_status_t gnn_spmm_noalloc(gnn_graph_t h, int transpose, gnn_weights_t wmode, const float* edge_w, int heads,
                              const void* X, gnn_dtype_t x_dt, int64_t ldx, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                              int64_t d, int relu, void* stream) {
    GNN_TRY(check_graph(h, "gnn_spmm_noalloc"));
    const Graph& g = h->g;
    if (transpose && !g.has_csc) return fail(GNN_ERR_GRAPH, "gnn_spmm_noalloc: transpose needs the CSC view");
    GNN_REQUIRE(d >= 1, "gnn_spmm_noalloc: d must be >= 1");
    const size_t need = spmm_partial_bytes(g.plan[transpose ? 1 : 0], d);
    if (need > kSpmmScratchBytes)
        return fail(GNN_ERR_UNSUPPORTED, "gnn_spmm_noalloc: the hub-row partials need " + std::to_string(need) +
                                             " bytes, more than its " + std::to_string(kSpmmScratchBytes) +
                                             "-byte device scratch; use gnn_spmm with a workspace");
    void* ws = nullptr;
    GNN_TRY(spmm_noalloc_scratch(&ws));
    // the same checks and kernels as gnn_spmm, with the scratch as its workspace
    return gnn_spmm(h, transpose, wmode, edge_w, heads, X, x_dt, ldx, Y, y_dt, ldy, d, relu, ws, kSpmmScratchBytes,
                    stream);
}

gnn_status_t gnn_edge_reduce(gnn_graph_t h, int by_src, const float* vals, int heads, float* out, void* stream) {
    GNN_TRY(check_graph(h, "gnn_edge_reduce"));
    const Graph& g = h->g;
    GNN_REQUIRE(heads >= 1, "gnn_edge_reduce: heads must be >= 1");
    GNN_REQUIRE(g.n == 0 || (vals && out), "gnn_edge_reduce: NULL pointer");
    if (by_src && !g.has_csc) return fail(GNN_ERR_GRAPH, "gnn_edge_reduce: out-edge sums need the CSC view");
    return launch_edge_reduce(by_src ? csc_view(g) : csr_view(g), vals, heads, out,
                              static_cast<hipStream_t>(stream));
}

gnn_status_t gnn_sddmm(gnn_graph_t h, int op, const void* src_feat, int64_t ld_src, const void* dst_feat,
                       int64_t ld_dst, gnn_dtype_t dt, int heads, int64_t d_head, float slope, float* out,
                       float* out_pre, void* stream) {
    GNN_TRY(check_graph(h, "gnn_sddmm"));
    const Graph& g = h->g;
    GNN_REQUIRE(op == 0 || op == 1, "gnn_sddmm: op must be 0 (add) or 1 (dot)");
    GNN_REQUIRE(heads >= 1 && d_head >= 1, "gnn_sddmm: heads and d_head must be >= 1");
    GNN_REQUIRE(!bad_dt(dt), "gnn_sddmm: unknown dtype");
    GNN_REQUIRE(g.n == 0 || (src_feat && dst_feat && out), "gnn_sddmm: NULL pointer");
    GNN_REQUIRE(ld_src >= heads * d_head && ld_dst >= heads * d_head, "gnn_sddmm: leading dimension too small");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (op == 0) {
        GNN_REQUIRE(d_head == 1, "gnn_sddmm(add): d_head must be 1 (one score per head)");
        GNN_REQUIRE(dt == GNN_F32, "gnn_sddmm(add): scores are f32");
        return launch_sddmm_add(csr_view(g), static_cast<const float*>(src_feat), ld_src,
                                static_cast<const float*>(dst_feat), ld_dst, heads, slope, out, out_pre, st);
    }
    GNN_REQUIRE(out_pre == nullptr, "gnn_sddmm(dot): out_pre must be NULL");
    return launch_sddmm_dot(csr_view(g), src_feat, ld_src, dst_feat, ld_dst, dt, heads, d_head, out, st);
}

gnn_status_t gnn_edge_softmax(gnn_graph_t h, const float* E, float* alpha, int heads, void* stream) {
    GNN_TRY(check_graph(h, "gnn_edge_softmax"));
    const Graph& g = h->g;
    GNN_REQUIRE(heads >= 1, "gnn_edge_softmax: heads must be >= 1");
    GNN_REQUIRE(g.n == 0 || (E && alpha), "gnn_edge_softmax: NULL pointer");
    return launch_edge_softmax(csr_view(g), E, alpha, heads, static_cast<hipStream_t>(stream));
}

gnn_status_t gnn_edge_softmax_bwd(gnn_graph_t h, const float* alpha, const float* dalpha, const float* lrelu_pre,
                                  float slope, float* dE, int heads, void* stream) {
    GNN_TRY(check_graph(h, "gnn_edge_softmax_bwd"));
    const Graph& g = h->g;
    GNN_REQUIRE(heads >= 1, "gnn_edge_softmax_bwd: heads must be >= 1");
    GNN_REQUIRE(g.n == 0 || (alpha && dalpha && dE), "gnn_edge_softmax_bwd: NULL pointer");
    return launch_edge_softmax_bwd(csr_view(g), alpha, dalpha, lrelu_pre, slope, dE, heads,
                                   static_cast<hipStream_t>(stream));
}

size_t gnn_gemm_workspace_size(int transA, int transB, int64_t M, int64_t N, int64_t K) {
    return gemm_ws_bytes(transA, transB, M, N, K);
}

gnn_status_t gnn_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, const void* A, gnn_dtype_t a_dt,
                      int64_t lda, const void* B, gnn_dtype_t b_dt, int64_t ldb, void* C, gnn_dtype_t c_dt,
                      int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
    GNN_REQUIRE(M >= 0 && N >= 0 && K >= 0, "gnn_gemm: negative size");
    GNN_REQUIRE(!bad_dt(a_dt) && !bad_dt(b_dt) && !bad_dt(c_dt), "gnn_gemm: unknown dtype");
    GNN_REQUIRE((transA == 0 || transA == 1) && (transB == 0 || transB == 1), "gnn_gemm: trans flags must be 0/1");
    GNN_REQUIRE(lda >= std::max<int64_t>(1, transA ? M : K), "gnn_gemm: lda too small");
    GNN_REQUIRE(ldb >= std::max<int64_t>(1, transB ? K : N), "gnn_gemm: ldb too small");
    GNN_REQUIRE(ldc >= std::max<int64_t>(1, N), "gnn_gemm: ldc too small");
    GNN_REQUIRE(M * N == 0 || C, "gnn_gemm: C is NULL");
    GNN_REQUIRE(M * N * K == 0 || (A && B), "gnn_gemm: A or B is NULL");
    return launch_gemm(transA, transB, M, N, K, A, a_dt, lda, B, b_dt, ldb, C, c_dt, ldc, ws, ws_bytes,
                       static_cast<hipStream_t>(stream));
}

size_t gnn_softmax_xent_workspace_size(int64_t n) { return n > 0 ? xent_ws_bytes(n) : 256; }

gnn_status_t gnn_softmax_xent(const float* logits, int64_t n, int64_t c, int64_t ld, const int32_t* labels,
                              float* loss, float* dlogits, int64_t ld_d, void* ws, size_t ws_bytes, void* stream) {
    GNN_REQUIRE(n >= 0 && c >= 1, "gnn_softmax_xent: need n >= 0, c >= 1");
    GNN_REQUIRE(ld >= c && (!dlogits || ld_d >= c), "gnn_softmax_xent: leading dimension too small");
    GNN_REQUIRE(loss && ws, "gnn_softmax_xent: loss or ws is NULL");
    GNN_REQUIRE(n == 0 || (logits && labels), "gnn_softmax_xent: NULL pointer");
    if (ws_bytes < gnn_softmax_xent_workspace_size(n))
        return fail(GNN_ERR_WORKSPACE, "gnn_softmax_xent: workspace too small");
    return launch_softmax_xent(logits, n, c, ld, labels, loss, dlogits, ld_d, static_cast<float*>(ws),
                               static_cast<hipStream_t>(stream));
}

gnn_status_t gnn_quantize(const float* H, int64_t ldh, int64_t d, const int32_t* rows, int64_t n_rows, int bits,
                          uint64_t seed, uint32_t stream_id, uint8_t* packed, float* scale, float* zero,
                          void* stream) {
    GNN_REQUIRE(bits == 2 || bits == 4 || bits == 8, "gnn_quantize: bits must be 2, 4 or 8");
    GNN_REQUIRE(d >= 1 && (d * bits) % 8 == 0, "gnn_quantize: d*bits must be a positive multiple of 8");
    GNN_REQUIRE(ldh >= d, "gnn_quantize: ldh must be >= d");
    GNN_REQUIRE(n_rows >= 0, "gnn_quantize: n_rows must be >= 0");
    GNN_REQUIRE(n_rows == 0 || (H && rows && packed && scale && zero), "gnn_quantize: NULL pointer");
    return launch_quantize(H, ldh, d, rows, n_rows, bits, seed, stream_id, packed, scale, zero,
                           static_cast<hipStream_t>(stream));
}

gnn_status_t gnn_dequantize(const uint8_t* packed, const float* scale, const float* zero, int64_t n_rows, int64_t d,
                            int bits, const int32_t* rows, float* H, int64_t ldh, void* stream) {
    GNN_REQUIRE(bits == 2 || bits == 4 || bits == 8, "gnn_dequantize: bits must be 2, 4 or 8");
    GNN_REQUIRE(d >= 1 && (d * bits) % 8 == 0, "gnn_dequantize: d*bits must be a positive multiple of 8");
    GNN_REQUIRE(ldh >= d, "gnn_dequantize: ldh must be >= d");
    GNN_REQUIRE(n_rows >= 0, "gnn_dequantize: n_rows must be >= 0");
    GNN_REQUIRE(n_rows == 0 || (H && rows && packed && scale && zero), "gnn_dequantize: NULL pointer");
    return launch_dequantize(packed, scale, zero, n_rows, d, bits, rows, H, ldh, static_cast<hipStream_t>(stream));
}

size_t gnn_gemm_q8_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return gemm_q8_ws_bytes(M, N, K);
}

gnn_status_t gnn_gemm_q8(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                         float* C, int64_t ldc, uint64_t seed, uint32_t stream_id, void* ws, size_t ws_bytes,
                         void* stream) {
    GNN_REQUIRE(M >= 0 && N >= 0 && K >= 0, "gnn_gemm_q8: sizes must be >= 0");
    GNN_REQUIRE(K <= 133000, "gnn_gemm_q8: K above 133,000 could overflow the int32 sums");
    GNN_REQUIRE(lda >= std::max<int64_t>(K, 1) && ldb >= std::max<int64_t>(N, 1) && ldc >= std::max<int64_t>(N, 1),
                "gnn_gemm_q8: leading dimensions too small");
    GNN_REQUIRE(M == 0 || N == 0 || (C && (K == 0 || (A && B))), "gnn_gemm_q8: NULL pointer");
    if (M == 0 || N == 0) return GNN_OK;
    const size_t need = gemm_q8_ws_bytes(M, N, K);
    if (!ws || ws_bytes < need) return fail(GNN_ERR_WORKSPACE, "gnn_gemm_q8: workspace too small");
    return launch_gemm_q8(M, N, K, A, lda, B, ldb, C, ldc, seed, stream_id, ws, static_cast<hipStream_t>(stream));
}

size_t gnn_sddmm_q8_workspace_size(gnn_graph_t h, int64_t d) {
    if (!h || d < 0) return 0;
    return sddmm_q8_ws_bytes(h->g.n, d);
}

gnn_status_t gnn_sddmm_q8(gnn_graph_t h, const float* src_feat, int64_t ld_src, const float* dst_feat,
                          int64_t ld_dst, int heads, int64_t d_head, uint64_t seed, uint32_t stream_id, float* out,
                          void* ws, size_t ws_bytes, void* stream) {
    GNN_TRY(check_graph(h, "gnn_sddmm_q8"));
    const Graph& g = h->g;
    GNN_REQUIRE(heads >= 1 && d_head >= 1, "gnn_sddmm_q8: heads and d_head must be >= 1");
    GNN_REQUIRE(sddmm_q8_supported(heads, d_head),
                "gnn_sddmm_q8: d_head must be 16 times a power of two (16 ... 256) and heads * d_head <= 1024");
    const int64_t d = heads * d_head;
    GNN_REQUIRE(ld_src >= d && ld_dst >= d, "gnn_sddmm_q8: leading dimension too small");
    GNN_REQUIRE(g.n == 0 || (src_feat && dst_feat && out), "gnn_sddmm_q8: NULL pointer");
    if (g.n == 0) return GNN_OK;
    const size_t need = sddmm_q8_ws_bytes(g.n, d);
    if (!ws || ws_bytes < need) return fail(GNN_ERR_WORKSPACE, "gnn_sddmm_q8: workspace too small");
    return launch_sddmm_q8(csr_view(g), src_feat, ld_src, dst_feat, ld_dst, heads, d_head, seed, stream_id, out, ws,
                           static_cast<hipStream_t>(stream));
}

gnn_status_t gnn_quant_stats(gnn_graph_t h, const float* edge_w, const float* H, int64_t ldh, int64_t d,
                             const int32_t* rows, int64_t n_rows, float* beta, float* range, void* stream) {
    GNN_TRY(check_graph(h, "gnn_quant_stats"));
    const Graph& g = h->g;
    GNN_REQUIRE(d >= 1 && ldh >= d, "gnn_quant_stats: need d >= 1 and ldh >= d");
    GNN_REQUIRE(n_rows >= 0, "gnn_quant_stats: n_rows must be >= 0");
    GNN_REQUIRE(n_rows == 0 || (H && rows && beta && range), "gnn_quant_stats: NULL pointer");
    const float* w = edge_w ? edge_w : g.wgcn;
    if (g.has_csc) return launch_quant_stats(csc_view(g), w, H, ldh, d, rows, n_rows, beta, range,
                                             static_cast<hipStream_t>(stream));
    return launch_quant_stats(csr_view(g), w, H, ldh, d, rows, n_rows, beta, range, static_cast<hipStream_t>(stream));
}

gnn_status_t gnn_assign_bits(int64_t m, const float* beta, int64_t d, double avg_bits, int32_t* bits) {
    GNN_REQUIRE(m >= 0 && d >= 1, "gnn_assign_bits: need m >= 0 and d >= 1");
    GNN_REQUIRE(m == 0 || (beta && bits), "gnn_assign_bits: NULL pointer");
    GNN_REQUIRE(avg_bits >= 2.0 && avg_bits <= 8.0, "gnn_assign_bits: avg_bits must be in [2, 8]");
    for (int64_t k = 0; k < m; ++k)
        GNN_REQUIRE(std::isfinite(beta[k]) && beta[k] >= 0.0f, "gnn_assign_bits: beta must be finite and >= 0");
    // budget in quarter-row units: a 2 -> 4 upgrade costs one (d/4 bytes), 4 -> 8 costs two
    const double extra_bytes = (avg_bits - 2.0) * static_cast<double>(m) * static_cast<double>(d) / 8.0;
    int64_t units = static_cast<int64_t>(std::floor(extra_bytes / (static_cast<double>(d) / 4.0) + 1e-9));
    // variance removed per quarter-row unit: beta (1/9 - 1/225) for 2 -> 4, beta (1/225 - 1/65025) / 2 for 4 -> 8
    const double g24 = 1.0 / 9.0 - 1.0 / 225.0, g48 = (1.0 / 225.0 - 1.0 / 65025.0) / 2.0;
    struct Cand {
        double gain;
        int64_t k;
        int stage;  // 0: 2 -> 4, 1: 4 -> 8
    };
    auto worse = [](const Cand& a, const Cand& b) { return a.gain < b.gain || (a.gain == b.gain && a.k > b.k); };
    std::vector<Cand> heap;
    heap.reserve(static_cast<size_t>(m));
    for (int64_t k = 0; k < m; ++k) {
        bits[k] = 2;
        heap.push_back(Cand{static_cast<double>(beta[k]) * g24, k, 0});
    }
    std::make_heap(heap.begin(), heap.end(), worse);
    while (!heap.empty() && units > 0) {
        std::pop_heap(heap.begin(), heap.end(), worse);
        const Cand c = heap.back();
        heap.pop_back();
        const int64_t cost = c.stage == 0 ? 1 : 2;
        if (cost > units) continue;
        units -= cost;
        if (c.stage == 0) {
            bits[c.k] = 4;
            heap.push_back(Cand{static_cast<double>(beta[c.k]) * g48, c.k, 1});
            std::push_heap(heap.begin(), heap.end(), worse);
        } else {
            bits[c.k] = 8;
        }
    }
    return GNN_OK;
}

gnn_status_t gnn_quant_slots(int64_t n, int n_groups, const int32_t* const* rows, const int64_t* counts,
                             int32_t* qslot, void* stream) {
    GNN_REQUIRE(n >= 0 && n < (int64_t(1) << 31), "gnn_quant_slots: n out of range");
    GNN_REQUIRE(n_groups >= 0 && n_groups <= 8, "gnn_quant_slots: at most 8 groups");
    GNN_REQUIRE(n == 0 || qslot, "gnn_quant_slots: qslot is NULL");
    GNN_REQUIRE(n_groups == 0 || (rows && counts), "gnn_quant_slots: rows or counts is NULL");
    for (int g = 0; g < n_groups; ++g) {
        GNN_REQUIRE(counts[g] >= 0 && counts[g] < (int64_t(1) << 27), "gnn_quant_slots: group row count out of range");
        GNN_REQUIRE(counts[g] == 0 || rows[g], "gnn_quant_slots: NULL row list");
    }
    return launch_quant_slots(n, n_groups, rows, counts, qslot, static_cast<hipStream_t>(stream));
}

size_t gnn_spmm_dequant_workspace_size(gnn_graph_t h, int64_t d) {
    if (!h || d < 1) return 0;
    const Graph& g = h->g;
    return align_up(spmm_partial_bytes(g.plan[0], d)) + align_up(quantised_source_record_bytes(g.n));
}

gnn_status_t gnn_spmm_dequant(gnn_graph_t h, const float* X, int64_t ldx, const int32_t* qslot,
                              const gnn_qgroup_t* groups, int n_groups, const float* Z, int64_t ldz, float* Y,
                              int64_t ldy, int64_t d, int relu, void* ws, size_t ws_bytes, void* stream) {
    GNN_TRY(check_graph(h, "gnn_spmm_dequant"));
    const Graph& g = h->g;
    GNN_REQUIRE(d >= 4 && d % 4 == 0, "gnn_spmm_dequant: d must be a positive multiple of 4");
    GNN_REQUIRE(ldx >= d && ldy >= d && ldx % 4 == 0, "gnn_spmm_dequant: ldx, ldy must be >= d, ldx a multiple of 4");
    GNN_REQUIRE(reinterpret_cast<uintptr_t>(X) % 16 == 0, "gnn_spmm_dequant: X must be 16-byte aligned");
    GNN_REQUIRE(relu == 0 || relu == 1, "gnn_spmm_dequant: relu must be 0 or 1");
    GNN_REQUIRE(n_groups >= 0 && n_groups <= 8, "gnn_spmm_dequant: at most 8 groups");
    GNN_REQUIRE(n_groups == 0 || groups, "gnn_spmm_dequant: groups is NULL");
    GNN_REQUIRE(g.n == 0 || (X && Y && qslot), "gnn_spmm_dequant: X, Y or qslot is NULL");
    GNN_REQUIRE(static_cast<const void*>(X) != static_cast<const void*>(Y), "gnn_spmm_dequant: X and Y must not overlap");
    for (int i = 0; i < n_groups; ++i) {
        const gnn_qgroup_t& q = groups[i];
        GNN_REQUIRE(q.bits == 2 || q.bits == 4 || q.bits == 8, "gnn_spmm_dequant: group bits must be 2, 4 or 8");
        GNN_REQUIRE(q.n_rows >= 0 && q.n_rows < (int64_t(1) << 27), "gnn_spmm_dequant: group row count out of range");
        GNN_REQUIRE(q.n_rows == 0 || (q.packed && q.scale && q.zero), "gnn_spmm_dequant: NULL group buffer");
        GNN_REQUIRE(reinterpret_cast<uintptr_t>(q.packed) % 4 == 0, "gnn_spmm_dequant: codes must be 4-byte aligned");
    }
    const size_t part = align_up(spmm_partial_bytes(g.plan[0], d));
    const size_t need = part + align_up(quantised_source_record_bytes(g.n));
    if (!ws || ws_bytes < need) return fail(GNN_ERR_WORKSPACE, "gnn_spmm_dequant: workspace too small");
    QuantSources qs;
    qs.qslot = qslot;
    qs.groups = groups;
    qs.n_groups = n_groups;
    qs.records = static_cast<char*>(ws) + part;
    GNN_REQUIRE(!Z || ldz >= d, "gnn_spmm_dequant: ldz must be >= d");
    GNN_REQUIRE(!Z || Z != Y || ldz == ldy, "gnn_spmm_dequant: Z may alias Y only with ldz == ldy");
    qs.addend = Z;
    qs.ld_add = ldz;
    return launch_spmm(csr_view(g), g.dinv, GNN_W_GCN, nullptr, 1, X, GNN_F32, ldx, Y, GNN_F32, ldy, d, relu,
                       Rank1Epilogue{}, static_cast<float*>(ws), static_cast<hipStream_t>(stream), MaskEpilogue{}, qs);
}

}  // extern "C"
