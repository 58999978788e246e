// layers.cpp -- GCN and GAT layers composed from the primitives.
//
// GCN (AdaQP Eqn. 3; Sancus Sec. 2): Y = sigma(A_hat X W).  The product runs
// on the narrower side: GEMM first when d_out <= d_in, otherwise the
// aggregation first.
// GAT (Tango, GAT running example, Fig. 1a forward / Fig. 1b backward).
//
// Workspaces are carved in 256-byte aligned slices; their sizes are returned
// by the *_workspace_size queries with the same arithmetic.

#include <algorithm>
#include <string>

#include "internal.h"

namespace gnnmp {
namespace {

struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* p) : base(static_cast<char*>(p)) {}
    void* take(size_t bytes) {
        void* p = base ? base + off : nullptr;
        off += align_up(bytes);
        return p;
    }
};

// GCN workspace: [G (masked gradient)] [T (aggregation or GEMM intermediate)]
//                [split-K partials] [SpMM partials].  Intermediate rows are
// padded so a gathered row touches as few cache lines as its size allows:
// f32 rows to a multiple of 64 bytes (the 41-wide aggregation: 0.535 ms in
// 176-byte rows, 0.513 ms in 192-byte rows), bf16 rows to whole 128-byte lines.
inline int64_t pad_row(int64_t d, gnn_dtype_t dt) {
    return dt == GNN_BF16 ? (d + 63) / 64 * 64 : (d + 15) / 16 * 16;
}
inline size_t row_bytes_max(int64_t d) {
    return static_cast<size_t>(std::max(pad_row(d, GNN_F32) * 4, pad_row(d, GNN_BF16) * 2));
}

struct GcnWs {
    size_t g, t, gemm, spmm;
    size_t total() const { return align_up(g) + align_up(t) + align_up(gemm) + align_up(spmm); }
};

GcnWs gcn_ws(const Graph& g, int64_t d_in, int64_t d_out) {
    GcnWs w;
    const int64_t n = g.n;
    const int64_t dmax = std::max(d_in, d_out);
    w.g = static_cast<size_t>(n) * row_bytes_max(d_out);
    w.t = static_cast<size_t>(n) * row_bytes_max(dmax);
    w.gemm = std::max(gemm_ws_bytes(1, 0, d_in, d_out, n), gemm_ws_bytes(0, 0, n, d_out, d_in));
    w.gemm = std::max(w.gemm, gemm_ws_bytes(0, 1, n, d_in, d_out));
    w.spmm = spmm_partial_bytes(g.plan[0], dmax);
    if (g.has_csc) w.spmm = std::max(w.spmm, spmm_partial_bytes(g.plan[1], dmax));
    return w;
}

// One graph-convolution layer, Y = sigma(A X W), with A the GCN operator
// A_hat or the mean operator; the backward applies A^T (the CSR view when A is
// a symmetrised graph's A_hat, else the CSC view).
gnn_status_t conv_fwd(const char* api, gnn_weights_t wmode, gnn_graph_t h, const void* X, gnn_dtype_t x_dt,
                      int64_t ldx, int64_t d_in,
                               const float* W, int64_t d_out, int relu, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                               void* saved, void* ws, size_t ws_bytes, void* stream) {
    GNN_REQUIRE(h, std::string(api) + ": graph handle is NULL");
    const Graph& g = h->g;
    GNN_REQUIRE(d_in >= 1 && d_out >= 1, std::string(api) + ": widths must be >= 1");
    GNN_REQUIRE(ldx >= d_in && ldy >= d_out, std::string(api) + ": leading dimensions too small");
    GNN_REQUIRE((x_dt == GNN_F32 || x_dt == GNN_BF16) && (y_dt == GNN_F32 || y_dt == GNN_BF16),
                std::string(api) + ": unknown dtype");
    GNN_REQUIRE(relu == 0 || relu == 1, std::string(api) + ": relu must be 0 or 1");
    GNN_REQUIRE(g.n == 0 || (X && W && Y), std::string(api) + ": NULL pointer");
    const bool gemm_first = d_out <= d_in;
    GNN_REQUIRE(gemm_first || g.n == 0 || saved, std::string(api) + ": saved is NULL (aggregate-first order)");
    const GcnWs w = gcn_ws(g, d_in, d_out);
    if (ws_bytes < w.total() || (!ws && w.total()))
        return fail(GNN_ERR_WORKSPACE, std::string(api) + ": workspace smaller than gnn_gcn_workspace_size()");
    if (g.n == 0) return GNN_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Carver c(ws);
    c.take(w.g);
    void* T = c.take(w.t);
    void* gws = c.take(w.gemm);
    float* sws = static_cast<float*>(c.take(w.spmm));
    if (gemm_first) {
        // Z = X W (padded rows), then Y = sigma(A_hat Z)
        const int64_t ldz = pad_row(d_out, x_dt);
        GNN_TRY(launch_gemm(0, 0, g.n, d_out, d_in, X, x_dt, ldx, W, GNN_F32, d_out, T, x_dt, ldz, gws, w.gemm, st));
        return launch_spmm(csr_view(g), g.dinv, wmode, nullptr, 1, T, x_dt, ldz, Y, y_dt, ldy, d_out, relu,
                           Rank1Epilogue{}, sws, st);
    }
    // saved = A_hat X (same layout as X), then Y = sigma(saved W)
    GNN_TRY(launch_spmm(csr_view(g), g.dinv, wmode, nullptr, 1, X, x_dt, ldx, saved, x_dt, ldx, d_in, 0,
                        Rank1Epilogue{}, sws, st));
    return launch_gemm(0, 0, g.n, d_out, d_in, saved, x_dt, ldx, W, GNN_F32, d_out, Y, y_dt, ldy, gws, w.gemm, st,
                       relu);
}

gnn_status_t conv_bwd(const char* api, gnn_weights_t wmode, gnn_graph_t h, const void* X, gnn_dtype_t x_dt,
                      int64_t ldx, int64_t d_in,
                               const float* W, int64_t d_out, int relu, int relu_in, const void* Y, const void* dY,
                               gnn_dtype_t y_dt, int64_t ldy, const void* saved, void* dX, float* dW, void* ws,
                               size_t ws_bytes, void* stream) {
    GNN_REQUIRE(h, std::string(api) + ": graph handle is NULL");
    const Graph& g = h->g;
    // the backward aggregates over the transposed operator: A_hat of a
    // symmetrised graph is symmetric (its CSR view serves); A_hat of any
    // other graph and the mean operator are not (CSC view: the GCN weight
    // dinv[u] * dinv[v] is formed there from the same two factors)
    const bool use_csr = wmode == GNN_W_GCN && g.symmetric;
    if (!use_csr && !g.has_csc)
        return fail(GNN_ERR_GRAPH, std::string(api) + ": the transposed aggregation needs the CSC view (graph not "
                                                      "symmetrised)");
    const AggView bview = use_csr ? csr_view(g) : csc_view(g);
    GNN_REQUIRE(d_in >= 1 && d_out >= 1, std::string(api) + ": widths must be >= 1");
    GNN_REQUIRE(ldx >= d_in && ldy >= d_out, std::string(api) + ": leading dimensions too small");
    GNN_REQUIRE((x_dt == GNN_F32 || x_dt == GNN_BF16) && (y_dt == GNN_F32 || y_dt == GNN_BF16),
                std::string(api) + ": unknown dtype");
    GNN_REQUIRE((relu == 0 || relu == 1) && (relu_in == 0 || relu_in == 1),
                std::string(api) + ": flags must be 0/1");
    GNN_REQUIRE(dW && W, std::string(api) + ": W or dW is NULL");
    GNN_REQUIRE(g.n == 0 || dY, std::string(api) + ": dY is NULL");
    GNN_REQUIRE(!relu || g.n == 0 || Y, std::string(api) + ": Y is NULL (needed for the ReLU mask)");
    GNN_REQUIRE(!relu_in || !dX || X, std::string(api) + ": X is NULL (needed for the input ReLU mask)");
    const bool gemm_first = d_out <= d_in;
    GNN_REQUIRE(g.n == 0 || (gemm_first ? X != nullptr : saved != nullptr),
                std::string(api) + ": X (GEMM-first) or saved (aggregate-first) is NULL");
    const GcnWs w = gcn_ws(g, d_in, d_out);
    if (ws_bytes < w.total() || (!ws && w.total()))
        return fail(GNN_ERR_WORKSPACE, std::string(api) + ": workspace smaller than gnn_gcn_workspace_size()");
    hipStream_t st = static_cast<hipStream_t>(stream);
    Carver c(ws);
    void* Gb = c.take(w.g);
    void* T = c.take(w.t);
    void* gws = c.take(w.gemm);
    float* sws = static_cast<float*>(c.take(w.spmm));
    // G = dY * [Y > 0]: materialised in the storage type when masked
    const void* G = dY;
    gnn_dtype_t g_dt = y_dt;
    int64_t ldg = ldy;
    if (relu && g.n) {
        ldg = pad_row(d_out, x_dt);
        GNN_TRY(launch_relu_mask(g.n, d_out, dY, ldy, Y, ldy, y_dt, Gb, ldg, x_dt, st));
        G = Gb;
        g_dt = x_dt;
    }
    // the input gradient, optionally times the previous layer's ReLU derivative [X > 0]
    MaskEpilogue mx;
    if (relu_in) {
        mx.M = X;
        mx.ld = ldx;
        mx.dt = x_dt;
    }
    if (gemm_first) {
        // dZ = A_hat G;  dW = X^T dZ;  dX = dZ W^T
        const int64_t ldz = pad_row(d_out, x_dt);
        GNN_TRY(launch_spmm(bview, g.dinv, wmode, nullptr, 1, G, g_dt, ldg, T, x_dt, ldz, d_out, 0,
                            Rank1Epilogue{}, sws, st));
        GNN_TRY(launch_gemm(1, 0, d_in, d_out, g.n, X, x_dt, ldx, T, x_dt, ldz, dW, GNN_F32, d_out, gws, w.gemm, st));
        if (dX)
            GNN_TRY(launch_gemm(0, 1, g.n, d_in, d_out, T, x_dt, ldz, W, GNN_F32, d_out, dX, x_dt, ldx, gws, w.gemm,
                                st, 0, mx));
        return GNN_OK;
    }
    // dW = (A_hat X)^T G;  dX = A_hat (G W^T)
    GNN_TRY(launch_gemm(1, 0, d_in, d_out, g.n, saved, x_dt, ldx, G, g_dt, ldg, dW, GNN_F32, d_out, gws, w.gemm, st));
    if (dX) {
        const int64_t ldt = pad_row(d_in, x_dt);
        GNN_TRY(launch_gemm(0, 1, g.n, d_in, d_out, G, g_dt, ldg, W, GNN_F32, d_out, T, x_dt, ldt, gws, w.gemm, st));
        GNN_TRY(launch_spmm(bview, g.dinv, wmode, nullptr, 1, T, x_dt, ldt, dX, x_dt, ldx, d_in, 0,
                            Rank1Epilogue{}, sws, st, mx));
    }
    return GNN_OK;
}

}  // namespace
}  // namespace gnnmp

using namespace gnnmp;

extern "C" {

size_t gnn_gcn_workspace_size(gnn_graph_t h, int64_t d_in, int64_t d_out) {
    if (!h || d_in <= 0 || d_out <= 0) return 0;
    return gcn_ws(h->g, d_in, d_out).total();
}

gnn_status_t gnn_gcn_layer_fwd(gnn_graph_t h, const void* X, gnn_dtype_t x_dt, int64_t ldx, int64_t d_in,
                               const float* W, int64_t d_out, int relu, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                               void* saved, void* ws, size_t ws_bytes, void* stream) {
    return conv_fwd("gnn_gcn_layer_fwd", GNN_W_GCN, h, X, x_dt, ldx, d_in, W, d_out, relu, Y, y_dt, ldy, saved, ws,
                    ws_bytes, stream);
}

gnn_status_t gnn_gcn_layer_bwd(gnn_graph_t h, const void* X, gnn_dtype_t x_dt, int64_t ldx, int64_t d_in,
                               const float* W, int64_t d_out, int relu, int relu_in, const void* Y, const void* dY,
                               gnn_dtype_t y_dt, int64_t ldy, const void* saved, void* dX, float* dW, void* ws,
                               size_t ws_bytes, void* stream) {
    return conv_bwd("gnn_gcn_layer_bwd", GNN_W_GCN, h, X, x_dt, ldx, d_in, W, d_out, relu, relu_in, Y, dY, y_dt, ldy,
                    saved, dX, dW, ws, ws_bytes, stream);
}

size_t gnn_sage_workspace_size(gnn_graph_t h, int64_t d_in, int64_t d_out) {
    return gnn_gcn_workspace_size(h, d_in, d_out);
}

gnn_status_t gnn_sage_layer_fwd(gnn_graph_t h, const void* X, gnn_dtype_t x_dt, int64_t ldx, int64_t d_in,
                                const float* W, int64_t d_out, int relu, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                                void* saved, void* ws, size_t ws_bytes, void* stream) {
    return conv_fwd("gnn_sage_layer_fwd", GNN_W_MEAN, h, X, x_dt, ldx, d_in, W, d_out, relu, Y, y_dt, ldy, saved, ws,
                    ws_bytes, stream);
}

gnn_status_t gnn_sage_layer_bwd(gnn_graph_t h, const void* X, gnn_dtype_t x_dt, int64_t ldx, int64_t d_in,
                                const float* W, int64_t d_out, int relu, int relu_in, const void* Y, const void* dY,
                                gnn_dtype_t y_dt, int64_t ldy, const void* saved, void* dX, float* dW, void* ws,
                                size_t ws_bytes, void* stream) {
    return conv_bwd("gnn_sage_layer_bwd", GNN_W_MEAN, h, X, x_dt, ldx, d_in, W, d_out, relu, relu_in, Y, dY, y_dt,
                    ldy, saved, dX, dW, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// GAT
// ---------------------------------------------------------------------------
size_t gnn_gat_saved_size(gnn_graph_t h, int heads, int64_t d_head) {
    if (!h || heads < 1 || d_head < 1) return 0;
    const Graph& g = h->g;
    const size_t n = g.n, hd = static_cast<size_t>(heads) * d_head;
    return align_up(n * hd * 4) + 4 * align_up(n * heads * 4);
}

size_t gnn_gat_workspace_size(gnn_graph_t h, int64_t d_in, int heads, int64_t d_head) {
    if (!h || heads < 1 || d_head < 1 || d_in < 1) return 0;
    const Graph& g = h->g;
    const size_t n = g.n, e = g.nnz;
    const int64_t hd = heads * d_head;
    size_t gemm = std::max(gemm_ws_bytes(0, 0, g.n, hd, d_in), gemm_ws_bytes(1, 0, d_in, hd, g.n));
    gemm = std::max(gemm, gemm_ws_bytes(0, 1, g.n, d_in, hd));
    // forward: GEMM workspace, then the edge pass's hub-row partials
    const size_t fwd = align_up(gemm) + align_up(gat_fused_fwd_partial_bytes(g.plan[0], heads, d_head));
    // backward: dE (CSC order: per-head planes, then per-edge records), the
    // per-destination records, dD, dS, dH', the CSC pass's chunk partials,
    // the column-sum partials, the GEMM workspace
    size_t bwd = 2 * align_up(e * heads * 4) + align_up(n * heads * 12) + 2 * align_up(n * heads * 4) +
                 align_up(n * hd * 4) + align_up(head_colsum_partial_bytes(g.n, heads, d_head)) + align_up(gemm);
    if (g.has_csc) bwd += align_up(gat_fused_bwd_partial_bytes(g.plan[1], heads, d_head));
    return std::max(fwd, bwd);
}

namespace {
struct GatSaved {
    float *Hp, *S, *D, *M, *Z;
};
GatSaved carve_saved(const Graph& g, void* saved, int heads, int64_t d_head) {
    Carver c(saved);
    const size_t n = g.n, hd = static_cast<size_t>(heads) * d_head;
    GatSaved s;
    s.Hp = static_cast<float*>(c.take(n * hd * 4));
    s.S = static_cast<float*>(c.take(n * heads * 4));
    s.D = static_cast<float*>(c.take(n * heads * 4));
    s.M = static_cast<float*>(c.take(n * heads * 4));
    s.Z = static_cast<float*>(c.take(n * heads * 4));
    return s;
}
bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
}  // namespace

gnn_status_t gnn_gat_layer_fwd(gnn_graph_t h, const float* X, int64_t d_in, const float* W, const float* a_src,
                               const float* a_dst, int heads, int64_t d_head, float slope, float* Y, void* saved,
                               void* ws, size_t ws_bytes, void* stream) {
    GNN_REQUIRE(h, "gnn_gat_layer_fwd: graph handle is NULL");
    const Graph& g = h->g;
    GNN_REQUIRE(d_in >= 1 && heads >= 1 && d_head >= 1, "gnn_gat_layer_fwd: sizes must be >= 1");
    GNN_REQUIRE(g.n == 0 || (X && W && a_src && a_dst && Y && saved), "gnn_gat_layer_fwd: NULL pointer");
    // the shapes the score, attention and aggregation kernels take, checked
    // before the first launch (the same heads and d_head as the backward)
    if (!gat_fused_bwd_supported(heads, d_head) || heads * d_head > 1024)
        return fail(GNN_ERR_UNSUPPORTED, "gnn_gat_layer_fwd: needs 1, 2, 4 or 8 heads, d_head a power of two from 4 "
                                         "to 256 and heads * d_head <= 1024");
    GNN_REQUIRE(g.n == 0 || (aligned16(Y) && aligned16(a_src) && aligned16(a_dst) && aligned16(saved)),
                "gnn_gat_layer_fwd: Y, a_src, a_dst and saved must be 16-byte aligned");
    const size_t need = gnn_gat_workspace_size(h, d_in, heads, d_head);
    if (ws_bytes < need || (!ws && need))
        return fail(GNN_ERR_WORKSPACE, "gnn_gat_layer_fwd: workspace smaller than gnn_gat_workspace_size()");
    if (g.n == 0) return GNN_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t hd = heads * d_head;
    GatSaved s = carve_saved(g, saved, heads, d_head);
    Carver c(ws);
    size_t gemm = std::max(gemm_ws_bytes(0, 0, g.n, hd, d_in), gemm_ws_bytes(1, 0, d_in, hd, g.n));
    gemm = std::max(gemm, gemm_ws_bytes(0, 1, g.n, d_in, hd));
    void* gws = c.take(gemm);
    float* part = static_cast<float*>(c.take(gat_fused_fwd_partial_bytes(g.plan[0], heads, d_head)));
    // H' = X W;  S, D per-head scores (S for the backward, D for both);
    // then one pass over the in-edges: E = LReLU(S[src] + D[dst]) with S[src]
    // formed from the gathered row H'[src], the softmax folded into
    // Y = (G . alpha) H', each row's maximum and 1/sum kept
    GNN_TRY(launch_gemm(0, 0, g.n, hd, d_in, X, GNN_F32, d_in, W, GNN_F32, hd, s.Hp, GNN_F32, hd, gws, gemm, st));
    GNN_TRY(launch_gat_scores(g.n, s.Hp, heads, d_head, a_src, a_dst, s.S, s.D, st));
    return launch_gat_fwd_fused(csr_view(g), heads, d_head, slope, s.Hp, s.D, a_src, Y, s.M, s.Z, part, st);
}

gnn_status_t gnn_gat_layer_bwd(gnn_graph_t h, const float* X, int64_t d_in, const float* W, const float* a_src,
                               const float* a_dst, int heads, int64_t d_head, float slope, const float* Y,
                               const float* dY, const void* saved, float* dX, float* dW, float* da_src,
                               float* da_dst, void* ws, size_t ws_bytes, void* stream) {
    GNN_REQUIRE(h, "gnn_gat_layer_bwd: graph handle is NULL");
    const Graph& g = h->g;
    GNN_REQUIRE(d_in >= 1 && heads >= 1 && d_head >= 1, "gnn_gat_layer_bwd: sizes must be >= 1");
    GNN_REQUIRE(dW && da_src && da_dst, "gnn_gat_layer_bwd: NULL gradient pointer");
    GNN_REQUIRE(g.n == 0 || (X && W && a_src && a_dst && Y && dY && saved), "gnn_gat_layer_bwd: NULL pointer");
    if (!g.has_csc) return fail(GNN_ERR_GRAPH, "gnn_gat_layer_bwd: the graph needs the CSC view");
    if (!gat_fused_bwd_supported(heads, d_head))
        return fail(GNN_ERR_UNSUPPORTED, "gnn_gat_layer_bwd: needs 1, 2, 4 or 8 heads and d_head a power of two "
                                         "from 4 to 256");
    GNN_REQUIRE(g.n == 0 || (aligned16(Y) && aligned16(dY) && aligned16(a_src) && aligned16(a_dst) &&
                             aligned16(saved)),
                "gnn_gat_layer_bwd: Y, dY, a_src, a_dst and saved must be 16-byte aligned");
    const size_t need = gnn_gat_workspace_size(h, d_in, heads, d_head);
    if (ws_bytes < need || (!ws && need))
        return fail(GNN_ERR_WORKSPACE, "gnn_gat_layer_bwd: workspace smaller than gnn_gat_workspace_size()");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t hd = heads * d_head;
    const size_t n = g.n, e = g.nnz;
    GatSaved s = carve_saved(g, const_cast<void*>(saved), heads, d_head);
    Carver c(ws);
    float* dEh = static_cast<float*>(c.take(e * heads * 4));
    float* dEc = static_cast<float*>(c.take(e * heads * 4));
    float* rec = static_cast<float*>(c.take(n * heads * 12));
    float* dD = static_cast<float*>(c.take(n * heads * 4));
    float* dS = static_cast<float*>(c.take(n * heads * 4));
    float* dHp = static_cast<float*>(c.take(n * hd * 4));
    float* cps = static_cast<float*>(c.take(head_colsum_partial_bytes(g.n, heads, d_head)));
    float* part = static_cast<float*>(c.take(gat_fused_bwd_partial_bytes(g.plan[1], heads, d_head)));
    size_t gemm = std::max(gemm_ws_bytes(0, 0, g.n, hd, d_in), gemm_ws_bytes(1, 0, d_in, hd, g.n));
    gemm = std::max(gemm, gemm_ws_bytes(0, 1, g.n, d_in, hd));
    void* gws = c.take(gemm);
    // dalpha, dE, dS and P = (G . alpha)^T dY + dS a_src in one pass over the
    // out-edges; dD in one pass over the in-edges
    GNN_TRY(launch_gat_bwd_fused(csr_view(g), csc_view(g), g.csr_cpos, g.nnz, heads, d_head, slope, s.Hp, s.D, s.M,
                                 s.Z, Y, dY, a_src, rec, dEh, dEc, part, dS, dD, dHp, st));
    // da_src = sum_v dS[v] H'[v], da_dst = sum_v dD[v] H'[v] per head
    GNN_TRY(launch_head_colsum(g.n, dS, dD, s.Hp, heads, d_head, da_src, da_dst, cps, st));
    // dW = X^T dH',  dX = dH' W^T, with dH' = P + dD a_dst (per head) formed
    // element by element as the products load it
    OperandRank1 r1;
    r1.s = dD;
    r1.ld = heads;
    r1.dh = d_head;
    r1.v = a_dst;
    GNN_TRY(launch_gemm(1, 0, d_in, hd, g.n, X, GNN_F32, d_in, dHp, GNN_F32, hd, dW, GNN_F32, hd, gws, gemm, st, 0,
                        MaskEpilogue{}, OperandRank1{}, r1));
    if (dX)
        GNN_TRY(launch_gemm(0, 1, g.n, d_in, hd, dHp, GNN_F32, hd, W, GNN_F32, hd, dX, GNN_F32, d_in, gws, gemm, st,
                            0, MaskEpilogue{}, r1));
    return GNN_OK;
}

}  // extern "C"
