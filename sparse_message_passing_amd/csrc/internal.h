// internal.h -- shared declarations of the gnnmp library (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/gnnmp.h"

namespace gnnmp {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
void set_error(const std::string& msg);
const char* last_error_cstr();
gnn_status_t fail(gnn_status_t s, const std::string& msg);
gnn_status_t hip_fail(hipError_t e, const char* what);
gnn_status_t launch_status(const char* what);  // checks hipGetLastError after launches

#define GNN_REQUIRE(cond, msg)                                                   \
    do {                                                                         \
        if (!(cond)) return ::gnnmp::fail(GNN_ERR_INVALID_ARG, (msg));           \
    } while (0)

#define GNN_HIP(call)                                                            \
    do {                                                                         \
        hipError_t e__ = (call);                                                 \
        if (e__ != hipSuccess) return ::gnnmp::hip_fail(e__, #call);             \
    } while (0)

#define GNN_TRY(call)                                                            \
    do {                                                                         \
        gnn_status_t s__ = (call);                                               \
        if (s__ != GNN_OK) return s__;                                           \
    } while (0)

// ---------------------------------------------------------------------------
// graph
// ---------------------------------------------------------------------------
// Rows whose degree exceeds the view's chunk length are cut into chunks of
// that many edges for the aggregation kernels; each chunk is an independent
// work item and the chunks of one row are summed afterwards in a fixed order.
// Measured: in-edge views with 512-edge chunks (the forward GAT pass on the
// 2^21-node directed R-MAT graph, 4 heads x 64: 128: 7.26 ms, 256: 6.80,
// 512: 6.49, 1024: 7.01; the 256-wide aggregation of the quantised
// exchange 3.40 -> 3.31 ms from 256 to 512, the 2.45M-node bf16 one
// unchanged, the 2^20-node GCN one 2.40 -> 2.43 ms), out-edge views with
// 2048 (the GAT backward's out-edge pass, 256: 9.36 ms, 512: 8.96, 1024:
// 8.75, 2048: 8.54, 4096: 8.88, 16384: 11.2); a hub row kept whole in one
// group is a straggler (73,549 in-edges: 25-27 ms per pass).
#ifndef GNN_CHUNK_CSR
#define GNN_CHUNK_CSR 512
#endif
#ifndef GNN_CHUNK_CSC
#define GNN_CHUNK_CSC 2048
#endif
constexpr int64_t kChunkCsr = GNN_CHUNK_CSR;  // CSR view (in-edges of each destination)
constexpr int64_t kChunkCsc = GNN_CHUNK_CSC;  // CSC view (out-edges of each source)
// Rows above this degree get a whole workgroup in the per-row edge kernels.
constexpr int64_t kBlockRow = 2048;
static_assert(kChunkCsr <= kBlockRow && kChunkCsc <= kBlockRow, "the degree buckets nest");

struct RowPlan {               // one per view (CSR by destination, CSC by source)
    int32_t* order = nullptr;      // [n] rows by degree desc, ties by id
    int64_t chunk = kChunkCsr;     // chunk length of this view's heavy rows
    int64_t n_heavy = 0;           // rows with degree > chunk: order[0 .. n_heavy)
    int64_t n_block = 0;           // rows with degree > kBlockRow: order[0 .. n_block)
    int64_t n_chunks = 0;          // chunks of the heavy rows
    int32_t* chunk_row = nullptr;  // [n_chunks] index into order of the chunk's row
    int32_t* chunk_first = nullptr;// [n_heavy + 1] first chunk of heavy row i
    int64_t max_degree = 0;
};

struct Graph {
    int64_t n = 0, nnz = 0;
    bool has_csc = false;
    bool symmetric = false;       // built with GNN_GRAPH_SYMMETRIZE: A_hat^T = A_hat
    int64_t* row_ptr = nullptr;   // [n+1]
    int32_t* col = nullptr;       // [nnz]
    float* dinv = nullptr;        // [n]
    float* wgcn = nullptr;        // [nnz] dinv[src] * dinv[dst] in CSR order
    float* dmean = nullptr;       // [n] 1 / row length (binary32 division), the mean-aggregation weight
    int64_t* col_ptr = nullptr;   // [n+1]
    int32_t* csc_row = nullptr;   // [nnz]
    int32_t* csc_eid = nullptr;   // [nnz]
    int32_t* csr_cpos = nullptr;  // [nnz] CSC slot of each CSR edge (the inverse of csc_eid)
    RowPlan plan[2];              // 0: CSR, 1: CSC
    std::vector<void*> allocations;
};

// Host-side construction (graph_build.cpp).
struct HostGraph {
    int64_t n = 0;
    std::vector<int64_t> row_ptr;
    std::vector<int32_t> col;
    std::vector<float> dinv;
    std::vector<int64_t> col_ptr;
    std::vector<int32_t> csc_row, csc_eid;
};
gnn_status_t build_host_graph(int64_t n, int64_t m, const int32_t* src, const int32_t* dst, bool symmetrize,
                              bool csc, HostGraph& out);
void degree_order(const std::vector<int64_t>& ptr, std::vector<int32_t>& order);

// ---------------------------------------------------------------------------
// launchers (one per kernel family); all validate nothing, the API does that
// ---------------------------------------------------------------------------
struct AggView {          // what an aggregation walks
    int64_t n;
    const int64_t* ptr;   // row_ptr or col_ptr
    const int32_t* idx;   // col or csc_row (the "other end" of each edge)
    const int32_t* eid;   // CSR slot of each entry (CSC only) or nullptr
    const RowPlan* plan;
    const float* wgcn;    // GCN weight per edge in this view's order (CSR only) or nullptr
    const float* dmean;   // [n] 1 / CSR row length: the mean weight of every in-edge of a row
};

AggView csr_view(const Graph& g);
AggView csc_view(const Graph& g);

struct Rank1Epilogue {    // Y[r, k*dh + j] += a[r, k] * va[k, j] + b[r, k] * vb[k, j]
    const float* a = nullptr;
    const float* va = nullptr;
    const float* b = nullptr;
    const float* vb = nullptr;
};

struct MaskEpilogue {     // out[r, f] *= [M[r, f] > 0]  (the ReLU derivative of a stored activation)
    const void* M = nullptr;
    int64_t ld = 0;
    gnn_dtype_t dt = GNN_F32;
};

// A binary32 operand read as X[r][c] + s[r, c / dh] * v[c] (one fmaf per
// element), r and c the row and column of the operand as stored: the GAT
// backward's dD a_dst term, applied where the two products that consume dH'
// load it instead of in a pass of its own.  dh a power of two >= 4, v
// 16-byte aligned.
struct OperandRank1 {
    const float* s = nullptr;  // [rows][ld]
    int64_t ld = 0;
    int64_t dh = 4;
    const float* v = nullptr;  // [cols]
    int dh_log2 = 2;           // set by the product from dh
};

struct QuantSources {      // dequantise-in-gather: source rows with qslot[u] >= 0 come from quantised groups
    const int32_t* qslot = nullptr;
    const gnn_qgroup_t* groups = nullptr;  // host array of n_groups descriptors
    int n_groups = 0;
    void* records = nullptr;               // device scratch of 16 bytes per node (quantised_source_record_bytes)
    const float* addend = nullptr;         // Y = A X~ + addend (may alias Y), before the ReLU
    int64_t ld_add = 0;
};
inline size_t quantised_source_record_bytes(int64_t n) { return static_cast<size_t>(n) * 16; }

gnn_status_t launch_spmm(const AggView& v, const float* dinv, gnn_weights_t wmode, const float* edge_w, int heads,
                         const void* X, gnn_dtype_t x_dt, int64_t ldx, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                         int64_t d, int relu, const Rank1Epilogue& r1, float* partial, hipStream_t st,
                         const MaskEpilogue& mask = MaskEpilogue{}, const QuantSources& qs = QuantSources{});
gnn_status_t launch_quantize_sym8(const float* X, int64_t ldx, int64_t rows, int64_t cols, const float* mptr,
                                  uint64_t seed, uint32_t stream_id, int8_t* out, int64_t out_ld, int transpose,
                                  float* s_out, hipStream_t st);
// max |X| over a rows x cols block: 512 partial maxima (partial[0..511]), then one
gnn_status_t launch_absmax(const float* X, int64_t ld, int64_t rows, int64_t cols, float* partial, float* out,
                           hipStream_t st);
size_t gemm_q8_ws_bytes(int64_t M, int64_t N, int64_t K);
// SDDMM dot on 8-bit codes (both operands quantised like the 8-bit GEMM's)
bool sddmm_q8_supported(int heads, int64_t d_head);
size_t sddmm_q8_ws_bytes(int64_t n, int64_t d);
gnn_status_t launch_sddmm_q8(const AggView& v, const float* src, int64_t ld_src, const float* dst, int64_t ld_dst,
                             int heads, int64_t d_head, uint64_t seed, uint32_t stream_id, float* out, void* ws,
                             hipStream_t st);
gnn_status_t launch_gemm_q8(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                            float* C, int64_t ldc, uint64_t seed, uint32_t stream_id, void* ws, hipStream_t st);
gnn_status_t launch_quant_stats(const AggView& v, const float* w, const float* H, int64_t ldh, int64_t d,
                                const int32_t* rows, int64_t n_rows, float* beta, float* range, hipStream_t st);
gnn_status_t launch_quant_slots(int64_t n, int n_groups, const int32_t* const* rows, const int64_t* counts,
                                int32_t* qslot, hipStream_t st);
size_t spmm_partial_bytes(const RowPlan& p, int64_t d);
// the allocation-free aggregation's device scratch: its size and its address
// on the current device (spmm.hip)
constexpr size_t kSpmmScratchBytes = size_t(64) << 20;
gnn_status_t spmm_noalloc_scratch(void** out);
// whether gathers from a rows x row_bytes matrix are worth cutting into column slabs

gnn_status_t launch_sddmm_add(const AggView& v, const float* S, int64_t lds, const float* D, int64_t ldd,
                              int heads, float slope, float* out, float* out_pre, hipStream_t st);
gnn_status_t launch_sddmm_dot(const AggView& v, const void* src_feat, int64_t ld_src, const void* dst_feat,
                              int64_t ld_dst, gnn_dtype_t dt, int heads, int64_t d_head, float* out, hipStream_t st);
gnn_status_t launch_edge_softmax(const AggView& v, const float* E, float* alpha, int heads, hipStream_t st);
// GAT backward edge pass: records, the fused out-edge pass (dalpha, dE, dS, transposed aggregation + dS a_src),
// hub fixups, and the in-edge sum dD (the dD a_dst term of dH' is left to the products that read dH')
bool gat_fused_bwd_supported(int heads, int64_t d_head);
size_t gat_fused_bwd_partial_bytes(const RowPlan& csc_plan, int heads, int64_t d_head);
gnn_status_t launch_gat_bwd_fused(const AggView& csr, const AggView& csc, const int32_t* cpos, int64_t nnz,
                                  int heads, int64_t d_head, float slope, const float* Hp, const float* D,
                                  const float* M, const float* Z, const float* Y, const float* dY,
                                  const float* a_src, float* rec, float* dEh, float* dEc,
                                  float* part, float* dS, float* dD, float* dHp, hipStream_t st);
// GAT forward edge pass (gat_fwd.hip): per destination and head, the scores from the gathered H' rows,
// LeakyReLU, the softmax folded into the weighted aggregation (running maximum); writes Y and each
// destination's softmax maximum M and 1 / sum Z ([n, heads]); chunk partials in `part`
size_t gat_fused_fwd_partial_bytes(const RowPlan& csr_plan, int heads, int64_t d_head);
gnn_status_t launch_gat_fwd_fused(const AggView& csr, int heads, int64_t d_head, float slope, const float* Hp,
                                  const float* D, const float* a_src, float* Y, float* M, float* Z, float* part,
                                  hipStream_t st);
gnn_status_t launch_edge_softmax_bwd(const AggView& v, const float* alpha, const float* dalpha,
                                     const float* pre, float slope, float* dE, int heads, hipStream_t st);
gnn_status_t launch_edge_reduce(const AggView& v, const float* vals, int heads, float* out, hipStream_t st);

gnn_status_t launch_gat_scores(int64_t n, const float* Hp, int heads, int64_t d_head, const float* a_src,
                               const float* a_dst, float* S, float* D, hipStream_t st);
size_t head_colsum_partial_bytes(int64_t n, int heads, int64_t d_head);
gnn_status_t launch_head_colsum(int64_t n, const float* coefA, const float* coefB, const float* Hp, int heads,
                                int64_t d_head, float* outA, float* outB, float* partial, hipStream_t st);

size_t gemm_ws_bytes(int transA, int transB, int64_t M, int64_t N, int64_t K);
// bf16 x bf16 weight gradient C = A^T B (gemm_bf16.hip): split-K partials [splits][M][N] into `part`
bool gemm_tn_bf16_supported(int64_t lda, int64_t ldb, const void* A, const void* B);
gnn_status_t launch_gemm_tn_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                                 int64_t ldb, float* part, int64_t splits, int64_t kper, hipStream_t st);
gnn_status_t launch_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, const void* A, gnn_dtype_t a_dt,
                         int64_t lda, const void* B, gnn_dtype_t b_dt, int64_t ldb, void* C, gnn_dtype_t c_dt,
                         int64_t ldc, void* ws, size_t ws_bytes, hipStream_t st, int relu = 0,
                         const MaskEpilogue& mask = MaskEpilogue{}, const OperandRank1& ra1 = OperandRank1{},
                         const OperandRank1& rb1 = OperandRank1{});

size_t xent_ws_bytes(int64_t n);
gnn_status_t launch_softmax_xent(const float* logits, int64_t n, int64_t c, int64_t ld, const int32_t* labels,
                                 float* loss, float* dlogits, int64_t ld_d, float* ws, hipStream_t st);
gnn_status_t launch_relu_mask(int64_t n, int64_t d, const void* dY, int64_t ldd, const void* Y, int64_t ldy,
                              gnn_dtype_t y_dt, void* G, int64_t ldg, gnn_dtype_t g_dt, hipStream_t st);

gnn_status_t launch_quantize(const float* H, int64_t ldh, int64_t d, const int32_t* rows, int64_t n_rows, int bits,
                             uint64_t seed, uint32_t stream_id, uint8_t* packed, float* scale, float* zero,
                             hipStream_t st);
gnn_status_t launch_dequantize(const uint8_t* packed, const float* scale, const float* zero, int64_t n_rows,
                               int64_t d, int bits, const int32_t* rows, float* H, int64_t ldh, hipStream_t st);

// ---------------------------------------------------------------------------
// kernel timers (timer.cpp): a launch inside a ScopedTimer's scope is
// bracketed by HIP events on its stream while timing is on and the timer's
// key (printf-formatted) matches the key gnn_timer_start asked for
// ---------------------------------------------------------------------------
bool timer_on();
class ScopedTimer {
public:
    ScopedTimer(hipStream_t st, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
    ~ScopedTimer();
    ScopedTimer(const ScopedTimer&) = delete;
    ScopedTimer& operator=(const ScopedTimer&) = delete;

private:
    hipStream_t st_;
    int slot_ = -1;
};
inline const char* dt_name(gnn_dtype_t t) { return t == GNN_BF16 ? "bf16" : "f32"; }

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }
inline size_t dt_size(gnn_dtype_t t) { return t == GNN_BF16 ? 2 : 4; }

}  // namespace gnnmp

struct gnn_graph {
    gnnmp::Graph g;
};
