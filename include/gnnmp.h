/*
 * gnnmp.h -- C ABI of the per-layer GNN message-passing library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operations follow the pages' statement of the problem:
 *   - AdaQP (arXiv 2306.01381): message passing as aggregation + update
 *     (Sec. 2.1, Eqn. 1 and the weighted-sum form Eqn. 3), per-row stochastic
 *     integer quantisation and dequantisation of exchanged messages
 *     (Eqn. 4, 5), the local/remote split of the aggregation (Eqn. 7).
 *   - Sancus (IJCAI'23 extended abstract), Sec. 2 Preliminaries: the GCN
 *     operator A_hat = Dbar^-1/2 (A + I) Dbar^-1/2 and the layer
 *     H(l+1) = sigma(A_hat H(l) W).
 *   - Tango (SC'23, arXiv 2308.00890), GAT running example (Fig. 1a/1b): the
 *     GAT forward and backward expressed with GEMM, SpMM and SDDMM.
 *
 * Conventions (all entry points)
 *   - Graphs are CSR by destination: row v lists the sources u of the edges
 *     u -> v in ascending order.  Edge-valued arrays are [nnz, heads]
 *     row-major in CSR order.
 *   - Dense matrices are row-major with a leading dimension in elements.
 *   - Every pointer is device memory unless its comment says "host".  The
 *     caller owns all device buffers; the library owns only graph handles.
 *   - Compute calls are asynchronous on the caller's HIP stream (`stream`,
 *     a hipStream_t; NULL = the default stream), never synchronise the host,
 *     and use no floating-point atomics: results are bitwise reproducible.
 *   - Arguments are validated before anything is launched.  On failure the
 *     call returns a non-zero status, launches nothing, and
 *     gnn_last_error() describes the problem (thread-local).
 *   - Floating-point sums accumulate in binary32.  GNN_BF16 tensors hold
 *     bfloat16 (round-to-nearest-even at every store).
 */
#ifndef GNNMP_H
#define GNNMP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GNN_OK = 0,
    GNN_ERR_INVALID_ARG = 1,   /* a pointer, size, flag or leading dimension is invalid */
    GNN_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement          */
    GNN_ERR_OUT_OF_MEMORY = 3, /* device or host allocation failed (graph creation)     */
    GNN_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed            */
    GNN_ERR_GRAPH = 5,         /* the graph lacks a view this call needs (e.g. CSC)     */
    GNN_ERR_WORKSPACE = 6      /* the workspace is smaller than the size query returned */
} gnn_status_t;

typedef enum { GNN_F32 = 0, GNN_BF16 = 1 } gnn_dtype_t;

/* Edge weights of an aggregation. */
typedef enum {
    GNN_W_GCN = 0,   /* A_hat entries dinv[u]*dinv[v] (Sancus Sec. 2), heads must be 1 */
    GNN_W_ONES = 1,  /* every weight 1 (Tango's "ones" SpMM)                          */
    GNN_W_EDGE = 2,  /* caller's edge_w[nnz, heads] in CSR order (GAT attention)       */
    GNN_W_MEAN = 3   /* 1 / (row length) of the destination: the mean over {v} u N(v)
                        (GraphSAGE's mean aggregator in AdaQP's weighted-sum form,
                        Eqn. 1); heads must be 1                                      */
} gnn_weights_t;

typedef struct gnn_graph* gnn_graph_t;

/* Status text and the calling thread's last error detail (never NULL). */
const char* gnn_status_string(gnn_status_t s);
const char* gnn_last_error(void);

/* ------------------------------------------------------------------------
 * Graph layer
 * ------------------------------------------------------------------------ */
#define GNN_GRAPH_SYMMETRIZE 0x1u  /* add the reverse of every edge                */
#define GNN_GRAPH_CSC        0x2u  /* also build the transposed (CSC + eid) view  */

/* Build a graph from an edge list (Sancus Sec. 2: Abar = A + I; Tango,
 * datasets paragraph: reverse edges and self-loops are added).  Self-loops
 * and repeated edges of the input are dropped, the reverse edges are added
 * when GNN_GRAPH_SYMMETRIZE is set, then exactly one self-loop per node is
 * added, so the degree Dbar_vv is the CSR row length.  Also computes
 * dinv[v] = 1/sqrt(Dbar_vv) (binary32, correctly rounded) and the order of
 * rows by in-degree, descending, ties by id (and of CSC columns by
 * out-degree when the CSC view is built).
 *   n        number of nodes, 0 <= n < 2^31
 *   m        number of input edges, m >= 0
 *   src,dst  host int32[m]; ids must lie in [0, n)
 *   flags    GNN_GRAPH_* bits
 *   out      receives the handle (host)
 * Synchronous: uploads the device arrays before it returns.  The result has
 * nnz < 2^31.  Errors: GNN_ERR_INVALID_ARG (ids out of range, n < 0, ...),
 * GNN_ERR_OUT_OF_MEMORY, GNN_ERR_HIP. */
gnn_status_t gnn_graph_create(int64_t n, int64_t m, const int32_t* src, const int32_t* dst,
                              uint32_t flags, gnn_graph_t* out);

/* Split of the aggregation by message origin (AdaQP Eqn. 7: the sum over a
 * node's local in-neighbours plus the sum over its remote ones).  marginal:
 * host uint8[n], nonzero for the source rows that arrive over the exchange.
 * Builds two graphs over the same n nodes: *local holds the in-edges whose
 * source is not marginal, *remote those whose source is; every edge keeps its
 * position order within its row and its GCN weight in g, so
 * A_hat = A_local + A_remote entry by entry (use GNN_W_GCN with them; their
 * dinv is g's).  Neither has a CSC view.  Both are destroyed with
 * gnn_graph_destroy; on error neither is created. */
gnn_status_t gnn_graph_split(gnn_graph_t g, const uint8_t* marginal, gnn_graph_t* local, gnn_graph_t* remote);

gnn_status_t gnn_graph_destroy(gnn_graph_t g);

typedef struct {
    int64_t n, nnz;
    int64_t max_in_degree, max_out_degree;   /* max_out_degree = 0 without CSC */
    int has_csc;
    /* device views, owned by the graph */
    const int64_t* row_ptr;   /* [n+1]                                      */
    const int32_t* col;       /* [nnz]  source of each CSR slot             */
    const float* dinv;        /* [n]    1/sqrt(row length)                  */
    const int32_t* perm;      /* [n]    rows by in-degree desc, ties by id  */
    const int64_t* col_ptr;   /* [n+1]  CSC (NULL without CSC)              */
    const int32_t* csc_row;   /* [nnz]  destination of each CSC slot        */
    const int32_t* csc_eid;   /* [nnz]  CSR slot of each CSC slot           */
    const int32_t* perm_t;    /* [n]    columns by out-degree desc, ties by id */
    int symmetric;            /* 1: built with GNN_GRAPH_SYMMETRIZE (A_hat^T = A_hat) */
    /* Degree buckets of the degree-ordered lists perm (in-degree) and perm_t
     * (out-degree; all zero without CSC): bucket i holds positions
     * [bucket_off[i], bucket_off[i+1]) -- degree > bucket_threshold[0], then
     * degree > bucket_threshold[1], then the rest -- so bucket_off =
     * {0, #rows with degree > 2048, #rows with degree > 512, n}; likewise
     * bucket_off_t with bucket_threshold_t = {2048, 2048}.  The aggregation
     * kernels give rows of the first bucket a whole workgroup in the per-row
     * edge kernels and cut rows of the first two into chunks of
     * bucket_threshold[1] (in-edges) or bucket_threshold_t[1] (out-edges)
     * edges; the thresholds are tuning choices of this library. */
    int64_t bucket_threshold[2];   /* {2048, 512} */
    int64_t bucket_off[4];
    int64_t bucket_off_t[4];
    int64_t bucket_threshold_t[2]; /* {2048, 2048}; zero without CSC */
} gnn_graph_info_t;

gnn_status_t gnn_graph_info(gnn_graph_t g, gnn_graph_info_t* out /* host */);

/* Copy views back to host buffers (any pointer may be NULL to skip it).
 * w receives the GCN edge weights dinv[src]*dinv[dst] in CSR order
 * (binary32 product of the two binary32 factors); bucket_off and
 * bucket_off_t receive int64[4] each, the bucket offsets of gnn_graph_info.
 * The CSC outputs (col_ptr, csc_row, csc_eid, perm_t, bucket_off_t) need the
 * CSC view (GNN_ERR_GRAPH otherwise).  Synchronous. */
gnn_status_t gnn_graph_export(gnn_graph_t g, int64_t* row_ptr, int32_t* col, float* dinv, float* w,
                              int32_t* perm, int64_t* bucket_off, int64_t* col_ptr, int32_t* csc_row,
                              int32_t* csc_eid, int32_t* perm_t, int64_t* bucket_off_t /* all host */);

/* ------------------------------------------------------------------------
 * Primitives
 * ------------------------------------------------------------------------ */

/* Aggregation (SpMM).  AdaQP Eqn. 3 aggregation sum_u alpha_uv h_u; Tango
 * GAT running example, "H(l) = (G . alpha) H'" (multi-head weighted SpMM):
 *   transpose = 0:  Y[v, f] = sum_{u -> v} w(e, f / (d/heads)) * X[u, f]
 *   transpose = 1:  Y[u, f] = sum_{u -> v} w(e, f / (d/heads)) * X[v, f]
 *                   (needs the CSC view; the gradient over the reversed graph)
 * then optionally ReLU (relu = 1).  X: [n, ldx] of x_dt, Y: [n, ldy] of y_dt,
 * d features (d >= 1, ldx, ldy >= d), heads >= 1 dividing d.  X and Y must
 * not overlap.  Needs a workspace of gnn_spmm_workspace_size() bytes for
 * the split of high-degree rows (ws may be NULL when that size is 0). */
size_t gnn_spmm_workspace_size(gnn_graph_t g, int transpose, int64_t d);
gnn_status_t gnn_spmm(gnn_graph_t g, int transpose, gnn_weights_t wmode, const float* edge_w, int heads,
                      const void* X, gnn_dtype_t x_dt, int64_t ldx, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                      int64_t d, int relu, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free variant of gnn_spmm, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments,
 * results (bitwise: the same kernels) and checks as gnn_spmm without the
 * workspace: the hub-row partial sums go to a fixed device scratch of
 * gnn_spmm_noalloc_max_scratch() bytes (64 MiB) that the library holds on
 * each GPU it runs on until the process ends, found on the first call on a
 * device (with the graph's device current).  Calls whose partials need more
 * than that (gnn_spmm_workspace_size(g, transpose, d) bytes) fail with
 * GNN_ERR_UNSUPPORTED before any launch.  Nothing in the scratch needs to
 * start at zero.  Every call on one GPU shares the scratch: calls that
 * overlap on one GPU (on different streams without ordering, or from
 * different host threads) race and must be serialised by the caller. */
size_t gnn_spmm_noalloc_max_scratch(void);
gnn_status_t gnn_spmm_noalloc(gnn_graph_t g, int transpose, gnn_weights_t wmode, const float* edge_w, int heads,
                              const void* X, gnn_dtype_t x_dt, int64_t ldx, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                              int64_t d, int relu, void* stream);

/* Edge -> node sums (Tango: dD = (G . dE) 1 over in-edges, dS = (G^T . dE) 1
 * over out-edges; the incidence-matrix SpMM).  by_src = 0 sums the in-edges
 * of every node, by_src = 1 its out-edges (needs CSC).  vals [nnz, heads]
 * f32, out [n, heads] f32. */
gnn_status_t gnn_edge_reduce(gnn_graph_t g, int by_src, const float* vals, int heads, float* out,
                             void* stream);

/* SDDMM (Tango, GAT running example: E = G . (S (+) D^T)).
 *   op = 0 (add):  out[e, k] = LReLU(src_feat[u, k] + dst_feat[v, k]) with
 *                  slope `slope` (NaN: no activation), out_pre[e, k] the
 *                  value before the activation (nullable).  d_head must be 1;
 *                  src_feat, dst_feat are [n, ld] f32 with heads columns.
 *                  One IEEE add and one multiply: bit-exact.
 *   op = 1 (dot):  out[e, k] = sum_j src_feat[u, k*d_head + j] * dst_feat[v, k*d_head + j]
 *                  (the attention gradient d(alpha) = dY[dst] . H'[src]);
 *                  features of dt, out_pre must be NULL.
 * out [nnz, heads] f32. */
gnn_status_t gnn_sddmm(gnn_graph_t g, int op, const void* src_feat, int64_t ld_src, const void* dst_feat,
                       int64_t ld_dst, gnn_dtype_t dt, int heads, int64_t d_head, float slope, float* out,
                       float* out_pre, void* stream);

/* Edge softmax over the in-edges of each destination, per head (Tango, GAT
 * running example, softmax step, with the per-destination maximum
 * subtracted first):  alpha[e,k] = exp(E[e,k] - m_vk) / sum_in(v) exp(E - m_vk).
 * E, alpha [nnz, heads] f32 (may alias). */
gnn_status_t gnn_edge_softmax(gnn_graph_t g, const float* E, float* alpha, int heads, void* stream);

/* Its backward (Tango, Fig. 1b): P[v,k] = sum_in(v) alpha * dalpha;
 * dE = alpha * (dalpha - P[dst]).  When lrelu_pre is not NULL the LeakyReLU
 * derivative is applied too: dE *= (lrelu_pre > 0 ? 1 : slope).
 * All [nnz, heads] f32; dE may alias dalpha. */
gnn_status_t gnn_edge_softmax_bwd(gnn_graph_t g, const float* alpha, const float* dalpha,
                                  const float* lrelu_pre, float slope, float* dE, int heads, void* stream);

/* Dense product C = op(A) * op(B) (the update H W of AdaQP Eqn. 3 / Sancus
 * Sec. 2, Tango's GEMM step; and its backward dW = H^T dZ, dH = dZ W^T),
 * on the matrix cores.  op(A) is M x K, op(B) is K x N, C is M x N:
 *   transA = 0: A is [M, lda] row-major;  1: A is [K, lda] (A^T used)
 *   transB = 0: B is [K, ldb];            1: B is [N, ldb] (B^T used)
 * Inputs of a_dt / b_dt (bf16 inputs are widened exactly), C of c_dt.
 * Workspace: gnn_gemm_workspace_size() bytes (split-K partials and a
 * transposed copy of a small B; 0 is possible). */
size_t gnn_gemm_workspace_size(int transA, int transB, int64_t M, int64_t N, int64_t K);
gnn_status_t gnn_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K,
                      const void* A, gnn_dtype_t a_dt, int64_t lda, const void* B, gnn_dtype_t b_dt, int64_t ldb,
                      void* C, gnn_dtype_t c_dt, int64_t ldc, void* ws, size_t ws_bytes, void* stream);

/* Quantisation-aware GEMM (Tango, SC'23: symmetric, tensor-level, dynamic
 * 8-bit quantisation with stochastic rounding; int8 x int8 products summed in
 * int32; the result dequantised in the epilogue).  For X in {A, B}:
 * m = max|X|, x = X * (127/m), q = floor(x) + [u < x - floor(x)] clamped to
 * [-127, 127], s = m/127 (binary32, one rounding per operation; m == 0 gives
 * q = 0, s = 0); u is the Philox4x32-10 draw of key (seed low, seed high),
 * counter (row, col/4, stream, 0), word col mod 4 of X's own element, with
 * stream = stream_id for A and stream_id + 1 for B.  C = f32(sum_k qA qB) *
 * (s_A * s_B) (the int32 sum converted with round-to-nearest-even): bit-exact
 * against any faithful implementation.  K <= 133,000 keeps the int32 sums
 * from overflowing (|q| <= 127).  A [M, lda] f32,
 * B [K, ldb] f32 (no transposes), C [M, ldc] f32.  Workspace (the quantised
 * copies, K padded to 64, and the scales): gnn_gemm_q8_workspace_size(). */
size_t gnn_gemm_q8_workspace_size(int64_t M, int64_t N, int64_t K);
gnn_status_t gnn_gemm_q8(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                         float* C, int64_t ldc, uint64_t seed, uint32_t stream_id, void* ws, size_t ws_bytes,
                         void* stream);

/* SDDMM dot on quantised inputs (Tango, SC'23, "SDDMM with on-the-fly
 * dequantization": a product of two quantised values is the product of their
 * codes times the product of their scales, so the dot runs on the 8-bit
 * codes, which a random gather reads at a quarter of the bytes).  Both
 * operands are quantised over the whole tensor exactly as gnn_gemm_q8
 * quantises its operands: src_feat ([n, ld_src] f32) with stream_id,
 * dst_feat ([n, ld_dst] f32) with stream_id + 1, counters (node, feature/4).
 * out[e, k] = f32(sum_j q_src[u, k*d_head + j] * q_dst[v, k*d_head + j]) *
 * (s_src * s_dst) for CSR edge e = u -> v (int32 sums, exact; bit-exact
 * against any faithful implementation); out [nnz, heads] f32 in CSR order.
 * d_head must be 16 times a power of two (16 ... 256) and heads * d_head
 * <= 1024 (GNN_ERR_INVALID_ARG otherwise).  Workspace (both quantised
 * copies, n x heads*d_head bytes each, and the scales):
 * gnn_sddmm_q8_workspace_size(g, heads*d_head). */
size_t gnn_sddmm_q8_workspace_size(gnn_graph_t g, int64_t d);
gnn_status_t gnn_sddmm_q8(gnn_graph_t g, const float* src_feat, int64_t ld_src, const float* dst_feat,
                          int64_t ld_dst, int heads, int64_t d_head, uint64_t seed, uint32_t stream_id, float* out,
                          void* ws, size_t ws_bytes, void* stream);

/* Mean softmax cross-entropy over n rows of c logits and its gradient:
 *   loss = (1/n) sum_v [logsumexp(z_v) - z_v[y_v]],  dz = (softmax(z_v) - onehot(y_v)) / n.
 * logits [n, ld] f32, labels int32[n] in [0, c), loss: one device float,
 * dlogits [n, ld_d] f32 (nullable).  The softmax and loss stay binary32
 * (Tango keeps the layer feeding the softmax in full precision).
 * Workspace gnn_softmax_xent_workspace_size(n) bytes. */
size_t gnn_softmax_xent_workspace_size(int64_t n);
gnn_status_t gnn_softmax_xent(const float* logits, int64_t n, int64_t c, int64_t ld, const int32_t* labels,
                              float* loss, float* dlogits, int64_t ld_d, void* ws, size_t ws_bytes, void* stream);

/* Per-row stochastic integer quantisation (AdaQP Eqn. 4).  For row r
 * (node rows[r] of H), with b = bits in {2, 4, 8}:
 *   Z = min, R = max - min, inv = (2^b-1)/R, S = R/(2^b-1)   (IEEE binary32)
 *   x = (h - Z) * inv   (two rounded operations, no contraction)
 *   q = min(floor(x) + [u < x - floor(x)], 2^b - 1)
 * with u the uniform of Philox4x32-10 (Salmon et al., SC'11) at
 * key (seed low, seed high), counter (rows[r], f/4, stream_id, 0), word f%4,
 * u = (word >> 8) * 2^-24.  A constant row gives q = 0, S = 0.
 * packed [n_rows, d*b/8] bytes (element j in byte j*b/8 at bit (j%(8/b))*b),
 * scale, zero [n_rows] f32.  d*b must be a multiple of 8.  Codes are
 * bit-exact against any other implementation of this definition. */
gnn_status_t gnn_quantize(const float* H, int64_t ldh, int64_t d, const int32_t* rows, int64_t n_rows, int bits,
                          uint64_t seed, uint32_t stream_id, uint8_t* packed, float* scale, float* zero, void* stream);

/* Dequantisation (AdaQP Eqn. 5): H[rows[r], f] = fma(q, S_r, Z_r), one
 * correctly rounded operation; rows not listed are untouched. */
gnn_status_t gnn_dequantize(const uint8_t* packed, const float* scale, const float* zero, int64_t n_rows,
                            int64_t d, int bits, const int32_t* rows, float* H, int64_t ldh, void* stream);

/* Bit-width statistics (AdaQP Sec. 3.2, the beta_k of Problem 11).  For each
 * listed row r (node k = rows[r]) of H [n, ldh] f32:
 *   range[r] = max(h_k) - min(h_k)   (binary32, the R gnn_quantize uses)
 *   beta[r]  = (S2 * d) * range^2 / 6,  S2 = sum of alpha^2 over the edges
 * from k to the nodes that aggregate it, alpha = edge_w[e] (f32 [nnz], CSR
 * order) or the GCN weight when edge_w is NULL.  The edges from k are its
 * out-edges (CSC view) when the graph has one, else its CSR row, which holds
 * the same edges and weights on a symmetrised GCN graph.  The stochastic
 * rounding variance a row adds is beta / (2^b - 1)^2.  beta, range: f32
 * [n_rows] device; every operation binary32 with one rounding. */
gnn_status_t gnn_quant_stats(gnn_graph_t g, const float* edge_w, const float* H, int64_t ldh, int64_t d,
                             const int32_t* rows, int64_t n_rows, float* beta, float* range, void* stream);

/* Greedy bit-width assignment, a stand-in for AdaQP's assignment MILP
 * (Problem 12, solved there with a third-party solver): with candidate widths
 * {2, 4, 8} and a byte budget of avg_bits * m * d / 8, minimise
 * sum_k beta_k / (2^b_k - 1)^2.  Every row starts at 2 bits; upgrades
 * (2 -> 4 costs d/4 bytes, 4 -> 8 costs d/2) are taken in decreasing order
 * of variance removed per byte, ties by smaller row index, each only if it
 * still fits; a row's 4 -> 8 is considered once its 2 -> 4 is taken.
 * Host arrays: beta [m] (>= 0, finite), bits [m] out.  2 <= avg_bits <= 8. */
gnn_status_t gnn_assign_bits(int64_t m, const float* beta, int64_t d, double avg_bits, int32_t* bits);

/* Dequantise-in-gather aggregation.  AdaQP (Sec. 3, Eqn. 4, 5 and 7): the
 * marginal rows a partition receives arrive as per-row codes with their scale
 * and zero point, and are aggregated with the central rows; Tango's
 * quantisation-aware aggregation reads the small quantised copy directly.
 * Here the gather dequantises in registers, so the binary32 copy of the
 * marginal rows is never written or re-read.
 *
 * A group is one bit-width buffer exactly as gnn_quantize writes it. */
typedef struct {
    const uint8_t* packed;  /* [n_rows, d*bits/8] device bytes, 4-byte aligned */
    const float* scale;     /* [n_rows] device */
    const float* zero;      /* [n_rows] device */
    int64_t n_rows;         /* < 2^27 */
    int bits;               /* 2, 4 or 8 */
} gnn_qgroup_t;

/* Slot map for gnn_spmm_dequant: qslot[v] = -1 for every v in [0, n), then
 * qslot[rows_g[r]] = (g << 27) | r for each group g in order (a node listed
 * twice keeps its last entry).  rows: host array of n_groups device pointers
 * (int32 node ids in [0, n)); counts: host array of n_groups row counts;
 * n_groups <= 8.  qslot: int32[n] device, written on `stream`. */
gnn_status_t gnn_quant_slots(int64_t n, int n_groups, const int32_t* const* rows, const int64_t* counts,
                             int32_t* qslot, void* stream);

/* Y = A_hat X~ (GCN weights, CSR view) with X~[u] = X[u] when qslot[u] < 0,
 * else the row of slot qslot[u] dequantised as gnn_dequantize does
 * (fma(q, S, Z), one rounding).  The result is bitwise that of
 * gnn_dequantize into a copy of X followed by gnn_spmm(GNN_W_GCN): the same
 * values summed in the same order.  Z (nullable) is added to each sum before
 * the ReLU, Y = A_hat X~ + Z, one rounding (AdaQP Eqn. 7: the remote part
 * added to the local part); Z may be Y itself (ldz == ldy).
 * X [n, ldx] f32 (rows with qslot >= 0 are
 * not read), Y [n, ldy] f32, d % 4 == 0, ldx % 4 == 0, X 16-byte aligned;
 * groups: host array of n_groups (<= 8) descriptors whose codes have row
 * length d*bits/8.  relu as in gnn_spmm.  Workspace:
 * gnn_spmm_dequant_workspace_size(g, d) bytes (hub-row partials plus one
 * 16-byte record per node, rebuilt from qslot and the groups on every call). */
size_t gnn_spmm_dequant_workspace_size(gnn_graph_t g, int64_t d);
gnn_status_t gnn_spmm_dequant(gnn_graph_t g, const float* X, int64_t ldx, const int32_t* qslot,
                              const gnn_qgroup_t* groups, int n_groups, const float* Z, int64_t ldz, float* Y,
                              int64_t ldy, int64_t d, int relu, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Layers (GCN: AdaQP Eqn. 3 / Sancus Sec. 2; GAT: Tango Fig. 1a/1b)
 * ------------------------------------------------------------------------ */

/* GCN layer Y = sigma(A_hat X W), sigma = ReLU when relu = 1.  The GEMM runs
 * first when d_out <= d_in, i.e. Y = sigma(A_hat (X W)); otherwise
 * Y = sigma((A_hat X) W) and A_hat X is written to `saved` (same layout as X:
 * [n, ldx] of x_dt), which the backward needs.  X [n, ldx] of x_dt,
 * W [d_in, d_out] f32 contiguous, Y [n, ldy] of y_dt.  Intermediates are
 * stored in x_dt.  Workspace: gnn_gcn_workspace_size() bytes. */
size_t gnn_gcn_workspace_size(gnn_graph_t g, int64_t d_in, int64_t d_out);
gnn_status_t gnn_gcn_layer_fwd(gnn_graph_t g, const void* X, gnn_dtype_t x_dt, int64_t ldx, int64_t d_in,
                               const float* W, int64_t d_out, int relu, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                               void* saved, void* ws, size_t ws_bytes, void* stream);

/* Its backward.  G = dY * [Y > 0] (ReLU'(0) = 0) when relu, else dY.
 *   GEMM-first:      dZ = A_hat^T G;  dW = X^T dZ;  dX = dZ W^T
 *   aggregate-first: dW = (A_hat X)^T G;  dX = A_hat^T (G W^T)
 * A_hat^T is applied over the CSR view when the graph was built with
 * GNN_GRAPH_SYMMETRIZE (A_hat^T = A_hat), otherwise over the CSC view
 * (GNN_ERR_GRAPH without one: a graph that is not symmetrised, such as the
 * parts gnn_graph_split returns, needs GNN_GRAPH_CSC for the backward).
 * dY, Y [n, ldy] of y_dt; dX [n, ldx] of x_dt (NULL:
 * not formed); dW [d_in, d_out] f32.  relu_in = 1 says X is itself a ReLU
 * output: dX is then returned times [X > 0], the gradient with respect to
 * the previous layer's pre-activation, and that layer's backward is called
 * with relu = 0 (this fuses the mask into the last kernel of this call). */
gnn_status_t gnn_gcn_layer_bwd(gnn_graph_t g, const void* X, gnn_dtype_t x_dt, int64_t ldx, int64_t d_in,
                               const float* W, int64_t d_out, int relu, int relu_in, const void* Y, const void* dY,
                               gnn_dtype_t y_dt, int64_t ldy, const void* saved, void* dX, float* dW, void* ws,
                               size_t ws_bytes, void* stream);

/* GraphSAGE layer with the mean aggregator in AdaQP's weighted-sum form
 * (Eqn. 1 with alpha_{u,v} = 1/|{v} u N(v)|): Y = sigma(M X W), M = the mean
 * operator (GNN_W_MEAN weights).  Same arguments, operand-order rule, saved
 * tensor and workspace as the GCN layer; the backward applies M^T and needs
 * the CSC view (M is not symmetric). */
size_t gnn_sage_workspace_size(gnn_graph_t g, int64_t d_in, int64_t d_out);
gnn_status_t gnn_sage_layer_fwd(gnn_graph_t g, const void* X, gnn_dtype_t x_dt, int64_t ldx, int64_t d_in,
                                const float* W, int64_t d_out, int relu, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                                void* saved, void* ws, size_t ws_bytes, void* stream);
gnn_status_t gnn_sage_layer_bwd(gnn_graph_t g, const void* X, gnn_dtype_t x_dt, int64_t ldx, int64_t d_in,
                                const float* W, int64_t d_out, int relu, int relu_in, const void* Y, const void* dY,
                                gnn_dtype_t y_dt, int64_t ldy, const void* saved, void* dX, float* dW, void* ws,
                                size_t ws_bytes, void* stream);

/* GAT layer forward (Tango, Fig. 1a):  H' = X W;  S = H' a_src, D = H' a_dst
 * per head;  E = LReLU(S[src] + D[dst]);  alpha = edge softmax(E);
 * Y[v, head k] = sum_in alpha[e,k] H'[u, head k] (heads concatenated, no bias,
 * no output activation).  X [n, d_in] f32, W [d_in, heads*d_head] f32,
 * a_src, a_dst [heads, d_head] f32, Y [n, heads*d_head] f32.
 * The edge part runs as one pass over each destination's in-edges: S[src] is
 * formed from the gathered row H'[src] (the same binary32 operations as the
 * stored S, so the same E), and the softmax is folded into the weighted sum
 * with a running maximum (the same quotient); alpha itself is not stored.
 * saved: gnn_gat_saved_size() bytes holding H' [n, heads*d_head], S, D,
 * each destination's softmax maximum M and Z = 1 / sum_in exp(E - M) per head
 * ([n, heads] each), in that order, each slice starting on a 256-byte
 * boundary; the attention weights are alpha[e,k] = exp(E[e,k] - M[dst,k]) *
 * Z[dst,k].  Needs the CSC view only for the backward.  Shapes: 1, 2, 4 or 8
 * heads, d_head a power of two from 4 to 256 and heads * d_head <= 1024
 * (GNN_ERR_UNSUPPORTED otherwise, before anything is launched); Y, a_src,
 * a_dst and saved 16-byte aligned (GNN_ERR_INVALID_ARG otherwise). */
size_t gnn_gat_saved_size(gnn_graph_t g, int heads, int64_t d_head);
size_t gnn_gat_workspace_size(gnn_graph_t g, int64_t d_in, int heads, int64_t d_head);
gnn_status_t gnn_gat_layer_fwd(gnn_graph_t g, const float* X, int64_t d_in, const float* W, const float* a_src,
                               const float* a_dst, int heads, int64_t d_head, float slope, float* Y, void* saved,
                               void* ws, size_t ws_bytes, void* stream);

/* GAT layer backward (Tango, Fig. 1b):
 *   dalpha[e] = dY[dst] . H'[src] per head            (SDDMM dot)
 *   dE = alpha (dalpha - P[dst]),  P = sum_in alpha dalpha,  then LReLU'
 *   dD[v] = sum_in(v) dE,  dS[u] = sum_out(u) dE       (edge -> node sums)
 *   dH' = (G . alpha)^T dY + dS a_src + dD a_dst        (SpMM on the CSC view)
 *   da_src[k] = sum_v dS[v,k] H'[v, head k], likewise da_dst
 *   dW = X^T dH',  dX = dH' W^T  (dX nullable).
 * Y is the forward's output [n, heads*d_head]: since Y[v] = sum_in alpha H'[u],
 * P[v, k] = <dY[v, head k], Y[v, head k]>, a row product taken before any
 * dE, which lets the SDDMM dot, dE, dS and the transposed SpMM run as one
 * pass over the out-edges (alpha formed again from S, D, M, Z).  Requires the
 * CSC view, 1, 2, 4 or 8 heads and d_head a power of two from 4 to 256
 * (GNN_ERR_UNSUPPORTED otherwise); Y, dY, a_src, a_dst and saved 16-byte
 * aligned (GNN_ERR_INVALID_ARG otherwise). */
gnn_status_t gnn_gat_layer_bwd(gnn_graph_t g, const float* X, int64_t d_in, const float* W, const float* a_src,
                               const float* a_dst, int heads, int64_t d_head, float slope, const float* Y,
                               const float* dY, const void* saved, float* dX, float* dW, float* da_src,
                               float* da_dst, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Kernel timers (measurement of this library's own kernels; not an
 * operation of the pages).  For callers that report the duration of one
 * kernel inside a larger step, e.g. a roofline fraction: while timing is on,
 * each instrumented launch whose key equals `key` (every instrumented launch
 * when key is NULL or "") is bracketed by two HIP events recorded on the
 * stream it is launched on.  Keys name the kernel and its shape, e.g.
 * "spmm_kernel d=256 h=1 f32->f32 csr", "gat_bwd_csc_kernel h=4 dh=64",
 * "attn_fwd_kernel h=4", "gemm M=... N=... K=... ta=0 tb=0 f32,f32->f32".
 *   gnn_timer_start   creates a pool of 2*capacity events (host call; events
 *                     are created here, never while launches are timed),
 *                     clears earlier records and turns timing on.
 *   gnn_timer_stop    turns timing off (records are kept).
 *   gnn_timer_result  waits for the recorded events of `key` and returns the
 *                     number of timed launches and their summed duration in
 *                     ms; GNN_ERR_WORKSPACE when launches were dropped
 *                     because the pool was full.
 *   gnn_timer_keys    every key launched while timing was on, one per line
 *                     (buf: host, len bytes incl. the terminating NUL).
 *   gnn_timer_release destroys the pool.
 * Timing is process-wide (one pool, guarded by a lock); the event records
 * add a few microseconds per timed launch to the stream. */
gnn_status_t gnn_timer_start(const char* key, int64_t capacity);
gnn_status_t gnn_timer_stop(void);
gnn_status_t gnn_timer_result(const char* key, int64_t* launches, double* total_ms);
gnn_status_t gnn_timer_keys(char* buf, size_t len);
gnn_status_t gnn_timer_release(void);

#ifdef __cplusplus
}
#endif
#endif /* GNNMP_H */
