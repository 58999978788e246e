/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the per-layer
 * GNN message-passing path.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * code, header or constant with the HIP library: it is written directly from
 * the definitions on the pages.
 *
 * Conventions
 *   - The graph is CSR by destination: row v lists the sources u of the edges
 *     u -> v (Tango, GAT running example: a destination aggregates its
 *     in-edges; the edge score is S[src] + D[dst]).
 *   - Edge arrays are [nnz, heads] in CSR order.
 *   - Floating-point inputs and sums are double (binary32 inputs convert
 *     exactly); results are returned as double and the Python side rounds
 *     them to the storage type at the store points.
 *   - The steps whose result the method fixes in single precision (the
 *     quantiser and the dequantiser) are computed in IEEE binary32 with one
 *     rounding per operation (built with -ffp-contract=off, no fast-math).
 *   - OpenMP splits only independent output rows, so every result is the
 *     same at any thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

/* Thread count of the row-parallel loops (results do not depend on it). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------------------
 * Aggregation as a sparse-dense product (SpMM).
 *
 * AdaQP (arXiv 2306.01381), Sec. 2.1, Eqn. 1-3: the aggregation of node v is
 * the weighted sum over its neighbours, sum_u alpha_uv h_u, with v itself in
 * the sum.  Tango (SC'23), GAT running example, step "H(l) = (G . alpha) H'":
 * a multi-head weighted SpMM in which head k of an edge scales feature block
 * k of the source row.
 *
 *   Y[v, f] = sum_{e in row v} w[e, f / (d/heads)] * X[col[e], f]
 *
 * w == NULL means every edge weight is 1 (the "ones" SpMM of the edge
 * softmax).  Y is [n, d] double, dense.
 * ------------------------------------------------------------------------- */
void orc_spmm(int64_t n, const int64_t* row_ptr, const int32_t* col,
              const double* w, int heads, const double* X, int64_t ldx,
              int64_t d, double* Y)
{
    const int64_t dh = d / heads;
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t v = 0; v < n; ++v) {
        double* y = Y + v * d;
        for (int64_t f = 0; f < d; ++f) y[f] = 0.0;
        for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e) {
            const double* x = X + (int64_t)col[e] * ldx;
            for (int64_t f = 0; f < d; ++f) {
                double we = w ? w[e * heads + f / dh] : 1.0;
                y[f] += we * x[f];
            }
        }
    }
}

/* SDDMM with the "dot" operator: out[e, k] = <A[v, head k], B[u, head k]>
 * for edge e = (u -> v).  Tango uses it for the attention gradient
 * d(alpha)[e] = dH(l)[dst] . H'[src] (quantised SDDMM paragraph, "dot"). */
void orc_sddmm_dot(int64_t n, const int64_t* row_ptr, const int32_t* col,
                   const double* A, int64_t lda, const double* B, int64_t ldb,
                   int heads, int64_t dh, double* out)
{
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t v = 0; v < n; ++v) {
        const double* a = A + v * lda;
        for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e) {
            const double* b = B + (int64_t)col[e] * ldb;
            for (int k = 0; k < heads; ++k) {
                double s = 0.0;
                for (int64_t j = 0; j < dh; ++j)
                    s += a[k * dh + j] * b[k * dh + j];
                out[e * heads + k] = s;
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Edge softmax over the in-edges of each destination, per head.
 *
 * Tango, GAT running example, softmax step: alpha = exp(E) / E', where E' is
 * the per-destination sum of exp(E) broadcast back to the in-edges.  The
 * per-(v, k) maximum is subtracted first; that leaves the quotient unchanged.
 * ------------------------------------------------------------------------- */
void orc_edge_softmax(int64_t n, const int64_t* row_ptr, const double* E,
                      int heads, double* alpha)
{
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t v = 0; v < n; ++v) {
        for (int k = 0; k < heads; ++k) {
            double m = -INFINITY, s = 0.0;
            for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e)
                if (E[e * heads + k] > m) m = E[e * heads + k];
            for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e)
                s += exp(E[e * heads + k] - m);
            for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e)
                alpha[e * heads + k] = exp(E[e * heads + k] - m) / s;
        }
    }
}

/* Edge-softmax backward.  Tango, GAT running example, backward (Fig. 1b):
 * P[v] = sum over in-edges of alpha * d(alpha); dE = alpha * (d(alpha) - P[dst]). */
void orc_edge_softmax_bwd(int64_t n, const int64_t* row_ptr, const double* alpha,
                          const double* dalpha, int heads, double* dE)
{
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t v = 0; v < n; ++v) {
        for (int k = 0; k < heads; ++k) {
            double P = 0.0;
            for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e)
                P += alpha[e * heads + k] * dalpha[e * heads + k];
            for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e)
                dE[e * heads + k] = alpha[e * heads + k] *
                                    (dalpha[e * heads + k] - P);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Edge -> node sums (the "ones" SpMM / incidence-matrix SpMM).
 * Tango, GAT running example: dD = (G . dE) 1 sums the in-edges of each node,
 * dS = (G^T . dE) 1 sums the out-edges; incidence-matrix SpMM paragraph.
 * ------------------------------------------------------------------------- */
void orc_edge_reduce_dst(int64_t n, const int64_t* row_ptr, const double* vals,
                         int heads, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < n; ++v)
        for (int k = 0; k < heads; ++k) {
            double s = 0.0;
            for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e)
                s += vals[e * heads + k];
            out[v * heads + k] = s;
        }
}

void orc_edge_reduce_src(int64_t n, const int64_t* row_ptr, const int32_t* col,
                         const double* vals, int heads, double* out)
{
    memset(out, 0, sizeof(double) * (size_t)(n * heads));
    for (int64_t v = 0; v < n; ++v)
        for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e)
            for (int k = 0; k < heads; ++k)
                out[(int64_t)col[e] * heads + k] += vals[e * heads + k];
}

/* ---------------------------------------------------------------------------
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
 * as 1, 2, 3", SC'11): a counter-based generator.  Each of the 10 rounds
 * multiplies counter words 0 and 2 by two fixed odd constants, takes the high
 * and low halves of the 64-bit products, and mixes them with words 1 and 3
 * and the round key; the key is bumped by two Weyl constants between rounds.
 * ------------------------------------------------------------------------- */
static const uint32_t PHILOX_M0 = 0xD2511F53u, PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t PHILOX_W0 = 0x9E3779B9u, PHILOX_W1 = 0xBB67AE85u;

void orc_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out)
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform of element f of node `node`: counter (node, f/4, stream, 0),
 * key (seed low word, seed high word), output word f mod 4, top 24 bits
 * scaled by 2^-24 (exact in binary32). */
static float philox_uniform(uint64_t seed, uint32_t stream, uint32_t node, uint32_t f)
{
    uint32_t ctr[4] = { node, f >> 2, stream, 0u };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t r[4];
    orc_philox4x32_10(ctr, key, r);
    return (float)(r[f & 3u] >> 8) * (1.0f / 16777216.0f);
}

void orc_philox_uniforms(uint64_t seed, uint32_t stream, const int32_t* nodes,
                         int64_t n_nodes, int64_t d, float* u)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_nodes; ++i)
        for (int64_t f = 0; f < d; ++f)
            u[i * d + f] = philox_uniform(seed, stream, (uint32_t)nodes[i], (uint32_t)f);
}

/* ---------------------------------------------------------------------------
 * Per-row stochastic integer quantisation, AdaQP, background on
 * stochastic integer quantisation, Eqn. 4:
 *   q = round_st((h - Z) / S),  Z = min(h),  S = (max(h) - min(h)) / (2^b - 1).
 * In binary32: R = max - min; inv = (2^b - 1) / R; x = (h - Z) * inv;
 * code = floor(x) + [u < x - floor(x)], clamped to 2^b - 1 (x can round a
 * hair above the top level); S = R / (2^b - 1).  A constant row (R == 0)
 * gets all-zero codes, S = 0.
 * Packing: element j of a row sits in byte j*b/8 at bit (j mod 8/b)*b.
 * Row r of the output is the quantised row rows[r] of H.
 * ------------------------------------------------------------------------- */
void orc_quantize(const float* H, int64_t ldh, int64_t d, const int32_t* rows,
                  int64_t n_rows, int bits, uint64_t seed, uint32_t stream,
                  uint8_t* packed, float* scale, float* zero)
{
    const int64_t row_bytes = d * bits / 8;
    const uint32_t top = (1u << bits) - 1u;
    const float levels = (float)top;
    const int per_byte = 8 / bits;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int32_t node = rows[r];
        const float* h = H + (int64_t)node * ldh;
        uint8_t* out = packed + r * row_bytes;
        /* min and max of the row; of two equal zeros the minimum is -0 and
         * the maximum +0, so the result does not depend on the scan order */
        float mn = h[0], mx = h[0];
        for (int64_t f = 1; f < d; ++f) {
            if (h[f] < mn || (h[f] == mn && signbit(h[f]))) mn = h[f];
            if (h[f] > mx || (h[f] == mx && !signbit(h[f]))) mx = h[f];
        }
        const float R = mx - mn;
        memset(out, 0, (size_t)row_bytes);
        zero[r] = mn;
        if (R == 0.0f) { scale[r] = 0.0f; continue; }
        const float inv = levels / R;
        scale[r] = R / levels;
        for (int64_t f = 0; f < d; ++f) {
            float t = h[f] - mn;
            float x = t * inv;
            float fl = floorf(x);
            float frac = x - fl;
            float u = philox_uniform(seed, stream, (uint32_t)node, (uint32_t)f);
            uint32_t code = (uint32_t)fl + (u < frac ? 1u : 0u);
            if (code > top) code = top;
            out[f / per_byte] |= (uint8_t)(code << ((f % per_byte) * bits));
        }
    }
}

/* Dequantisation, AdaQP, same background passage, Eqn. 5: the linear inverse map
 * h_hat = q * S + Z, one correctly rounded fused multiply-add, written into
 * row rows[r] of H (other rows untouched). */
void orc_dequantize(const uint8_t* packed, const float* scale, const float* zero,
                    int64_t n_rows, int64_t d, int bits, const int32_t* rows,
                    float* H, int64_t ldh)
{
    const int64_t row_bytes = d * bits / 8;
    const uint32_t mask = (1u << bits) - 1u;
    const int per_byte = 8 / bits;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        const uint8_t* in = packed + r * row_bytes;
        float* h = H + (int64_t)rows[r] * ldh;
        for (int64_t f = 0; f < d; ++f) {
            uint32_t q = (in[f / per_byte] >> ((f % per_byte) * bits)) & mask;
            h[f] = fmaf((float)q, scale[r], zero[r]);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Tango (SC'23), quantisation background and the quantisation-aware GEMM:
 * symmetric, tensor-level, dynamic 8-bit quantisation with stochastic
 * rounding.  m = max |X| over the whole tensor, s = m / 127; a value maps to
 * x = X * (127 / m) in [-127, 127] and rounds stochastically,
 * q = floor(x) + [u < x - floor(x)], clamped to [-127, 127]; X ~ q * s.
 * In binary32 with one rounding per operation.  The uniform of element
 * (r, c) is the Philox draw of counter (r, c/4, stream, 0), word c mod 4.
 * m == 0 gives q = 0 and s = 0.  q is [rows, cols] row-major.
 * ------------------------------------------------------------------------- */
void orc_quantize_sym8(const float* X, int64_t ldx, int64_t rows, int64_t cols,
                       uint64_t seed, uint32_t stream, int8_t* q, float* s)
{
    float m = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(X[r * ldx + c]);
            if (a > m) m = a;
        }
    *s = m / 127.0f;
    if (m == 0.0f) {
        memset(q, 0, (size_t)(rows * cols));
        *s = 0.0f;
        return;
    }
    const float inv = 127.0f / m;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float x = X[r * ldx + c] * inv;
            float fl = floorf(x);
            float frac = x - fl;
            float u = philox_uniform(seed, stream, (uint32_t)r, (uint32_t)c);
            int32_t v = (int32_t)fl + (u < frac ? 1 : 0);
            if (v > 127) v = 127;
            if (v < -127) v = -127;
            q[r * cols + c] = (int8_t)v;
        }
}
