// quant.hip -- per-row stochastic integer quantisation and dequantisation of
// exchanged message rows (AdaQP, arXiv 2306.01381, Eqn. 4 and 5).
//
// Quantise, row r (node rows[r]) with b bits:
//   Z = min(h), R = max(h) - min(h), inv = (2^b - 1)/R, S = R/(2^b - 1)
//   x = (h - Z) * inv,  q = min(floor(x) + [u < x - floor(x)], 2^b - 1)
// every operation an IEEE binary32 operation with one rounding (no
// contraction), so the codes agree bit for bit with any other faithful
// implementation.  u comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11): counter
// (node, f/4, stream, 0), key (seed low, seed high), word f%4, top 24 bits
// times 2^-24.  Stateless, so a rerun draws the same numbers.
//
// One wave per row.  Lane l owns feature quads l, l + 64, ... (features
// 4l..4l+3, 4l+256.., read as 16-byte vectors when the rows allow); one Philox
// call yields exactly the four uniforms of a quad, and a quad's codes fill
// b/2 whole bytes (2-bit: 1 byte, 4-bit: 2, 8-bit: 4), so each lane writes
// its own bytes with one store and the row is written contiguously.
// Dequantise: h = fma(q, S, Z), one rounding.

#include "device.h"
#include "internal.h"

// Built with -ffp-contract=off (see build.py): a fused t*inv - floor(x)
// would change codes.
#pragma clang fp contract(off)

namespace gnnmp {

namespace {

constexpr int kMaxQuads = 4;  // d <= 1024

struct U4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                            uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // one 32 x 32 -> 64-bit product per multiplier (a single
        // v_mad_u64_u32, where separate low and high halves take two
        // multiplies)
        const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0, p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
        const uint32_t lo0 = static_cast<uint32_t>(p0), hi0 = static_cast<uint32_t>(p0 >> 32);
        const uint32_t lo1 = static_cast<uint32_t>(p1), hi1 = static_cast<uint32_t>(p1 >> 32);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0, c1 = lo1, c2 = n2, c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return U4{c0, c1, c2, c3};
}

// minimum / maximum with -0 < +0, so the result is independent of the order
// in which the row is scanned
__device__ __forceinline__ float min_z(float a, float b) { return (b < a || (b == a && signbit(b))) ? b : a; }
__device__ __forceinline__ float max_z(float a, float b) { return (b > a || (b == a && !signbit(b))) ? b : a; }

__device__ __forceinline__ float u24(uint32_t w) { return static_cast<float>(w >> 8) * (1.0f / 16777216.0f); }

// NQ = feature quads per lane (d <= 256 NQ); RW rows per wave (two for rows
// of at most 256 features, so two rows' loads are in flight at once).  The
// rows' loads are issued first and the lane's Philox blocks computed while
// they are in flight (the uniforms do not depend on the data); a flat row
// ignores them.
template <int NQ, int RW>
__global__ __launch_bounds__(256) void quantize_kernel(const float* H, int64_t ldh, int64_t d, const int32_t* rows,
                                                       int64_t n_rows, int bits, uint32_t k0, uint32_t k1,
                                                       uint32_t stream_id, uint8_t* packed, float* scale,
                                                       float* zero, int vec) {
    const int lane = threadIdx.x & 63;
    const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RW;
    if (r0 >= n_rows) return;
    const int64_t nq = (d + 3) / 4;
    uint32_t node[RW];
    float x[RW][NQ][4];
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        const bool on = r0 + k < n_rows;
        node[k] = on ? static_cast<uint32_t>(rows[r0 + k]) : 0u;
        const float* h = H + static_cast<int64_t>(node[k]) * ldh;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int64_t q = lane + 64 * i;
            if (on && vec && 4 * q + 4 <= d) {
                const float4 t = *reinterpret_cast<const float4*>(h + 4 * q);
                x[k][i][0] = t.x, x[k][i][1] = t.y, x[k][i][2] = t.z, x[k][i][3] = t.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) x[k][i][j] = (on && q < nq && 4 * q + j < d) ? h[4 * q + j] : 0.0f;
            }
        }
    }
    U4 rnd[RW][NQ];
#pragma unroll
    for (int k = 0; k < RW; ++k)
#pragma unroll
        for (int i = 0; i < NQ; ++i)
            rnd[k][i] = philox4x32_10(node[k], static_cast<uint32_t>(lane + 64 * i), stream_id, 0u, k0, k1);
    float mn[RW], mx[RW];
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        mn[k] = INFINITY, mx[k] = -INFINITY;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int64_t q = lane + 64 * i;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (q < nq && 4 * q + j < d) {
                    mn[k] = min_z(mn[k], x[k][i][j]);
                    mx[k] = max_z(mx[k], x[k][i][j]);
                }
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
        for (int k = 0; k < RW; ++k) {
            mn[k] = min_z(mn[k], __shfl_xor(mn[k], o, 64));
            mx[k] = max_z(mx[k], __shfl_xor(mx[k], o, 64));
        }
    }
    const uint32_t top = (1u << bits) - 1u;
    const float levels = static_cast<float>(top);
    const int64_t row_bytes = d * bits / 8;
    const bool wide = (row_bytes % 4 == 0) && (reinterpret_cast<uintptr_t>(packed) % 4 == 0);
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        const int64_t r = r0 + k;
        if (r >= n_rows) break;
        const float R = __fsub_rn(mx[k], mn[k]);
        const bool flat = !(R != 0.0f);
        const float inv = flat ? 0.0f : __fdiv_rn(levels, R);
        if (lane == 0) {
            zero[r] = mn[k];
            scale[r] = flat ? 0.0f : __fdiv_rn(R, levels);
        }
        uint8_t* out = packed + r * row_bytes;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int64_t q = lane + 64 * i;
            if (q >= nq) break;
            uint32_t code[4] = {0u, 0u, 0u, 0u};
            if (!flat) {
                const uint32_t w[4] = {rnd[k][i].x, rnd[k][i].y, rnd[k][i].z, rnd[k][i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float t = __fsub_rn(x[k][i][j], mn[k]);
                    const float xs = __fmul_rn(t, inv);
                    const float fl = floorf(xs);
                    const float frac = __fsub_rn(xs, fl);
                    uint32_t c = static_cast<uint32_t>(fl) + (u24(w[j]) < frac ? 1u : 0u);
                    code[j] = c > top ? top : c;
                }
            }
            const int64_t nvalid = min<int64_t>(4, d - 4 * q);
            if (bits == 8) {
                if (nvalid == 4 && wide) {
                    *reinterpret_cast<uint32_t*>(out + 4 * q) =
                        code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
                } else {
                    for (int j = 0; j < nvalid; ++j) out[4 * q + j] = static_cast<uint8_t>(code[j]);
                }
            } else if (bits == 4) {
                const uint32_t lo = code[0] | (code[1] << 4), hi = code[2] | (code[3] << 4);
                if (nvalid == 4 && wide) {
                    *reinterpret_cast<uint16_t*>(out + 2 * q) = static_cast<uint16_t>(lo | (hi << 8));
                } else {
                    out[2 * q] = static_cast<uint8_t>(lo);  // d even: a partial quad holds 2 features
                    if (nvalid == 4) out[2 * q + 1] = static_cast<uint8_t>(hi);
                }
            } else {
                out[q] = static_cast<uint8_t>(code[0] | (code[1] << 2) | (code[2] << 4) | (code[3] << 6));
            }
        }
    }
}

__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* packed, const float* scale, const float* zero,
                                                         int64_t n_rows, int64_t d, int bits, const int32_t* rows,
                                                         float* H, int64_t ldh) {
    const int lane = threadIdx.x & 63;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;
    const float S = scale[r], Z = zero[r];
    const int64_t row_bytes = d * bits / 8;
    const uint8_t* in = packed + r * row_bytes;
    float* h = H + static_cast<int64_t>(rows[r]) * ldh;
    const int64_t nq = (d + 3) / 4;
    const uint32_t mask = (1u << bits) - 1u;
    const bool vec = (ldh % 4 == 0) && (reinterpret_cast<uintptr_t>(H) % 16 == 0);
    const bool wide = (row_bytes % 4 == 0) && (reinterpret_cast<uintptr_t>(packed) % 4 == 0);
    for (int64_t q = lane; q < nq; q += 64) {
        const int64_t nvalid = min<int64_t>(4, d - 4 * q);
        uint32_t word;
        if (bits == 8) {
            if (nvalid == 4 && wide) word = *reinterpret_cast<const uint32_t*>(in + 4 * q);
            else {
                word = 0;
                for (int j = 0; j < nvalid; ++j) word |= static_cast<uint32_t>(in[4 * q + j]) << (8 * j);
            }
        } else if (bits == 4) {
            if (nvalid == 4 && wide) word = *reinterpret_cast<const uint16_t*>(in + 2 * q);
            else word = static_cast<uint32_t>(in[2 * q]) | (nvalid == 4 ? static_cast<uint32_t>(in[2 * q + 1]) << 8 : 0u);
        } else {
            word = in[q];
        }
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = __fmaf_rn(static_cast<float>((word >> (j * bits)) & mask), S, Z);
        if (vec && nvalid == 4) {
            *reinterpret_cast<float4*>(h + 4 * q) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
            for (int j = 0; j < nvalid; ++j) h[4 * q + j] = o[j];
        }
    }
}

// Bit-width statistics of AdaQP Sec. 3.2 (the beta_k of Problem 11): for
// listed row r (node k = rows[r]) the range R = max(h_k) - min(h_k) and
//   beta = (sum over k's edges of alpha^2) * D * R^2 / 6,
// alpha the edge's GCN weight.  One wave per row: the row's features for
// the range (minimum and maximum as the quantiser takes them, so R is the
// quantiser's R bit for bit), then the squared weights of the node's edges.
__global__ __launch_bounds__(256) void quant_stats_kernel(const float* H, int64_t ldh, int64_t d,
                                                          const int32_t* rows, int64_t n_rows, const int64_t* ptr,
                                                          const int32_t* eid, const float* w, float* beta,
                                                          float* range) {
    const int lane = threadIdx.x & 63;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;
    const int64_t k = rows[r];
    const float* h = H + k * ldh;
    float mn = INFINITY, mx = -INFINITY;
    for (int64_t f = lane; f < d; f += 64) {
        const float x = h[f];
        mn = min_z(mn, x);
        mx = max_z(mx, x);
    }
    float s2 = 0.0f;
    for (int64_t e = ptr[k] + lane; e < ptr[k + 1]; e += 64) {
        const float a = w[eid ? static_cast<int64_t>(eid[e]) : e];
        s2 = __fmaf_rn(a, a, s2);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = min_z(mn, __shfl_xor(mn, o, 64));
        mx = max_z(mx, __shfl_xor(mx, o, 64));
        s2 = __fadd_rn(s2, __shfl_xor(s2, o, 64));
    }
    if (lane == 0) {
        const float R = __fsub_rn(mx, mn);
        range[r] = R;
        beta[r] = __fdiv_rn(__fmul_rn(__fmul_rn(s2, static_cast<float>(d)), __fmul_rn(R, R)), 6.0f);
    }
}

// Tango's symmetric, tensor-level, dynamic 8-bit quantisation (quantisation
// background section) with stochastic rounding: m = max|X| (computed before,
// read from device memory), x = X * (127 / m), q = floor(x) + [u < x -
// floor(x)] clamped to [-127, 127], s = m / 127 (m == 0: q = 0, s = 0).
// u is the Philox draw of counter (r, c/4, stream, 0), word c mod 4 -- one
// call per thread covers four consecutive columns.  The output is
// k-contiguous with out_ld >= the k extent, the padding filled with zero
// codes: transpose = 0 writes out[r][c] (k = c), transpose = 1 writes
// out[c][r] (k = r).
__global__ __launch_bounds__(256) void quantize_sym8_kernel(const float* X, int64_t ldx, int64_t rows, int64_t cols,
                                                            const float* mptr, uint32_t k0, uint32_t k1,
                                                            uint32_t stream_id, int8_t* out, int64_t out_ld,
                                                            int transpose, int64_t rows_ext, int64_t cq,
                                                            float* s_out) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (t >= rows_ext * cq) return;
    const int64_t r = t / cq, c4 = (t % cq) * 4;
    const float m = *mptr;
    if (t == 0) s_out[0] = m == 0.0f ? 0.0f : __fdiv_rn(m, 127.0f);
    int q[4] = {0, 0, 0, 0};
    if (r < rows && c4 < cols && m != 0.0f) {
        const float inv = __fdiv_rn(127.0f, m);
        const U4 rnd = philox4x32_10(static_cast<uint32_t>(r), static_cast<uint32_t>(c4 >> 2), stream_id, 0u, k0, k1);
        const uint32_t w[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
        float xin[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        const float* xr = X + r * ldx + c4;
        if (c4 + 4 <= cols && (reinterpret_cast<uintptr_t>(xr) & 15) == 0) {
            const float4 v = *reinterpret_cast<const float4*>(xr);
            xin[0] = v.x, xin[1] = v.y, xin[2] = v.z, xin[3] = v.w;
        } else {
            for (int j = 0; j < 4 && c4 + j < cols; ++j) xin[j] = xr[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (c4 + j >= cols) break;
            const float x = __fmul_rn(xin[j], inv);
            const float fl = floorf(x);
            const float frac = __fsub_rn(x, fl);
            int v = static_cast<int>(fl) + (u24(w[j]) < frac ? 1 : 0);
            q[j] = v > 127 ? 127 : (v < -127 ? -127 : v);
        }
    }
    if (!transpose) {
        if (r < rows) {
            const uint32_t packed = (static_cast<uint32_t>(q[0]) & 0xFFu) | ((static_cast<uint32_t>(q[1]) & 0xFFu) << 8) |
                                    ((static_cast<uint32_t>(q[2]) & 0xFFu) << 16) |
                                    ((static_cast<uint32_t>(q[3]) & 0xFFu) << 24);
            *reinterpret_cast<uint32_t*>(out + r * out_ld + c4) = packed;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (c4 + j < cols) out[(c4 + j) * out_ld + r] = static_cast<int8_t>(q[j]);
    }
}

__global__ __launch_bounds__(256) void slots_fill_kernel(int64_t n, int32_t* qslot) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) qslot[i] = -1;
}

__global__ __launch_bounds__(256) void slots_scatter_kernel(const int32_t* rows, int64_t count, int32_t tag,
                                                            int32_t* qslot) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (r < count) qslot[rows[r]] = tag | static_cast<int32_t>(r);
}

}  // namespace

gnn_status_t launch_quant_stats(const AggView& v, const float* w, const float* H, int64_t ldh, int64_t d,
                                const int32_t* rows, int64_t n_rows, float* beta, float* range, hipStream_t st) {
    if (n_rows == 0) return GNN_OK;
    hipLaunchKernelGGL(quant_stats_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, st, H, ldh, d, rows, n_rows, v.ptr,
                       v.eid, w, beta, range);
    return launch_status("gnn_quant_stats");
}

// rows x cols f32 -> int8 codes, k-contiguous; k extent padded to out_ld
gnn_status_t launch_quantize_sym8(const float* X, int64_t ldx, int64_t rows, int64_t cols, const float* mptr,
                                  uint64_t seed, uint32_t stream_id, int8_t* out, int64_t out_ld, int transpose,
                                  float* s_out, hipStream_t st) {
    // non-transposed: every row, columns up to out_ld (zero padding);
    // transposed: rows (k) up to out_ld, columns in quads
    const int64_t rows_ext = transpose ? out_ld : rows;
    const int64_t cq = transpose ? (cols + 3) / 4 : out_ld / 4;
    const int64_t total = rows_ext * cq;
    if (total > 0)
        hipLaunchKernelGGL(quantize_sym8_kernel, dim3((total + 255) / 256), dim3(256), 0, st, X, ldx, rows, cols, mptr,
                           static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), stream_id, out, out_ld,
                           transpose, rows_ext, cq, s_out);
    return launch_status("8-bit symmetric quantisation");
}

// Slot map of the dequantise-in-gather aggregation: -1 everywhere, then
// (group << 27) | r at rows_g[r].  Groups are scattered one launch after the
// other on the same stream, so a node listed in two groups keeps the later.
gnn_status_t launch_quant_slots(int64_t n, int n_groups, const int32_t* const* rows, const int64_t* counts,
                                int32_t* qslot, hipStream_t st) {
    if (n > 0) hipLaunchKernelGGL(slots_fill_kernel, dim3((n + 255) / 256), dim3(256), 0, st, n, qslot);
    for (int g = 0; g < n_groups; ++g)
        if (counts[g] > 0)
            hipLaunchKernelGGL(slots_scatter_kernel, dim3((counts[g] + 255) / 256), dim3(256), 0, st, rows[g],
                               counts[g], static_cast<int32_t>(g) << 27, qslot);
    return launch_status("gnn_quant_slots");
}

gnn_status_t launch_quantize(const float* H, int64_t ldh, int64_t d, const int32_t* rows, int64_t n_rows, int bits,
                             uint64_t seed, uint32_t stream_id, uint8_t* packed, float* scale, float* zero,
                             hipStream_t st) {
    if (n_rows == 0) return GNN_OK;
    if (d > 64 * 4 * kMaxQuads) return fail(GNN_ERR_UNSUPPORTED, "gnn_quantize: d must be at most 1024");
    const int64_t blocks = (n_rows + 3) / 4;
    const int vec = ldh % 4 == 0 && reinterpret_cast<uintptr_t>(H) % 16 == 0;
    const int nq4 = static_cast<int>(((d + 3) / 4 + 63) / 64);  // quads per lane
    ScopedTimer t(st, "quantize_kernel b=%d d=%lld", bits, static_cast<long long>(d));
#define GNN_Q(NQv, RWv, BLK)                                                                                         \
    hipLaunchKernelGGL((quantize_kernel<NQv, RWv>), dim3(BLK), dim3(256), 0, st, H, ldh, d, rows, n_rows, bits,    \
                       static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), stream_id, packed, scale, zero, \
                       vec)
    switch (nq4) {
        case 1: GNN_Q(1, 2, (n_rows + 7) / 8); break;
        case 2: GNN_Q(2, 1, blocks); break;
        case 3: GNN_Q(3, 1, blocks); break;
        default: GNN_Q(4, 1, blocks); break;
    }
#undef GNN_Q
    return launch_status("gnn_quantize");
}

gnn_status_t launch_dequantize(const uint8_t* packed, const float* scale, const float* zero, int64_t n_rows,
                               int64_t d, int bits, const int32_t* rows, float* H, int64_t ldh, hipStream_t st) {
    if (n_rows == 0) return GNN_OK;
    const int64_t blocks = (n_rows + 3) / 4;
    ScopedTimer t(st, "dequantize_kernel b=%d d=%lld", bits, static_cast<long long>(d));
    hipLaunchKernelGGL(dequantize_kernel, dim3(blocks), dim3(256), 0, st, packed, scale, zero, n_rows, d, bits, rows,
                       H, ldh);
    return launch_status("gnn_dequantize");
}

}  // namespace gnnmp
