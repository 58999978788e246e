// gemm_q8.hip -- Tango's quantisation-aware GEMM on the CDNA4 int8 matrix
// cores (Tango, SC'23, "novel quantization-aware matrix multiplication" and
// "GEMM with on-the-fly quantization"): both operands quantised symmetric,
// tensor-level and dynamic to int8 (the quantiser is in quant.hip), products
// accumulated exactly in int32, and the result dequantised in the epilogue,
// C = f32(acc) * (s_A * s_B).  Tango's DP4A on V100 becomes
// v_mfma_i32_16x16x64_i8 here (64 k values per instruction).
//
//  * the tensor-wide maxima |A|, |B| come from a two-stage max reduction
//    (order free, so the result is exact and deterministic; a contiguous
//    operand is read as one run of 16-byte loads);
//  * the quantised copies are k-contiguous, rows padded with zero codes to a
//    multiple of 64 k, so the GEMM needs no k bounds;
//  * a 256-thread workgroup computes a 128 x 128 tile of C, its four waves
//    64 x 64 each as 4 x 4 blocks of 16 x 16; 64-byte k slabs are
//    double-buffered in LDS (rows of 80 bytes: the 16-byte fragment reads of
//    16 consecutive rows hit distinct banks); lane l supplies the 16 k values
//    16(l/16) .. +15 of its row of both operands, and the transposed tile
//    leaves it four consecutive columns of one row of C for the epilogue.

#include <algorithm>

#include "device.h"
#include "internal.h"

namespace gnnmp {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int QBM = 128, QBN = 128, QBK = 64, QPAD = 16;

__device__ __forceinline__ float absmax4(float m, float4 v) {
    return fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
}

__global__ __launch_bounds__(256) void absmax_stage1(const float* X, int64_t ld, int64_t rows, int64_t cols,
                                                     float* partial) {
    __shared__ float sh[4];
    float m = 0.0f;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nthr = static_cast<int64_t>(gridDim.x) * 256;
    if (ld == cols && (reinterpret_cast<uintptr_t>(X) & 15) == 0) {
        // one contiguous run of rows * cols floats: 16-byte loads, eight in
        // flight per thread, then the tail
        const int64_t total = rows * cols, n4 = total / 4;
        const float4* X4 = reinterpret_cast<const float4*>(X);
        int64_t i = tid;
        for (; i + 7 * nthr < n4; i += 8 * nthr) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = X4[i + u * nthr];
#pragma unroll
            for (int u = 0; u < 8; ++u) m = absmax4(m, v[u]);
        }
        for (; i < n4; i += nthr) m = absmax4(m, X4[i]);
        for (int64_t j = n4 * 4 + tid; j < total; j += nthr) m = fmaxf(m, fabsf(X[j]));
    } else {
        // strided rows: dealt round-robin to the waves, columns across the lanes
        const int lane = threadIdx.x & 63;
        for (int64_t r = tid >> 6; r < rows; r += nthr >> 6) {
            const float* x = X + r * ld;
            for (int64_t c = lane; c < cols; c += 64) m = fmaxf(m, fabsf(x[c]));
        }
    }
    m = group_max<64>(m);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

__global__ __launch_bounds__(256) void absmax_stage2(const float* partial, int n, float* out) {
    __shared__ float sh[4];
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, partial[i]);
    m = group_max<64>(m);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) out[0] = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

struct Q8Args {
    int64_t M, N, Kp;
    const int8_t* A;   // [M][Kp]
    const int8_t* B;   // [N][Kp] (B transposed: k-contiguous)
    const float* s;    // s[0] = s_A, s[1] = s_B
    float* C;
    int64_t ldc;
    int64_t tiles_n, nblocks, per_xcd;
    int vec_c;
};

__global__ __launch_bounds__(256) void gemm_q8_kernel(Q8Args g) {
    constexpr int ROW = QBK + QPAD;  // bytes per LDS row
    __shared__ __align__(16) int8_t As[2][QBM * ROW];
    __shared__ __align__(16) int8_t Bs[2][QBN * ROW];
    const int64_t bid = blockIdx.x;
    const int64_t L = (bid % 8) * g.per_xcd + bid / 8;  // XCD-aware: neighbouring tiles on one XCD
    if (L >= g.nblocks) return;
    const int64_t m0 = (L / g.tiles_n) * QBM, n0 = (L % g.tiles_n) * QBN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // piece p of a slab: row (tid + 256p) / 4, 16-byte chunk (tid % 4)
    v4i ra[2], rb[2];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int q = tid + 256 * p, r = q >> 2, c = (q & 3) * 16;
            const int64_t ma = m0 + r, nb = n0 + r;
            ra[p] = ma < g.M ? *reinterpret_cast<const v4i*>(g.A + ma * g.Kp + k0 + c) : v4i{0, 0, 0, 0};
            rb[p] = nb < g.N ? *reinterpret_cast<const v4i*>(g.B + nb * g.Kp + k0 + c) : v4i{0, 0, 0, 0};
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int q = tid + 256 * p, r = q >> 2, c = (q & 3) * 16;
            *reinterpret_cast<v4i*>(&As[buf][r * ROW + c]) = ra[p];
            *reinterpret_cast<v4i*>(&Bs[buf][r * ROW + c]) = rb[p];
        }
    };

    const int64_t nslab = g.Kp / QBK;
    if (nslab > 0) {
        load(0);
        store(0);
    }
    __syncthreads();
    const int koff = 16 * (lane >> 4);
    for (int64_t s = 0; s < nslab; ++s) {
        const int buf = static_cast<int>(s & 1);
        if (s + 1 < nslab) load((s + 1) * QBK);
        v4i af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const v4i*>(&As[buf][(wm * 64 + i * 16 + (lane & 15)) * ROW + koff]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = *reinterpret_cast<const v4i*>(&Bs[buf][(wn * 64 + j * 16 + (lane & 15)) * ROW + koff]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf[j], af[i], acc[i][j], 0, 0, 0);
        if (s + 1 < nslab) store(buf ^ 1);
        __syncthreads();
    }

    // dequantise: C = f32(acc) * (s_A * s_B), two roundings (the product of
    // the scales, then the product with the converted sum)
    const float scale = __fmul_rn(g.s[0], g.s[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 64 + i * 16 + (lane & 15);
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t nb = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = __fmul_rn(static_cast<float>(acc[i][j][r]), scale);
            float* c = g.C + m * g.ldc + nb;
            if (nb + 4 <= g.N && g.vec_c) {
                *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < g.N) c[r] = v[r];
            }
        }
    }
}

}  // namespace

int64_t q8_padded_k(int64_t K) { return (K + QBK - 1) / QBK * QBK; }

gnn_status_t launch_absmax(const float* X, int64_t ld, int64_t rows, int64_t cols, float* partial, float* out,
                           hipStream_t st) {
    hipLaunchKernelGGL(absmax_stage1, dim3(512), dim3(256), 0, st, X, ld, rows, cols, partial);
    hipLaunchKernelGGL(absmax_stage2, dim3(1), dim3(256), 0, st, partial, 512, out);
    return launch_status("8-bit quantisation (maxima)");
}

size_t gemm_q8_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t Kp = q8_padded_k(K);
    return align_up(static_cast<size_t>(M) * Kp) + align_up(static_cast<size_t>(N) * Kp) + align_up(1024 * 4) +
           align_up(4 * 4);
}

gnn_status_t launch_gemm_q8(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                            float* C, int64_t ldc, uint64_t seed, uint32_t stream_id, void* ws, hipStream_t st) {
    const int64_t Kp = q8_padded_k(K);
    char* w = static_cast<char*>(ws);
    int8_t* Aq = reinterpret_cast<int8_t*>(w);
    w += align_up(static_cast<size_t>(M) * Kp);
    int8_t* Bq = reinterpret_cast<int8_t*>(w);
    w += align_up(static_cast<size_t>(N) * Kp);
    float* partial = reinterpret_cast<float*>(w);
    w += align_up(1024 * 4);
    float* stat = reinterpret_cast<float*>(w);  // [max|A|, max|B|, s_A, s_B]
    // tensor-wide maxima (512 partial blocks per operand)
    GNN_TRY(launch_absmax(A, lda, M, K, partial, stat + 0, st));
    GNN_TRY(launch_absmax(B, ldb, K, N, partial + 512, stat + 1, st));
    // quantised copies: A as is, B transposed, both k-contiguous with zero padding
    GNN_TRY(launch_quantize_sym8(A, lda, M, K, stat + 0, seed, stream_id, Aq, Kp, 0, stat + 2, st));
    GNN_TRY(launch_quantize_sym8(B, ldb, K, N, stat + 1, seed, stream_id + 1, Bq, Kp, 1, stat + 3, st));
    Q8Args g;
    g.M = M, g.N = N, g.Kp = Kp;
    g.A = Aq, g.B = Bq, g.s = stat + 2;
    g.C = C, g.ldc = ldc;
    g.tiles_n = (N + QBN - 1) / QBN;
    g.nblocks = ((M + QBM - 1) / QBM) * g.tiles_n;
    g.per_xcd = (g.nblocks + 7) / 8;
    g.vec_c = ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0;
    if (g.nblocks > 0) hipLaunchKernelGGL(gemm_q8_kernel, dim3(8 * g.per_xcd), dim3(256), 0, st, g);
    return launch_status("gnn_gemm_q8");
}

}  // namespace gnnmp
