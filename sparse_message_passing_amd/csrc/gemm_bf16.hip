// gemm_bf16.hip -- the weight gradient dW = X^T dZ with both operands stored
// as bfloat16 (the bf16-storage GCN's backward; AdaQP Eqn. 3's update, its
// gradient), on gfx950's bf16 matrix cores, v_mfma_f32_16x16x32_bf16.
//
// C[m][n] = sum_k A[k][m] B[k][n] over K = the number of nodes (A = X or the
// saved aggregate, B = the layer's output gradient), M, N = the two widths.
// Both operands are k-major in memory (a node's row is contiguous), while the
// instruction takes eight consecutive k of one row of each operand per lane.
// So each slab of BK = 32 nodes is written to LDS transposed: a thread loads
// eight consecutive m (16 bytes) of two consecutive nodes and writes the
// eight (node, node + 1) pairs as eight 4-byte LDS stores into [m][k] rows;
// every lane then reads its eight k of one row with a single 16-byte LDS
// read.  Products of bf16 values are exact in binary32 and accumulate in
// binary32, so only the summation order differs from any other faithful
// product.  The K range is split over workgroups (the output is small and
// K is the node count); each split writes a binary32 partial tile and the
// fixed-order reduction of the f32 path adds them: no atomics, bitwise
// reproducible.
//
// Tile: 128 x 128 of C per 256-thread workgroup, four waves of 64 x 64, each
// a 4 x 4 grid of 16 x 16 MFMA blocks; two LDS buffers and two slabs of
// global loads in flight (each split runs a few hundred slabs back to back,
// so memory latency, not the matrix cores, sets the pace).

#include "device.h"
#include "internal.h"

namespace gnnmp {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int TBM = 128, TBN = 128, TBK = 32;

struct TnArgs {
    int64_t M, N, K;
    const bf16_t* A;  // [K][lda]
    int64_t lda;
    const bf16_t* B;  // [K][ldb]
    int64_t ldb;
    float* part;      // [splits][M][N]
    int64_t kper;     // nodes per split (multiple of TBK)
    int64_t tiles_m, tiles_n, nblocks, per_xcd;
};

// LDS tile [rows][TBK] bf16, rows of 64 bytes with the four 16-byte k chunks
// of row r permuted by (r / 8) mod 4 (element (r, k) in chunk
// (k / 8) ^ ((r / 8) & 3)): a wave's 4-byte transposing stores then spread
// over the banks four lanes deep instead of sixteen, and its 16-byte
// fragment reads stay conflict-free.
__device__ __forceinline__ int lds_at(int r, int k) { return r * TBK + (((k >> 3) ^ ((r >> 3) & 3)) << 3) + (k & 7); }

// eight bf16 of row k, columns c..c+7 (zero outside [0, K) x [0, C))
__device__ __forceinline__ uint4 load8(const bf16_t* X, int64_t ld, int64_t k, int64_t kend, int64_t c, int64_t C) {
    if (k >= kend) return make_uint4(0u, 0u, 0u, 0u);
    const bf16_t* p = X + k * ld + c;
    if (c + 8 <= C) return *reinterpret_cast<const uint4*>(p);
    uint16_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = c + i < C ? p[i] : 0;
    return make_uint4(v[0] | (uint32_t(v[1]) << 16), v[2] | (uint32_t(v[3]) << 16), v[4] | (uint32_t(v[5]) << 16),
                      v[6] | (uint32_t(v[7]) << 16));
}

// the eight (node k, node k + 1) pairs of columns c..c+7 into LDS rows c..c+7
__device__ __forceinline__ void store_pairs(bf16_t* S, int c, int k, uint4 r0, uint4 r1) {
    const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w}, b[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        *reinterpret_cast<uint32_t*>(S + lds_at(c + 2 * h, k)) = (a[h] & 0xFFFFu) | (b[h] << 16);
        *reinterpret_cast<uint32_t*>(S + lds_at(c + 2 * h + 1, k)) = (a[h] >> 16) | (b[h] & 0xFFFF0000u);
    }
}

struct Slab {  // one thread's share of a slab of both operands
    uint4 a0, a1, b0, b1;
};

__global__ __launch_bounds__(256) void gemm_tn_bf16_kernel(TnArgs g) {
    __shared__ __attribute__((aligned(16))) bf16_t As[2][TBM * TBK];
    __shared__ __attribute__((aligned(16))) bf16_t Bs[2][TBN * TBK];
    const int64_t bid = blockIdx.x;
    const int64_t L = (bid % 8) * g.per_xcd + bid / 8;  // XCD-aware: an XCD's blocks take a contiguous range
    if (L >= g.nblocks) return;
    const int64_t tiles = g.tiles_m * g.tiles_n;
    const int64_t split = L / tiles;
    const int64_t t = L % tiles;
    const int64_t m0 = (t / g.tiles_n) * TBM, n0 = (t % g.tiles_n) * TBN;
    const int64_t kbeg = split * g.kper;
    const int64_t kend = min(g.K, kbeg + g.kper);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // this thread's piece of a slab: columns c..c+7 of nodes 2kp, 2kp + 1
    // (sixteen consecutive threads read one node's 256 contiguous bytes)
    const int c = (tid & 15) * 8, kp = tid >> 4;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    auto load = [&](Slab& x, int64_t k0) {
        const int64_t k = k0 + 2 * kp;  // nodes at or past kend read as zero
        x.a0 = load8(g.A, g.lda, k, kend, m0 + c, g.M);
        x.a1 = load8(g.A, g.lda, k + 1, kend, m0 + c, g.M);
        x.b0 = load8(g.B, g.ldb, k, kend, n0 + c, g.N);
        x.b1 = load8(g.B, g.ldb, k + 1, kend, n0 + c, g.N);
    };
    auto store = [&](int buf, const Slab& x) {
        store_pairs(As[buf], c, 2 * kp, x.a0, x.a1);
        store_pairs(Bs[buf], c, 2 * kp, x.b0, x.b1);
    };
    auto compute = [&](int buf) {
        // lane l: row l % 16 of a block, k = 8 (l / 16) .. + 7 (one 16-byte read)
        const int r = lane & 15, kq = 8 * (lane >> 4);
        bf16x8 af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][lds_at(wm * 64 + i * 16 + r, kq)]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][lds_at(wn * 64 + j * 16 + r, kq)]);
        // B's rows as the instruction's first operand, A's as its second: the
        // block computed is C^T, so lane l ends holding C[m = l % 16][n = 4 (l / 16) + q]
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    };

    // Two slabs of loads in flight: LDS buffer 0 holds slab s and register
    // set r1 slab s + 1 at the top of each trip, which handles two slabs; the
    // slab count is rounded up to even (the padding slab reads as zeros).
    const int64_t nslab = (kend - kbeg + TBK - 1) / TBK;
    const int64_t ns = (nslab + 1) & ~int64_t(1);
    Slab r0, r1;
    if (ns > 0) {
        load(r0, kbeg);
        store(0, r0);
        load(r1, kbeg + TBK);
    }
    __syncthreads();
    for (int64_t s = 0; s < ns; s += 2) {
        if (s + 2 < ns) load(r0, kbeg + (s + 2) * TBK);
        compute(0);
        store(1, r1);
        __syncthreads();
        if (s + 3 < ns) load(r1, kbeg + (s + 3) * TBK);
        compute(1);
        if (s + 2 < ns) store(0, r0);
        __syncthreads();
    }

    // the split's partial tile: lane l holds C[m][nb .. nb + 3] of each block
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 64 + i * 16 + (lane & 15);
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t nb = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
            float* w = g.part + (split * g.M + m) * g.N + nb;
            if (nb + 4 <= g.N && g.N % 4 == 0) {
                *reinterpret_cast<float4*>(w) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (nb + q < g.N) w[q] = acc[i][j][q];
            }
        }
    }
}

}  // namespace

bool gemm_tn_bf16_supported(int64_t lda, int64_t ldb, const void* A, const void* B) {
    return lda % 8 == 0 && ldb % 8 == 0 && reinterpret_cast<uintptr_t>(A) % 16 == 0 &&
           reinterpret_cast<uintptr_t>(B) % 16 == 0;
}

gnn_status_t launch_gemm_tn_bf16(int64_t M, int64_t N, int64_t K, const bf16_t* A, int64_t lda, const bf16_t* B,
                                 int64_t ldb, float* part, int64_t splits, int64_t kper, hipStream_t st) {
    TnArgs g;
    g.M = M, g.N = N, g.K = K;
    g.A = A, g.lda = lda, g.B = B, g.ldb = ldb;
    g.part = part;
    g.kper = kper;
    g.tiles_m = (M + TBM - 1) / TBM;
    g.tiles_n = (N + TBN - 1) / TBN;
    g.nblocks = g.tiles_m * g.tiles_n * splits;
    g.per_xcd = (g.nblocks + 7) / 8;
    hipLaunchKernelGGL(gemm_tn_bf16_kernel, dim3(8 * g.per_xcd), dim3(256), 0, st, g);
    return launch_status("gnn_gemm (bf16 weight gradient)");
}

}  // namespace gnnmp
