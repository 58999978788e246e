// gemm.hip -- dense products on the CDNA4 matrix cores.
//
// The update step H W (AdaQP Eqn. 3; Sancus Sec. 2; Tango's GEMM step
// "H' = H(l-1) W") and its backward dW = H^T dZ, dH = dZ W^T.
//
// Design (gfx950, wave64, v_mfma_f32_16x16x4_f32):
//  * a workgroup of WM x WN waves computes a BM x BN tile of C (four waves;
//    eight for the deep f32 NN products, below); each wave owns
//    (BM/WM) x (BN/WN) as a grid of 16x16 MFMA blocks held in accumulation
//    registers;
//  * K advances in slabs of 16 through double-buffered LDS; each operand
//    keeps its global contiguity in LDS (k-contiguous rows, or k-major
//    planes), so every global->LDS store is a 16-byte write; the next slab's
//    global loads are issued before the current slab's MFMAs and its LDS
//    stores after them, one barrier per slab;
//  * the weight-gradient products (A transposed, K = number of nodes) and
//    the products with a bf16 A use a second instantiation whose interior
//    tiles keep two slabs of loads in flight (registers for slab s + 1 and
//    s + 2), so a load has two slabs of MFMAs to arrive instead of one; it
//    holds more registers (two waves per SIMD instead of three), which loses
//    on the f32 NN updates with four waves;
//  * the f32 NN products with K >= 256 (the GAT layer's H' = XW and dX =
//    dH' W^T, the GCN's 256-deep updates) and the f32 weight gradients split
//    the 128 x 128 tile over eight waves of 64 x 32 instead, which fits the
//    two-slab pipeline in four waves per SIMD (2^21 x 256 x 256: 2.54 ->
//    2.44-2.50 ms, with the rank-1 term 2.83 -> 2.66-2.70 ms; the 256 x 256
//    weight gradient over 2^20 rows 1.12 -> 1.07 ms); shallower NN products
//    keep four waves (a 128-deep update lost with eight: 0.75 -> 0.86 ms);
//  * operand fragments: in MFMA j of a slab, lane l supplies
//    B[k0 + 4(l/16) + j][n0 + l%16] as the instruction's first operand and
//    A[m0 + l%16][k0 + 4(l/16) + j] as its second, so a k-contiguous
//    operand's four values come from one 16-byte LDS read, and the block
//    computed is the transposed tile: lane l ends holding C[m0 + l%16][n0 +
//    4(l/16) + r], r = 0..3, four consecutive columns of one row, stored with
//    one 16-byte write;
//  * interior tiles load full slabs from running offsets with no per-element
//    checks; only edge tiles and the last partial slab take the checked path;
//  * the workgroup -> tile map keeps the tiles that share rows of A on one XCD
//    (workgroups are dealt round-robin over the 8 XCDs, each with its own L2);
//  * tall reductions (K = number of nodes, for dW) are split over K; each
//    split writes a binary32 partial tile and a second pass adds the splits
//    in order.  No atomics: bitwise reproducible;
//  * an operand may carry a per-head rank-1 term, X[r][c] + s[r, head of c]
//    v[c], formed with one fmaf as each piece goes to LDS (a compile-time
//    variant, so other products keep their registers): the GAT backward's
//    dD a_dst term of dH', which otherwise costs a read and a write of all of
//    dH' (2^21 x 256 f32: the in-edge pass 1.92 -> 0.90 ms, the dX product
//    2.54 -> 2.85 ms, the dW product unchanged; results bitwise the same).

#include <algorithm>
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace gnnmp {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef short bf16x4 __attribute__((ext_vector_type(4)));

// four widened bf16 values back to bf16 (exact: their low 16 bits are zero)
__device__ __forceinline__ bf16x4 to_bf16x4(const float (&v)[4]) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = static_cast<short>(__float_as_uint(v[i]) >> 16);
    return r;
}

constexpr int BK = 16;
// LDS padding.  k-contiguous tiles: rows of BK + 4 = 20 floats, so the
// 16-byte fragment reads of 8 consecutive lanes (rows r..r+7) cover the 32
// banks once.  k-major planes: rows of (BM or BN) + 4 floats, so the k rows
// 4g + j that lane groups g = 0, 1 (and 2, 3) read at the same time start
// 16 banks apart.
constexpr int PAD = 4;
constexpr int PADM = 4;

struct GemmArgs {
    int64_t M, N, K;
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    void* C;
    int64_t ldc;
    float* ws;       // split-K partials [splits][M][N]
    int64_t kper;    // K range per split (multiple of BK)
    int splits;
    int64_t tiles_m, tiles_n;
    int64_t nblocks; // real work items (tiles * splits)
    int64_t per_xcd; // ceil(nblocks / 8)
    int relu;        // ReLU epilogue (applied after the split-K sum)
    int vec_c;       // C rows take 16-byte (bf16: 8-byte) stores
    int vec_mask;    // mask rows take 16-byte (bf16: 8-byte) loads
    int vec_ws;      // split-K partial rows (stride N) take 16-byte stores
    MaskEpilogue mask;  // C *= [M > 0] (after the split-K sum)
    OperandRank1 r1;    // kernels with R1 = 1: A (stored [M][K]) read as A + s v, s per (row m, head of k);
                        // R1 = 2: B (stored [K][N]) read as B + s v, s per (row k, head of n)
};

__device__ __forceinline__ bool mask_on(const MaskEpilogue& m, int64_t r, int64_t c) {
    if (!m.M) return true;
    if (m.dt == GNN_BF16) return Elem<bf16_t>::load(static_cast<const bf16_t*>(m.M) + r * m.ld + c) > 0.0f;
    return Elem<float>::load(static_cast<const float*>(m.M) + r * m.ld + c) > 0.0f;
}

// Piece q of a k-contiguous slab (rows x BK): four consecutive lanes take the
// four k quads of one row, so each 16-lane quarter of a load instruction
// reads four whole 64-byte row pieces (a quarter of sixteen rows at one quad
// each, the earlier mapping, touched four times as many cache lines per
// instruction: 1-3% slower across the products measured).
__device__ __forceinline__ int kc_row(int q) { return q >> 2; }
__device__ __forceinline__ int kc_k(int q) { return (q & 3) * 4; }

template <typename T, bool VEC>
__device__ __forceinline__ void load4(const T* base, int64_t off, bool full, int valid, float (&r)[4]) {
    if (VEC && full) {
        float4 t = Elem<T>::load4(base + off);
        r[0] = t.x, r[1] = t.y, r[2] = t.z, r[3] = t.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = i < valid ? Elem<T>::load(base + off + i) : 0.0f;
    }
}

// The rank-1 term of a piece (stored row r, columns c..c+3, c a multiple of
// 4 and so inside one head): its coefficient s[r, c / dh] and the four v[c + i]
// are loaded with the piece, and added with one fmaf per element when the
// piece is written to LDS, so the piece's global load is not waited for any
// earlier than without the term.  Elements past the operand's edge get w = 0
// or v = 0 (and are zero themselves): they stay zero.
template <int NP>
struct Rank1Regs {
    float w[NP];
    float v[NP][4];
};

__device__ __forceinline__ void rank1_v(const OperandRank1& o, int64_t c, int valid, float (&v)[4]) {
    if (valid == 4) {
        const float4 t = *reinterpret_cast<const float4*>(o.v + c);
        v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = i < valid ? o.v[c + i] : 0.0f;
    }
}

__device__ __forceinline__ float rank1_w(const OperandRank1& o, int64_t r, int64_t c, int valid) {
    return valid > 0 ? o.s[r * o.ld + (c >> o.dh_log2)] : 0.0f;
}

// TRANS_A: A given as [K][lda] (element (m,k) at A[k*lda+m]); else [M][lda].
// TRANS_B: B given as [N][ldb] (element (k,n) at B[n*ldb+k]); else [K][ldb].
// R1: 0, or the operand (1: A, 2: B) that carries the rank-1 term g.r1.
template <int BM, int BN, int WM, int WN, bool TRANS_A, bool TRANS_B, bool VA, bool VB, bool PF, typename TA,
          typename TB, typename TC, int R1 = 0>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(GemmArgs g) {
    constexpr int NT = WM * WN * 64;  // threads
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int A_LOADS = BM * BK / 4 / NT;  // float4-sized pieces per thread
    constexpr int B_LOADS = BN * BK / 4 / NT;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small");
    static_assert(R1 == 0 || (R1 == 1 && !TRANS_A) || (R1 == 2 && !TRANS_B), "rank-1 term on an untransposed operand");
    constexpr int R1N = R1 == 1 ? A_LOADS : R1 == 2 ? B_LOADS : 1;
    // An operand contiguous along k is kept k-contiguous in LDS ([rows][BK+PAD]),
    // one contiguous along m / n is kept k-major ([BK][rows+PAD]): either way the
    // global->LDS store is one 16-byte write per thread and piece, and the
    // fragment reads of 16 consecutive rows hit distinct banks.  Two buffers:
    // the next slab is written while the current one is read.
    constexpr bool A_KC = !TRANS_A, B_KC = TRANS_B;
    constexpr bool kBf16Pair = std::is_same<TA, bf16_t>::value && std::is_same<TB, bf16_t>::value;
    constexpr int A_SZ = A_KC ? BM * (BK + PAD) : BK * (BM + PADM);
    constexpr int B_SZ = B_KC ? BN * (BK + PAD) : BK * (BN + PADM);
    __shared__ float As[2][A_SZ];
    __shared__ float Bs[2][B_SZ];

    // XCD-aware tile map: the blocks dealt to one XCD take a contiguous range
    const int64_t bid = blockIdx.x;
    const int64_t L = (bid % 8) * g.per_xcd + bid / 8;
    if (L >= g.nblocks) return;
    const int64_t tiles = g.tiles_m * g.tiles_n;
    const int64_t split = L / tiles;
    const int64_t t = L % tiles;
    const int64_t tm = t / g.tiles_n, tn = t % g.tiles_n;
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t kbeg = split * g.kper;
    const int64_t kend = min(g.K, kbeg + g.kper);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const TA* A = static_cast<const TA*>(g.A);
    const TB* B = static_cast<const TB*>(g.B);

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    float ra[A_LOADS][4], rb[B_LOADS][4];
    float ra1[A_LOADS][4], rb1[B_LOADS][4];  // slab s + 1 while s + 2 loads (PF)
    Rank1Regs<R1N> rr, rr1;                  // the rank-1 terms of those two register sets
    // With the term on B, a thread's pieces all cover columns n0 + 4 (tid % (BN / 4)) .. + 3 in every slab,
    // so their v is loaded once (zero past column N).
    float vb_r1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (R1 == 2) {
        const int64_t c = n0 + (tid % (BN / 4)) * 4;
        rank1_v(g.r1, c, static_cast<int>(max<int64_t>(0, min<int64_t>(4, g.N - c))), vb_r1);
    }

    // Interior tiles (every row / column of the tile in range, 16-byte
    // aligned operands) load full slabs without per-element checks, from
    // per-thread offsets that advance by one slab per call.
    const bool a_full = VA && m0 + BM <= g.M;
    const bool b_full = VB && n0 + BN <= g.N;
    int64_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
    for (int p = 0; p < A_LOADS; ++p) {
        const int q = tid + p * NT;
        if constexpr (!TRANS_A) a_off[p] = (m0 + kc_row(q)) * g.lda + kbeg + kc_k(q);
        else a_off[p] = (kbeg + q / (BM / 4)) * g.lda + m0 + (q % (BM / 4)) * 4;
    }
#pragma unroll
    for (int p = 0; p < B_LOADS; ++p) {
        const int q = tid + p * NT;
        if constexpr (!TRANS_B) b_off[p] = (kbeg + q / (BN / 4)) * g.ldb + n0 + (q % (BN / 4)) * 4;
        else b_off[p] = (n0 + kc_row(q)) * g.ldb + kbeg + kc_k(q);
    }
    const int64_t a_step = TRANS_A ? BK * g.lda : BK;
    const int64_t b_step = TRANS_B ? BK : BK * g.ldb;

    auto load_slab = [&](int64_t k0) {
        const bool full_k = k0 + BK <= kend;
#pragma unroll
        for (int p = 0; p < A_LOADS; ++p) {
            const int q = tid + p * NT;
            if (a_full && full_k) {
                load4<TA, true>(A, a_off[p], true, 4, ra[p]);
                if constexpr (R1 == 1) {  // the pieces of a thread share their columns k0 + kc_k(tid)
                    rr.w[p] = rank1_w(g.r1, m0 + kc_row(q), k0 + kc_k(q), 4);
                    if (p == 0) rank1_v(g.r1, k0 + kc_k(q), 4, rr.v[0]);
                    else
#pragma unroll
                        for (int i = 0; i < 4; ++i) rr.v[p][i] = rr.v[0][i];
                }
            } else if constexpr (!TRANS_A) {  // contiguous along k: q -> (m, k4)
                const int mm = kc_row(q), kk = kc_k(q);
                const int64_t m = m0 + mm, k = k0 + kk;
                const int valid = (m < g.M) ? static_cast<int>(max<int64_t>(0, min<int64_t>(4, kend - k))) : 0;
                load4<TA, VA>(A, m * g.lda + k, valid == 4, valid, ra[p]);
                if constexpr (R1 == 1) {  // edge tiles and slabs: always reloaded
                    rr.w[p] = rank1_w(g.r1, m, k, valid);
                    rank1_v(g.r1, k, valid, rr.v[p]);
                }
            } else {                   // contiguous along m: q -> (k, m4)
                const int kk = q / (BM / 4), mm = (q % (BM / 4)) * 4;
                const int64_t m = m0 + mm, k = k0 + kk;
                const int valid = (k < kend) ? static_cast<int>(max<int64_t>(0, min<int64_t>(4, g.M - m))) : 0;
                load4<TA, VA>(A, k * g.lda + m, valid == 4, valid, ra[p]);
            }
            a_off[p] += a_step;
        }
#pragma unroll
        for (int p = 0; p < B_LOADS; ++p) {
            const int q = tid + p * NT;
            if (b_full && full_k) {
                load4<TB, true>(B, b_off[p], true, 4, rb[p]);
                if constexpr (R1 == 2) rr.w[p] = rank1_w(g.r1, k0 + q / (BN / 4), n0 + (q % (BN / 4)) * 4, 4);
            } else if constexpr (!TRANS_B) {  // contiguous along n: q -> (k, n4)
                const int kk = q / (BN / 4), nn = (q % (BN / 4)) * 4;
                const int64_t n = n0 + nn, k = k0 + kk;
                const int valid = (k < kend) ? static_cast<int>(max<int64_t>(0, min<int64_t>(4, g.N - n))) : 0;
                load4<TB, VB>(B, k * g.ldb + n, valid == 4, valid, rb[p]);
                if constexpr (R1 == 2) rr.w[p] = rank1_w(g.r1, k, n, valid);
            } else {                   // contiguous along k: q -> (n, k4)
                const int nn = kc_row(q), kk = kc_k(q);
                const int64_t n = n0 + nn, k = k0 + kk;
                const int valid = (n < g.N) ? static_cast<int>(max<int64_t>(0, min<int64_t>(4, kend - k))) : 0;
                load4<TB, VB>(B, n * g.ldb + k, valid == 4, valid, rb[p]);
            }
            b_off[p] += b_step;
        }
    };
    auto store_slab = [&](int buf) {
        if constexpr (R1 == 1) {
#pragma unroll
            for (int p = 0; p < A_LOADS; ++p)
#pragma unroll
                for (int i = 0; i < 4; ++i) ra[p][i] = fmaf(rr.w[p], rr.v[p][i], ra[p][i]);
        }
        if constexpr (R1 == 2) {
#pragma unroll
            for (int p = 0; p < B_LOADS; ++p)
#pragma unroll
                for (int i = 0; i < 4; ++i) rb[p][i] = fmaf(rr.w[p], vb_r1[i], rb[p][i]);
        }
#pragma unroll
        for (int p = 0; p < A_LOADS; ++p) {
            const int q = tid + p * NT;
            if constexpr (A_KC) {
                const int mm = kc_row(q), kk = kc_k(q);
                *reinterpret_cast<float4*>(&As[buf][mm * (BK + PAD) + kk]) =
                    make_float4(ra[p][0], ra[p][1], ra[p][2], ra[p][3]);
            } else {
                const int kk = q / (BM / 4), mm = (q % (BM / 4)) * 4;
                *reinterpret_cast<float4*>(&As[buf][kk * (BM + PADM) + mm]) =
                    make_float4(ra[p][0], ra[p][1], ra[p][2], ra[p][3]);
            }
        }
#pragma unroll
        for (int p = 0; p < B_LOADS; ++p) {
            const int q = tid + p * NT;
            if constexpr (B_KC) {
                const int nn = kc_row(q), kk = kc_k(q);
                *reinterpret_cast<float4*>(&Bs[buf][nn * (BK + PAD) + kk]) =
                    make_float4(rb[p][0], rb[p][1], rb[p][2], rb[p][3]);
            } else {
                const int kk = q / (BN / 4), nn = (q % (BN / 4)) * 4;
                *reinterpret_cast<float4*>(&Bs[buf][kk * (BN + PADM) + nn]) =
                    make_float4(rb[p][0], rb[p][1], rb[p][2], rb[p][3]);
            }
        }
    };

    const int64_t nslab = (kend - kbeg + BK - 1) / BK;
    // the MFMAs of the slab held in LDS buffer buf
    auto compute = [&](const int buf) {
        // Fragments of the whole slab.  MFMA j of the slab takes k = 4g + j from
        // lane group g = lane / 16 (any assignment of the slab's 16 k values to
        // (j, g) pairs gives the same products, as long as A and B agree), so a
        // k-contiguous operand is read with one 16-byte LDS load per row and
        // slab, and a k-major one with four 4-byte loads.
        const int g4 = 4 * (lane >> 4);
        float af[FM][4], bfr[FN][4];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * TM + i * 16 + (lane & 15);
            if constexpr (A_KC) {
                const float4 t = *reinterpret_cast<const float4*>(&As[buf][row * (BK + PAD) + g4]);
                af[i][0] = t.x, af[i][1] = t.y, af[i][2] = t.z, af[i][3] = t.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) af[i][j] = As[buf][(g4 + j) * (BM + PADM) + row];
            }
        }
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
            const int col = wn * TN + jj * 16 + (lane & 15);
            if constexpr (B_KC) {
                const float4 t = *reinterpret_cast<const float4*>(&Bs[buf][col * (BK + PAD) + g4]);
                bfr[jj][0] = t.x, bfr[jj][1] = t.y, bfr[jj][2] = t.z, bfr[jj][3] = t.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) bfr[jj][j] = Bs[buf][(g4 + j) * (BN + PADM) + col];
            }
        }
        if constexpr (kBf16Pair) {
            // Both operands stored as bf16: the slab's 16 k values go through
            // one bf16 MFMA per block (lane group g supplies k = 4g..4g+3, the
            // instruction's own layout).  bf16 x bf16 products are exact in
            // binary32 and accumulate in binary32, so only the summation order
            // differs from the f32 path.  The LDS holds the widened values; the
            // top 16 bits of each are the bf16 it came from.
            bf16x4 ab[FM], bb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) ab[i] = to_bf16x4(af[i]);
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) bb[jj] = to_bf16x4(bfr[jj]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int jj = 0; jj < FN; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bb[jj], ab[i], acc[i][jj], 0, 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int jj = 0; jj < FN; ++jj)
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(bfr[jj][j], af[i][j], acc[i][jj], 0, 0, 0);
        }
    };
    // interior tile, whole slabs (PF): unchecked loads from the running
    // offsets into register set x, and that set's LDS stores.  They repeat
    // load_slab / store_slab with the register set as a parameter; routing
    // the one-slab loop through these made the compiler copy registers in
    // every instantiation's loop (the NN update 1.25 -> 1.48 ms).
    int64_t k_full = kbeg;  // first k of the slab load_full reads next
    auto load_full = [&](float (&xa)[A_LOADS][4], float (&xb)[B_LOADS][4], Rank1Regs<R1N>& xr) {
#pragma unroll
        for (int p = 0; p < A_LOADS; ++p) {
            load4<TA, true>(A, a_off[p], true, 4, xa[p]);
            if constexpr (R1 == 1) {
                xr.w[p] = rank1_w(g.r1, m0 + kc_row(tid + p * NT), k_full + kc_k(tid + p * NT), 4);
                if (p == 0) rank1_v(g.r1, k_full + kc_k(tid), 4, xr.v[0]);
                else
#pragma unroll
                    for (int i = 0; i < 4; ++i) xr.v[p][i] = xr.v[0][i];
            }
            a_off[p] += a_step;
        }
#pragma unroll
        for (int p = 0; p < B_LOADS; ++p) {
            load4<TB, true>(B, b_off[p], true, 4, xb[p]);
            if constexpr (R1 == 2)
                xr.w[p] = rank1_w(g.r1, k_full + (tid + p * NT) / (BN / 4), n0 + ((tid + p * NT) % (BN / 4)) * 4, 4);
            b_off[p] += b_step;
        }
        k_full += BK;
    };
    auto store_full = [&](int buf, const float (&xa)[A_LOADS][4], const float (&xb)[B_LOADS][4],
                          const Rank1Regs<R1N>& xr) {
#pragma unroll
        for (int p = 0; p < A_LOADS; ++p) {
            const int q = tid + p * NT;
            float t[4] = {xa[p][0], xa[p][1], xa[p][2], xa[p][3]};
            if constexpr (R1 == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) t[i] = fmaf(xr.w[p], xr.v[p][i], t[i]);
            }
            if constexpr (A_KC) {
                *reinterpret_cast<float4*>(&As[buf][kc_row(q) * (BK + PAD) + kc_k(q)]) =
                    make_float4(t[0], t[1], t[2], t[3]);
            } else {
                *reinterpret_cast<float4*>(&As[buf][(q / (BM / 4)) * (BM + PADM) + (q % (BM / 4)) * 4]) =
                    make_float4(t[0], t[1], t[2], t[3]);
            }
        }
#pragma unroll
        for (int p = 0; p < B_LOADS; ++p) {
            const int q = tid + p * NT;
            float t[4] = {xb[p][0], xb[p][1], xb[p][2], xb[p][3]};
            if constexpr (R1 == 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) t[i] = fmaf(xr.w[p], vb_r1[i], t[i]);
            }
            if constexpr (B_KC) {
                *reinterpret_cast<float4*>(&Bs[buf][kc_row(q) * (BK + PAD) + kc_k(q)]) =
                    make_float4(t[0], t[1], t[2], t[3]);
            } else {
                *reinterpret_cast<float4*>(&Bs[buf][(q / (BN / 4)) * (BN + PADM) + (q % (BN / 4)) * 4]) =
                    make_float4(t[0], t[1], t[2], t[3]);
            }
        }
    };
    if (PF && a_full && b_full && (kend - kbeg) % BK == 0 && nslab >= 2) {
        // Two slabs of loads in flight.  Straight-line code (the loop handles
        // two slabs per trip, each register set with a fixed role) lets the
        // compiler wait for exactly the older slab's loads; the scheduling
        // barriers keep the loads ahead of the MFMAs they overlap.
        load_full(ra, rb, rr);
        store_full(0, ra, rb, rr);
        load_full(ra1, rb1, rr1);
        __syncthreads();
        int64_t s = 0;
        // here LDS buffer 0 holds slab s and (ra1, rb1) slab s + 1
        for (; s + 3 < nslab; s += 2) {
            load_full(ra, rb, rr);  // slab s + 2
            __builtin_amdgcn_sched_barrier(0);
            compute(0);
            store_full(1, ra1, rb1, rr1);
            __syncthreads();
            load_full(ra1, rb1, rr1);  // slab s + 3
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            store_full(0, ra, rb, rr);
            __syncthreads();
        }
        if (s + 3 == nslab) {  // three slabs left
            load_full(ra, rb, rr);
            compute(0);
            store_full(1, ra1, rb1, rr1);
            __syncthreads();
            compute(1);
            store_full(0, ra, rb, rr);
            __syncthreads();
            compute(0);
        } else {  // two slabs left
            compute(0);
            store_full(1, ra1, rb1, rr1);
            __syncthreads();
            compute(1);
        }
    } else {
        if (nslab > 0) {
            load_slab(kbeg);
            store_slab(0);
        }
        __syncthreads();
        for (int64_t s = 0; s < nslab; ++s) {
            const int buf = static_cast<int>(s & 1);
            if (s + 1 < nslab) load_slab(kbeg + (s + 1) * BK);
            compute(buf);
            // the other buffer was last read in iteration s-1, which every wave
            // has left (barrier below), so it can be refilled now
            if (s + 1 < nslab) store_slab(buf ^ 1);
            __syncthreads();
        }
    }

    // epilogue: the block (i, jj) leaves lane l holding C[m][nb + r], r = 0..3
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = m0 + wm * TM + i * 16 + (lane & 15);
        if (m >= g.M) continue;
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
            const int64_t nb = n0 + wn * TN + jj * 16 + 4 * (lane >> 4);
            float v[4] = {acc[i][jj][0], acc[i][jj][1], acc[i][jj][2], acc[i][jj][3]};
            const bool full = nb + 4 <= g.N;
            if (g.splits > 1) {
                float* w = g.ws + (split * g.M + m) * g.N + nb;
                if (full && g.vec_ws) {
                    *reinterpret_cast<float4*>(w) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (nb + r < g.N) w[r] = v[r];
                }
                continue;
            }
            if (g.relu) {
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = fmaxf(v[r], 0.0f);
            }
            if (g.mask.M) {
                float mk[4];
                if (full && g.vec_mask) {
                    float4 t;
                    if (g.mask.dt == GNN_BF16)
                        t = Elem<bf16_t>::load4(static_cast<const bf16_t*>(g.mask.M) + m * g.mask.ld + nb);
                    else
                        t = Elem<float>::load4(static_cast<const float*>(g.mask.M) + m * g.mask.ld + nb);
                    mk[0] = t.x, mk[1] = t.y, mk[2] = t.z, mk[3] = t.w;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) mk[r] = (nb + r < g.N && mask_on(g.mask, m, nb + r)) ? 1.0f : 0.0f;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = mk[r] > 0.0f ? v[r] : 0.0f;
            }
            TC* c = static_cast<TC*>(g.C) + m * g.ldc + nb;
            if (full && g.vec_c) {
                Elem<TC>::store4(c, make_float4(v[0], v[1], v[2], v[3]));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < g.N) Elem<TC>::store(c + r, v[r]);
            }
        }
    }
}

// C = sum over splits in a fixed order: four thread groups each add every
// fourth split (z = g, g+4, ...), then the four sums are added in order.
template <typename TC>
__global__ __launch_bounds__(256) void splitk_reduce(const float* ws, int splits, int64_t M, int64_t N, TC* C,
                                                     int64_t ldc, int relu, MaskEpilogue mask) {
    __shared__ float part[4][64];
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + (threadIdx.x & 63);
    const int grp = threadIdx.x >> 6;
    // split z goes to group z mod 4, and within the group to accumulator
    // (z / 4) mod 4: a fixed order with four loads in flight per thread
    float p4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (i < M * N) {
        int z = grp;
        for (; z + 12 < splits; z += 16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) p4[q] += ws[(z + 4 * q) * M * N + i];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (z + 4 * q < splits) p4[q] += ws[(z + 4 * q) * M * N + i];
    }
    const float s = (p4[0] + p4[1]) + (p4[2] + p4[3]);
    part[grp][threadIdx.x & 63] = s;
    __syncthreads();
    if (grp == 0 && i < M * N) {
        const int t = threadIdx.x;
        float tot = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
        const int64_t r = i / N, c = i % N;
        if (relu) tot = fmaxf(tot, 0.0f);
        if (!mask_on(mask, r, c)) tot = 0.0f;
        Elem<TC>::store(C + r * ldc + c, tot);
    }
}

// out[k][n] = B[n][k]  (B: N rows of K, leading dimension ldb; out: K rows of N)
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* B, int64_t ldb, int64_t N, int64_t K, T* out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= N * K) return;
    const int64_t k = i / N, n = i % N;
    out[i] = B[n * ldb + k];
}

struct Plan {
    int bm, bn, wm, wn;
    int splits;
    int64_t kper;
};

Plan make_plan(int64_t M, int64_t N, int64_t K) {
    Plan p;
    p.splits = 1;
    p.kper = 0;
    if (N <= 64) {
        p.bm = 128, p.bn = 64, p.wm = 4, p.wn = 1;
    } else {
        p.bm = 128, p.bn = 128, p.wm = 2, p.wn = 2;
    }
    if (K <= 0) return p;
    const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
    // split K when there are too few tiles to fill the chip and K is tall
    if (tiles < 512 && K >= 4096) {
        int64_t want = (1024 + tiles - 1) / tiles;
        int64_t maxs = K / 2048;
        p.splits = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(want, std::min<int64_t>(maxs, 512))));
    }
    const int64_t ks = (K + p.splits - 1) / p.splits;
    p.kper = (ks + BK - 1) / BK * BK;
    p.splits = static_cast<int>((K + p.kper - 1) / p.kper);
    if (p.splits < 1) p.splits = 1;
    return p;
}

template <int BM, int BN, int WM, int WN, bool TA_, bool TB_, typename TA, typename TB, typename TC, int R1 = 0>
void launch_shape(GemmArgs& g, bool va, bool vb, hipStream_t st) {
    const int64_t grid = 8 * g.per_xcd;
    // Two slabs of loads in flight for the transposed-A products (weight
    // gradients, K = nodes) and the products with a bf16 A, in 128 x 128
    // tiles.  Measured per launch: f32 weight gradient over 2^20 rows 1.00 ->
    // 0.95 ms, bf16 over 2.45M rows 2.31 -> 1.45 ms, bf16 x f32 update over
    // 2.45M rows 3.09 -> 2.92 ms; the same variant lost on 128 x 64 tiles
    // (0.43 -> 0.72 ms) and on the f32 NN updates in a whole step (1.25 ->
    // 1.30 ms).  The eight-wave f32 tiles (chosen only for vectorisable
    // operands and a K span of 256 or more) always take it.
    if constexpr (WN == 4) {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, TA_, TB_, true, true, true, TA, TB, TC, R1>), dim3(grid),
                           dim3(WM * WN * 64), 0, st, g);
    } else {
        if constexpr ((TA_ || std::is_same<TA, bf16_t>::value) && BN == 128) {
            if (va && vb && (g.splits > 1 ? g.kper : g.K) >= 256) {
                hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, TA_, TB_, true, true, true, TA, TB, TC, R1>),
                                   dim3(grid), dim3(WM * WN * 64), 0, st, g);
                return;
            }
        }
        if (va && vb)
            hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, TA_, TB_, true, true, false, TA, TB, TC, R1>), dim3(grid),
                               dim3(WM * WN * 64), 0, st, g);
        else if (va)
            hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, TA_, TB_, true, false, false, TA, TB, TC, R1>),
                               dim3(grid), dim3(WM * WN * 64), 0, st, g);
        else if (vb)
            hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, TA_, TB_, false, true, false, TA, TB, TC, R1>),
                               dim3(grid), dim3(WM * WN * 64), 0, st, g);
        else
            hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, TA_, TB_, false, false, false, TA, TB, TC, R1>),
                               dim3(grid), dim3(WM * WN * 64), 0, st, g);
    }
}

template <bool TA_, bool TB_, typename TA, typename TB, typename TC, int R1 = 0>
void launch_types(GemmArgs& g, const Plan& p, bool va, bool vb, hipStream_t st) {
    constexpr bool f32 = !TB_ && std::is_same<TB, float>::value &&
                         (std::is_same<TA, float>::value || (!TA_ && std::is_same<TA, bf16_t>::value));
    if (p.bn == 64) {
        launch_shape<128, 64, 4, 1, TA_, TB_, TA, TB, TC, R1>(g, va, vb, st);
    } else {
        bool eight = false;
        if constexpr (f32) {
            eight = va && vb && (TA_ ? (g.splits > 1 ? g.kper : g.K) >= 256 : g.splits == 1 && g.K >= 256);
            if (eight) launch_shape<128, 128, 2, 4, TA_, TB_, TA, TB, TC, R1>(g, va, vb, st);
        }
        if (!eight) launch_shape<128, 128, 2, 2, TA_, TB_, TA, TB, TC, R1>(g, va, vb, st);
    }
    if (g.splits > 1) {
        const int64_t tot = g.M * g.N;
        hipLaunchKernelGGL((splitk_reduce<TC>), dim3((tot + 63) / 64), dim3(256), 0, st, g.ws, g.splits, g.M, g.N,
                           static_cast<TC*>(g.C), g.ldc, g.relu, g.mask);
    }
}

template <bool TA_, bool TB_>
gnn_status_t launch_trans(GemmArgs& g, const Plan& p, gnn_dtype_t a, gnn_dtype_t b, gnn_dtype_t c, bool va, bool vb,
                          int r1, hipStream_t st) {
    // binary32 products with a rank-1 operand term (the host checks the types)
    if constexpr (!TA_) {  // B transposed too when it is too large to transpose in the workspace
        if (r1 == 1) {
            launch_types<TA_, TB_, float, float, float, 1>(g, p, va, vb, st);
            return launch_status("gnn_gemm");
        }
    }
    if constexpr (!TB_) {
        if (r1 == 2) {
            launch_types<TA_, TB_, float, float, float, 2>(g, p, va, vb, st);
            return launch_status("gnn_gemm");
        }
    }
#define GNN_GEMM_CASE(TAt, TBt, TCt)                                                     \
    launch_types<TA_, TB_, TAt, TBt, TCt>(g, p, va, vb, st);                             \
    return launch_status("gnn_gemm");
    if (a == GNN_F32 && b == GNN_F32 && c == GNN_F32) { GNN_GEMM_CASE(float, float, float) }
    if (a == GNN_F32 && b == GNN_F32 && c == GNN_BF16) { GNN_GEMM_CASE(float, float, bf16_t) }
    if (a == GNN_BF16 && b == GNN_F32 && c == GNN_F32) { GNN_GEMM_CASE(bf16_t, float, float) }
    if (a == GNN_BF16 && b == GNN_F32 && c == GNN_BF16) { GNN_GEMM_CASE(bf16_t, float, bf16_t) }
    if (a == GNN_BF16 && b == GNN_BF16 && c == GNN_F32) { GNN_GEMM_CASE(bf16_t, bf16_t, float) }
    if (a == GNN_BF16 && b == GNN_BF16 && c == GNN_BF16) { GNN_GEMM_CASE(bf16_t, bf16_t, bf16_t) }
    if (a == GNN_F32 && b == GNN_BF16 && c == GNN_F32) { GNN_GEMM_CASE(float, bf16_t, float) }
    { GNN_GEMM_CASE(float, bf16_t, bf16_t) }
#undef GNN_GEMM_CASE
}

}  // namespace

// A small B given transposed (a weight matrix in dX = dZ W^T) is transposed
// once into the workspace and the product runs in the NN form, whose
// k-major B tile loads and fragment reads are the faster of the two.
constexpr int64_t kSmallB = int64_t(1) << 22;

bool transpose_b_first(int transA, int transB, int64_t N, int64_t K) {
    return !transA && transB && N >= 1 && K >= 1 && N * K <= kSmallB;
}

size_t split_bytes(const Plan& p, int64_t M, int64_t N) {
    return p.splits > 1 ? align_up(static_cast<size_t>(p.splits) * M * N * sizeof(float)) : 0;
}

size_t gemm_ws_bytes(int transA, int transB, int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    Plan p = make_plan(M, N, K);
    size_t b = split_bytes(p, M, N);
    if (transpose_b_first(transA, transB, N, K)) b += align_up(static_cast<size_t>(N) * K * sizeof(float));
    return b;
}

gnn_status_t launch_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, const void* A, gnn_dtype_t a_dt,
                         int64_t lda, const void* B, gnn_dtype_t b_dt, int64_t ldb, void* C, gnn_dtype_t c_dt,
                         int64_t ldc, void* ws, size_t ws_bytes, hipStream_t st, int relu,
                         const MaskEpilogue& mask, const OperandRank1& ra1, const OperandRank1& rb1) {
    if (M == 0 || N == 0) return GNN_OK;
    auto r1_ok = [](const OperandRank1& o) {
        return o.s && o.v && o.ld >= 1 && o.dh >= 4 && reinterpret_cast<uintptr_t>(o.v) % 16 == 0;
    };
    if ((ra1.s && (ra1.dh & (ra1.dh - 1))) || (rb1.s && (rb1.dh & (rb1.dh - 1))))
        return fail(GNN_ERR_UNSUPPORTED, "gnn_gemm: a rank-1 operand term needs a power-of-two head width");
    if ((ra1.s && rb1.s) || (ra1.s && (transA || a_dt != GNN_F32 || !r1_ok(ra1))) ||
        (rb1.s && (transB || b_dt != GNN_F32 || !r1_ok(rb1))) ||
        ((ra1.s || rb1.s) && (a_dt != GNN_F32 || b_dt != GNN_F32 || c_dt != GNN_F32)))
        return fail(GNN_ERR_UNSUPPORTED, "gnn_gemm: a rank-1 operand term needs binary32 operands, an "
                                         "untransposed operand, a head width that is a multiple of 4 and a "
                                         "16-byte aligned vector");
    const int r1 = ra1.s ? 1 : rb1.s ? 2 : 0;
    {  // every column's head must have a coefficient: (cols - 1) / dh < ld
        const OperandRank1& o = r1 == 1 ? ra1 : rb1;
        const int64_t cols = r1 == 1 ? K : N;
        if (r1 && cols > 0 && (cols - 1) / o.dh >= o.ld)
            return fail(GNN_ERR_UNSUPPORTED, "gnn_gemm: a rank-1 operand term needs a coefficient for every head");
    }
    Plan p = make_plan(M, N, K);
    if (ws_bytes < gemm_ws_bytes(transA, transB, M, N, K))
        return fail(GNN_ERR_WORKSPACE, "gnn_gemm: workspace smaller than gnn_gemm_workspace_size()");
    if (transpose_b_first(transA, transB, N, K)) {
        void* Bt = static_cast<char*>(ws) + split_bytes(p, M, N);
        const int64_t total = N * K;
        if (b_dt == GNN_BF16)
            hipLaunchKernelGGL((transpose_kernel<bf16_t>), dim3((total + 255) / 256), dim3(256), 0, st,
                               static_cast<const bf16_t*>(B), ldb, N, K, static_cast<bf16_t*>(Bt));
        else
            hipLaunchKernelGGL((transpose_kernel<float>), dim3((total + 255) / 256), dim3(256), 0, st,
                               static_cast<const float*>(B), ldb, N, K, static_cast<float*>(Bt));
        GNN_TRY(launch_status("gnn_gemm (B transpose)"));
        B = Bt;
        ldb = N;
        transB = 0;
    }
    GemmArgs g;
    g.M = M, g.N = N, g.K = K;
    g.A = A, g.lda = lda, g.B = B, g.ldb = ldb, g.C = C, g.ldc = ldc;
    g.ws = static_cast<float*>(ws);
    g.relu = relu;
    g.mask = mask;
    g.r1 = r1 == 1 ? ra1 : rb1;
    g.r1.dh_log2 = 0;
    while ((int64_t(1) << g.r1.dh_log2) < g.r1.dh) ++g.r1.dh_log2;
    g.kper = p.kper;
    g.splits = p.splits;
    g.tiles_m = (M + p.bm - 1) / p.bm;
    g.tiles_n = (N + p.bn - 1) / p.bn;
    g.nblocks = g.tiles_m * g.tiles_n * p.splits;
    g.per_xcd = (g.nblocks + 7) / 8;
    if (K == 0) {
        // C = 0: run the kernel with an empty K range
        g.kper = 0;
        g.splits = 1;
        g.nblocks = g.tiles_m * g.tiles_n;
        g.per_xcd = (g.nblocks + 7) / 8;
    }
    const size_t as = dt_size(a_dt), bs = dt_size(b_dt), cs = dt_size(c_dt);
    g.vec_c = ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % (4 * cs) == 0;
    g.vec_mask = mask.M && mask.ld % 4 == 0 && reinterpret_cast<uintptr_t>(mask.M) % (4 * dt_size(mask.dt)) == 0;
    g.vec_ws = N % 4 == 0;
    const bool va = lda % 4 == 0 && reinterpret_cast<uintptr_t>(A) % (4 * as) == 0;
    const bool vb = ldb % 4 == 0 && reinterpret_cast<uintptr_t>(B) % (4 * bs) == 0;
    // bf16 x bf16 weight gradients (A transposed, K = nodes, split over K) on
    // the 16x16x32 bf16 matrix cores, with no more splits than this plan's
    // (so the workspace the size query returned holds the partials).
    // Measured on the 2.45M-node graph: 256 x 256 1.41 -> 0.70 ms, 100 x 256
    // ~1.5 -> 0.74 ms; 256 x 47 0.72 -> 0.77 ms (the 128-wide tile is mostly
    // padding there), so products 64 wide or less keep the 128 x 64 tiles.
    if (transA && !transB && a_dt == GNN_BF16 && b_dt == GNN_BF16 && p.splits > 1 && N > 64 && !relu && !mask.M &&
        gemm_tn_bf16_supported(lda, ldb, A, B)) {
        const int64_t kper = ((K + p.splits - 1) / p.splits + 31) / 32 * 32;
        const int64_t splits = (K + kper - 1) / kper;
        ScopedTimer t(st, "gemm M=%lld N=%lld K=%lld ta=%d tb=%d %s,%s->%s", static_cast<long long>(M),
                      static_cast<long long>(N), static_cast<long long>(K), transA, transB, dt_name(a_dt),
                      dt_name(b_dt), dt_name(c_dt));
        GNN_TRY(launch_gemm_tn_bf16(M, N, K, static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(B), ldb,
                                    static_cast<float*>(ws), splits, kper, st));
        const int64_t tot = M * N;
        if (c_dt == GNN_BF16)
            hipLaunchKernelGGL((splitk_reduce<bf16_t>), dim3((tot + 63) / 64), dim3(256), 0, st,
                               static_cast<const float*>(ws), static_cast<int>(splits), M, N, static_cast<bf16_t*>(C),
                               ldc, 0, MaskEpilogue{});
        else
            hipLaunchKernelGGL((splitk_reduce<float>), dim3((tot + 63) / 64), dim3(256), 0, st,
                               static_cast<const float*>(ws), static_cast<int>(splits), M, N, static_cast<float*>(C),
                               ldc, 0, MaskEpilogue{});
        return launch_status("gnn_gemm (split-K reduction)");
    }
    // timed: the product and, when split over K, its fixed-order reduction
    ScopedTimer t(st, "gemm M=%lld N=%lld K=%lld ta=%d tb=%d %s,%s->%s%s", static_cast<long long>(M),
                  static_cast<long long>(N), static_cast<long long>(K), transA, transB, dt_name(a_dt), dt_name(b_dt),
                  dt_name(c_dt), r1 == 1 ? " +rank1 A" : r1 == 2 ? " +rank1 B" : "");
    if (!transA && !transB) return launch_trans<false, false>(g, p, a_dt, b_dt, c_dt, va, vb, r1, st);
    if (!transA && transB) return launch_trans<false, true>(g, p, a_dt, b_dt, c_dt, va, vb, r1, st);
    if (transA && !transB) return launch_trans<true, false>(g, p, a_dt, b_dt, c_dt, va, vb, r1, st);
    return launch_trans<true, true>(g, p, a_dt, b_dt, c_dt, va, vb, r1, st);
}

}  // namespace gnnmp
