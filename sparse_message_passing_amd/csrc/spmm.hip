// spmm.hip -- aggregation Y = (G . w) X over the CSR (in-edges) or CSC
// (out-edges) view.
//
// AdaQP (arXiv 2306.01381) Eqn. 3: the aggregation of node v is the weighted
// sum of its neighbours' rows; Tango (SC'23), GAT running example:
// "H(l) = (G . alpha) H'" with one weight per (edge, head), and the
// backward SpMM over the reversed graph.
//
// Work decomposition (gfx950, wave64):
//  * a "group" of LANES lanes owns one output row; lane l holds features
//    (c*LANES + l)*VEC .. +VEC-1, so every gathered source row is read with
//    fully coalesced 16-byte (fp32) or 8-byte (bf16) loads;
//  * the group first loads LANES edge indices (and weights) in one coalesced
//    access, then walks them by broadcasting each index from its lane
//    (v_readlane for whole-wave groups, ds_bpermute otherwise), four source
//    rows in flight per lane;
//  * wide rows over a graph whose source matrix is larger than the
//    memory-side cache are processed in column slabs: the grid is
//    slab-major, so all items gather columns [0, W) first, then [W, 2W), ...
//    and each slab's working set (rows x W) stays cache resident while the
//    gathers of that slab run; only the edge indices and weights are read
//    once per slab;
//  * rows are visited in degree-descending order (the graph's `order`), and a
//    row longer than the view's chunk length (512 in-edges, 2048 out-edges)
//    is cut into chunks of that many edges that are
//    independent work items writing binary32 partial rows; a second kernel
//    adds each row's partials in chunk order.  No atomics: bitwise
//    reproducible.

#include <algorithm>
#include <mutex>

#include "device.h"
#include "internal.h"

// Scratch of the allocation-free aggregation (gnn_spmm_noalloc): the hub-row
// partial sums live here instead of in a caller workspace.  Each GPU the
// library runs on holds one copy until the process ends; host code reaches
// it only through the device address hipGetSymbolAddress returns (see
// spmm_noalloc_scratch), never through this name.
static __device__ __align__(256) unsigned char scratch[gnnmp::kSpmmScratchBytes];

namespace gnnmp {

namespace {

constexpr int kMaxHeads = 8;

// Column-slab budget: the source rows' slab must fit in this many bytes (the
// size of the memory-side cache), and a slab row is never narrower than 256
// bytes (two cache lines; one-line slabs pay more in re-read edge indices
// than they gain in hits).  Measured on a 2^20-node R-MAT graph, 256 wide:
// 3.22 ms unslabbed, 2.42 ms in 64-column slabs, bitwise the same result.
#ifndef GNN_SPMM_SLAB_BYTES
#define GNN_SPMM_SLAB_BYTES (256ll << 20)
#endif
#ifndef GNN_SPMM_SLAB_MIN_BYTES
#define GNN_SPMM_SLAB_MIN_BYTES 256
#endif
constexpr int64_t kSlabBytes = GNN_SPMM_SLAB_BYTES;
constexpr int64_t kSlabMinBytes = GNN_SPMM_SLAB_MIN_BYTES;

constexpr int kMaxQGroups = 8;

struct QGroupDev {        // one bit-width buffer of quantised rows
    const uint8_t* packed;
    const float* scale;
    const float* zero;
    int64_t row_bytes;
    int bits;
};

struct SpmmArgs {
    int64_t n;
    const int64_t* ptr;
    const int32_t* idx;
    const int32_t* eid;
    const int32_t* order;
    int64_t n_heavy, n_chunks, chunk;
    const int32_t* chunk_row;
    const int32_t* chunk_first;
    const float* dinv;
    const float* edge_w;
    int wmode;
    int heads;
    int64_t dh;
    const void* X;
    int64_t ldx;
    void* Y;
    int64_t ldy;
    int64_t d;
    int64_t pd;          // row stride of the partial buffer (d rounded up to 4)
    int64_t slab_blocks; // workgroups per column slab (grid = slab_blocks x number of slabs)
    int relu;
    int vec_store;       // Y rows take 16-byte (8-byte for bf16) stores
    Rank1Epilogue r1;
    MaskEpilogue mask;   // Y *= [M > 0]
    float* partial;
    const float* wgcn;   // GCN edge weights in this view's edge order (NULL: dinv[u]*dinv[v] on the fly)
    const float* dmean;  // [n] 1 / CSR row length (mean weights)
    const int32_t* qslot;           // dequantise-in-gather: slot of each source node, -1 = row of X
    QGroupDev qg[kMaxQGroups];
    int q_words;                    // every group's code rows are whole 4-byte words
    const uint4* qrec;              // per-node records (QRec), zero for rows of X
    const float* addend;            // Y = (G . w) X + addend (may be Y itself), before the ReLU
    int64_t ld_add;
};

// Dequantise-in-gather.  A per-node record, built once per call, holds for
// every quantised source its code-row address (bits in the top byte, which
// device addresses leave free), its scale S and zero point Z, so the gather
// needs no per-edge group lookup: the lane that owns an edge loads the record
// with the edge's index and broadcasts it.  dq_load fetches the lane's code
// bits for features f..f+3 (one aligned 4-byte load when every group's code
// rows are whole words) and returns them raw, so the loads of the four edges
// in flight are all issued before any of them is waited on; dq_decode turns
// them into fma(q, S, Z), one correctly rounded operation each, exactly as the
// dequantisation kernel does.
struct QRec {
    uint32_t lo, hi;  // code-row address, bits << 24 in hi
    float S, Z;
};

__device__ __forceinline__ float4 dq_load(const SpmmArgs& a, uint32_t lo, uint32_t hi, float S, float Z, int64_t f) {
    const int b = static_cast<int>(hi >> 24);
    const uint8_t* row = reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi & 0xFFFFFFu) << 32) | lo);
    const int64_t o = (f * b) >> 3;
    uint32_t w;
    if (a.q_words) {
        w = *reinterpret_cast<const uint32_t*>(row + (o & ~int64_t(3))) >> (8 * (o & 3));
    } else {
        const uint8_t* cp = row + o;
        if (b == 8) w = *reinterpret_cast<const uint32_t*>(cp);
        else if (b == 4) w = *reinterpret_cast<const uint16_t*>(cp);
        else w = *cp;
    }
    return make_float4(S, Z, __uint_as_float(w), __int_as_float(b));
}

__device__ __forceinline__ void dq_decode(float (&v)[4]) {
    const float S = v[0], Z = v[1];
    const uint32_t w = __float_as_uint(v[2]);
    const int b = __float_as_int(v[3]);
    const uint32_t m = (1u << b) - 1u;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __fmaf_rn(static_cast<float>((w >> (i * b)) & m), S, Z);
}

template <typename TO>
__device__ __forceinline__ float mask_of(const MaskEpilogue& m, int64_t row, int64_t f) {
    if (m.dt == GNN_BF16) return Elem<bf16_t>::load(static_cast<const bf16_t*>(m.M) + row * m.ld + f) > 0.0f ? 1.0f : 0.0f;
    return Elem<float>::load(static_cast<const float*>(m.M) + row * m.ld + f) > 0.0f ? 1.0f : 0.0f;
}

template <int VEC>
struct Acc {
    float v[VEC];
};

template <int LANES, int VEC, int NCH, typename TI, typename TO, bool QS>
__global__ __launch_bounds__(256) void spmm_kernel(SpmmArgs a) {
    static_assert(VEC != 8 || sizeof(TI) == 2, "eight features per lane are bf16 sources");
    const int lane = threadIdx.x % LANES;
    const int64_t slab = blockIdx.x / a.slab_blocks;
    const int64_t gid = static_cast<int64_t>(blockIdx.x - slab * a.slab_blocks) * (256 / LANES) + threadIdx.x / LANES;
    const int64_t fbase = slab * (LANES * VEC * NCH) + static_cast<int64_t>(lane) * VEC;  // first feature of pass c = 0
    int64_t row, eb, ee;
    bool heavy;
    if (gid < a.n_chunks) {
        const int oi = a.chunk_row[gid];
        row = a.order[oi];
        const int64_t c = gid - a.chunk_first[oi];
        eb = a.ptr[row] + c * a.chunk;
        ee = min(eb + a.chunk, a.ptr[row + 1]);
        heavy = true;
    } else {
        const int64_t li = gid - a.n_chunks + a.n_heavy;
        if (li >= a.n) return;
        row = a.order[li];
        eb = a.ptr[row];
        ee = a.ptr[row + 1];
        heavy = false;
    }
    const TI* X = static_cast<const TI*>(a.X);

    float acc[NCH][VEC];
    int hd[NCH];
    bool act[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t f = fbase + static_cast<int64_t>(c * LANES * VEC);
        act[c] = f < a.d;
        hd[c] = act[c] ? static_cast<int>(f / a.dh) : 0;
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[c][i] = 0.0f;
    }
    // per-row factor: dinv of the row (GCN), or the row's mean weight (CSR view)
    const float dv = a.wmode == GNN_W_GCN                ? a.dinv[row]
                     : (a.wmode == GNN_W_MEAN && !a.eid) ? a.dmean[row]
                                                         : 1.0f;
    const int heads = a.heads;
    // heads this slab's columns belong to (all heads when one pass covers the row)
    const int64_t slab_f0 = slab * (LANES * VEC * NCH);
    const int klo = static_cast<int>(slab_f0 / a.dh);
    const int khi = static_cast<int>(min(a.d, slab_f0 + LANES * VEC * NCH) - 1) / static_cast<int>(a.dh);

    for (int64_t e0 = eb; e0 < ee; e0 += LANES) {
        const int cnt = static_cast<int>(min(static_cast<int64_t>(LANES), ee - e0));
        int u_my = static_cast<int>(row);
        uint4 r_my = make_uint4(0u, 0u, 0u, 0u);  // quantised-source record (QS)
        float w_my[kMaxHeads];
#pragma unroll
        for (int k = 0; k < kMaxHeads; ++k) w_my[k] = 0.0f;
        if (lane < cnt) {
            const int64_t e = e0 + lane;
            u_my = a.idx[e];
            if constexpr (QS) r_my = a.qrec[u_my];
            if (a.wmode == GNN_W_GCN) {
                w_my[0] = a.wgcn ? a.wgcn[e] : a.dinv[u_my] * dv;
            } else if (a.wmode == GNN_W_ONES) {
                w_my[0] = 1.0f;
            } else if (a.wmode == GNN_W_MEAN) {
                // an in-edge of row v weighs 1/len(v); over the CSC view the
                // edge's destination is the other end
                w_my[0] = a.eid ? a.dmean[u_my] : dv;
            } else {
                const int64_t ce = a.eid ? static_cast<int64_t>(a.eid[e]) : e;
#pragma unroll
                for (int k = 0; k < kMaxHeads; ++k)
                    if (k >= klo && k <= khi) w_my[k] = a.edge_w[ce * heads + k];
            }
        }
        for (int j = 0; j < cnt; j += 4) {
            int u[4];
            uint32_t qlo[4], qhi[4];
            float qS[4], qZ[4];
            float w[4][NCH];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int src = (j + q < cnt) ? j + q : j;
                u[q] = group_bcast<LANES>(u_my, src);
                if constexpr (QS) {
                    qlo[q] = static_cast<uint32_t>(group_bcast<LANES>(static_cast<int>(r_my.x), src));
                    qhi[q] = static_cast<uint32_t>(group_bcast<LANES>(static_cast<int>(r_my.y), src));
                    qS[q] = group_bcast<LANES>(__uint_as_float(r_my.z), src);
                    qZ[q] = group_bcast<LANES>(__uint_as_float(r_my.w), src);
                } else {
                    qlo[q] = qhi[q] = 0u;
                    qS[q] = qZ[q] = 0.0f;
                }
                if (heads == 1) {
                    const float w0 = group_bcast<LANES>(w_my[0], src);
#pragma unroll
                    for (int c = 0; c < NCH; ++c) w[q][c] = w0;
                } else {
#pragma unroll
                    for (int c = 0; c < NCH; ++c) w[q][c] = 0.0f;
#pragma unroll
                    for (int k = 0; k < kMaxHeads; ++k) {
                        if (k >= klo && k <= khi) {
                            const float wk = group_bcast<LANES>(w_my[k], src);
#pragma unroll
                            for (int c = 0; c < NCH; ++c) w[q][c] = hd[c] == k ? wk : w[q][c];
                        }
                    }
                }
                if (j + q >= cnt) {
#pragma unroll
                    for (int c = 0; c < NCH; ++c) w[q][c] = 0.0f;
                }
            }
            Acc<VEC> xv[4][NCH];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int64_t f = fbase + static_cast<int64_t>(c * LANES * VEC);
                    if (act[c] && j + q < cnt) {
                        const TI* p = X + static_cast<int64_t>(u[q]) * a.ldx + f;
                        if constexpr (VEC == 8) {  // eight bf16 in one 16-byte load
                            const uint4 r = *reinterpret_cast<const uint4*>(p);
                            const uint32_t w8[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                            for (int h = 0; h < 4; ++h) {
                                xv[q][c].v[2 * h] = __uint_as_float(w8[h] << 16);
                                xv[q][c].v[2 * h + 1] = __uint_as_float(w8[h] & 0xFFFF0000u);
                            }
                        } else if constexpr (VEC == 4) {
                            float4 t;
                            if (QS && qhi[q] != 0u) t = dq_load(a, qlo[q], qhi[q], qS[q], qZ[q], f);  // raw
                            else t = Elem<TI>::load4(p);
                            xv[q][c].v[0] = t.x;
                            xv[q][c].v[1] = t.y;
                            xv[q][c].v[2] = t.z;
                            xv[q][c].v[3] = t.w;
                        } else {
                            xv[q][c].v[0] = Elem<TI>::load(p);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < VEC; ++i) xv[q][c].v[i] = 0.0f;
                    }
                }
            }
            if constexpr (QS && VEC == 4) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
                        if (qhi[q] != 0u && j + q < cnt) dq_decode(xv[q][c].v);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < NCH; ++c)
#pragma unroll
                    for (int i = 0; i < VEC; ++i) acc[c][i] = fmaf(w[q][c], xv[q][c].v[i], acc[c][i]);
        }
    }

#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (!act[c]) continue;
        const int64_t f = fbase + static_cast<int64_t>(c * LANES * VEC);
        const int nv = static_cast<int>(min(static_cast<int64_t>(VEC), a.d - f));  // valid features of this lane
        if (heavy) {
            float* P = a.partial + gid * a.pd + f;
            if constexpr (VEC == 8) {
                *reinterpret_cast<float4*>(P) = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
                *reinterpret_cast<float4*>(P + 4) = make_float4(acc[c][4], acc[c][5], acc[c][6], acc[c][7]);
            } else if constexpr (VEC == 4) {
                *reinterpret_cast<float4*>(P) = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
            } else {
                P[0] = acc[c][0];
            }
            continue;
        }
        if (a.addend) {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                if (i < nv) acc[c][i] = acc[c][i] + a.addend[row * a.ld_add + f + i];
        }
        if (a.r1.a) {
            const float ra = a.r1.a[row * heads + hd[c]];
            const float rb = a.r1.b[row * heads + hd[c]];
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                if (i < nv) acc[c][i] = acc[c][i] + (ra * a.r1.va[f + i] + rb * a.r1.vb[f + i]);
        }
        if (a.relu) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[c][i] = fmaxf(acc[c][i], 0.0f);
        }
        if (a.mask.M) {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                if (i < nv) acc[c][i] = mask_of<TO>(a.mask, row, f + i) > 0.0f ? acc[c][i] : 0.0f;
        }
        TO* Y = static_cast<TO*>(a.Y) + row * a.ldy + f;
        if constexpr (VEC == 8) {
            if (nv == 8 && a.vec_store) {
                Elem<TO>::store4(Y, make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]));
                Elem<TO>::store4(Y + 4, make_float4(acc[c][4], acc[c][5], acc[c][6], acc[c][7]));
            } else {
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    if (i < nv) Elem<TO>::store(Y + i, acc[c][i]);
            }
        } else if constexpr (VEC == 4) {
            if (nv == 4 && a.vec_store) {
                Elem<TO>::store4(Y, make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]));
            } else {
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    if (i < nv) Elem<TO>::store(Y + i, acc[c][i]);
            }
        } else {
            Elem<TO>::store(Y, acc[c][0]);
        }
    }
}

// Per-node records of the dequantise-in-gather sources: zero for rows of X,
// else (code-row address | bits << 56, S, Z) of the node's slot.
__global__ __launch_bounds__(256) void qrec_kernel(SpmmArgs a, QRec* rec) {
    const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (v >= a.n) return;
    const int slot = a.qslot[v];
    QRec r{0u, 0u, 0.0f, 0.0f};
    if (slot >= 0) {
        const int g = slot >> 27;
        const int64_t i = slot & ((1 << 27) - 1);
        const QGroupDev& G = a.qg[g];
        const uint64_t addr = reinterpret_cast<uint64_t>(G.packed + i * G.row_bytes);
        r.lo = static_cast<uint32_t>(addr);
        r.hi = static_cast<uint32_t>(addr >> 32) | (static_cast<uint32_t>(G.bits) << 24);
        r.S = G.scale[i];
        r.Z = G.zero[i];
    }
    *reinterpret_cast<uint4*>(rec + v) = make_uint4(r.lo, r.hi, __float_as_uint(r.S), __float_as_uint(r.Z));
}

// Sum the partial rows of each heavy row, then the epilogue.  Chunk c goes to
// accumulator (c - c0) mod 8 and the eight are added pairwise at the end: a
// fixed order (deterministic) with eight loads in flight, so the longest hub
// row (over a hundred chunks) does not wait on one load per chunk.
template <typename TO>
__global__ __launch_bounds__(256) void spmm_fixup(SpmmArgs a) {
    const int64_t i = blockIdx.x;
    const int64_t row = a.order[i];
    const int64_t c0 = a.chunk_first[i], c1 = a.chunk_first[i + 1];
    for (int64_t f = threadIdx.x; f < a.d; f += blockDim.x) {
        float p8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        int64_t c = c0;
        for (; c + 8 <= c1; c += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) p8[u] += a.partial[(c + u) * a.pd + f];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c + u < c1) p8[u] += a.partial[(c + u) * a.pd + f];
        float s = ((p8[0] + p8[1]) + (p8[2] + p8[3])) + ((p8[4] + p8[5]) + (p8[6] + p8[7]));
        if (a.addend) s = s + a.addend[row * a.ld_add + f];
        if (a.r1.a) {
            const int64_t h = f / a.dh;
            s = s + (a.r1.a[row * a.heads + h] * a.r1.va[f] + a.r1.b[row * a.heads + h] * a.r1.vb[f]);
        }
        if (a.relu) s = fmaxf(s, 0.0f);
        if (a.mask.M && !(mask_of<TO>(a.mask, row, f) > 0.0f)) s = 0.0f;
        Elem<TO>::store(static_cast<TO*>(a.Y) + row * a.ldy + f, s);
    }
}

template <int LANES, int VEC, int NCH, typename TI, typename TO, bool QS = false>
void launch_t(SpmmArgs a, hipStream_t st) {
    const int64_t groups = a.n_chunks + (a.n - a.n_heavy);
    const int64_t gpb = 256 / LANES;
    const int64_t width = LANES * VEC * NCH;  // features one pass covers
    const int64_t slabs = (a.d + width - 1) / width;
    a.slab_blocks = (groups + gpb - 1) / gpb;
    if (a.slab_blocks > 0) {
        ScopedTimer t(st, "spmm_kernel d=%lld h=%d %s->%s %s%s", static_cast<long long>(a.d), a.heads,
                      sizeof(TI) == 2 ? "bf16" : "f32", sizeof(TO) == 2 ? "bf16" : "f32", a.eid ? "csc" : "csr",
                      QS ? " dequant" : "");
        hipLaunchKernelGGL((spmm_kernel<LANES, VEC, NCH, TI, TO, QS>), dim3(a.slab_blocks * slabs), dim3(256), 0, st,
                           a);
    }
    if (a.n_heavy > 0) hipLaunchKernelGGL((spmm_fixup<TO>), dim3(a.n_heavy), dim3(256), 0, st, a);
}

template <typename TI, typename TO, bool QS = false>
gnn_status_t dispatch(const SpmmArgs& a, int vec, int lanes, int nch, hipStream_t st) {
    if constexpr (QS) {
        // Whole-wave groups over the whole row: every edge's record, and so
        // its decode branch, is wave uniform (broadcast with v_readlane).
        // Measured on the quantised-exchange workload (2^20 nodes, 30%
        // marginal rows, 256 wide): 3.47 ms, against 3.40 ms for the
        // slabbed binary32 aggregation plus 0.10 ms of dequantisation (the
        // smaller code rows make up for the lost column slabs); 16-lane
        // groups in 64-column slabs took 4.2 ms (per-edge record broadcasts
        // and divergent decodes), one feature per lane in 64-column slabs
        // 8.9 ms (four times the instructions).
        if (nch == 1) launch_t<64, 4, 1, TI, TO, true>(a, st);
        else if (nch == 2) launch_t<64, 4, 2, TI, TO, true>(a, st);
        else launch_t<64, 4, 4, TI, TO, true>(a, st);
        return launch_status("gnn_spmm_dequant");
    }
    if (vec == 4) {
        if (nch == 1) {
            if (lanes == 8) launch_t<8, 4, 1, TI, TO, QS>(a, st);
            else if (lanes == 16) launch_t<16, 4, 1, TI, TO, QS>(a, st);
            else if (lanes == 32) launch_t<32, 4, 1, TI, TO, QS>(a, st);
            else launch_t<64, 4, 1, TI, TO, QS>(a, st);
        } else if (nch == 2) {
            launch_t<64, 4, 2, TI, TO, QS>(a, st);
        } else {
            launch_t<64, 4, 4, TI, TO, QS>(a, st);
        }
    } else if constexpr (!QS) {
        if (nch == 1) launch_t<64, 1, 1, TI, TO>(a, st);
        else if (nch == 2) launch_t<64, 1, 2, TI, TO>(a, st);
        else launch_t<64, 1, 4, TI, TO>(a, st);
    }
    return launch_status(QS ? "gnn_spmm_dequant" : "gnn_spmm");
}

}  // namespace

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; HIP errors are reported.
gnn_status_t spmm_noalloc_scratch(void** out) {
    static std::mutex mu;
    static std::vector<void*> ptrs;
    int dev = 0;
    GNN_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs.empty()) {
        int count = 0;
        GNN_HIP(hipGetDeviceCount(&count));
        ptrs.assign(static_cast<size_t>(count), nullptr);
    }
    if (dev < 0 || static_cast<size_t>(dev) >= ptrs.size())
        return fail(GNN_ERR_HIP, "gnn_spmm_noalloc: current device out of range");
    if (!ptrs[dev]) {
        void* p = nullptr;
        GNN_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return GNN_OK;
}

size_t spmm_partial_bytes(const RowPlan& p, int64_t d) {
    const int64_t pd = (d + 7) / 8 * 8;
    return p.n_chunks > 0 ? align_up(static_cast<size_t>(p.n_chunks) * pd * sizeof(float)) : 0;
}

gnn_status_t launch_spmm(const AggView& v, const float* dinv, gnn_weights_t wmode, const float* edge_w, int heads,
                         const void* X, gnn_dtype_t x_dt, int64_t ldx, void* Y, gnn_dtype_t y_dt, int64_t ldy,
                         int64_t d, int relu, const Rank1Epilogue& r1, float* partial, hipStream_t st,
                         const MaskEpilogue& mask, const QuantSources& qs) {
    if (v.n == 0 || d == 0) return GNN_OK;
    if (heads > kMaxHeads) return fail(GNN_ERR_UNSUPPORTED, "gnn_spmm: at most 8 heads");
    SpmmArgs a;
    a.n = v.n;
    a.ptr = v.ptr;
    a.idx = v.idx;
    a.eid = v.eid;
    a.order = v.plan->order;
    a.n_heavy = v.plan->n_heavy;
    a.n_chunks = v.plan->n_chunks;
    a.chunk = v.plan->chunk;
    a.chunk_row = v.plan->chunk_row;
    a.chunk_first = v.plan->chunk_first;
    a.dinv = dinv;
    a.edge_w = edge_w;
    a.wmode = wmode;
    a.heads = heads;
    a.dh = d / heads;
    a.X = X;
    a.ldx = ldx;
    a.Y = Y;
    a.ldy = ldy;
    a.d = d;
    a.relu = relu;
    a.r1 = r1;
    a.mask = mask;
    a.partial = partial;
    a.wgcn = v.wgcn;
    a.dmean = v.dmean;
    a.qslot = qs.qslot;
    a.qrec = nullptr;
    a.addend = qs.addend;
    a.ld_add = qs.ld_add;
    a.q_words = 1;
    for (int i = 0; i < qs.n_groups; ++i)
        if ((d * qs.groups[i].bits / 8) % 4 || reinterpret_cast<uintptr_t>(qs.groups[i].packed) % 4) a.q_words = 0;
    for (int i = 0; i < kMaxQGroups; ++i) a.qg[i] = QGroupDev{nullptr, nullptr, nullptr, 0, 0};
    for (int i = 0; i < qs.n_groups && i < kMaxQGroups; ++i)
        a.qg[i] = QGroupDev{qs.groups[i].packed, qs.groups[i].scale, qs.groups[i].zero, d * qs.groups[i].bits / 8,
                            qs.groups[i].bits};
    a.pd = (d + 7) / 8 * 8;  // partial rows: room for a lane's last eight features
    const int64_t pd4 = (d + 3) / 4 * 4;
    const size_t xs = dt_size(x_dt), ys = dt_size(y_dt);
    // 4-wide loads need 4-element aligned rows with room for the last quad;
    // 4-wide stores additionally need the same of Y (else stores go one by one)
    const bool vec = ldx % 4 == 0 && ldx >= pd4 && reinterpret_cast<uintptr_t>(X) % (4 * xs) == 0 &&
                     (heads == 1 || a.dh % 4 == 0);
    a.vec_store = ldy % 4 == 0 && reinterpret_cast<uintptr_t>(Y) % (4 * ys) == 0;
    int64_t need = vec ? pd4 / 4 : d;  // lanes for one pass over the features
    // Column slabs, except where each edge's weights are reached through the
    // CSC-to-CSR edge map: those scattered weight reads would repeat in every
    // slab (measured: slabs slow the transposed 4-head GAT aggregation down).
    if (vec && !(wmode == GNN_W_EDGE && v.eid)) {
        // halve the pass width while the source rows' slab (rows x width)
        // exceeds the cache budget, down to the minimum slab row
        const int64_t rows = v.n;
        int64_t w = 8;
        while (w < need) w *= 2;
        const int64_t min_w = std::max<int64_t>(8, kSlabMinBytes / (4 * static_cast<int64_t>(xs)));
        while (w > min_w && rows * w * 4 * static_cast<int64_t>(xs) > kSlabBytes) w /= 2;
        need = std::min(need, w);
    }
    int lanes, nch;
    if (vec && need <= 8) lanes = 8, nch = 1;
    else if (vec && need <= 16) lanes = 16, nch = 1;
    else if (vec && need <= 32) lanes = 32, nch = 1;
    else {
        lanes = 64;
        nch = need <= 64 ? 1 : need <= 128 ? 2 : need <= 256 ? 4 : 0;
    }
    const int vw = vec ? 4 : 1;
    if (nch == 0) return fail(GNN_ERR_UNSUPPORTED, "gnn_spmm: d too large (max 1024 for 16-byte rows, 256 otherwise)");
    if (qs.qslot) {
        if (!vec || heads != 1 || x_dt != GNN_F32 || y_dt != GNN_F32 || qs.n_groups > kMaxQGroups || !qs.records)
            return fail(GNN_ERR_UNSUPPORTED, "gnn_spmm_dequant: needs f32 rows in 16-byte vectors, one head, <= 8 groups");
        const int64_t full = a.pd / 4;  // lanes for the whole row, no slabs
        nch = full <= 64 ? 1 : full <= 128 ? 2 : full <= 256 ? 4 : 0;
        if (nch == 0) return fail(GNN_ERR_UNSUPPORTED, "gnn_spmm_dequant: d must be at most 1024");
        a.qrec = static_cast<const uint4*>(qs.records);
        hipLaunchKernelGGL(qrec_kernel, dim3((v.n + 255) / 256), dim3(256), 0, st, a, static_cast<QRec*>(qs.records));
        return dispatch<float, float, true>(a, vw, lanes, nch, st);
    }
    // bf16 sources: eight features per lane, so every gather is one 16-byte
    // load (four bf16 would be 8 bytes) and a wave holds twice the rows.
    // Measured on the 2.45M-node bf16 workload: 256 wide 14.6 -> 9.8 ms, 100
    // wide in 104-element rows 7.5 -> 5.7 ms; binary32 sources keep four
    // features per lane (eight were slower: 2.47 -> 2.77 ms at 256 wide).
    if (x_dt == GNN_BF16 && vec && ldx % 8 == 0 && ldx >= a.pd && reinterpret_cast<uintptr_t>(X) % 16 == 0 &&
        (heads == 1 || a.dh % 8 == 0)) {
        int64_t need8 = a.pd / 8;
        if (!(wmode == GNN_W_EDGE && v.eid)) {
            int64_t w = 8;
            while (w < need8) w *= 2;
            const int64_t min_w8 = std::max<int64_t>(8, kSlabMinBytes / (8 * static_cast<int64_t>(xs)));
            while (w > min_w8 && v.n * w * 8 * static_cast<int64_t>(xs) > kSlabBytes) w /= 2;
            need8 = std::min(need8, w);
        }
        if (need8 >= 8 && need8 <= 64) {
            const int l8 = need8 <= 8 ? 8 : need8 <= 16 ? 16 : need8 <= 32 ? 32 : 64;
            if (y_dt == GNN_F32) {
                if (l8 == 8) launch_t<8, 8, 1, bf16_t, float>(a, st);
                else if (l8 == 16) launch_t<16, 8, 1, bf16_t, float>(a, st);
                else if (l8 == 32) launch_t<32, 8, 1, bf16_t, float>(a, st);
                else launch_t<64, 8, 1, bf16_t, float>(a, st);
            } else {
                if (l8 == 8) launch_t<8, 8, 1, bf16_t, bf16_t>(a, st);
                else if (l8 == 16) launch_t<16, 8, 1, bf16_t, bf16_t>(a, st);
                else if (l8 == 32) launch_t<32, 8, 1, bf16_t, bf16_t>(a, st);
                else launch_t<64, 8, 1, bf16_t, bf16_t>(a, st);
            }
            return launch_status("gnn_spmm");
        }
    }
    if (x_dt == GNN_F32 && y_dt == GNN_F32) return dispatch<float, float>(a, vw, lanes, nch, st);
    if (x_dt == GNN_F32 && y_dt == GNN_BF16) return dispatch<float, bf16_t>(a, vw, lanes, nch, st);
    if (x_dt == GNN_BF16 && y_dt == GNN_F32) return dispatch<bf16_t, float>(a, vw, lanes, nch, st);
    return dispatch<bf16_t, bf16_t>(a, vw, lanes, nch, st);
}

}  // namespace gnnmp
