// gat_bwd.hip -- the edge part of the GAT backward (Tango, SC'23, GAT running
// example, Fig. 1b) organised around the transposed aggregation.
//
// Per head k, with p = S[u] + D[v] on edge u -> v, E = LReLU(p) and
// alpha = exp(E - m[v]) / z[v] (m, z: the destination's softmax maximum and
// sum, kept by the forward):
//   dalpha[e] = <dY[v, k], H'[u, k]>
//   dE[e]     = alpha (dalpha - c[v]) * LReLU'(p),  c[v] = sum_in(v) alpha dalpha
//   dS[u]     = sum_out(u) dE,   dD[v] = sum_in(v) dE
//   dH'[u]    = sum_out(u) alpha dY[v] + dS[u] a_src + dD[u] a_dst
// The SDDMM dot and the transposed SpMM gather the same row dY[v] for the
// same edge, so one pass over the CSC view (sources, out-edges) does both:
// it re-forms alpha from S, D, m and z instead of reading a stored copy,
// forms dE, and sums dS and the transposed aggregation as it goes.  c[v] is
// needed before any dE, and since sum_in alpha H'[u] is the forward's output
// row, c[v] = <dY[v, k], Y[v, k]>: a dense row product, not an edge sum.
// dD needs the in-edge sum, so dE is also written (CSC order) and summed per
// destination through the CSR -> CSC slot map.  The dD a_dst term of dH' is
// not added here: the two products that read dH' (dW = X^T dH' and
// dX = dH' W^T) add it as they load each element, with the same single
// fmaf, which saves a read and a write of the whole of dH'.
//
// The CSC pass runs one head at a time (a column slab of H' and dY, slab-
// major over the grid) so each gathered slab of dY stays in the memory-side
// cache; per-destination records {D, m, 1/z, c} of the head are packed into
// one 16-byte read, and dE goes to the head's own plane (coalesced stores),
// re-laid afterwards as one record of all heads per edge for the in-edge sum.
// Out-edge hubs are cut into chunks whose partial rows are summed afterwards
// in a fixed order: deterministic, no atomics.

#include "device.h"
#include "internal.h"

namespace gnnmp {

namespace {

struct Rec3 {  // a per-destination record, stored and loaded with one 12-byte access
    float x, y, z;
};

// c = <dY[v, head k], Y[v, head k]> and the 12-byte record {D, m - log(1/z),
// c} of (v, k), head-major: rec[3 (k n + v) ..].  alpha = exp(E - m) / z =
// exp(E - (m - log(1/z))): one exponential, and a record that covers fewer
// cache lines per gathered destination.  One wave per row, HL = d_head / 4
// lanes a head.
template <int HL>
__global__ __launch_bounds__(256) void gat_rec_kernel(int64_t n, int heads, int64_t dh, const float* Y,
                                                      const float* dY, const float* D, const float* M,
                                                      const float* Z, float* rec) {
    const int lane = threadIdx.x & 63;
    const int64_t v = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (v >= n) return;
    const int64_t d = heads * dh;
    for (int64_t f0 = 0; f0 < d; f0 += 256) {
        const int64_t f = f0 + lane * 4;
        float c = 0.0f;
        if (f < d) {
            const float4 y = *reinterpret_cast<const float4*>(Y + v * d + f);
            const float4 g = *reinterpret_cast<const float4*>(dY + v * d + f);
            c = g.x * y.x;
            c = fmaf(g.y, y.y, c);
            c = fmaf(g.z, y.z, c);
            c = fmaf(g.w, y.w, c);
        }
        c = group_sum<HL>(c);
        if (f < d && (lane % HL) == 0) {
            const int64_t k = f / dh;
            const int64_t i = v * heads + k;
            // Z = 1/sum > 0 wherever the record is read (v has an in-edge there)
            *reinterpret_cast<Rec3*>(rec + (k * n + v) * 3) = Rec3{D[i], M[i] - __logf(Z[i]), c};
        }
    }
}

struct GatBwdArgs {
    int64_t n;
    const int64_t* ptr;          // CSC: out-edges of each source
    const int32_t* idx;          // destination of each CSC entry
    const int32_t* order;        // sources by out-degree, descending
    int64_t n_heavy, n_chunks, chunk;
    const int32_t* chunk_row;
    const int32_t* chunk_first;
    int heads;
    int64_t dh;
    int64_t slab_blocks;         // workgroups per head (grid = slab_blocks x heads)
    const float* Hp;             // H' [n, heads*dh]
    const float* rec;            // [heads, n, 3] {D, m - log(1/z), c}
    const float* dY;             // [n, heads*dh]
    const float* a_src;          // [heads, dh]
    float slope;
    int act;
    int64_t nnz;
    float* dEh;                  // [heads, nnz] dE in CSC order, one plane per head
    float* dS;                   // [n, heads]
    float* dHp;                  // [n, heads*dh]
    float* part;                 // [n_chunks, heads, dh] partial rows of the chunks
    float* pds;                  // [n_chunks, heads] partial dS of the chunks
};

// One group of L = dh/4 lanes per work item (a source row or a chunk of its
// out-edges); lane i holds features 4i..4i+3 of the head.  The lane that owns
// an edge (edge e0 + i of a group-width batch) loads its destination and
// record and forms alpha, then the batch is walked four edges at a time with
// the destination and alpha broadcast; the four dY gathers are issued before
// any is used.
template <int L>
__global__ __launch_bounds__(256) void gat_bwd_csc_kernel(GatBwdArgs a) {
    const int lane = threadIdx.x % L;
    const int k = static_cast<int>(blockIdx.x / a.slab_blocks);
    const int64_t gid =
        static_cast<int64_t>(blockIdx.x - static_cast<int64_t>(k) * a.slab_blocks) * (256 / L) + threadIdx.x / L;
    int64_t u, eb, ee;
    bool heavy;
    if (gid < a.n_chunks) {
        const int oi = a.chunk_row[gid];
        u = a.order[oi];
        eb = a.ptr[u] + (gid - a.chunk_first[oi]) * a.chunk;
        ee = min(eb + a.chunk, a.ptr[u + 1]);
        heavy = true;
    } else {
        const int64_t li = gid - a.n_chunks + a.n_heavy;
        if (li >= a.n) return;
        u = a.order[li];
        eb = a.ptr[u];
        ee = a.ptr[u + 1];
        heavy = false;
    }
    const int H = a.heads;
    const int64_t hd = H * a.dh;
    const int64_t fo = static_cast<int64_t>(k) * a.dh + lane * 4;
    const float4 hu = *reinterpret_cast<const float4*>(a.Hp + u * hd + fo);
    const float4 as = *reinterpret_cast<const float4*>(a.a_src + fo);
    // S[u] = <H'[u, head k], a_src[k]> again from the row in registers, in
    // the scores pass's order (the same bits as the saved S), instead of a
    // scattered 4-byte read per source row
    float su = hu.x * as.x;
    su = fmaf(hu.y, as.y, su);
    su = fmaf(hu.z, as.z, su);
    su = fmaf(hu.w, as.w, su);
    su = group_sum<L>(su);
    const float* rk = a.rec + static_cast<int64_t>(k) * a.n * 3;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float dsl = 0.0f;
    for (int64_t e0 = eb; e0 < ee; e0 += L) {
        const int cnt = static_cast<int>(min(static_cast<int64_t>(L), ee - e0));
        int v_my = 0;
        float a_my = 0.0f, c_my = 0.0f, dot_my = 0.0f;
        bool neg_my = false;
        if (lane < cnt) {
            v_my = a.idx[e0 + lane];
            const Rec3 r = *reinterpret_cast<const Rec3*>(rk + static_cast<int64_t>(v_my) * 3);
            const float p = su + r.x;
            neg_my = a.act && !(p > 0.0f);
            const float x = neg_my ? a.slope * p : p;
            a_my = __expf(x - r.y);
            c_my = r.z;
        }
        for (int j = 0; j < cnt; j += 4) {
            int vq[4];
            float aq[4];
            float4 y[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int src = (j + q < cnt) ? j + q : j;
                vq[q] = group_bcast<L>(v_my, src);
                aq[q] = j + q < cnt ? group_bcast<L>(a_my, src) : 0.0f;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                y[q] = j + q < cnt ? *reinterpret_cast<const float4*>(a.dY + static_cast<int64_t>(vq[q]) * hd + fo)
                                   : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = f4_fma(aq[q], y[q], acc);
                float pq = hu.x * y[q].x;
                pq = fmaf(hu.y, y[q].y, pq);
                pq = fmaf(hu.z, y[q].z, pq);
                pq = fmaf(hu.w, y[q].w, pq);
                pq = group_sum<L>(pq);
                if (lane == j + q) dot_my = pq;
            }
        }
        if (lane < cnt) {
            float dE = a_my * (dot_my - c_my);
            if (neg_my) dE = dE * a.slope;
            a.dEh[k * a.nnz + e0 + lane] = dE;
            dsl += dE;
        }
    }
    const float ds = group_sum<L>(dsl);
    if (heavy) {
        *reinterpret_cast<float4*>(a.part + (gid * H + k) * a.dh + lane * 4) = acc;
        if (lane == 0) a.pds[gid * H + k] = ds;
        return;
    }
    if (lane == 0) a.dS[u * H + k] = ds;
    *reinterpret_cast<float4*>(a.dHp + u * hd + fo) =
        make_float4(fmaf(ds, as.x, acc.x), fmaf(ds, as.y, acc.y), fmaf(ds, as.z, acc.z), fmaf(ds, as.w, acc.w));
}

// hub sources: sum the chunks' partial rows and dS, then the dS a_src term.
// One wave per (hub row, head).  Chunk c goes to accumulator (c - c0) mod 4,
// the four added pairwise at the end: a fixed order with four loads in flight.
__global__ __launch_bounds__(256) void gat_bwd_fixup_kernel(GatBwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int H = a.heads;
    if (w >= a.n_heavy * H) return;
    const int64_t i = w / H;
    const int k = static_cast<int>(w - i * H);
    const int64_t u = a.order[i];
    const int64_t c0 = a.chunk_first[i], c1 = a.chunk_first[i + 1];
    float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    {
        int64_t c = c0;
        for (; c + 4 <= c1; c += 4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) d4[q] += a.pds[(c + q) * H + k];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (c + q < c1) d4[q] += a.pds[(c + q) * H + k];
    }
    const float ds = (d4[0] + d4[1]) + (d4[2] + d4[3]);
    const int64_t hd = H * a.dh;
    for (int64_t f = lane * 4; f < a.dh; f += 256) {
        float4 p4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) p4[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        int64_t c = c0;
        for (; c + 4 <= c1; c += 4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 p = *reinterpret_cast<const float4*>(a.part + ((c + q) * H + k) * a.dh + f);
                p4[q].x += p.x;
                p4[q].y += p.y;
                p4[q].z += p.z;
                p4[q].w += p.w;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (c + q < c1) {
                const float4 p = *reinterpret_cast<const float4*>(a.part + ((c + q) * H + k) * a.dh + f);
                p4[q].x += p.x;
                p4[q].y += p.y;
                p4[q].z += p.z;
                p4[q].w += p.w;
            }
        }
        float4 acc;
        acc.x = (p4[0].x + p4[1].x) + (p4[2].x + p4[3].x);
        acc.y = (p4[0].y + p4[1].y) + (p4[2].y + p4[3].y);
        acc.z = (p4[0].z + p4[1].z) + (p4[2].z + p4[3].z);
        acc.w = (p4[0].w + p4[1].w) + (p4[2].w + p4[3].w);
        const float4 as = *reinterpret_cast<const float4*>(a.a_src + k * a.dh + f);
        *reinterpret_cast<float4*>(a.dHp + u * hd + k * a.dh + f) =
            make_float4(fmaf(ds, as.x, acc.x), fmaf(ds, as.y, acc.y), fmaf(ds, as.z, acc.z), fmaf(ds, as.w, acc.w));
    }
    if (lane == 0) a.dS[u * H + k] = ds;
}

// the per-head planes of dE re-laid as one record of all heads per edge (CSC
// order), so the in-edge sum below fetches an edge's dE in one read
template <int H>
__global__ __launch_bounds__(256) void de_records_kernel(int64_t nnz, const float* dEh, float* dEc) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= nnz) return;
    float r[H];
#pragma unroll
    for (int k = 0; k < H; ++k) r[k] = dEh[k * nnz + e];
    if constexpr (H == 4) {
        *reinterpret_cast<float4*>(dEc + e * 4) = make_float4(r[0], r[1], r[2], r[3]);
    } else {
#pragma unroll
        for (int k = 0; k < H; ++k) dEc[e * H + k] = r[k];
    }
}

struct InSumArgs {
    int64_t n;
    const int64_t* ptr;          // CSR: in-edges of each destination
    const int32_t* order;        // destinations by in-degree, descending
    int64_t n_block;             // rows that take a whole workgroup: order[0 .. n_block)
    const int32_t* cpos;         // CSC slot of each CSR edge
    const float* dEc;            // [nnz, H] CSC order
    float* dD;                   // [n, H]
};

template <int H>
__device__ __forceinline__ void add_edge(float (&acc)[H], const float* p) {
    if constexpr (H == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        acc[0] += t.x, acc[1] += t.y, acc[2] += t.z, acc[3] += t.w;
    } else {
#pragma unroll
        for (int k = 0; k < H; ++k) acc[k] += p[k];
    }
}

constexpr int kInLanes = 16;  // lanes per destination row

template <int H>
__global__ __launch_bounds__(256) void gat_in_sum_kernel(InSumArgs a) {
    __shared__ float sh[4][H];
    float acc[H];
#pragma unroll
    for (int k = 0; k < H; ++k) acc[k] = 0.0f;
    if (blockIdx.x < a.n_block) {
        // one long row per workgroup
        const int64_t v = a.order[blockIdx.x];
        for (int64_t e = a.ptr[v] + threadIdx.x; e < a.ptr[v + 1]; e += 256)
            add_edge<H>(acc, a.dEc + static_cast<int64_t>(a.cpos[e]) * H);
#pragma unroll
        for (int k = 0; k < H; ++k) acc[k] = group_sum<64>(acc[k]);
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
#pragma unroll
            for (int k = 0; k < H; ++k) sh[wave][k] = acc[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < H; ++k) acc[k] = ((sh[0][k] + sh[1][k]) + sh[2][k]) + sh[3][k];
        if (threadIdx.x == 0) {
#pragma unroll
            for (int k = 0; k < H; ++k) a.dD[v * H + k] = acc[k];
        }
        return;
    }
    const int lane = threadIdx.x % kInLanes;
    const int64_t li = a.n_block + static_cast<int64_t>(blockIdx.x - a.n_block) * (256 / kInLanes) +
                       threadIdx.x / kInLanes;
    if (li >= a.n) return;
    const int64_t v = a.order[li];
    for (int64_t e = a.ptr[v] + lane; e < a.ptr[v + 1]; e += kInLanes)
        add_edge<H>(acc, a.dEc + static_cast<int64_t>(a.cpos[e]) * H);
#pragma unroll
    for (int k = 0; k < H; ++k) acc[k] = group_sum<kInLanes>(acc[k]);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < H; ++k) a.dD[v * H + k] = acc[k];
    }
}

}  // namespace

bool gat_fused_bwd_supported(int heads, int64_t d_head) {
    const bool h = heads == 1 || heads == 2 || heads == 4 || heads == 8;
    return h && d_head >= 4 && d_head <= 256 && (d_head & (d_head - 1)) == 0;
}

size_t gat_fused_bwd_partial_bytes(const RowPlan& csc_plan, int heads, int64_t d_head) {
    return static_cast<size_t>(csc_plan.n_chunks) * heads * (d_head + 1) * 4;
}

gnn_status_t launch_gat_bwd_fused(const AggView& csr, const AggView& csc, const int32_t* cpos, int64_t nnz, int heads,
                                  int64_t d_head, float slope, const float* Hp, const float* D,
                                  const float* M, const float* Z, const float* Y, const float* dY,
                                  const float* a_src, float* rec, float* dEh, float* dEc,
                                  float* part, float* dS, float* dD, float* dHp, hipStream_t st) {
    const int64_t n = csr.n;
    if (n == 0) return GNN_OK;
    if (!gat_fused_bwd_supported(heads, d_head))
        return fail(GNN_ERR_UNSUPPORTED, "gnn_gat_layer_bwd: needs 1, 2, 4 or 8 heads and d_head a power of two "
                                         "from 4 to 256");
    const int hl = static_cast<int>(d_head / 4);
    const int64_t wave_blocks = (n + 3) / 4;
#define GNN_REC(HLv)                                                                                       \
    hipLaunchKernelGGL((gat_rec_kernel<HLv>), dim3(wave_blocks), dim3(256), 0, st, n, heads, d_head, Y, dY, D, M, \
                       Z, rec)
    switch (hl) {
        case 1: GNN_REC(1); break;
        case 2: GNN_REC(2); break;
        case 4: GNN_REC(4); break;
        case 8: GNN_REC(8); break;
        case 16: GNN_REC(16); break;
        case 32: GNN_REC(32); break;
        default: GNN_REC(64); break;
    }
#undef GNN_REC

    GatBwdArgs a;
    const RowPlan& p = *csc.plan;
    a.n = n;
    a.ptr = csc.ptr;
    a.idx = csc.idx;
    a.order = p.order;
    a.n_heavy = p.n_heavy;
    a.n_chunks = p.n_chunks;
    a.chunk = p.chunk;
    a.chunk_row = p.chunk_row;
    a.chunk_first = p.chunk_first;
    a.heads = heads;
    a.dh = d_head;
    a.Hp = Hp;
    a.rec = rec;
    a.dY = dY;
    a.a_src = a_src;
    a.act = slope == slope;  // NaN: no activation
    a.slope = a.act ? slope : 0.0f;
    a.nnz = nnz;
    a.dEh = dEh;
    a.dS = dS;
    a.dHp = dHp;
    a.part = part;
    a.pds = part + static_cast<size_t>(p.n_chunks) * heads * d_head;
    const int64_t items = p.n_chunks + (n - p.n_heavy);
    const int64_t gpb = 256 / hl;
    a.slab_blocks = (items + gpb - 1) / gpb;
#define GNN_CSC(Lv) \
    hipLaunchKernelGGL((gat_bwd_csc_kernel<Lv>), dim3(a.slab_blocks * heads), dim3(256), 0, st, a)
    {
    ScopedTimer t(st, "gat_bwd_csc_kernel h=%d dh=%lld", heads, static_cast<long long>(d_head));
    switch (hl) {
        case 1: GNN_CSC(1); break;
        case 2: GNN_CSC(2); break;
        case 4: GNN_CSC(4); break;
        case 8: GNN_CSC(8); break;
        case 16: GNN_CSC(16); break;
        case 32: GNN_CSC(32); break;
        default: GNN_CSC(64); break;
    }
    }
#undef GNN_CSC
    if (p.n_heavy > 0)
        hipLaunchKernelGGL(gat_bwd_fixup_kernel, dim3((p.n_heavy * heads + 3) / 4), dim3(256), 0, st, a);

    switch (heads) {
        case 1: hipLaunchKernelGGL((de_records_kernel<1>), dim3((nnz + 255) / 256), dim3(256), 0, st, nnz, dEh, dEc); break;
        case 2: hipLaunchKernelGGL((de_records_kernel<2>), dim3((nnz + 255) / 256), dim3(256), 0, st, nnz, dEh, dEc); break;
        case 4: hipLaunchKernelGGL((de_records_kernel<4>), dim3((nnz + 255) / 256), dim3(256), 0, st, nnz, dEh, dEc); break;
        default: hipLaunchKernelGGL((de_records_kernel<8>), dim3((nnz + 255) / 256), dim3(256), 0, st, nnz, dEh, dEc); break;
    }

    InSumArgs b;
    b.n = n;
    b.ptr = csr.ptr;
    b.order = csr.plan->order;
    b.n_block = csr.plan->n_block;
    b.cpos = cpos;
    b.dEc = dEc;
    b.dD = dD;
    const int64_t light = n - b.n_block;
    const int64_t blocks = b.n_block + (light + (256 / kInLanes) - 1) / (256 / kInLanes);
    ScopedTimer t(st, "gat_in_sum_kernel h=%d dh=%lld", heads, static_cast<long long>(d_head));
    switch (heads) {
        case 1: hipLaunchKernelGGL((gat_in_sum_kernel<1>), dim3(blocks), dim3(256), 0, st, b); break;
        case 2: hipLaunchKernelGGL((gat_in_sum_kernel<2>), dim3(blocks), dim3(256), 0, st, b); break;
        case 4: hipLaunchKernelGGL((gat_in_sum_kernel<4>), dim3(blocks), dim3(256), 0, st, b); break;
        default: hipLaunchKernelGGL((gat_in_sum_kernel<8>), dim3(blocks), dim3(256), 0, st, b); break;
    }
    return launch_status("gnn_gat_layer_bwd (edge pass)");
}

}  // namespace gnnmp
