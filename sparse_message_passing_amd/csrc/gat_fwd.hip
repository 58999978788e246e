// gat_fwd.hip -- the edge part of the GAT forward (Tango, SC'23, GAT running
// example, Fig. 1a) in one pass over the in-edges of every destination.
//
// Per destination v and head k the layer computes
//   E[e]  = LReLU(S[u] + D[v])              (SDDMM with (+) = add)
//   a[e]  = exp(E[e] - m) / sum_in(v) exp(E - m),  m = max_in(v) E
//   Y[v]  = sum_in(v) a[e] H'[u]             (weighted aggregation)
// The aggregation gathers the row H'[u, head k] of every in-edge anyway, so
// the pass forms S[u] = <H'[u, head k], a_src[k]> from that row instead of
// gathering it (one random read per edge less), and folds the softmax into
// the sum with a running maximum: for each batch of edges the running sum of
// exponentials and the running weighted row are rescaled by
// exp(m_old - m_new) and the batch's exp(E - m_new) are added (the online
// softmax: the same quotient as the two-pass definition).  The attention
// weights are never stored: the destination's final maximum M and
// Z = 1 / sum of exponentials are, and the backward forms
// a[e] = exp(E - M) Z again from them.
//
// Work decomposition: one head per column slab (slab-major over the grid, so
// a slab's gathered rows share the caches), a group of L = d_head / 4 lanes
// per destination row (lane i holds features 4i..4i+3 of the head), rows in
// degree-descending order, rows over 512 in-edges cut into chunks whose
// partial (maximum, sum, weighted row) are merged afterwards in a fixed
// order.  No atomics: bitwise reproducible.

#include "device.h"
#include "internal.h"

namespace gnnmp {

namespace {

struct GatFwdArgs {
    int64_t n;
    const int64_t* ptr;          // CSR: in-edges of each destination
    const int32_t* idx;          // source of each CSR entry
    const int32_t* order;        // destinations by in-degree, descending
    int64_t n_heavy, n_chunks, chunk;
    const int32_t* chunk_row;
    const int32_t* chunk_first;
    int heads;
    int64_t dh;
    int64_t slab_blocks;         // workgroups per head (grid = slab_blocks x heads)
    const float* Hp;             // H' [n, heads*dh]
    const float* D;              // [n, heads]
    const float* a_src;          // [heads, dh]
    float slope;
    int act;
    float* Y;                    // [n, heads*dh]
    float* M;                    // [n, heads] softmax maximum
    float* Z;                    // [n, heads] 1 / sum of exponentials
    float* part;                 // [n_chunks, heads, dh] weighted rows of the chunks
    float* pmz;                  // [n_chunks, heads, 2] (maximum, sum) of the chunks
};

__device__ __forceinline__ float4 f4_scale(float4 a, float c) {
    return make_float4(a.x * c, a.y * c, a.z * c, a.w * c);
}

template <int L>
__global__ __launch_bounds__(256) void gat_fwd_kernel(GatFwdArgs a) {
    const int lane = threadIdx.x % L;
    const int k = static_cast<int>(blockIdx.x / a.slab_blocks);
    const int64_t gid =
        static_cast<int64_t>(blockIdx.x - static_cast<int64_t>(k) * a.slab_blocks) * (256 / L) + threadIdx.x / L;
    int64_t v, eb, ee;
    bool heavy;
    if (gid < a.n_chunks) {
        const int oi = a.chunk_row[gid];
        v = a.order[oi];
        eb = a.ptr[v] + (gid - a.chunk_first[oi]) * a.chunk;
        ee = min(eb + a.chunk, a.ptr[v + 1]);
        heavy = true;
    } else {
        const int64_t li = gid - a.n_chunks + a.n_heavy;
        if (li >= a.n) return;
        v = a.order[li];
        eb = a.ptr[v];
        ee = a.ptr[v + 1];
        heavy = false;
    }
    const int H = a.heads;
    const int64_t hd = H * a.dh;
    const int64_t fo = static_cast<int64_t>(k) * a.dh + lane * 4;
    const float4 as = *reinterpret_cast<const float4*>(a.a_src + fo);
    const float dv = a.D[v * H + k];
    float m = -INFINITY, z = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int64_t e0 = eb; e0 < ee; e0 += L) {
        const int cnt = static_cast<int>(min(static_cast<int64_t>(L), ee - e0));
        const int u_my = lane < cnt ? a.idx[e0 + lane] : 0;
        for (int j = 0; j < cnt; j += 4) {
            int uq[4];
            float4 hq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) uq[q] = group_bcast<L>(u_my, (j + q < cnt) ? j + q : j);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                hq[q] = j + q < cnt ? *reinterpret_cast<const float4*>(a.Hp + static_cast<int64_t>(uq[q]) * hd + fo)
                                    : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            // the batch's scores E = LReLU(<H'[u], a_src> + D[v]); -inf past the row's end
            float eq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s = hq[q].x * as.x;
                s = fmaf(hq[q].y, as.y, s);
                s = fmaf(hq[q].z, as.z, s);
                s = fmaf(hq[q].w, as.w, s);
                s = group_sum<L>(s);
                const float x = s + dv;
                const float e = (a.act && !(x > 0.0f)) ? a.slope * x : x;
                eq[q] = j + q < cnt ? e : -INFINITY;
            }
            // rescale the running sums to the new maximum, then add the batch
            const float mn = fmaxf(m, fmaxf(fmaxf(eq[0], eq[1]), fmaxf(eq[2], eq[3])));
            const float c = __expf(m - mn);  // m = -inf on the first batch: c = 0
            acc = f4_scale(acc, c);
            z *= c;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float p = __expf(eq[q] - mn);  // 0 past the row's end
                acc = f4_fma(p, hq[q], acc);
                z += p;
            }
            m = mn;
        }
    }
    if (heavy) {
        *reinterpret_cast<float4*>(a.part + (gid * H + k) * a.dh + lane * 4) = acc;
        if (lane == 0) *reinterpret_cast<float2*>(a.pmz + (gid * H + k) * 2) = make_float2(m, z);
        return;
    }
    const float zi = z > 0.0f ? 1.0f / z : 0.0f;  // a row without in-edges aggregates nothing
    *reinterpret_cast<float4*>(a.Y + v * hd + fo) = f4_scale(acc, zi);
    if (lane == 0) {
        a.M[v * H + k] = m;
        a.Z[v * H + k] = zi;
    }
}

// Hub destinations: merge the chunks' (maximum, sum, weighted row) -- the
// maximum over the chunks, then each chunk's sum and row scaled by
// exp(its maximum - the maximum) -- and finish the row.  One wave per (hub
// row, head); a hub row has up to a few hundred chunks, so the wave's lanes
// split them: lane l takes chunks c0 + l, c0 + l + 64, ... for the maximum
// and the sum (then a butterfly over the wave), and for the row each of the
// G = 64 / (d_head / 4) lane groups takes every G-th chunk for its four
// features (then a butterfly over the groups).  A fixed order: bitwise
// reproducible.
__global__ __launch_bounds__(256) void gat_fwd_fixup_kernel(GatFwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int H = a.heads;
    if (w >= a.n_heavy * H) return;
    const int64_t i = w / H;
    const int k = static_cast<int>(w - i * H);
    const int64_t v = a.order[i];
    const int64_t c0 = a.chunk_first[i], c1 = a.chunk_first[i + 1];
    float m = -INFINITY;
    for (int64_t c = c0 + lane; c < c1; c += 64) m = fmaxf(m, a.pmz[(c * H + k) * 2]);
    m = group_max<64>(m);
    float z = 0.0f;
    for (int64_t c = c0 + lane; c < c1; c += 64) {
        const float2 mz = *reinterpret_cast<const float2*>(a.pmz + (c * H + k) * 2);
        z = fmaf(mz.y, __expf(mz.x - m), z);
    }
    z = group_sum<64>(z);
    const float zi = z > 0.0f ? 1.0f / z : 0.0f;
    const int q = static_cast<int>(a.dh / 4);  // feature quads (d_head <= 256: q <= 64)
    const int fq = lane % q, grp = lane / q, G = 64 / q;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int64_t c = c0 + grp; c < c1; c += G) {
        const float sc = __expf(a.pmz[(c * H + k) * 2] - m);
        acc = f4_fma(sc, *reinterpret_cast<const float4*>(a.part + (c * H + k) * a.dh + fq * 4), acc);
    }
    for (int o = q; o < 64; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o);
        acc.y += __shfl_xor(acc.y, o);
        acc.z += __shfl_xor(acc.z, o);
        acc.w += __shfl_xor(acc.w, o);
    }
    const int64_t hd = H * a.dh;
    if (grp == 0) *reinterpret_cast<float4*>(a.Y + v * hd + k * a.dh + fq * 4) = f4_scale(acc, zi);
    if (lane == 0) {
        a.M[v * H + k] = m;
        a.Z[v * H + k] = zi;
    }
}

}  // namespace

size_t gat_fused_fwd_partial_bytes(const RowPlan& csr_plan, int heads, int64_t d_head) {
    return align_up(static_cast<size_t>(csr_plan.n_chunks) * heads * d_head * 4) +
           align_up(static_cast<size_t>(csr_plan.n_chunks) * heads * 2 * 4);
}

gnn_status_t launch_gat_fwd_fused(const AggView& csr, int heads, int64_t d_head, float slope, const float* Hp,
                                  const float* D, const float* a_src, float* Y, float* M, float* Z, float* part,
                                  hipStream_t st) {
    const int64_t n = csr.n;
    if (n == 0) return GNN_OK;
    if (!gat_fused_bwd_supported(heads, d_head))
        return fail(GNN_ERR_UNSUPPORTED, "gnn_gat_layer_fwd: needs 1, 2, 4 or 8 heads and d_head a power of two "
                                         "from 4 to 256");
    const RowPlan& p = *csr.plan;
    GatFwdArgs a;
    a.n = n;
    a.ptr = csr.ptr;
    a.idx = csr.idx;
    a.order = p.order;
    a.n_heavy = p.n_heavy;
    a.n_chunks = p.n_chunks;
    a.chunk = p.chunk;
    a.chunk_row = p.chunk_row;
    a.chunk_first = p.chunk_first;
    a.heads = heads;
    a.dh = d_head;
    a.Hp = Hp;
    a.D = D;
    a.a_src = a_src;
    a.act = slope == slope;  // NaN: no activation
    a.slope = a.act ? slope : 0.0f;
    a.Y = Y;
    a.M = M;
    a.Z = Z;
    a.part = part;
    a.pmz = reinterpret_cast<float*>(reinterpret_cast<char*>(part) +
                                     align_up(static_cast<size_t>(p.n_chunks) * heads * d_head * 4));
    const int hl = static_cast<int>(d_head / 4);
    const int64_t items = p.n_chunks + (n - p.n_heavy);
    const int64_t gpb = 256 / hl;
    a.slab_blocks = (items + gpb - 1) / gpb;
    {
        ScopedTimer t(st, "gat_fwd_kernel h=%d dh=%lld", heads, static_cast<long long>(d_head));
#define GNN_FWD(Lv) hipLaunchKernelGGL((gat_fwd_kernel<Lv>), dim3(a.slab_blocks * heads), dim3(256), 0, st, a)
        switch (hl) {
            case 1: GNN_FWD(1); break;
            case 2: GNN_FWD(2); break;
            case 4: GNN_FWD(4); break;
            case 8: GNN_FWD(8); break;
            case 16: GNN_FWD(16); break;
            case 32: GNN_FWD(32); break;
            default: GNN_FWD(64); break;
        }
#undef GNN_FWD
    }
    if (p.n_heavy > 0)
        hipLaunchKernelGGL(gat_fwd_fixup_kernel, dim3((p.n_heavy * heads + 3) / 4), dim3(256), 0, st, a);
    return launch_status("gnn_gat_layer_fwd (edge pass)");
}

}  // namespace gnnmp
