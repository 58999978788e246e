// edge.hip -- edge-valued steps of the GAT chain (Tango, SC'23, GAT running
// example, Fig. 1a forward and Fig. 1b backward):
//   * per-head attention scores S = H' a_src, D = H' a_dst;
//   * SDDMM with (+) = add followed by LeakyReLU, and SDDMM with the dot
//     product (the attention gradient dY[dst] . H'[src]);
//   * edge softmax over each destination's in-edges, and its backward
//     dE = alpha (dalpha - sum_in alpha dalpha), with LeakyReLU';
//   * edge -> node sums over in-edges (CSR) or out-edges (CSC + eid);
//   * the per-head column sums da = sum_v dS[v, k] H'[v, head k].
//
// Edge arrays are [nnz, heads] in CSR order; with 4 heads one edge is one
// 16-byte vector.  Per-row kernels give a group of 16 lanes to each row
// (lane i walks edges i, i+16, ...) and a whole 256-thread workgroup to the
// few rows longer than kBlockRow; edge-parallel kernels reuse the row/chunk
// schedule of the aggregation so that hub rows are cut into independent
// chunks.  Reductions are fixed-order butterflies: no atomics.

#include "device.h"
#include "internal.h"

namespace gnnmp {

namespace {

constexpr int G = 16;  // lanes per row in the per-row edge kernels
constexpr int kCache = 4;  // edges per lane kept in registers by the softmax kernels (rows up to 64 edges)

template <int H>
struct HV {
    float v[H];
};

template <int H>
__device__ __forceinline__ HV<H> ld(const float* p) {
    HV<H> r;
    if constexpr (H == 4) {
        float4 t = *reinterpret_cast<const float4*>(p);
        r.v[0] = t.x, r.v[1] = t.y, r.v[2] = t.z, r.v[3] = t.w;
    } else if constexpr (H == 2) {
        float2 t = *reinterpret_cast<const float2*>(p);
        r.v[0] = t.x, r.v[1] = t.y;
    } else if constexpr (H == 8) {
        float4 t = *reinterpret_cast<const float4*>(p);
        float4 u = *reinterpret_cast<const float4*>(p + 4);
        r.v[0] = t.x, r.v[1] = t.y, r.v[2] = t.z, r.v[3] = t.w;
        r.v[4] = u.x, r.v[5] = u.y, r.v[6] = u.z, r.v[7] = u.w;
    } else {
#pragma unroll
        for (int k = 0; k < H; ++k) r.v[k] = p[k];
    }
    return r;
}

template <int H>
__device__ __forceinline__ void st(float* p, const HV<H>& r) {
    if constexpr (H == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(r.v[0], r.v[1], r.v[2], r.v[3]);
    } else if constexpr (H == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(r.v[0], r.v[1]);
    } else if constexpr (H == 8) {
        *reinterpret_cast<float4*>(p) = make_float4(r.v[0], r.v[1], r.v[2], r.v[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(r.v[4], r.v[5], r.v[6], r.v[7]);
    } else {
#pragma unroll
        for (int k = 0; k < H; ++k) p[k] = r.v[k];
    }
}

// ---------------------------------------------------------------------------
// work items shared by the edge-parallel kernels: heavy-row chunks first,
// then the remaining rows in degree order
// ---------------------------------------------------------------------------
struct Sched {
    int64_t n;
    const int64_t* ptr;
    const int32_t* idx;
    const int32_t* eid;
    const int32_t* order;
    int64_t n_heavy, n_chunks, n_block, chunk;
    const int32_t* chunk_row;
    const int32_t* chunk_first;
};

Sched make_sched(const AggView& v) {
    Sched s;
    s.n = v.n;
    s.ptr = v.ptr;
    s.idx = v.idx;
    s.eid = v.eid;
    s.order = v.plan->order;
    s.n_heavy = v.plan->n_heavy;
    s.n_chunks = v.plan->n_chunks;
    s.n_block = v.plan->n_block;
    s.chunk = v.plan->chunk;
    s.chunk_row = v.plan->chunk_row;
    s.chunk_first = v.plan->chunk_first;
    return s;
}

__device__ __forceinline__ bool work_item(const Sched& s, int64_t gid, int64_t& row, int64_t& eb, int64_t& ee) {
    if (gid < s.n_chunks) {
        const int oi = s.chunk_row[gid];
        row = s.order[oi];
        eb = s.ptr[row] + (gid - s.chunk_first[oi]) * s.chunk;
        ee = min(eb + s.chunk, s.ptr[row + 1]);
        return true;
    }
    const int64_t li = gid - s.n_chunks + s.n_heavy;
    if (li >= s.n) return false;
    row = s.order[li];
    eb = s.ptr[row];
    ee = s.ptr[row + 1];
    return true;
}

inline int64_t sched_items(const Sched& s) { return s.n_chunks + (s.n - s.n_heavy); }

// ---------------------------------------------------------------------------
// SDDMM add + LeakyReLU
// ---------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(256) void sddmm_add_kernel(Sched s, const float* S, int64_t lds, const float* D,
                                                        int64_t ldd, float slope, int act, float* out,
                                                        float* out_pre) {
    const int lane = threadIdx.x % G;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * (256 / G) + threadIdx.x / G;
    int64_t v, eb, ee;
    if (!work_item(s, gid, v, eb, ee)) return;
    float dv[H];
#pragma unroll
    for (int k = 0; k < H; ++k) dv[k] = D[v * ldd + k];
    for (int64_t e = eb + lane; e < ee; e += G) {
        const int64_t u = s.idx[e];
        HV<H> p, r;
#pragma unroll
        for (int k = 0; k < H; ++k) {
            p.v[k] = S[u * lds + k] + dv[k];
            r.v[k] = (act && !(p.v[k] > 0.0f)) ? slope * p.v[k] : p.v[k];
        }
        st<H>(out + e * H, r);
        if (out_pre) st<H>(out_pre + e * H, p);
    }
}

// ---------------------------------------------------------------------------
// SDDMM dot: out[e, k] = sum_j src[u, k*dh + j] * dst[v, k*dh + j]
// a group of LANES = d/4 lanes per row, each lane 4 features; the head's
// lanes (dh/4 of them) are reduced with a butterfly
// ---------------------------------------------------------------------------
template <int LANES, int HL, typename T>
__global__ __launch_bounds__(256) void sddmm_dot_kernel(Sched s, const T* src, int64_t ld_src, const T* dst,
                                                        int64_t ld_dst, int heads, float* out) {
    const int lane = threadIdx.x % LANES;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * (256 / LANES) + threadIdx.x / LANES;
    int64_t v, eb, ee;
    if (!work_item(s, gid, v, eb, ee)) return;
    const int f = lane * 4;
    const float4 dvec = Elem<T>::load4(dst + v * ld_dst + f);
    const int head = lane / HL;
    for (int64_t e0 = eb; e0 < ee; e0 += LANES) {
        const int cnt = static_cast<int>(min(static_cast<int64_t>(LANES), ee - e0));
        const int u_my = lane < cnt ? s.idx[e0 + lane] : 0;
        for (int j = 0; j < cnt; j += 4) {
            float4 x[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = group_bcast<LANES>(u_my, j + q < cnt ? j + q : j);
                x[q] = Elem<T>::load4(src + static_cast<int64_t>(u) * ld_src + f);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float p = x[q].x * dvec.x;
                p = fmaf(x[q].y, dvec.y, p);
                p = fmaf(x[q].z, dvec.z, p);
                p = fmaf(x[q].w, dvec.w, p);
                p = group_sum<HL>(p);
                if (j + q < cnt && (lane % HL) == 0) out[(e0 + j + q) * heads + head] = p;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// SDDMM dot on 8-bit codes (Tango: the dot of two quantised rows is the dot
// of their codes times the product of the scales).  A group of LQ lanes per
// row, each lane 16 code bytes of the row (four v_dot4 steps, int32 sums,
// exact); the HQ = d_head/16 lanes of a head are summed with a butterfly and
// the head's first lane writes f32(sum) * (s_src * s_dst).  A gathered row is
// d bytes instead of 4d.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ int group_isum(int v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
    return v;
}

template <int LQ, int HQ>
__global__ __launch_bounds__(256) void sddmm_q8_kernel(Sched s, const int8_t* src, const int8_t* dst, int64_t d,
                                                       int heads, const float* sc, float* out) {
    const int lane = threadIdx.x % LQ;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * (256 / LQ) + threadIdx.x / LQ;
    int64_t v, eb, ee;
    if (!work_item(s, gid, v, eb, ee)) return;
    const bool act = static_cast<int64_t>(lane) * 16 < d;  // lanes past the row's d/16 contribute zeros
    const int64_t f = static_cast<int64_t>(lane) * 16;
    const int4 zero4 = make_int4(0, 0, 0, 0);
    const int4 dv = act ? *reinterpret_cast<const int4*>(dst + v * d + f) : zero4;
    const int head = lane / HQ;
    const float scale = __fmul_rn(sc[0], sc[1]);
    for (int64_t e0 = eb; e0 < ee; e0 += LQ) {
        const int cnt = static_cast<int>(min(static_cast<int64_t>(LQ), ee - e0));
        const int u_my = lane < cnt ? s.idx[e0 + lane] : 0;
        for (int j = 0; j < cnt; j += 4) {
            int4 x[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = group_bcast<LQ>(u_my, j + q < cnt ? j + q : j);
                x[q] = act ? *reinterpret_cast<const int4*>(src + static_cast<int64_t>(u) * d + f) : zero4;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int p = __builtin_amdgcn_sdot4(x[q].x, dv.x, 0, false);
                p = __builtin_amdgcn_sdot4(x[q].y, dv.y, p, false);
                p = __builtin_amdgcn_sdot4(x[q].z, dv.z, p, false);
                p = __builtin_amdgcn_sdot4(x[q].w, dv.w, p, false);
                p = group_isum<HQ>(p);
                if (act && j + q < cnt && (lane % HQ) == 0)
                    out[(e0 + j + q) * heads + head] = __fmul_rn(static_cast<float>(p), scale);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// edge softmax and its backward: per-row groups for rows of degree <=
// kBlockRow, one workgroup per longer row
// ---------------------------------------------------------------------------
template <int H>
__device__ __forceinline__ void hv_fill(HV<H>& a, float x) {
#pragma unroll
    for (int k = 0; k < H; ++k) a.v[k] = x;
}

template <int H, int W>
__device__ __forceinline__ void hv_group_max(HV<H>& a) {
#pragma unroll
    for (int k = 0; k < H; ++k) a.v[k] = group_max<W>(a.v[k]);
}
template <int H, int W>
__device__ __forceinline__ void hv_group_sum(HV<H>& a) {
#pragma unroll
    for (int k = 0; k < H; ++k) a.v[k] = group_sum<W>(a.v[k]);
}

// block-wide reduction of H values (256 threads = 4 waves), result in every thread
template <int H, bool MAX>
__device__ __forceinline__ void hv_block_reduce(HV<H>& a, float (*sh)[H]) {
    if (MAX) hv_group_max<H, 64>(a);
    else hv_group_sum<H, 64>(a);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int k = 0; k < H; ++k) sh[wave][k] = a.v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < H; ++k) {
        float r = sh[0][k];
        for (int w = 1; w < 4; ++w) r = MAX ? fmaxf(r, sh[w][k]) : r + sh[w][k];
        a.v[k] = r;
    }
}

// Running maximum m and sum z of exp(x - m) of one value per head: a value
// above the maximum rescales the sum by exp(m_old - x) (an empty sum stays 0,
// so the first value gives z = 1); a -inf while the maximum is still -inf
// adds nothing (as exp(x - m) does once a finite maximum exists).
template <int H>
__device__ __forceinline__ void online_add(HV<H>& m, HV<H>& z, const HV<H>& x) {
#pragma unroll
    for (int k = 0; k < H; ++k) {
        if (x.v[k] > m.v[k]) {
            z.v[k] = fmaf(z.v[k], __expf(m.v[k] - x.v[k]), 1.0f);
            m.v[k] = x.v[k];
        } else if (m.v[k] != -INFINITY) {
            z.v[k] += __expf(x.v[k] - m.v[k]);
        }
    }
}

// the G lanes' (m, z) merged: the row maximum, and each lane's sum brought to
// it before the group sum
template <int H>
__device__ __forceinline__ void group_merge(HV<H>& m, HV<H>& z) {
    HV<H> mt = m;
    hv_group_max<H, G>(m);
#pragma unroll
    for (int k = 0; k < H; ++k) z.v[k] = mt.v[k] == -INFINITY ? 0.0f : z.v[k] * __expf(mt.v[k] - m.v[k]);
    hv_group_sum<H, G>(z);
}

template <int H>
__device__ __forceinline__ void softmax_fwd_rows(const Sched& s, const float* E, float* alpha, int64_t blk) {
    const int lane = threadIdx.x % G;
    const int64_t li = s.n_block + static_cast<int64_t>(blk) * (256 / G) + threadIdx.x / G;
    if (li >= s.n) return;
    const int64_t v = s.order[li];
    const int64_t eb = s.ptr[v], ee = s.ptr[v + 1];
    HV<H> m;
    hv_fill<H>(m, -INFINITY);
    if (ee - eb <= G * kCache) {
        // short row: each lane keeps its (up to kCache) edges in registers, so
        // E is read once; the same per-lane orders as the general path below
        HV<H> x[kCache];
#pragma unroll
        for (int c = 0; c < kCache; ++c) {
            const int64_t e = eb + lane + c * G;
            if (e < ee) {
                x[c] = ld<H>(E + e * H);
#pragma unroll
                for (int k = 0; k < H; ++k) m.v[k] = fmaxf(m.v[k], x[c].v[k]);
            }
        }
        hv_group_max<H, G>(m);
        HV<H> z;
        hv_fill<H>(z, 0.0f);
#pragma unroll
        for (int c = 0; c < kCache; ++c)
            if (eb + lane + c * G < ee) {
#pragma unroll
                for (int k = 0; k < H; ++k) z.v[k] += __expf(x[c].v[k] - m.v[k]);
            }
        hv_group_sum<H, G>(z);
#pragma unroll
        for (int k = 0; k < H; ++k) z.v[k] = 1.0f / z.v[k];
#pragma unroll
        for (int c = 0; c < kCache; ++c) {
            const int64_t e = eb + lane + c * G;
            if (e < ee) {
#pragma unroll
                for (int k = 0; k < H; ++k) x[c].v[k] = __expf(x[c].v[k] - m.v[k]) * z.v[k];
                st<H>(alpha + e * H, x[c]);
            }
        }
        return;
    }
    // long row: the maximum and the sum of exponentials in one pass (each
    // lane keeps a running maximum and rescales its sum when it grows; the
    // lanes' sums are brought to the row maximum before they are added), then
    // one pass that writes alpha: E is read twice instead of three times
    HV<H> z;
    hv_fill<H>(z, 0.0f);
    for (int64_t e = eb + lane; e < ee; e += G) {
        HV<H> x = ld<H>(E + e * H);
        online_add<H>(m, z, x);
    }
    group_merge<H>(m, z);
#pragma unroll
    for (int k = 0; k < H; ++k) z.v[k] = 1.0f / z.v[k];
    for (int64_t e = eb + lane; e < ee; e += G) {
        HV<H> x = ld<H>(E + e * H);
#pragma unroll
        for (int k = 0; k < H; ++k) x.v[k] = __expf(x.v[k] - m.v[k]) * z.v[k];
        st<H>(alpha + e * H, x);
    }
}

template <int H>
__device__ __forceinline__ void softmax_fwd_block(const Sched& s, const float* E, float* alpha, int64_t blk, float (*sh)[H]) {
    const int64_t v = s.order[blk];
    const int64_t eb = s.ptr[v], ee = s.ptr[v + 1];
    // the maximum and the sum of exponentials in one pass (as for long rows
    // above), then the pass that writes alpha
    HV<H> m;
    hv_fill<H>(m, -INFINITY);
    HV<H> z;
    hv_fill<H>(z, 0.0f);
    for (int64_t e = eb + threadIdx.x; e < ee; e += 256) {
        HV<H> x = ld<H>(E + e * H);
        online_add<H>(m, z, x);
    }
    HV<H> mt = m;
    hv_block_reduce<H, true>(m, sh);
#pragma unroll
    for (int k = 0; k < H; ++k) z.v[k] = mt.v[k] == -INFINITY ? 0.0f : z.v[k] * __expf(mt.v[k] - m.v[k]);
    hv_block_reduce<H, false>(z, sh);
#pragma unroll
    for (int k = 0; k < H; ++k) z.v[k] = 1.0f / z.v[k];
    for (int64_t e = eb + threadIdx.x; e < ee; e += 256) {
        HV<H> x = ld<H>(E + e * H);
#pragma unroll
        for (int k = 0; k < H; ++k) x.v[k] = __expf(x.v[k] - m.v[k]) * z.v[k];
        st<H>(alpha + e * H, x);
    }
}

template <int H>
__device__ __forceinline__ HV<H> dE_of(const HV<H>& a, const HV<H>& da, const HV<H>& P, const float* pre,
                                       int64_t e, float slope) {
    HV<H> r;
#pragma unroll
    for (int k = 0; k < H; ++k) r.v[k] = a.v[k] * (da.v[k] - P.v[k]);
    if (pre) {
        HV<H> p = ld<H>(pre + e * H);
#pragma unroll
        for (int k = 0; k < H; ++k) r.v[k] = p.v[k] > 0.0f ? r.v[k] : r.v[k] * slope;
    }
    return r;
}

template <int H>
__device__ __forceinline__ void softmax_bwd_rows(const Sched& s, const float* alpha, const float* dalpha,
                                                 const float* pre, float slope, float* dE, int64_t blk) {
    const int lane = threadIdx.x % G;
    const int64_t li = s.n_block + static_cast<int64_t>(blk) * (256 / G) + threadIdx.x / G;
    if (li >= s.n) return;
    const int64_t v = s.order[li];
    const int64_t eb = s.ptr[v], ee = s.ptr[v + 1];
    HV<H> P;
    hv_fill<H>(P, 0.0f);
    if (ee - eb <= G * kCache) {
        // short row: alpha and dalpha of the lane's edges stay in registers
        HV<H> a[kCache], da[kCache];
#pragma unroll
        for (int c = 0; c < kCache; ++c) {
            const int64_t e = eb + lane + c * G;
            if (e < ee) {
                a[c] = ld<H>(alpha + e * H);
                da[c] = ld<H>(dalpha + e * H);
#pragma unroll
                for (int k = 0; k < H; ++k) P.v[k] = fmaf(a[c].v[k], da[c].v[k], P.v[k]);
            }
        }
        hv_group_sum<H, G>(P);
#pragma unroll
        for (int c = 0; c < kCache; ++c) {
            const int64_t e = eb + lane + c * G;
            if (e < ee) st<H>(dE + e * H, dE_of<H>(a[c], da[c], P, pre, e, slope));
        }
        return;
    }
    for (int64_t e = eb + lane; e < ee; e += G) {
        HV<H> a = ld<H>(alpha + e * H), da = ld<H>(dalpha + e * H);
#pragma unroll
        for (int k = 0; k < H; ++k) P.v[k] = fmaf(a.v[k], da.v[k], P.v[k]);
    }
    hv_group_sum<H, G>(P);
    for (int64_t e = eb + lane; e < ee; e += G) {
        HV<H> a = ld<H>(alpha + e * H), da = ld<H>(dalpha + e * H);
        st<H>(dE + e * H, dE_of<H>(a, da, P, pre, e, slope));
    }
}

template <int H>
__device__ __forceinline__ void softmax_bwd_block(const Sched& s, const float* alpha, const float* dalpha,
                                                  const float* pre, float slope, float* dE, int64_t blk,
                                                  float (*sh)[H]) {
    const int64_t v = s.order[blk];
    const int64_t eb = s.ptr[v], ee = s.ptr[v + 1];
    HV<H> P;
    hv_fill<H>(P, 0.0f);
    for (int64_t e = eb + threadIdx.x; e < ee; e += 256) {
        HV<H> a = ld<H>(alpha + e * H), da = ld<H>(dalpha + e * H);
#pragma unroll
        for (int k = 0; k < H; ++k) P.v[k] = fmaf(a.v[k], da.v[k], P.v[k]);
    }
    hv_block_reduce<H, false>(P, sh);
    for (int64_t e = eb + threadIdx.x; e < ee; e += 256) {
        HV<H> a = ld<H>(alpha + e * H), da = ld<H>(dalpha + e * H);
        st<H>(dE + e * H, dE_of<H>(a, da, P, pre, e, slope));
    }
}

// ---------------------------------------------------------------------------
// edge -> node sums; over the CSC view the values are gathered through eid
// ---------------------------------------------------------------------------
template <int H>
__device__ __forceinline__ void reduce_rows(const Sched& s, const float* vals, float* out, int64_t blk) {
    const int lane = threadIdx.x % G;
    const int64_t li = s.n_block + static_cast<int64_t>(blk) * (256 / G) + threadIdx.x / G;
    if (li >= s.n) return;
    const int64_t v = s.order[li];
    HV<H> acc;
    hv_fill<H>(acc, 0.0f);
    for (int64_t e = s.ptr[v] + lane; e < s.ptr[v + 1]; e += G) {
        const int64_t ce = s.eid ? static_cast<int64_t>(s.eid[e]) : e;
        HV<H> x = ld<H>(vals + ce * H);
#pragma unroll
        for (int k = 0; k < H; ++k) acc.v[k] += x.v[k];
    }
    hv_group_sum<H, G>(acc);
    if (lane == 0) st<H>(out + v * H, acc);
}

template <int H>
__device__ __forceinline__ void reduce_block(const Sched& s, const float* vals, float* out, int64_t blk,
                                             float (*sh)[H]) {
    const int64_t v = s.order[blk];
    HV<H> acc;
    hv_fill<H>(acc, 0.0f);
    for (int64_t e = s.ptr[v] + threadIdx.x; e < s.ptr[v + 1]; e += 256) {
        const int64_t ce = s.eid ? static_cast<int64_t>(s.eid[e]) : e;
        HV<H> x = ld<H>(vals + ce * H);
#pragma unroll
        for (int k = 0; k < H; ++k) acc.v[k] += x.v[k];
    }
    hv_block_reduce<H, false>(acc, sh);
    if (threadIdx.x == 0) st<H>(out + v * H, acc);
}

// One launch per op: the first n_block workgroups each take one long row (the
// longest first), the rest take 16 short rows each, so the long rows run
// alongside the short ones instead of in a launch of their own.
template <int H>
__global__ __launch_bounds__(256) void softmax_fwd_kernel(Sched s, const float* E, float* alpha) {
    __shared__ float sh[4][H];
    if (blockIdx.x < s.n_block) softmax_fwd_block<H>(s, E, alpha, blockIdx.x, sh);
    else softmax_fwd_rows<H>(s, E, alpha, blockIdx.x - s.n_block);
}

template <int H>
__global__ __launch_bounds__(256) void softmax_bwd_kernel(Sched s, const float* alpha, const float* dalpha,
                                                          const float* pre, float slope, float* dE) {
    __shared__ float sh[4][H];
    if (blockIdx.x < s.n_block) softmax_bwd_block<H>(s, alpha, dalpha, pre, slope, dE, blockIdx.x, sh);
    else softmax_bwd_rows<H>(s, alpha, dalpha, pre, slope, dE, blockIdx.x - s.n_block);
}

template <int H>
__global__ __launch_bounds__(256) void reduce_kernel(Sched s, const float* vals, float* out) {
    __shared__ float sh[4][H];
    if (blockIdx.x < s.n_block) reduce_block<H>(s, vals, out, blockIdx.x, sh);
    else reduce_rows<H>(s, vals, out, blockIdx.x - s.n_block);
}

// ---------------------------------------------------------------------------
// GAT scores: S[v,k] = <H'[v, head k], a_src[k]>, D likewise (one wave per row)
// ---------------------------------------------------------------------------
// Two rows per wave (both rows' loads in flight before either is reduced).
template <int HL>
__global__ __launch_bounds__(256) void gat_scores_kernel(int64_t n, const float* Hp, int64_t d, int heads,
                                                         const float* a_src, const float* a_dst, float* S, float* D) {
    const int lane = threadIdx.x & 63;
    const int64_t v0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 2;
    if (v0 >= n) return;
    for (int64_t f0 = 0; f0 < d; f0 += 256) {
        const int64_t f = f0 + lane * 4;
        float4 x[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            x[j] = (f < d && v0 + j < n) ? *reinterpret_cast<const float4*>(Hp + (v0 + j) * d + f)
                                         : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float4 as = make_float4(0.0f, 0.0f, 0.0f, 0.0f), ad = as;
        if (f < d) {
            as = *reinterpret_cast<const float4*>(a_src + f);
            ad = *reinterpret_cast<const float4*>(a_dst + f);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float ps = x[j].x * as.x;
            ps = fmaf(x[j].y, as.y, ps);
            ps = fmaf(x[j].z, as.z, ps);
            ps = fmaf(x[j].w, as.w, ps);
            float pd = x[j].x * ad.x;
            pd = fmaf(x[j].y, ad.y, pd);
            pd = fmaf(x[j].z, ad.z, pd);
            pd = fmaf(x[j].w, ad.w, pd);
            ps = group_sum<HL>(ps);
            pd = group_sum<HL>(pd);
            const int64_t v = v0 + j;
            if (f < d && v < n && (lane % HL) == 0) {
                const int64_t k = f / (HL * 4);
                S[v * heads + k] = ps;
                D[v * heads + k] = pd;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// per-head column sums: outA[f] = sum_v coefA[v, f/dh] * Hp[v, f] (and B)
// stage 1: each block sums a range of rows; stage 2: blocks in order
// ---------------------------------------------------------------------------
constexpr int64_t kColRows = 2048;

__global__ __launch_bounds__(256) void colsum_stage1(int64_t n, const float* cA, const float* cB, const float* Hp,
                                                     int64_t d, int heads, int64_t dh, float* partial) {
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kColRows;
    const int64_t r1 = min(n, r0 + kColRows);
    for (int64_t f = threadIdx.x; f < d; f += 256) {
        const int64_t k = f / dh;
        float sa = 0.0f, sb = 0.0f;
#pragma unroll 8
        for (int64_t v = r0; v < r1; ++v) {
            const float x = Hp[v * d + f];
            sa = fmaf(cA[v * heads + k], x, sa);
            sb = fmaf(cB[v * heads + k], x, sb);
        }
        partial[(static_cast<int64_t>(blockIdx.x) * 2 + 0) * d + f] = sa;
        partial[(static_cast<int64_t>(blockIdx.x) * 2 + 1) * d + f] = sb;
    }
}

// out[f] (f < 2d: A then B) = sum over blocks b of partial[b][f], in a fixed
// order: four thread groups take every fourth block, then their sums are added
// in order.  One workgroup per 64 outputs.
__global__ __launch_bounds__(256) void colsum_stage2(int64_t nblk, int64_t d, const float* partial, float* outA,
                                                     float* outB) {
    __shared__ float sh[4][64];
    const int64_t o = static_cast<int64_t>(blockIdx.x) * 64 + (threadIdx.x & 63);  // in [0, 2d)
    const int grp = threadIdx.x >> 6;
    // block b goes to group b mod 4, and within the group to accumulator
    // (b / 4) mod 4: a fixed order with four loads in flight per thread
    float p4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (o < 2 * d) {
        int64_t b = grp;
        for (; b + 12 < nblk; b += 16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) p4[q] += partial[(b + 4 * q) * 2 * d + o];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (b + 4 * q < nblk) p4[q] += partial[(b + 4 * q) * 2 * d + o];
    }
    const float s = (p4[0] + p4[1]) + (p4[2] + p4[3]);
    sh[grp][threadIdx.x & 63] = s;
    __syncthreads();
    if (grp == 0 && o < 2 * d) {
        const int t = threadIdx.x;
        const float tot = ((sh[0][t] + sh[1][t]) + sh[2][t]) + sh[3][t];
        if (o < d) outA[o] = tot;
        else outB[o - d] = tot;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define GNN_HEADS_SWITCH(heads, CALL)                                                       \
    switch (heads) {                                                                         \
        case 1: { constexpr int H = 1; CALL; } break;                                        \
        case 2: { constexpr int H = 2; CALL; } break;                                        \
        case 4: { constexpr int H = 4; CALL; } break;                                        \
        case 8: { constexpr int H = 8; CALL; } break;                                        \
        default: return fail(GNN_ERR_UNSUPPORTED, "edge kernels support 1, 2, 4 or 8 heads"); \
    }

gnn_status_t launch_sddmm_add(const AggView& v, const float* S, int64_t lds, const float* D, int64_t ldd, int heads,
                              float slope, float* out, float* out_pre, hipStream_t st) {
    if (v.n == 0) return GNN_OK;
    Sched s = make_sched(v);
    const int64_t blocks = (sched_items(s) + (256 / G) - 1) / (256 / G);
    const int act = slope == slope;  // NaN: no activation
    ScopedTimer t(st, "sddmm_add_kernel h=%d", heads);
    GNN_HEADS_SWITCH(heads, hipLaunchKernelGGL((sddmm_add_kernel<H>), dim3(blocks), dim3(256), 0, st, s, S, lds, D,
                                               ldd, act ? slope : 0.0f, act, out, out_pre));
    return launch_status("gnn_sddmm(add)");
}

bool sddmm_q8_supported(int heads, int64_t d_head) {
    const int64_t hq = d_head / 16;
    return heads >= 1 && d_head % 16 == 0 && hq >= 1 && hq <= 16 && (hq & (hq - 1)) == 0 && heads * d_head <= 1024;
}

size_t sddmm_q8_ws_bytes(int64_t n, int64_t d) {
    return 2 * align_up(static_cast<size_t>(n) * d) + align_up(1024 * 4) + align_up(4 * 4);
}

gnn_status_t launch_sddmm_q8(const AggView& v, const float* src, int64_t ld_src, const float* dst, int64_t ld_dst,
                             int heads, int64_t d_head, uint64_t seed, uint32_t stream_id, float* out, void* ws,
                             hipStream_t st) {
    const int64_t n = v.n, d = heads * d_head;
    if (n == 0) return GNN_OK;
    char* w = static_cast<char*>(ws);
    int8_t* qs = reinterpret_cast<int8_t*>(w);
    w += align_up(static_cast<size_t>(n) * d);
    int8_t* qd = reinterpret_cast<int8_t*>(w);
    w += align_up(static_cast<size_t>(n) * d);
    float* partial = reinterpret_cast<float*>(w);
    w += align_up(1024 * 4);
    float* stat = reinterpret_cast<float*>(w);  // [max|src|, max|dst|, s_src, s_dst]
    // tensor-level scales and the sequential quantisation pass over each operand
    GNN_TRY(launch_absmax(src, ld_src, n, d, partial, stat + 0, st));
    GNN_TRY(launch_absmax(dst, ld_dst, n, d, partial + 512, stat + 1, st));
    GNN_TRY(launch_quantize_sym8(src, ld_src, n, d, stat + 0, seed, stream_id, qs, d, 0, stat + 2, st));
    GNN_TRY(launch_quantize_sym8(dst, ld_dst, n, d, stat + 1, seed, stream_id + 1, qd, d, 0, stat + 3, st));
    Sched s = make_sched(v);
    const int64_t need = (d + 15) / 16;
    const int lq = need <= 4 ? 4 : need <= 8 ? 8 : need <= 16 ? 16 : need <= 32 ? 32 : 64;
    const int hq = static_cast<int>(d_head / 16);
    const int64_t blocks = (sched_items(s) + (256 / lq) - 1) / (256 / lq);
#define GNN_Q8(L, HQv) \
    hipLaunchKernelGGL((sddmm_q8_kernel<L, HQv>), dim3(blocks), dim3(256), 0, st, s, qs, qd, d, heads, stat + 2, out)
#define GNN_Q8_H(L)                                           \
    switch (hq) {                                             \
        case 1: GNN_Q8(L, 1); break;                          \
        case 2: GNN_Q8(L, 2); break;                          \
        case 4: GNN_Q8(L, 4); break;                          \
        case 8: if (L >= 8) { GNN_Q8(L, 8); } break;          \
        default: if (L >= 16) { GNN_Q8(L, 16); } break;       \
    }
    switch (lq) {
        case 4: GNN_Q8_H(4) break;
        case 8: GNN_Q8_H(8) break;
        case 16: GNN_Q8_H(16) break;
        case 32: GNN_Q8_H(32) break;
        default: GNN_Q8_H(64) break;
    }
#undef GNN_Q8_H
#undef GNN_Q8
    return launch_status("gnn_sddmm_q8");
}

gnn_status_t launch_sddmm_dot(const AggView& v, const void* src_feat, int64_t ld_src, const void* dst_feat,
                              int64_t ld_dst, gnn_dtype_t dt, int heads, int64_t d_head, float* out, hipStream_t st) {
    if (v.n == 0) return GNN_OK;
    const int64_t d = heads * d_head;
    if (d_head % 4 || ld_src % 4 || ld_dst % 4 || d > 256)
        return fail(GNN_ERR_UNSUPPORTED, "gnn_sddmm(dot): needs d_head, leading dims multiple of 4 and heads*d_head <= 256");
    const int64_t hl = d_head / 4;
    if (hl & (hl - 1)) return fail(GNN_ERR_UNSUPPORTED, "gnn_sddmm(dot): d_head/4 must be a power of two");
    const int64_t need = d / 4;
    const int lanes = need <= 16 ? 16 : need <= 32 ? 32 : 64;
    if (need != lanes) return fail(GNN_ERR_UNSUPPORTED, "gnn_sddmm(dot): heads*d_head must be 64, 128 or 256");
    Sched s = make_sched(v);
    const int64_t blocks = (sched_items(s) + (256 / lanes) - 1) / (256 / lanes);
    ScopedTimer t(st, "sddmm_dot_kernel h=%d dh=%lld %s", heads, static_cast<long long>(d_head), dt_name(dt));
#define GNN_DOT(L, HLv, T)                                                                                         \
    hipLaunchKernelGGL((sddmm_dot_kernel<L, HLv, T>), dim3(blocks), dim3(256), 0, st, s,                          \
                       static_cast<const T*>(src_feat), ld_src, static_cast<const T*>(dst_feat), ld_dst, heads, out)
#define GNN_DOT_HL(L, T)                                                                                           \
    switch (hl) {                                                                                                  \
        case 1: GNN_DOT(L, 1, T); break;                                                                           \
        case 2: GNN_DOT(L, 2, T); break;                                                                           \
        case 4: GNN_DOT(L, 4, T); break;                                                                           \
        case 8: GNN_DOT(L, 8, T); break;                                                                           \
        case 16: GNN_DOT(L, 16, T); break;                                                                         \
        case 32: if (L >= 32) { GNN_DOT(L, 32, T); } break;                                                        \
        default: if (L == 64) { GNN_DOT(L, 64, T); } break;                                                        \
    }
    if (dt == GNN_F32) {
        if (lanes == 16) { GNN_DOT_HL(16, float) }
        else if (lanes == 32) { GNN_DOT_HL(32, float) }
        else { GNN_DOT_HL(64, float) }
    } else {
        if (lanes == 16) { GNN_DOT_HL(16, bf16_t) }
        else if (lanes == 32) { GNN_DOT_HL(32, bf16_t) }
        else { GNN_DOT_HL(64, bf16_t) }
    }
#undef GNN_DOT_HL
#undef GNN_DOT
    return launch_status("gnn_sddmm(dot)");
}

gnn_status_t launch_edge_softmax(const AggView& v, const float* E, float* alpha, int heads, hipStream_t st) {
    if (v.n == 0) return GNN_OK;
    Sched s = make_sched(v);
    const int64_t light = s.n - s.n_block;
    const int64_t blocks = (light + (256 / G) - 1) / (256 / G);
    ScopedTimer t(st, "softmax_fwd_kernel h=%d", heads);
    GNN_HEADS_SWITCH(heads, {
        hipLaunchKernelGGL((softmax_fwd_kernel<H>), dim3(s.n_block + blocks), dim3(256), 0, st, s, E, alpha);
    });
    return launch_status("gnn_edge_softmax");
}

gnn_status_t launch_edge_softmax_bwd(const AggView& v, const float* alpha, const float* dalpha, const float* pre,
                                     float slope, float* dE, int heads, hipStream_t st) {
    if (v.n == 0) return GNN_OK;
    Sched s = make_sched(v);
    const int64_t light = s.n - s.n_block;
    const int64_t blocks = (light + (256 / G) - 1) / (256 / G);
    ScopedTimer t(st, "softmax_bwd_kernel h=%d", heads);
    GNN_HEADS_SWITCH(heads, {
        hipLaunchKernelGGL((softmax_bwd_kernel<H>), dim3(s.n_block + blocks), dim3(256), 0, st, s, alpha, dalpha,
                           pre, slope, dE);
    });
    return launch_status("gnn_edge_softmax_bwd");
}

gnn_status_t launch_edge_reduce(const AggView& v, const float* vals, int heads, float* out, hipStream_t st) {
    if (v.n == 0) return GNN_OK;
    Sched s = make_sched(v);
    const int64_t light = s.n - s.n_block;
    const int64_t blocks = (light + (256 / G) - 1) / (256 / G);
    GNN_HEADS_SWITCH(heads, {
        hipLaunchKernelGGL((reduce_kernel<H>), dim3(s.n_block + blocks), dim3(256), 0, st, s, vals, out);
    });
    return launch_status("gnn_edge_reduce");
}

gnn_status_t launch_gat_scores(int64_t n, const float* Hp, int heads, int64_t d_head, const float* a_src,
                               const float* a_dst, float* S, float* D, hipStream_t st) {
    if (n == 0) return GNN_OK;
    const int64_t d = heads * d_head;
    const int64_t hl = d_head / 4;
    if (d_head % 4 || (hl & (hl - 1)) || hl > 64 || (d > 256 && 256 % d_head))
        return fail(GNN_ERR_UNSUPPORTED, "GAT scores: d_head must be 4 * a power of two, at most 256");
    const int64_t blocks = (n + 7) / 8;  // four waves of two rows
#define GNN_SC(HLv) \
    hipLaunchKernelGGL((gat_scores_kernel<HLv>), dim3(blocks), dim3(256), 0, st, n, Hp, d, heads, a_src, a_dst, S, D)
    switch (hl) {
        case 1: GNN_SC(1); break;
        case 2: GNN_SC(2); break;
        case 4: GNN_SC(4); break;
        case 8: GNN_SC(8); break;
        case 16: GNN_SC(16); break;
        case 32: GNN_SC(32); break;
        default: GNN_SC(64); break;
    }
#undef GNN_SC
    return launch_status("GAT scores");
}

size_t head_colsum_partial_bytes(int64_t n, int heads, int64_t d_head) {
    const int64_t nblk = (n + kColRows - 1) / kColRows;
    return align_up(static_cast<size_t>(nblk) * 2 * heads * d_head * sizeof(float));
}

gnn_status_t launch_head_colsum(int64_t n, const float* coefA, const float* coefB, const float* Hp, int heads,
                                int64_t d_head, float* outA, float* outB, float* partial, hipStream_t st) {
    const int64_t d = heads * d_head;
    const int64_t nblk = (n + kColRows - 1) / kColRows;
    if (nblk > 0)
        hipLaunchKernelGGL(colsum_stage1, dim3(nblk), dim3(256), 0, st, n, coefA, coefB, Hp, d, heads, d_head,
                           partial);
    hipLaunchKernelGGL(colsum_stage2, dim3((2 * d + 63) / 64), dim3(256), 0, st, nblk, d, partial, outA, outB);
    return launch_status("GAT attention-vector gradient");
}

}  // namespace gnnmp
