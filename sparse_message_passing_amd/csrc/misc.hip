// misc.hip -- the loss and the ReLU gradient mask.
//
// Mean softmax cross-entropy over all rows (the loss of a node-classification
// GCN; the pages train with full-graph gradient descent, AdaQP Eqn. 8):
//   loss = (1/n) sum_v [logsumexp(z_v) - z_v[y_v]],  dz = (softmax(z_v) - onehot(y_v)) / n.
// Tango keeps the layer that feeds the softmax in full precision, so the
// logits, their gradient and the loss are binary32.  The per-row losses are
// added in a fixed order (per group, per block, then over blocks).

#include "device.h"
#include "internal.h"

namespace gnnmp {

namespace {

constexpr int kRowsPerBlock = 64;
constexpr int kRowCache = 4;  // row entries a lane keeps in registers (rows of up to 4 LG classes)

// A group of LG lanes per row (LG = 16 when the row has at most 64 classes,
// else a whole wave), 256/LG groups per workgroup, each taking the block's
// rows g, g + 256/LG, ...; the block's loss is the sum over its groups in
// group order, each group's rows added in row order.
template <int LG>
__global__ __launch_bounds__(256) void xent_rows(const float* z, int64_t n, int64_t c, int64_t ld,
                                                 const int32_t* labels, float* dz, int64_t ldd, float inv_n,
                                                 float* block_loss) {
    constexpr int NG = 256 / LG;
    __shared__ float sh[NG];
    const int lane = threadIdx.x % LG, grp = threadIdx.x / LG;
    float grp_loss = 0.0f;
    for (int k = grp; k < kRowsPerBlock; k += NG) {
        const int64_t v = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + k;
        if (v >= n) break;
        const float* zr = z + v * ld;
        const int32_t y = labels[v];
        if (c <= LG * kRowCache) {
            // the row read once into registers (lane holds j = lane + LG i);
            // the same operations in the same order as the general path
            float zv[kRowCache];
#pragma unroll
            for (int i = 0; i < kRowCache; ++i) {
                const int64_t j = lane + LG * i;
                zv[i] = j < c ? zr[j] : -INFINITY;
            }
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < kRowCache; ++i)
                if (lane + LG * i < c) m = fmaxf(m, zv[i]);
            m = group_max<LG>(m);
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < kRowCache; ++i)
                if (lane + LG * i < c) s += __expf(zv[i] - m);
            s = group_sum<LG>(s);
            const float lse = m + __logf(s);
            grp_loss += lse - zr[y];
            if (dz) {
                const float is = 1.0f / s;
#pragma unroll
                for (int i = 0; i < kRowCache; ++i) {
                    const int64_t j = lane + LG * i;
                    if (j < c) {
                        float p = __expf(zv[i] - m) * is;
                        if (j == y) p -= 1.0f;
                        dz[v * ldd + j] = p * inv_n;
                    }
                }
            }
            continue;
        }
        float m = -INFINITY;
        for (int64_t j = lane; j < c; j += LG) m = fmaxf(m, zr[j]);
        m = group_max<LG>(m);
        float s = 0.0f;
        for (int64_t j = lane; j < c; j += LG) s += __expf(zr[j] - m);
        s = group_sum<LG>(s);
        const float lse = m + __logf(s);
        grp_loss += lse - zr[y];
        if (dz) {
            const float is = 1.0f / s;
            for (int64_t j = lane; j < c; j += LG) {
                float p = __expf(zr[j] - m) * is;
                if (j == y) p -= 1.0f;
                dz[v * ldd + j] = p * inv_n;
            }
        }
    }
    if (lane == 0) sh[grp] = grp_loss;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = sh[0];
        for (int g = 1; g < NG; ++g) t += sh[g];
        block_loss[blockIdx.x] = t;
    }
}

__global__ __launch_bounds__(256) void xent_total(const float* block_loss, int64_t nb, float inv_n, float* loss) {
    __shared__ float sh[256];
    // entry i goes to accumulator (i / 256) mod 4: a fixed order with four
    // loads in flight per thread
    float p4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t i = threadIdx.x;
    for (; i + 768 < nb; i += 1024) {
#pragma unroll
        for (int q = 0; q < 4; ++q) p4[q] += block_loss[i + 256 * q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (i + 256 * q < nb) p4[q] += block_loss[i + 256 * q];
    sh[threadIdx.x] = (p4[0] + p4[1]) + (p4[2] + p4[3]);
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) *loss = sh[0] * inv_n;
}

// G[r, f] = dY[r, f] * [Y[r, f] > 0] over an n x d block with leading dims;
// V = 4: four consecutive features per thread (16-byte f32 / 8-byte bf16
// accesses) where d, the leading dims and the pointers allow it
template <typename TY, typename TG, int V>
__global__ __launch_bounds__(256) void relu_mask_kernel(int64_t n, int64_t d, const TY* dY, int64_t ldd, const TY* Y,
                                                        int64_t ldy, TG* G, int64_t ldg) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t dv = d / V;
    if (i >= n * dv) return;
    const int64_t r = i / dv, f = (i - r * dv) * V;
    if constexpr (V == 4) {
        const float4 y = Elem<TY>::load4(Y + r * ldy + f);
        const float4 g = Elem<TY>::load4(dY + r * ldd + f);
        Elem<TG>::store4(G + r * ldg + f, make_float4(y.x > 0.0f ? g.x : 0.0f, y.y > 0.0f ? g.y : 0.0f,
                                                      y.z > 0.0f ? g.z : 0.0f, y.w > 0.0f ? g.w : 0.0f));
    } else {
        Elem<TG>::store(G + r * ldg + f,
                        Elem<TY>::load(Y + r * ldy + f) > 0.0f ? Elem<TY>::load(dY + r * ldd + f) : 0.0f);
    }
}

}  // namespace

size_t xent_ws_bytes(int64_t n) {
    return align_up(static_cast<size_t>((n + kRowsPerBlock - 1) / kRowsPerBlock) * sizeof(float));
}

gnn_status_t launch_softmax_xent(const float* logits, int64_t n, int64_t c, int64_t ld, const int32_t* labels,
                                 float* loss, float* dlogits, int64_t ld_d, float* ws, hipStream_t st) {
    const int64_t nb = (n + kRowsPerBlock - 1) / kRowsPerBlock;
    const float inv_n = n > 0 ? 1.0f / static_cast<float>(n) : 0.0f;
    if (nb > 0 && c <= 64)
        hipLaunchKernelGGL((xent_rows<16>), dim3(nb), dim3(256), 0, st, logits, n, c, ld, labels, dlogits, ld_d,
                           inv_n, ws);
    else if (nb > 0)
        hipLaunchKernelGGL((xent_rows<64>), dim3(nb), dim3(256), 0, st, logits, n, c, ld, labels, dlogits, ld_d,
                           inv_n, ws);
    hipLaunchKernelGGL(xent_total, dim3(1), dim3(256), 0, st, ws, nb, inv_n, loss);
    return launch_status("gnn_softmax_xent");
}

gnn_status_t launch_relu_mask(int64_t n, int64_t d, const void* dY, int64_t ldd, const void* Y, int64_t ldy,
                              gnn_dtype_t y_dt, void* G, int64_t ldg, gnn_dtype_t g_dt, hipStream_t st) {
    if (n == 0 || d == 0) return GNN_OK;
    const size_t ys = y_dt == GNN_BF16 ? 2 : 4, gs = g_dt == GNN_BF16 ? 2 : 4;
    const bool v4 = d % 4 == 0 && ldd % 4 == 0 && ldy % 4 == 0 && ldg % 4 == 0 &&
                    reinterpret_cast<uintptr_t>(dY) % (4 * ys) == 0 && reinterpret_cast<uintptr_t>(Y) % (4 * ys) == 0 &&
                    reinterpret_cast<uintptr_t>(G) % (4 * gs) == 0;
    const int64_t blocks = (n * (v4 ? d / 4 : d) + 255) / 256;
#define GNN_RM(TY, TG)                                                                                       \
    do {                                                                                                     \
        if (v4)                                                                                              \
            hipLaunchKernelGGL((relu_mask_kernel<TY, TG, 4>), dim3(blocks), dim3(256), 0, st, n, d,          \
                               static_cast<const TY*>(dY), ldd, static_cast<const TY*>(Y), ldy,              \
                               static_cast<TG*>(G), ldg);                                                    \
        else                                                                                                 \
            hipLaunchKernelGGL((relu_mask_kernel<TY, TG, 1>), dim3(blocks), dim3(256), 0, st, n, d,          \
                               static_cast<const TY*>(dY), ldd, static_cast<const TY*>(Y), ldy,              \
                               static_cast<TG*>(G), ldg);                                                    \
    } while (0)
    if (y_dt == GNN_F32 && g_dt == GNN_F32) GNN_RM(float, float);
    else if (y_dt == GNN_F32) GNN_RM(float, bf16_t);
    else if (g_dt == GNN_F32) GNN_RM(bf16_t, float);
    else GNN_RM(bf16_t, bf16_t);
#undef GNN_RM
    return launch_status("ReLU gradient mask");
}

}  // namespace gnnmp
