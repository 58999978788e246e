// calib.hip -- reference kernels of known traffic and known flops on one
// MI355X (gfx950): they measure the achievable peaks the roofline fractions
// are read against, and calibrate the HBM byte counters (a kernel whose
// bytes are known shows what a counter reads per byte moved).
//
//   gnn_calib_read    streams a buffer once (16-byte loads), one float per
//                     workgroup written
//   gnn_calib_copy    dst = src (16-byte loads and stores)
//   gnn_calib_gather  gathers rows of `row_bytes` from a table by an index
//                     list (the access pattern of an aggregation), summing
//                     them per lane group; one float per thread written
//   gnn_calib_mfma    back-to-back independent matrix-core products from
//                     registers: f32 16x16x4, bf16 16x16x32, i8 16x16x64
//
// All pointers are device memory; every call is asynchronous on `stream`.
// Sizes are checked on the host before a launch; an index must lie in
// [0, rows) (the caller's list; the kernels do not check it).

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void read_kernel(const float4* __restrict__ src, int64_t n, float* out) {
    float s = 0.0f;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const float4 v = src[i];
        s += (v.x + v.y) + (v.z + v.w);
    }
    __shared__ float red[kThreads];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                        int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
        dst[i] = src[i];
}

// L lanes per row (16 bytes each); each group walks its share of the index
// list, four rows in flight.
template <int L>
__global__ __launch_bounds__(kThreads) void gather_kernel(const float4* __restrict__ table, int64_t row_vec,
                                                          const int32_t* __restrict__ idx, int64_t n_idx,
                                                          float* out) {
    const int lane = threadIdx.x % L;
    const int64_t groups = static_cast<int64_t>(gridDim.x) * (kThreads / L);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * (kThreads / L) + threadIdx.x / L;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int64_t i = g * 4; i < n_idx; i += groups * 4) {
        float4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t j = i + q;
            v[q] = j < n_idx && lane < row_vec ? table[static_cast<int64_t>(idx[j]) * row_vec + lane]
                                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc.x += v[q].x;
            acc.y += v[q].y;
            acc.z += v[q].z;
            acc.w += v[q].w;
        }
    }
    out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = (acc.x + acc.y) + (acc.z + acc.w);
}

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Eight independent accumulators per wave keep the matrix pipe busy; the
// operands are formed in registers once.
constexpr int kChains = 8;

__global__ __launch_bounds__(kThreads) void mfma_f32_kernel(int iters, float* out) {
    const float a = 1.0f + threadIdx.x * 1e-3f, b = 0.5f - threadIdx.x * 1e-4f;
    v4f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
    out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(int iters, float* out) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(1.0f + (threadIdx.x + i) * 1e-3f);
        b[i] = static_cast<__bf16>(0.5f - i * 1e-2f);
    }
    v4f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
    out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void mfma_i8_kernel(int iters, float* out) {
    const int base = static_cast<int>(threadIdx.x) * 0x01010101;
    const v4i a = v4i{base, base ^ 0x02020202, base ^ 0x04040404, base ^ 0x08080808};
    const v4i b = v4i{0x01020304, 0x05060708, 0x090A0B0C, 0x0D0E0F10};
    v4i acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = v4i{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
    out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = static_cast<float>(s);
}

}  // namespace

extern "C" {

// 0 on success, -1 on a bad argument, else the HIP error code of the launch.
int gnn_calib_read(const void* src, int64_t bytes, float* out, int64_t out_floats, void* stream) {
    if (!src || !out || bytes <= 0 || bytes % 16 || out_floats < 1) return -1;
    const int64_t blocks = out_floats < 4096 ? out_floats : 4096;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const float4*>(src), bytes / 16, out);
    return static_cast<int>(hipGetLastError());
}

int gnn_calib_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16) return -1;
    hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const float4*>(src), static_cast<float4*>(dst), bytes / 16);
    return static_cast<int>(hipGetLastError());
}

// table: [rows, row_bytes]; idx: int32[n_idx] in [0, rows); out: float[blocks * 256]
int gnn_calib_gather(const void* table, int64_t row_bytes, const int32_t* idx, int64_t n_idx, float* out,
                     int64_t blocks, void* stream) {
    if (!table || !idx || !out || n_idx <= 0 || blocks < 1) return -1;
    if (row_bytes != 64 && row_bytes != 128 && row_bytes != 256 && row_bytes != 512 && row_bytes != 1024) return -1;
    const int64_t rv = row_bytes / 16;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const float4* t = static_cast<const float4*>(table);
    switch (rv) {
        case 4: hipLaunchKernelGGL((gather_kernel<4>), dim3(blocks), dim3(kThreads), 0, st, t, rv, idx, n_idx, out); break;
        case 8: hipLaunchKernelGGL((gather_kernel<8>), dim3(blocks), dim3(kThreads), 0, st, t, rv, idx, n_idx, out); break;
        case 16: hipLaunchKernelGGL((gather_kernel<16>), dim3(blocks), dim3(kThreads), 0, st, t, rv, idx, n_idx, out); break;
        case 32: hipLaunchKernelGGL((gather_kernel<32>), dim3(blocks), dim3(kThreads), 0, st, t, rv, idx, n_idx, out); break;
        default: hipLaunchKernelGGL((gather_kernel<64>), dim3(blocks), dim3(kThreads), 0, st, t, rv, idx, n_idx, out); break;
    }
    return static_cast<int>(hipGetLastError());
}

// kind 0: f32 16x16x4 (2048 flops per wave instruction), 1: bf16 16x16x32
// (16384), 2: i8 16x16x64 (32768 integer ops); out: float[blocks * 256].
// Returns the flops (or integer ops) of the launch in *work.
int gnn_calib_mfma(int kind, int64_t blocks, int iters, float* out, double* work, void* stream) {
    if (!out || !work || blocks < 1 || iters < 1 || kind < 0 || kind > 2) return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const double per = kind == 0 ? 2.0 * 16 * 16 * 4 : kind == 1 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 64;
    *work = per * kChains * static_cast<double>(iters) * (kThreads / 64) * static_cast<double>(blocks);
    if (kind == 0) hipLaunchKernelGGL(mfma_f32_kernel, dim3(blocks), dim3(kThreads), 0, st, iters, out);
    else if (kind == 1) hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(kThreads), 0, st, iters, out);
    else hipLaunchKernelGGL(mfma_i8_kernel, dim3(blocks), dim3(kThreads), 0, st, iters, out);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
