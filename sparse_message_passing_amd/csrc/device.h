// device.h -- small device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gnnmp {

typedef uint16_t bf16_t;  // bfloat16 storage

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// round-to-nearest-even; infinities stay infinite, and a NaN stays a NaN of
// the same sign (quiet bit set: a payload only in the low 16 bits would
// otherwise round into the exponent and read as an infinity)
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
    __device__ __forceinline__ static float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ static void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};
template <> struct Elem<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p) { return bf2f(*p); }
    __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f2bf(v); }
    __device__ __forceinline__ static float4 load4(const bf16_t* p) {
        uint2 r = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
    }
    __device__ __forceinline__ static void store4(bf16_t* p, float4 v) {
        uint2 r;
        r.x = static_cast<uint32_t>(f2bf(v.x)) | (static_cast<uint32_t>(f2bf(v.y)) << 16);
        r.y = static_cast<uint32_t>(f2bf(v.z)) | (static_cast<uint32_t>(f2bf(v.w)) << 16);
        *reinterpret_cast<uint2*>(p) = r;
    }
};

// value of `v` held by lane `src` of the aligned group of `width` lanes
template <int WIDTH>
__device__ __forceinline__ int group_bcast(int v, int src_in_group) {
    if constexpr (WIDTH == 64) {
        return __builtin_amdgcn_readlane(v, src_in_group);
    } else {
        return __shfl(v, src_in_group, WIDTH);
    }
}
template <int WIDTH>
__device__ __forceinline__ float group_bcast(float v, int src_in_group) {
    return __int_as_float(group_bcast<WIDTH>(__float_as_int(v), src_in_group));
}

// butterfly sum / max within aligned groups of WIDTH lanes (all lanes get the result)
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
    return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WIDTH));
    return v;
}

__device__ __forceinline__ float4 f4_fma(float w, float4 x, float4 a) {
    a.x = fmaf(w, x.x, a.x);
    a.y = fmaf(w, x.y, a.y);
    a.z = fmaf(w, x.z, a.z);
    a.w = fmaf(w, x.w, a.w);
    return a;
}

}  // namespace gnnmp
