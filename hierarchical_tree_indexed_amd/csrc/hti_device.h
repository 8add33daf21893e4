// hti_device.h -- device helpers shared by the library's HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hti {

constexpr int kWave = 64;

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf2f(uint32_t u16) { return __uint_as_float(u16 << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite values).
__device__ __forceinline__ uint16_t f2bf(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Round an fp32 value to the storage precision of T and back.
template <typename T> __device__ __forceinline__ float round_to(float x);
template <> __device__ __forceinline__ float round_to<float>(float x) { return x; }
template <> __device__ __forceinline__ float round_to<bf16_t>(float x)
{
    return bf2f(f2bf(x));
}

template <typename T> __device__ __forceinline__ void store_elem(T *p, float x);
template <> __device__ __forceinline__ void store_elem<float>(float *p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_elem<bf16_t>(bf16_t *p, float x) { *p = f2bf(x); }

// Load N consecutive elements (N * sizeof(T) bytes, naturally aligned) as fp32.
template <typename T, int N> struct VecLoad;

template <> struct VecLoad<float, 2> {
    __device__ __forceinline__ static void run(const float *p, float *o)
    {
        float2 v = *reinterpret_cast<const float2 *>(p);
        o[0] = v.x; o[1] = v.y;
    }
};
template <> struct VecLoad<float, 4> {
    __device__ __forceinline__ static void run(const float *p, float *o)
    {
        float4 v = *reinterpret_cast<const float4 *>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
};
template <> struct VecLoad<float, 8> {
    __device__ __forceinline__ static void run(const float *p, float *o)
    {
        VecLoad<float, 4>::run(p, o);
        VecLoad<float, 4>::run(p + 4, o + 4);
    }
};
template <> struct VecLoad<float, 1> {
    __device__ __forceinline__ static void run(const float *p, float *o) { o[0] = *p; }
};
template <> struct VecLoad<bf16_t, 1> {
    __device__ __forceinline__ static void run(const bf16_t *p, float *o) { o[0] = bf2f(*p); }
};
template <> struct VecLoad<bf16_t, 2> {
    __device__ __forceinline__ static void run(const bf16_t *p, float *o)
    {
        uint32_t v = *reinterpret_cast<const uint32_t *>(p);
        o[0] = bf2f(v & 0xffffu); o[1] = bf2f(v >> 16);
    }
};
template <> struct VecLoad<bf16_t, 4> {
    __device__ __forceinline__ static void run(const bf16_t *p, float *o)
    {
        uint2 v = *reinterpret_cast<const uint2 *>(p);
        o[0] = bf2f(v.x & 0xffffu); o[1] = bf2f(v.x >> 16);
        o[2] = bf2f(v.y & 0xffffu); o[3] = bf2f(v.y >> 16);
    }
};
template <> struct VecLoad<bf16_t, 8> {
    __device__ __forceinline__ static void run(const bf16_t *p, float *o)
    {
        uint4 v = *reinterpret_cast<const uint4 *>(p);
        o[0] = bf2f(v.x & 0xffffu); o[1] = bf2f(v.x >> 16);
        o[2] = bf2f(v.y & 0xffffu); o[3] = bf2f(v.y >> 16);
        o[4] = bf2f(v.z & 0xffffu); o[5] = bf2f(v.z >> 16);
        o[6] = bf2f(v.w & 0xffffu); o[7] = bf2f(v.w >> 16);
    }
};

template <typename T, int N>
__device__ __forceinline__ void load_vec(const T *p, float *o) { VecLoad<T, N>::run(p, o); }

// Butterfly reductions over groups of `W` lanes (W a power of two <= 64);
// every lane of the group ends with the result.
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int off = W / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int off = W / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

} // namespace hti
