// hti_device.h -- device helpers shared by the library's HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// DPP-based reductions (no LDS round trip).  16-lane all-reduce: quad
// permutations [1,0,3,2] and [2,3,0,1], then row half-mirror and row mirror;
// the four 16-lane rows are combined through readlane.
template <int CTRL>
__device__ __forceinline__ float dppf(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float rlane(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float sum16(float v)
{
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    v += dppf<0x141>(v);
    v += dppf<0x140>(v);
    return v;
}
__device__ __forceinline__ float max16(float v)
{
    v = fmaxf(v, dppf<0xB1>(v));
    v = fmaxf(v, dppf<0x4E>(v));
    v = fmaxf(v, dppf<0x141>(v));
    v = fmaxf(v, dppf<0x140>(v));
    return v;
}
__device__ __forceinline__ int min16i(int v)
{
    v = min(v, dppi<0xB1>(v));
    v = min(v, dppi<0x4E>(v));
    v = min(v, dppi<0x141>(v));
    v = min(v, dppi<0x140>(v));
    return v;
}
__device__ __forceinline__ int sum16i(int v)
{
    v += dppi<0xB1>(v);
    v += dppi<0x4E>(v);
    v += dppi<0x141>(v);
    v += dppi<0x140>(v);
    return v;
}
// Value of lane n of this lane's 16-lane row (DPP row_newbcast); n must fold
// to a constant after unrolling.
__device__ __forceinline__ int row_bcast(int v, int n)
{
    switch (n) {
    case 0: return dppi<0x150>(v);
    case 1: return dppi<0x151>(v);
    case 2: return dppi<0x152>(v);
    case 3: return dppi<0x153>(v);
    case 4: return dppi<0x154>(v);
    case 5: return dppi<0x155>(v);
    case 6: return dppi<0x156>(v);
    case 7: return dppi<0x157>(v);
    case 8: return dppi<0x158>(v);
    case 9: return dppi<0x159>(v);
    case 10: return dppi<0x15A>(v);
    case 11: return dppi<0x15B>(v);
    case 12: return dppi<0x15C>(v);
    case 13: return dppi<0x15D>(v);
    case 14: return dppi<0x15E>(v);
    default: return dppi<0x15F>(v);
    }
}
// Sums over the 16 lanes of a row of the G values z[0..G) at once, as a
// transposed butterfly: at each lane bit from 3 down, the lanes with the bit
// set keep the upper half of the values still open and swap the other half
// with their partner.  Lane `sub` ends with the sum of value sub / (16 / G).
template <int G>
__device__ __forceinline__ float row_sums(const float (&z)[G], int sub)
{
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "G in {1, 2, 4, 8}");
    float a[G];
#pragma unroll
    for (int h = 0; h < G; ++h) a[h] = z[h];
    auto half = [&](auto ctrl, int n, bool hi) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < n; ++h) {
            const float keep = hi ? a[h + n] : a[h];
            const float send = hi ? a[h] : a[h + n];
            a[h] = keep + dppf<decltype(ctrl)::value>(send);
        }
    };
    using Mirror = std::integral_constant<int, 0x140>;      // lane i <-> 15 - i
    using HalfMirror = std::integral_constant<int, 0x141>;  // i <-> 7 - i within each half
    using Swap2 = std::integral_constant<int, 0x4E>;        // i <-> i ^ 2
    if constexpr (G >= 2) half(Mirror{}, G / 2, (sub & 8) != 0);
    else a[0] += dppf<0x140>(a[0]);
    if constexpr (G >= 4) half(HalfMirror{}, G / 4, (sub & 4) != 0);
    else a[0] += dppf<0x141>(a[0]);
    if constexpr (G >= 8) half(Swap2{}, 1, (sub & 2) != 0);
    else a[0] += dppf<0x4E>(a[0]);
    a[0] += dppf<0xB1>(a[0]);
    return a[0];
}

// Sum over the G values a lane group holds after row_sums (the values differ
// across lane bits 3, 2, 1 for G = 2, 4, 8 and are equal within a group).
template <int G>
__device__ __forceinline__ float head_total(float v)
{
    if constexpr (G >= 8) v += dppf<0x4E>(v);
    if constexpr (G >= 4) v += dppf<0x141>(v);
    if constexpr (G >= 2) v += dppf<0x140>(v);
    return v;
}

// Sum of v over lanes l and l ^ 16 (rows 2r and 2r+1 exchanged by one
// v_permlane16_swap) and over lanes l and l ^ 32 (halves exchanged by one
// v_permlane32_swap), in every lane.
__device__ __forceinline__ float xsum16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xmax16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// wave-wide results, uniform across the wave
__device__ __forceinline__ float wave_sum(float v)
{
    v = sum16(v);
    return (rlane(v, 0) + rlane(v, 16)) + (rlane(v, 32) + rlane(v, 48));
}
__device__ __forceinline__ float wave_max(float v)
{
    v = max16(v);
    return fmaxf(fmaxf(rlane(v, 0), rlane(v, 16)), fmaxf(rlane(v, 32), rlane(v, 48)));
}
__device__ __forceinline__ int wave_min_i(int v)
{
    v = min16i(v);
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// One 16-byte-per-lane gather straight into LDS (gfx950 global_load_lds_dwordx4):
// lane l's 16 bytes land at lds + 16 * l; `lds` must be wave-uniform.
__device__ __forceinline__ void gather16_to_lds(const void *g, void *lds)
{
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

} // namespace hti
