// hti_trav_common.h -- pieces shared by the traversal kernels.
#pragma once

#include "hti_device.h"

namespace hti {

// Raw register images of N consecutive elements.
template <typename T, int N> struct Raw;
template <> struct Raw<bf16_t, 1> { using type = uint16_t; };
template <> struct Raw<bf16_t, 2> { using type = uint32_t; };
template <> struct Raw<bf16_t, 4> { using type = uint2; };
template <> struct Raw<float, 1> { using type = float; };
template <> struct Raw<float, 2> { using type = float2; };
template <> struct Raw<float, 4> { using type = float4; };

__device__ __forceinline__ void cvt(uint16_t r, float *o) { o[0] = bf2f(r); }
__device__ __forceinline__ void cvt(uint32_t r, float *o)
{
    o[0] = bf2f(r & 0xffffu);
    o[1] = bf2f(r >> 16);
}
__device__ __forceinline__ void cvt(uint2 r, float *o)
{
    cvt(r.x, o);
    cvt(r.y, o + 2);
}
// E4M3 router keys: raw images of N consecutive codes, decoded by the vector
// unit's packed 8-bit float conversion (OCP E4M3 on this target).
template <int N> struct Raw8;
template <> struct Raw8<2> { using type = uint16_t; };
template <> struct Raw8<4> { using type = uint32_t; };
template <int N> __device__ __forceinline__ void cvt8(uint32_t r, float *o)
{
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)r, false);
    o[0] = lo[0];
    o[1] = lo[1];
    if constexpr (N == 4) {
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)r, true);
        o[2] = hi[0];
        o[3] = hi[1];
    }
}
// E4M3 codes held in the low bytes of a key register image
__device__ __forceinline__ void put8(uint2 &k, uint32_t w) { k = make_uint2(w, 0u); }
__device__ __forceinline__ void put8(uint32_t &k, uint32_t w) { k = w; }
__device__ __forceinline__ uint32_t get8(const uint2 &k) { return k.x; }
__device__ __forceinline__ uint32_t get8(const uint32_t &k) { return k; }
// (fp32 caches: 8-bit router keys are rejected before any launch)
template <typename K> __device__ __forceinline__ void put8(K &, uint32_t) {}
template <typename K> __device__ __forceinline__ uint32_t get8(const K &) { return 0u; }
__device__ __forceinline__ void cvt(float r, float *o) { o[0] = r; }
__device__ __forceinline__ void cvt(float2 r, float *o)
{
    o[0] = r.x;
    o[1] = r.y;
}
__device__ __forceinline__ void cvt(float4 r, float *o)
{
    o[0] = r.x;
    o[1] = r.y;
    o[2] = r.z;
    o[3] = r.w;
}

// Candidate list of one level: children of the kept parents (in parent order)
// followed by the level's orphans; the top level is [0, n_top).
struct Cands {
    const int *selp;
    int nprev;
    int b;
    uint32_t binv;      // ceil(2^32 / b): i / b == umulhi(i, binv) for i < 2^16
    int64_t orph0;
    bool top;
    // Branch-free (selects only), so that gathers addressed by it can be
    // issued back to back: the parent slot is clamped into the kept list and
    // read even for orphans and at the top level, where it is not used.
    __device__ __forceinline__ int64_t id(int i) const
    {
        const int nb = nprev * b;
        const int q = (int)__umulhi((uint32_t)i, binv);
        const int qs = min(q, nprev > 0 ? nprev - 1 : 0);
        const int64_t child = (int64_t)selp[qs] * b + (i - q * b);
        const int64_t orphan = orph0 + (i - nb);
        return top ? (int64_t)i : (i < nb ? child : orphan);
    }
};

constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Pointer into global memory, so that loads through it are global (not flat)
// loads even when the pointer itself came through LDS: a flat load also counts
// against the LDS wait counter, and every later LDS wait would then wait for
// the gather too.
template <typename T> using gptr = const __attribute__((address_space(1))) T *;
template <typename T> __device__ __forceinline__ gptr<T> to_global(const void *p)
{
    return (gptr<T>)(const T *)p;
}
// loads of the HIP vector types go through the matching native vector type
template <typename V> struct NativeOf { using type = V; };
template <> struct NativeOf<uint2> { using type = unsigned __attribute__((ext_vector_type(2))); };
template <> struct NativeOf<uint4> { using type = unsigned __attribute__((ext_vector_type(4))); };
template <> struct NativeOf<float2> { using type = float __attribute__((ext_vector_type(2))); };
template <> struct NativeOf<float4> { using type = float __attribute__((ext_vector_type(4))); };
template <typename V, typename T> __device__ __forceinline__ V gload(gptr<T> p)
{
    using N = typename NativeOf<V>::type;
    const N n = *(gptr<N>)p;
    V v;
    __builtin_memcpy(&v, &n, sizeof(V));
    return v;
}

} // namespace hti
