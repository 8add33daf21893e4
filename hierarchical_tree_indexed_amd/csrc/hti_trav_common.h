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

} // namespace hti
