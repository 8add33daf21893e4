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
    __device__ __forceinline__ int64_t id(int i) const
    {
        if (top) return i;
        if (i < nprev * b) {
            const int q = (int)__umulhi((uint32_t)i, binv);
            return (int64_t)selp[q] * b + (i - q * b);
        }
        return orph0 + (i - nprev * b);
    }
};

constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

} // namespace hti
