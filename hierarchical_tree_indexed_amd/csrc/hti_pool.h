// hti_pool.h -- pooling of one tree node by one wavefront, shared by the tree
// build, the per-token append and the decode step that appends.
//
// "Recursive Sparse Attention" (abstract: one key and one mean-pooled value
// per node, one pooler shared by every level) and "Subquadratic Attention
// with a Hierarchical Tree-Structured Indexer" (Figure 3 caption: a chunk of
// contiguous key nodes is summarised by an attention-weighted sum of its
// keys, the attention taken w.r.t. reference queries, one key per reference
// stored in parallel; Table VIII: only full nodes).
//
// Layout of the work: the node's b children are contiguous rows (b * d
// elements), so a wave streams them with 16-byte loads: lane = (row group
// rg = lane / 16) x (slice sub = lane % 16); row group rg holds children rg,
// rg + 4, ..., slice sub holds d/16 contiguous elements of each.  Dot
// products reduce over the 16 lanes of a row group, the softmax and the
// weighted sums over the 4 row groups (DPP within a row, lane-swap
// instructions across rows: no LDS round trips).
#pragma once

#include "hti_device.h"
#include "hti_internal.h"

namespace hti {

// ----------------------------------------------------------------------------
// One wave pools node `node` of level `lvl` (children at level lvl-1) for
// (sequence, KV head) slot bh, head index h.  CPL = children per lane-row
// (ceil(b / 4)).
// ----------------------------------------------------------------------------
template <typename T, int D>
__device__ __forceinline__ void store_slice(T *p, const float *v);

template <>
__device__ __forceinline__ void store_slice<bf16_t, 128>(bf16_t *p, const float *v)
{
    uint4 o;
    o.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    o.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    o.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
    o.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
    *reinterpret_cast<uint4 *>(p) = o;
}
template <>
__device__ __forceinline__ void store_slice<bf16_t, 64>(bf16_t *p, const float *v)
{
    uint2 o;
    o.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    o.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *reinterpret_cast<uint2 *>(p) = o;
}
template <>
__device__ __forceinline__ void store_slice<float, 128>(float *p, const float *v)
{
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ __forceinline__ void store_slice<float, 64>(float *p, const float *v)
{
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T, int D, int CPL>
__device__ void pool_node(const TreeArgs &t, int lvl, int64_t bh, int h, int64_t node, int lane)
{
    constexpr int EPL = D / 16;                  // elements per lane of a child row
    const int sub = lane & 15, rg = lane >> 4;
    const int b = t.b, R = t.R;
    const int64_t c0 = node * b;                 // first child (level lvl-1 index)
    const int64_t nchild_cap = t.ncap[lvl - 1];

    // Children rg, rg + 4, ...: a slot past the last child reads child b-1
    // and carries no weight, so that every load is unconditional and all of
    // them (values included) are in flight together.
    bool valid[CPL];
    int64_t crow[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int child = rg + 4 * c;
        valid[c] = child < b;
        crow[c] = bh * nchild_cap + c0 + min(child, b - 1);
    }
    const T *vbase = (lvl == 1) ? (const T *)t.vc : (const T *)t.lv[lvl - 2];
    float vx[CPL][EPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) load_vec<T, EPL>(vbase + crow[c] * D + sub * EPL, vx[c]);

    float kx[CPL][EPL];
    for (int j = 0; j < R; ++j) {
        if (lvl >= 2 || j == 0) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const T *kp = (lvl == 1) ? (const T *)t.kc + crow[c] * D
                                         : (const T *)t.lk[lvl - 2] + (crow[c] * R + j) * D;
                load_vec<T, EPL>(kp + sub * EPL, kx[c]);
            }
        }
        float r[EPL];
        load_vec<float, EPL>(t.refs + ((int64_t)h * R + j) * D + sub * EPL, r);

        // logits of the children against reference j
        float a[CPL];
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dot += r[e] * kx[c][e];
            dot = sum16(dot) * t.scale;
            a[c] = valid[c] ? dot : -INFINITY;
            mx = fmaxf(mx, a[c]);
        }
        mx = xmax32(xmax16(mx));
        float den = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            a[c] = valid[c] ? expf(a[c] - mx) : 0.f;
            den += a[c];
        }
        den = xsum32(xsum16(den));

        // pooled key = sum_c softmax_c * k_c
        float acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float w = a[c] / den;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] += w * kx[c][e];
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = xsum32(xsum16(acc[e]));
        if (rg == 0) {
            T *out = (T *)t.lk[lvl - 1] + (((bh * t.ncap[lvl] + node) * R + j) * D) + sub * EPL;
            store_slice<T, D>(out, acc);
        }
    }

    // mean-pooled value
    float vs[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) vs[e] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        if (valid[c]) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) vs[e] += vx[c][e];
        }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        vs[e] = xsum32(xsum16(vs[e])) / (float)b;
    }
    if (rg == 0) {
        T *out = (T *)t.lv[lvl - 1] + (bh * t.ncap[lvl] + node) * D + sub * EPL;
        store_slice<T, D>(out, vs);
    }
}

} // namespace hti
