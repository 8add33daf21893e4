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
// instructions across rows: no LDS round trips).  With 8-bit router keys
// every pooled key row is also written as E4M3 codes with a power-of-two row
// scale, taken from its stored (cache-dtype) value.
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

// E4M3 code (OCP 8-bit float: 4 exponent bits, bias 7, 3 mantissa bits) of
// x, |x| < 256, rounded to the nearest value, ties to even.  With e the
// binade of |x| (floor(log2 |x|), at least -6, the subnormal binade's) the
// value is q * 2^(e-3), q = rint(|x| * 2^(3-e)) in [0, 16], and the code is
// 8 (e + 7) + q - 8: a q of 16 carries into the next binade's exponent field,
// and the subnormals (e = -6, q < 8) land on codes 0..7.
__device__ __forceinline__ uint32_t e4m3_code(float x)
{
    const float a = fabsf(x);
    int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    e = e < -6 ? -6 : e;
    const int q = (int)rintf(ldexpf(a, 3 - e));
    return (uint32_t)(8 * e + 48 + q) | ((__float_as_uint(x) >> 24) & 0x80u);
}

// Router copy of one pooled key row, held as EPL elements by each of the 16
// lanes of a row group (the values as stored: rounded to the cache dtype):
// the row scale 2^(e-8) for amax = f * 2^e, f in [0.5, 1) (1 when the row is
// zero), and the codes of the scaled elements.  Lanes of row group 0 store.
template <int D, int EPL>
__device__ __forceinline__ void store_router_row(const TreeArgs &t, int lvl, int64_t row, const float *k, int sub,
                                                 bool store)
{
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(k[e]));
    amax = max16(amax);
    const int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 8;
    uint32_t w[EPL / 4];
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
        w[i] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[i] |= e4m3_code(ldexpf(k[4 * i + e], 8 - ex)) << (8 * e);
    }
    if (store) {
        uint8_t *q = t.lkq[lvl - 1] + row * D + sub * EPL;
        if constexpr (EPL == 8)
            *reinterpret_cast<uint2 *>(q) = make_uint2(w[0], w[1]);
        else
            *reinterpret_cast<uint32_t *>(q) = w[0];
        if (sub == 0) t.lks[lvl - 1][row] = ldexpf(1.f, ex - 8);
    }
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
        if (t.rfp8) {
            float kr[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) kr[e] = round_to<T>(acc[e]);
            store_router_row<D, EPL>(t, lvl, (bh * t.ncap[lvl] + node) * R + j, kr, sub, rg == 0);
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
