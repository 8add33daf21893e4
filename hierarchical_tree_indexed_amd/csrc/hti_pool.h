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
// products reduce over the 16 lanes of a row group (DPP), the softmax over
// the 4 row groups (lane swaps), and each weighted sum with a reduce-scatter
// over the row groups that leaves every lane of the wave a quarter of its
// slice (EPL/2 + EPL/4 lane swaps instead of 2 EPL), so that all 64 lanes
// store a quarter of the row: no LDS round trips.  With 8-bit router keys
// every pooled key row is also written as E4M3 codes with a power-of-two row
// scale, taken from its stored (cache-dtype) value.
#pragma once

#include "hti_device.h"
#include "hti_internal.h"

namespace hti {

// Sums over the four row groups of this lane's EPL partial values, scattered:
// the lanes of row group rg end with the totals of slice elements
// rg * EPL/4 + i, i < EPL/4.  A swap of the upper 32 lanes of x with the
// lower 32 of y, then a sum, leaves rows 0-1 with x summed over rows (0, 2)
// and (1, 3) and rows 2-3 with y summed likewise; a swap of the odd rows of x
// with the even rows of y, then a sum, finishes each row's pair.
template <int EPL>
__device__ __forceinline__ void rg_reduce_scatter(const float (&x)[EPL], float (&out)[EPL / 4])
{
    float h[EPL / 2];
#pragma unroll
    for (int e = 0; e < EPL / 2; ++e) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[e]), __float_as_uint(x[e + EPL / 2]),
                                                        false, false);
        h[e] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int e = 0; e < EPL / 4; ++e) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(h[e]), __float_as_uint(h[e + EPL / 4]),
                                                        false, false);
        out[e] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

// N contiguous elements of a row (N = 1 or 2), rounded to T.
template <typename T, int N>
__device__ __forceinline__ void store_part(T *p, const float (&v)[N])
{
    if constexpr (sizeof(T) == 2) {
        if constexpr (N == 2)
            *reinterpret_cast<uint32_t *>(p) = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        else
            *reinterpret_cast<uint16_t *>(p) = f2bf(v[0]);
    } else {
        if constexpr (N == 2)
            *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
        else
            *reinterpret_cast<float *>(p) = v[0];
    }
}

// EPL elements of a child row read once (the tree build): a non-temporal
// load, so that the streamed rows do not push other lines out of the caches.
template <typename T, int EPL, bool NT>
__device__ __forceinline__ void load_child(const T *p, float *o)
{
    if constexpr (NT && sizeof(T) * EPL == 16) {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[2 * i] = __uint_as_float(v[i] << 16);
                o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
        }
    } else {
        load_vec<T, EPL>(p, o);
    }
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

// Router copy of one pooled key row, spread over the wave as N elements per
// lane at column col (the values as stored: rounded to the cache dtype): the
// row scale 2^(e-8) for amax = f * 2^e, f in [0.5, 1) (1 when the row is
// zero), and the codes of the scaled elements.
template <int D, int N>
__device__ __forceinline__ void store_router_part(const TreeArgs &t, int lvl, int64_t row, const float (&k)[N],
                                                  int col, int lane)
{
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) amax = fmaxf(amax, fabsf(k[e]));
    amax = xmax32(xmax16(max16(amax)));
    const int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 8;
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) w |= e4m3_code(ldexpf(k[e], 8 - ex)) << (8 * e);
    uint8_t *q = t.lkq[lvl - 1] + row * D + col;
    if constexpr (N == 2)
        *reinterpret_cast<uint16_t *>(q) = (uint16_t)w;
    else
        *q = (uint8_t)w;
    if (lane == 0) t.lks[lvl - 1][row] = ldexpf(1.f, ex - 8);
}

// This lane's part (NP = EPL/4 elements, see rg_reduce_scatter) of the pooled
// key sum_c softmax_c(r . k_c * scale) k_c over the node's children c (kx:
// this lane's slices of the children's keys; a padded slot is invalid and
// carries no weight).
template <int D, int CPL>
__device__ __forceinline__ void pool_key(float scale, const float *r_j, const float (&kx)[CPL][D / 16],
                                         const bool (&valid)[CPL], int sub, float (&part)[D / 64])
{
    constexpr int EPL = D / 16;
    float r[EPL];
    load_vec<float, EPL>(r_j + sub * EPL, r);
    // logits in base 2 (scale * log2 e folded into one multiply), so that
    // each weight is one exp2; the weights' sum is at least 1, so its
    // hardware reciprocal (1 ulp) needs no range care
    const float zs = scale * 1.44269504088896340736f;
    float a[CPL];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot += r[e] * kx[c][e];
        dot = sum16(dot) * zs;
        a[c] = valid[c] ? dot : -INFINITY;
        mx = fmaxf(mx, a[c]);
    }
    mx = xmax32(xmax16(mx));
    float den = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        a[c] = valid[c] ? __builtin_amdgcn_exp2f(a[c] - mx) : 0.f;
        den += a[c];
    }
    const float inv = __builtin_amdgcn_rcpf(xsum32(xsum16(den)));
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const float w = a[c] * inv;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += w * kx[c][e];
    }
    rg_reduce_scatter<EPL>(acc, part);
}

// Pooled key row `row` of level lvl (and its router copy): each lane stores
// its part, at column col.
template <typename T, int D>
__device__ __forceinline__ void store_key_row(const TreeArgs &t, int lvl, int64_t row, const float (&part)[D / 64],
                                              int col, int lane)
{
    constexpr int NP = D / 64;
    store_part<T, NP>((T *)t.lk[lvl - 1] + row * D + col, part);
    if (t.rfp8) {
        float kr[NP];
#pragma unroll
        for (int e = 0; e < NP; ++e) kr[e] = round_to<T>(part[e]);
        store_router_part<D, NP>(t, lvl, row, kr, col, lane);
    }
}

// One wave pools node `node` of level `lvl` (children at level lvl-1: b
// tokens at level 1, fan nodes above) for (sequence, KV head) slot bh.
// CPL = children per lane-row (ceil(children / 4)).
// LV: 1 when lvl is 1, 2 when lvl is at least 2, 0 when either (known at run
// time only).  refs() is called by every wave once its child loads are in
// flight, active or not (so it may hold a block barrier), and returns the R
// reference rows of the head ([R, D] fp32): from global memory, or staged in
// LDS (then the per-reference loop of level 1 issues no global load, and so
// never waits on the previous reference's stores).  An inactive wave stores
// nothing and returns after refs().
template <typename T, int D, int CPL, int LV, typename Refs>
__device__ __forceinline__ void pool_node_refs(const TreeArgs &t, int lvl, int64_t bh, int64_t node, int lane,
                                               bool active, Refs refs)
{
    constexpr int EPL = D / 16;                  // elements per lane of a child row
    constexpr int NP = D / 64;                   // elements per lane of a pooled row
    const int sub = lane & 15, rg = lane >> 4;
    const int col = sub * EPL + rg * NP;         // this lane's column of a pooled row
    const int b = LV == 1 ? t.b : LV == 2 ? t.fan : fan_in(t, lvl), R = t.R;   // children of the node
    // An inactive wave reads the children of a node clamped into the level
    // (every launch has at least one node there) and discards them: the
    // loads are unconditional, so the compiler keeps the rows packed until
    // their use, and they need not wait for what decides `active`.
    const int64_t c0 = min(node, t.ncap[lvl] - 1) * b;   // first child (level lvl-1 index)
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
    // keys of reference 0 (level 1: the token keys, shared by every reference)
    // (index clamped: an out-of-range lk[-1], even unselected, makes the
    // compiler copy the whole argument block to scratch)
    const T *kbase = lvl == 1 ? (const T *)t.kc : (const T *)t.lk[lvl >= 2 ? lvl - 2 : 0];
    const int kstride = (lvl == 1) ? 1 : R;      // key rows per child
    float vx[CPL][EPL], kx[CPL][EPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) load_child<T, EPL, LV != 0>(vbase + crow[c] * D + sub * EPL, vx[c]);
#pragma unroll
    for (int c = 0; c < CPL; ++c) load_child<T, EPL, LV != 0>(kbase + crow[c] * kstride * D + sub * EPL, kx[c]);
    const float *refs_h = refs();
    if (!active) return;

    // mean-pooled value first: it frees the value registers before the keys
    {
        float vs[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) vs[e] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            if (valid[c]) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) vs[e] += vx[c][e];
            }
        float part[NP];
        rg_reduce_scatter<EPL>(vs, part);
#pragma unroll
        for (int e = 0; e < NP; ++e) part[e] /= (float)b;
        store_part<T, NP>((T *)t.lv[lvl - 1] + (bh * t.ncap[lvl] + node) * D + col, part);
    }

    // pooled keys, one per reference.  Key j - 1 is stored after the child
    // keys of reference j are requested (levels >= 2; level 1 shares one set
    // of keys, loaded above), so waiting for those never waits for that store.
    const bool upper = LV == 2 || (LV == 0 && lvl >= 2);
    const int64_t row0 = (bh * t.ncap[lvl] + node) * R;
    float part[NP];
    for (int j = 0; j < R; ++j) {
        if (j > 0) {
            if (upper) {
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    load_child<T, EPL, LV != 0>(kbase + (crow[c] * R + j) * D + sub * EPL, kx[c]);
            }
            store_key_row<T, D>(t, lvl, row0 + j - 1, part, col, lane);
        }
        pool_key<D, CPL>(t.scale, refs_h + j * D, kx, valid, sub, part);
    }
    store_key_row<T, D>(t, lvl, row0 + R - 1, part, col, lane);
}

// One wave pools reference j of node `node` of level lvl >= 2, whose
// children hold R keys each: key j of the node is made from the children's
// keys j alone, so the R references of a node are independent work (the
// wave of reference 0 also pools the mean value).  One round trip per wave:
// the children's keys j, (j = 0) their values and the reference row go out
// together.  An inactive wave (node past the level's last full node) stores
// nothing; its loads are clamped into the level.
template <typename T, int D, int CPL>
__device__ __forceinline__ void pool_node_one_ref(const TreeArgs &t, int lvl, int64_t bh, int h, int64_t node, int j,
                                                  int lane, bool active)
{
    constexpr int EPL = D / 16;
    constexpr int NP = D / 64;
    const int sub = lane & 15, rg = lane >> 4;
    const int col = sub * EPL + rg * NP;
    const int b = t.fan, R = t.R;                // children of a node above level 1
    const int64_t c0 = min(node, t.ncap[lvl] - 1) * b;
    const int64_t nchild_cap = t.ncap[lvl - 1];
    bool valid[CPL];
    int64_t crow[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int child = rg + 4 * c;
        valid[c] = child < b;
        crow[c] = bh * nchild_cap + c0 + min(child, b - 1);
    }
    const T *kbase = (const T *)t.lk[lvl >= 2 ? lvl - 2 : 0];
    float kx[CPL][EPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) load_child<T, EPL, true>(kbase + (crow[c] * R + j) * D + sub * EPL, kx[c]);
    if (j == 0) {
        const T *vbase = (const T *)t.lv[lvl >= 2 ? lvl - 2 : 0];
        float vx[CPL][EPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) load_child<T, EPL, true>(vbase + crow[c] * D + sub * EPL, vx[c]);
        float vs[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) vs[e] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            if (valid[c]) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) vs[e] += vx[c][e];
            }
        float part[NP];
        rg_reduce_scatter<EPL>(vs, part);
#pragma unroll
        for (int e = 0; e < NP; ++e) part[e] /= (float)b;
        if (active) store_part<T, NP>((T *)t.lv[lvl - 1] + (bh * t.ncap[lvl] + node) * D + col, part);
    }
    float part[NP];
    pool_key<D, CPL>(t.scale, t.refs + ((int64_t)h * R + j) * D, kx, valid, sub, part);
    if (active) store_key_row<T, D>(t, lvl, (bh * t.ncap[lvl] + node) * R + j, part, col, lane);
}

// The same, reading the reference rows of head h from global memory.
template <typename T, int D, int CPL>
__device__ void pool_node(const TreeArgs &t, int lvl, int64_t bh, int h, int64_t node, int lane)
{
    const float *refs_h = t.refs + (int64_t)h * t.R * D;
    pool_node_refs<T, D, CPL, 0>(t, lvl, bh, node, lane, true, [=]() { return refs_h; });
}

} // namespace hti
