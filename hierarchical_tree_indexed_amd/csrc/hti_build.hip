// hti_build.hip -- tree construction: RoPE table, level-by-level pooling, and
// the per-token append with its cascade of completed nodes.
//
// Pooling follows "Recursive Sparse Attention" (abstract: one key and one
// mean-pooled value per node, one pooler shared by every level) and
// "Subquadratic Attention with a Hierarchical Tree-Structured Indexer"
// (Figure 3 caption: a chunk of contiguous key nodes is summarised by an
// attention-weighted sum of its keys, the attention taken w.r.t. reference
// queries, one key per reference stored in parallel, higher levels built from
// the lower summaries; Table VIII: only full nodes, n_l = floor(n_{l-1} / b)).
//
// Layout of the work: one wavefront pools one node.  The node's b children
// are contiguous rows (b * d elements), so a wave streams them with 16-byte
// loads: lane = (row group rg = lane / 16) x (slice sub = lane % 16); row
// group rg holds children rg, rg + 4, ..., slice sub holds d/16 contiguous
// elements of each.  Dot products reduce over the 16 lanes of a row group,
// the softmax and the weighted sums over the 4 row groups.  Every child byte
// is read from HBM once; the node is written once.
#include <type_traits>

#include "hti_device.h"
#include "hti_internal.h"

namespace hti {

// ----------------------------------------------------------------------------
// RoPE table: cos/sin(pos * base^(-2j/d)), angle formed in double.
// ----------------------------------------------------------------------------
__global__ void k_rope_init(float2 *rope, int npos, int D, double base)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int half = D / 2;
    if (idx >= (int64_t)npos * half) return;
    const int pos = (int)(idx / half), j = (int)(idx % half);
    const double theta = pow(base, -2.0 * (double)j / (double)D);
    const double ang = (double)pos * theta;
    rope[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t launch_rope_init(const TreeArgs &t, double base, hipStream_t s)
{
    const int64_t n = (int64_t)t.rope_npos * (t.D / 2);
    if (n == 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_rope_init, dim3((unsigned)blocks), dim3(256), 0, s,
                       const_cast<float2 *>(t.rope), t.rope_npos, t.D, base);
    return hipGetLastError();
}

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
            dot = group_sum<16>(dot) * t.scale;
            a[c] = valid[c] ? dot : -INFINITY;
            mx = fmaxf(mx, a[c]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        float den = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            a[c] = valid[c] ? expf(a[c] - mx) : 0.f;
            den += a[c];
        }
        den += __shfl_xor(den, 16, kWave);
        den += __shfl_xor(den, 32, kWave);

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
        for (int e = 0; e < EPL; ++e) {
            acc[e] += __shfl_xor(acc[e], 16, kWave);
            acc[e] += __shfl_xor(acc[e], 32, kWave);
        }
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
        vs[e] += __shfl_xor(vs[e], 16, kWave);
        vs[e] += __shfl_xor(vs[e], 32, kWave);
        vs[e] = vs[e] / (float)b;
    }
    if (rg == 0) {
        T *out = (T *)t.lv[lvl - 1] + (bh * t.ncap[lvl] + node) * D + sub * EPL;
        store_slice<T, D>(out, vs);
    }
}

// Level `lvl` of every (sequence, head): 4 nodes per 256-thread block.
template <typename T, int D, int CPL>
__global__ __launch_bounds__(256) void k_build_level(TreeArgs t, int lvl)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t node = (int64_t)blockIdx.x * 4 + wave;
    const int64_t bh = blockIdx.y;
    const int bi = (int)(bh / t.Hkv), h = (int)(bh % t.Hkv);
    int64_t n = t.len[bi];
    for (int l = 0; l < lvl; ++l) n /= t.b;
    if (node >= n) return;
    pool_node<T, D, CPL>(t, lvl, bh, h, node, lane);
}

// Append one token per sequence: one block per sequence, one wave per KV head
// (MAXT: the largest block, 64 * Hkv threads, which sets the register budget).
template <typename T, int D, int CPL, int MAXT>
__global__ __launch_bounds__(MAXT) void k_append(TreeArgs t, const T *kn, const T *vn)
{
    const int h = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int bi = blockIdx.x;
    const int64_t bh = (int64_t)bi * t.Hkv + h;
    // the new row does not depend on the length: its loads go out with the
    // length's (stores predicated on the length, not behind a branch)
    constexpr int EPW = (D + 2 * kWave - 1) / (2 * kWave);   // bf16 / fp32 pairs per lane
    uint64_t kr[EPW], vr[EPW];
    static_assert(sizeof(T) <= 4, "element size");
    using W2 = typename std::conditional<sizeof(T) == 2, uint32_t, uint64_t>::type;
#pragma unroll
    for (int u = 0; u < EPW; ++u) {
        const int e = min(2 * (lane + u * kWave), D - 2);
        kr[u] = *reinterpret_cast<const W2 *>(kn + bh * D + e);
        vr[u] = *reinterpret_cast<const W2 *>(vn + bh * D + e);
    }
    const int64_t L = t.len[bi];
    const bool full = L >= t.ncap[0];                  // cache full: unchanged
    T *kc = (T *)t.kc + (bh * t.ncap[0] + (full ? 0 : L)) * D;
    T *vc = (T *)t.vc + (bh * t.ncap[0] + (full ? 0 : L)) * D;
#pragma unroll
    for (int u = 0; u < EPW; ++u) {
        const int e = 2 * (lane + u * kWave);
        if (!full && e < D) {
            *reinterpret_cast<W2 *>(kc + e) = (W2)kr[u];
            *reinterpret_cast<W2 *>(vc + e) = (W2)vr[u];
        }
    }
    if (full) return;
    __syncthreads();
    int64_t idx = L + 1;                               // node count after the append
    for (int lvl = 1; lvl <= t.levels; ++lvl) {
        if (idx % t.b != 0) break;                     // no node completed at this level
        idx /= t.b;
        pool_node<T, D, CPL>(t, lvl, bh, h, idx - 1, lane);
        __syncthreads();
    }
    if (threadIdx.x == 0) t.len[bi] = L + 1;
}

template <typename T, int D>
static hipError_t build_level_d(const TreeArgs &t, int lvl, int64_t max_nodes, hipStream_t s)
{
    dim3 grid((unsigned)((max_nodes + 3) / 4), (unsigned)(t.B * t.Hkv));
    if (t.b <= 8)
        hipLaunchKernelGGL((k_build_level<T, D, 2>), grid, dim3(256), 0, s, t, lvl);
    else if (t.b <= 16)
        hipLaunchKernelGGL((k_build_level<T, D, 4>), grid, dim3(256), 0, s, t, lvl);
    else if (t.b <= 32)
        hipLaunchKernelGGL((k_build_level<T, D, 8>), grid, dim3(256), 0, s, t, lvl);
    else
        hipLaunchKernelGGL((k_build_level<T, D, 16>), grid, dim3(256), 0, s, t, lvl);
    return hipGetLastError();
}

hipError_t launch_build_level(const TreeArgs &t, int lvl, int64_t max_nodes, hipStream_t s)
{
    if (max_nodes <= 0) return hipSuccess;
    if (t.dtype == HTI_BF16)
        return t.D == 128 ? build_level_d<bf16_t, 128>(t, lvl, max_nodes, s)
                          : build_level_d<bf16_t, 64>(t, lvl, max_nodes, s);
    return t.D == 128 ? build_level_d<float, 128>(t, lvl, max_nodes, s)
                      : build_level_d<float, 64>(t, lvl, max_nodes, s);
}

template <typename T, int D, int MAXT>
static void append_b(const TreeArgs &t, const T *k, const T *v, hipStream_t s)
{
    dim3 grid(t.B), block(64 * t.Hkv);
    if (t.b <= 8)
        hipLaunchKernelGGL((k_append<T, D, 2, MAXT>), grid, block, 0, s, t, k, v);
    else if (t.b <= 16)
        hipLaunchKernelGGL((k_append<T, D, 4, MAXT>), grid, block, 0, s, t, k, v);
    else if (t.b <= 32)
        hipLaunchKernelGGL((k_append<T, D, 8, MAXT>), grid, block, 0, s, t, k, v);
    else
        hipLaunchKernelGGL((k_append<T, D, 16, MAXT>), grid, block, 0, s, t, k, v);
}

template <typename T, int D>
static hipError_t append_d(const TreeArgs &t, const void *kn, const void *vn, hipStream_t s)
{
    const T *k = (const T *)kn, *v = (const T *)vn;
    if (t.Hkv <= 8) append_b<T, D, 512>(t, k, v, s);
    else append_b<T, D, 1024>(t, k, v, s);
    return hipGetLastError();
}

hipError_t launch_append(const TreeArgs &t, const void *k_new, const void *v_new, hipStream_t s)
{
    if (t.dtype == HTI_BF16)
        return t.D == 128 ? append_d<bf16_t, 128>(t, k_new, v_new, s)
                          : append_d<bf16_t, 64>(t, k_new, v_new, s);
    return t.D == 128 ? append_d<float, 128>(t, k_new, v_new, s)
                      : append_d<float, 64>(t, k_new, v_new, s);
}

} // namespace hti
