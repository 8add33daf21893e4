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
#include "hti_pool.h"

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

// Level `lvl` of every (sequence, head): 4 nodes per 256-thread block at
// level 1 (a node's references share its token keys), 4 (node, reference)
// items above (LV = 2).  EXT false: every full node over the first len[s]
// tokens (node = the block's offset, so the child loads go out before len[s]
// arrives).  EXT true: only the nodes that tokens len[s] .. len[s] + ext - 1
// (clamped to the cache) complete, len[s] still being the old length.
template <typename T, int D, int CPL, int LV, bool EXT>
__global__ __launch_bounds__(256) void k_build_level(TreeArgs t, int lvl, int64_t ext)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int bhy = (int)blockIdx.y;                   // 32-bit: the divisions stay short
    const int64_t bh = bhy;
    const int bi = bhy / t.Hkv, h = bhy % t.Hkv;
    const int64_t L = t.len[bi];
    // node range: floor(floor(x / f1) / f2) = floor(x / (f1 f2)), so one
    // division by the span (the product of the fan-ins up to lvl) for each
    // end; both ends are below the cache capacity (< 2^31), so a span clamped
    // to 2^31 divides them the same, in 32 bits
    uint32_t span = 1;
    for (int l = 1; l <= lvl; ++l) span = (uint32_t)min((uint64_t)span * (uint64_t)fan_in(t, l), (uint64_t)1 << 31);
    const int64_t lo = EXT ? (int64_t)((uint32_t)L / span) : 0;
    const int64_t hi = (int64_t)((uint32_t)(EXT ? min(L + ext, t.ncap[0]) : L) / span);
    if constexpr (LV == 2) {
        // levels >= 2: one wave per (node, reference)
        const int64_t item = (int64_t)blockIdx.x * 4 + wave;
        const int64_t node = lo + item / t.R;
        pool_node_one_ref<T, D, CPL>(t, lvl, bh, h, node, (int)(item % t.R), lane, node < hi);
        return;
    }
    const int64_t node = lo + (int64_t)blockIdx.x * 4 + wave;

    // The block's four nodes share head h: its reference rows (at most
    // HTI_MAX_R * D floats, one float4 per thread) go to LDS once.  Their
    // load is issued before the child loads and written to LDS after them,
    // so the barrier does not hold the child rows back.
    static_assert(HTI_MAX_R * D <= 4 * 256, "one float4 of reference rows per thread");
    __shared__ __align__(16) float sref[HTI_MAX_R * D];
    const int i4 = 4 * (int)threadIdx.x;
    const bool has = i4 < t.R * D;
    float4 rv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has) rv = *reinterpret_cast<const float4 *>(t.refs + (int64_t)h * t.R * D + i4);
    pool_node_refs<T, D, CPL, LV>(t, lvl, bh, node, lane, node < hi, [&]() {
        if (has) *reinterpret_cast<float4 *>(sref + i4) = rv;
        __syncthreads();
        return (const float *)sref;
    });
}

// Rows of a block of T tokens per sequence ([B, T, Hkv, D], the prefill
// block layout) into the cache at len[s] .., as far as the cache holds them;
// 16 bytes per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_extend_rows(TreeArgs t, const T *kb, const T *vb, int T_)
{
    constexpr int EPC = 16 / sizeof(T);                 // elements per 16-byte chunk
    const int cpr = t.D / EPC;                          // chunks per row
    const int64_t bh = blockIdx.y;
    const int bi = (int)(bh / t.Hkv), h = (int)(bh % t.Hkv);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T_ * cpr) return;
    const int tok = (int)(i / cpr), ch = (int)(i % cpr);
    const int64_t row = t.len[bi] + tok;
    if (row >= t.ncap[0]) return;
    const int64_t src = (((int64_t)bi * T_ + tok) * t.Hkv + h) * t.D + ch * EPC;
    const int64_t dst = (bh * t.ncap[0] + row) * t.D + ch * EPC;
    *reinterpret_cast<uint4 *>((T *)t.kc + dst) = *reinterpret_cast<const uint4 *>(kb + src);
    *reinterpret_cast<uint4 *>((T *)t.vc + dst) = *reinterpret_cast<const uint4 *>(vb + src);
}

// len[s] += T, clamped to the cache
__global__ void k_extend_len(int64_t *len, int B, int64_t T_, int64_t cap)
{
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s < B) len[s] = min(len[s] + T_, cap);
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
        const int f = fan_in(t, lvl);
        if (idx % f != 0) break;                       // no node completed at this level
        idx /= f;
        pool_node<T, D, CPL>(t, lvl, bh, h, idx - 1, lane);
        __syncthreads();
    }
    if (threadIdx.x == 0) t.len[bi] = L + 1;
}

template <typename T, int D, int LV, bool EXT>
static void build_level_lv(const TreeArgs &t, int lvl, dim3 grid, int64_t ext, hipStream_t s)
{
    const int f = fan_in(t, lvl);
    if (f <= 8)
        hipLaunchKernelGGL((k_build_level<T, D, 2, LV, EXT>), grid, dim3(256), 0, s, t, lvl, ext);
    else if (f <= 16)
        hipLaunchKernelGGL((k_build_level<T, D, 4, LV, EXT>), grid, dim3(256), 0, s, t, lvl, ext);
    else if (f <= 32)
        hipLaunchKernelGGL((k_build_level<T, D, 8, LV, EXT>), grid, dim3(256), 0, s, t, lvl, ext);
    else
        hipLaunchKernelGGL((k_build_level<T, D, 16, LV, EXT>), grid, dim3(256), 0, s, t, lvl, ext);
}

template <typename T, int D>
static hipError_t build_level_d(const TreeArgs &t, int lvl, int64_t max_nodes, int64_t ext, hipStream_t s)
{
    // four waves per block: nodes at level 1, (node, reference) items above
    const int64_t items = lvl == 1 ? max_nodes : max_nodes * t.R;
    dim3 grid((unsigned)((items + 3) / 4), (unsigned)(t.B * t.Hkv));
    if (lvl == 1)
        ext > 0 ? build_level_lv<T, D, 1, true>(t, lvl, grid, ext, s) : build_level_lv<T, D, 1, false>(t, lvl, grid, ext, s);
    else
        ext > 0 ? build_level_lv<T, D, 2, true>(t, lvl, grid, ext, s) : build_level_lv<T, D, 2, false>(t, lvl, grid, ext, s);
    return hipGetLastError();
}

static hipError_t build_level_any(const TreeArgs &t, int lvl, int64_t max_nodes, int64_t ext, hipStream_t s)
{
    if (max_nodes <= 0) return hipSuccess;
    if (t.dtype == HTI_BF16)
        return t.D == 128 ? build_level_d<bf16_t, 128>(t, lvl, max_nodes, ext, s)
                          : build_level_d<bf16_t, 64>(t, lvl, max_nodes, ext, s);
    return t.D == 128 ? build_level_d<float, 128>(t, lvl, max_nodes, ext, s)
                      : build_level_d<float, 64>(t, lvl, max_nodes, ext, s);
}

hipError_t launch_build_level(const TreeArgs &t, int lvl, int64_t max_nodes, hipStream_t s)
{
    return build_level_any(t, lvl, max_nodes, 0, s);
}

hipError_t launch_extend(const TreeArgs &t, const void *k_blk, const void *v_blk, int T_, hipStream_t s)
{
    if (T_ <= 0) return hipSuccess;
    const int epc = t.dtype == HTI_BF16 ? 8 : 4;
    const int64_t chunks = (int64_t)T_ * (t.D / epc);
    const dim3 rgrid((unsigned)((chunks + 255) / 256), (unsigned)(t.B * t.Hkv));
    if (t.dtype == HTI_BF16)
        hipLaunchKernelGGL(k_extend_rows<bf16_t>, rgrid, dim3(256), 0, s, t, (const bf16_t *)k_blk,
                           (const bf16_t *)v_blk, T_);
    else
        hipLaunchKernelGGL(k_extend_rows<float>, rgrid, dim3(256), 0, s, t, (const float *)k_blk,
                           (const float *)v_blk, T_);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // T tokens complete at most floor(T / (span of a level-l node)) + 1
    // nodes of level l
    int64_t span = T_;
    for (int l = 1; l <= t.levels; ++l) {
        span /= fan_in(t, l);
        e = build_level_any(t, l, span + 1, T_, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_extend_len, dim3((unsigned)((t.B + 63) / 64)), dim3(64), 0, s, t.len, t.B,
                       (int64_t)T_, t.ncap[0]);
    return hipGetLastError();
}

template <typename T, int D, int MAXT>
static void append_b(const TreeArgs &t, const T *k, const T *v, hipStream_t s)
{
    dim3 grid(t.B), block(64 * t.Hkv);
    const int f = t.b > t.fan ? t.b : t.fan;          // the larger fan-in of the levels
    if (f <= 8)
        hipLaunchKernelGGL((k_append<T, D, 2, MAXT>), grid, block, 0, s, t, k, v);
    else if (f <= 16)
        hipLaunchKernelGGL((k_append<T, D, 4, MAXT>), grid, block, 0, s, t, k, v);
    else if (f <= 32)
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
