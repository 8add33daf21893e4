// hti_prefill_nodes.hip -- the token level of a prefill block, node-inverted.
//
// "Recursive Sparse Attention", abstract: after the summary levels, every
// query attends exactly to the tokens of the level-1 nodes it kept (plus the
// orphan tokens), each token at its index among the query's token-level
// candidates.  For a block of queries this reads the same node rows once per
// query that kept them; here the queries are grouped by kept node instead, so
// that each node's b token rows are read once per block.
//
// Positions.  A query at candidate position P that kept level-1 node n at rank
// r (its r-th kept node) sees token j of n at position r*b + j.  Rotations of
// rotate-half RoPE compose (R(x)^T R(y) = R(y - x)), so
//     <R(P) q, R(r*b + j) k_j> = <R(P - r*b) q, R(j) k_j>:
// the keys are turned by their offset inside the node -- the same for every
// query -- and each (query, node) pair turns its query by P - r*b.  The logits
// of a node are then one plain product [pairs * G, d] x [d, b] on the matrix
// cores, and so is the probability-weighted value sum.  Token logits decide no
// selection, so bf16 operands (fp32 accumulation) only move the outputs by far
// less than their tolerance.
//
// Passes (one launch each, after the traversal of the summary levels, which
// leaves each unit's kept level-1 list and counts the units per node):
//   k_pairs_scan     per tree: exclusive scan of the per-node counts (in place)
//   k_pairs_scatter  every (unit, rank) pair to its node's run of the tree's
//                    pair list
//   k_token_nodes    one wave per kPairsPerWave consecutive pairs: for each
//                    node in its range, the node's keys (turned) and values
//                    (transposed through LDS) once, then S^T = K' Q'^T and
//                    O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 for 16 / G pairs
//                    at a time; each pair leaves its normalised output (bf16)
//                    with its max and denominator
//   k_token_merge    one wave per (unit, head): the traversal's partial state
//                    and the unit's pair states merged into one online-softmax
//                    state, which the in-block kernel then seeds from.
#include <algorithm>

#include "hti_device.h"
#include "hti_internal.h"

namespace hti {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float floatx4;

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t pack_bf(float a, float b)
{
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// Turn eight rotate-half pairs (lo[e], hi[e]) = (x_i, x_{i + d/2}), i = i0 + e,
// by the (cos, sin) rows cs (8 pairs, as 4 float4) and round to bf16: the
// first halves go to `a`, the second halves to `b`.
__device__ __forceinline__ void turn8(const uint4 &lo, const uint4 &hi, const float4 *cs, bf16x8 &a, bf16x8 &b)
{
    const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w}, hw[4] = {hi.x, hi.y, hi.z, hi.w};
    uint32_t ra[4], rb[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float4 c = cs[w];   // (cos, sin) of pairs i0 + 2w, i0 + 2w + 1
        const float x0 = bf2f(lw[w] & 0xffffu), x1 = bf2f(lw[w] >> 16);
        const float y0 = bf2f(hw[w] & 0xffffu), y1 = bf2f(hw[w] >> 16);
        ra[w] = pack_bf(x0 * c.x - y0 * c.y, x1 * c.z - y1 * c.w);
        rb[w] = pack_bf(x0 * c.y + y0 * c.x, x1 * c.w + y1 * c.z);
    }
    a = __builtin_bit_cast(bf16x8, make_uint4(ra[0], ra[1], ra[2], ra[3]));
    b = __builtin_bit_cast(bf16x8, make_uint4(rb[0], rb[1], rb[2], rb[3]));
}

// Exclusive scan of one tree's per-node counts, in place; the tree's total
// goes to ptot.  One workgroup of 1024 threads per tree, 8 counts per thread
// per round.
__global__ __launch_bounds__(1024) void k_pairs_scan(uint32_t *cnt, int64_t n, uint32_t *ptot)
{
    __shared__ uint32_t wsum[16];
    uint32_t *c = cnt + (int64_t)blockIdx.x * n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t carry = 0;
    for (int64_t base = 0; base < n; base += 1024 * 8) {
        const int64_t i0 = base + (int64_t)tid * 8;
        uint32_t v[8], s = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t x = (i0 + e < n) ? c[i0 + e] : 0u;
            v[e] = s;
            s += x;
        }
        uint32_t inc = s;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t y = (uint32_t)__shfl_up((int)inc, d);
            if (lane >= d) inc += y;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        uint32_t wpre = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const uint32_t x = wsum[w];
            wpre += (w < wave) ? x : 0u;
            tot += x;
        }
        const uint32_t off = carry + wpre + inc - s;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (i0 + e < n) c[i0 + e] = off + v[e];
        carry += tot;
        __syncthreads();
    }
    if (tid == 0) ptot[blockIdx.x] = carry;
}

// Every kept (unit, rank) pair into its node's run of its tree's pair list,
// with what the node kernel needs of it: the query's rotation position
// P - rank * b (P = its position after the token-level candidates: the kept
// nodes' tokens and the orphans, then block row qi) and its first q row.  The
// order inside a run depends on the atomics; each pair's result does not.
__global__ __launch_bounds__(256) void k_pairs_scatter(NodeArgs a, int64_t n)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const int64_t unit = idx / a.keff;
    const int r = (int)(idx - unit * a.keff);
    const int nsel = a.nsel1[unit];
    if (r >= nsel) return;
    const int node = a.kept1[idx];
    const int Hr = a.t.Hkv, b = a.t.b;
    const int64_t g = unit % Hr;
    const int64_t bq = unit / Hr;                 // bi * T + qi
    const int64_t bi = bq / a.T;
    const int64_t qi = bq - bi * a.T;
    const int64_t tree = bi * (Hr / a.t.hdiv) + g / a.t.hdiv;
    const int64_t L = a.t.len[bi];
    const int64_t P = (int64_t)nsel * b + (L % b) + qi;
    const uint32_t pos = atomicAdd(&a.cnt[tree * a.t.ncap[1] + node], 1u);
    a.pairs[tree * a.cap_t + pos] =
        make_uint4((uint32_t)node, (uint32_t)idx, (uint32_t)(P - (int64_t)r * b),
                   (uint32_t)(bq * a.t.Hq + g * a.t.G));
}

// Pairs per wave of the node kernel: the runs of one wave's pairs are
// handled one after the other, so fewer pairs per wave give more waves (and
// more loads in flight) at the price of reading a node twice where its run
// crosses a wave boundary.
constexpr int kPairsPerWave = 16;

// V^T rows in LDS: 32 token slots (bf16) per d plus 8 bytes of padding, which
// spreads the 16-byte fragment reads of 16 consecutive rows over the banks.
constexpr int kVtWords = 20;

template <int D, int G, int NT>
__global__ __launch_bounds__(256) void k_token_nodes(NodeArgs a)
{
    constexpr int KS = D / 32;   // k-steps of S^T = K' Q'^T
    constexpr int KH = KS / 2;   // k-steps that cover the first rotate-half
    constexpr int DT = D / 16;   // d-tiles of O^T = V^T P^T
    constexpr int PT = 16 / G;   // pairs per 16-row tile
    static_assert(NT == 1 || NT == 2, "b <= 32");
    __shared__ __attribute__((aligned(16))) uint32_t vts[4][D * kVtWords];

    const TreeArgs &t = a.t;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    constexpr int CH = kPairsPerWave;
    const int64_t wpt = (a.cap_t + CH - 1) / CH;
    const int64_t w = (int64_t)blockIdx.x * 4 + wave;
    const int tree = (int)(w / wpt);
    if (tree >= a.ntrees) return;
    const int64_t base = (w - (int64_t)tree * wpt) * CH;
    const int64_t tot = a.ptot[tree];
    if (base >= tot) return;
    const int npair = (int)std::min<int64_t>(CH, tot - base);
    // lane p < npair holds pair base + p
    uint4 rec = make_uint4(0xffffffffu, 0u, 0u, 0u);
    if (lane < npair) rec = a.pairs[tree * a.cap_t + base + lane];
    const uint32_t mynode = rec.x;
    const uint32_t prevnode = (uint32_t)__shfl((int)mynode, lane > 0 ? lane - 1 : 0);
    // runs of equal nodes among the wave's pairs
    uint64_t starts = __ballot(lane < npair && (lane == 0 || mynode != prevnode));

    const int b = t.b;
    const bf16_t *kc = (const bf16_t *)t.kc + (int64_t)tree * t.ncap[0] * D;
    const bf16_t *vc = (const bf16_t *)t.vc + (int64_t)tree * t.ncap[0] * D;
    uint32_t *vl = vts[wave];

    while (starts) {
        const int s0 = __builtin_ctzll(starts);
        starts &= starts - 1;
        const int s1 = starts ? __builtin_ctzll(starts) : npair;
        const int64_t node = (uint32_t)__builtin_amdgcn_readlane((int)mynode, s0);
        const bf16_t *k0 = kc + node * b * D;
        const bf16_t *v0 = vc + node * b * D;

        // K' (A operand of S^T): token 16 tt + col turned by its offset in the
        // node; tokens past b read row b - 1 and are masked out below
        bf16x8 ak[NT][KS];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int tk = std::min(16 * tt + col, b - 1);
            const bf16_t *kr = k0 + (int64_t)tk * D;
#pragma unroll
            for (int s = 0; s < KH; ++s) {
                const int i0 = 8 * grp + 32 * s;
                const uint4 lo = *reinterpret_cast<const uint4 *>(kr + i0);
                const uint4 hi = *reinterpret_cast<const uint4 *>(kr + i0 + D / 2);
                const float4 *cs = reinterpret_cast<const float4 *>(t.rope + (int64_t)tk * (D / 2) + i0);
                turn8(lo, hi, cs, ak[tt][s], ak[tt][s + KH]);
            }
        }
        // V^T into LDS: token t of the node goes to slot 8*((t%16)/4) + 4*(t/16)
        // + t%4, the order in which a lane holds its probabilities after
        // S^T; tokens past b are zero.  A lane moves tokens (2p, 2p+1) of 8
        // columns at a time (adjacent slots: one 32-bit word per column).
#pragma unroll
        for (int u = 0; u < D / 32; ++u) {
            const int item = lane + 64 * u;
            const int tp = item & 15, dc = item >> 4;
            const int t0 = 2 * tp;
            uint4 x = *reinterpret_cast<const uint4 *>(v0 + (int64_t)std::min(t0, b - 1) * D + 8 * dc);
            uint4 y = *reinterpret_cast<const uint4 *>(v0 + (int64_t)std::min(t0 + 1, b - 1) * D + 8 * dc);
            if (t0 >= b) x = make_uint4(0u, 0u, 0u, 0u);
            if (t0 + 1 >= b) y = make_uint4(0u, 0u, 0u, 0u);
            const int sl = 8 * ((t0 & 15) >> 2) + 4 * (t0 >> 4) + (t0 & 3);
            uint32_t *dst = vl + (8 * dc) * kVtWords + (sl >> 1);
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dst[(2 * e) * kVtWords] = (xs[e] & 0xffffu) | (ys[e] << 16);
                dst[(2 * e + 1) * kVtWords] = (xs[e] >> 16) | (ys[e] & 0xffff0000u);
            }
        }
        wave_sync();

        // the run's pairs, PT at a time: row col of the tile is head col % G
        // of pair p0 + col / G
        for (int p0 = s0; p0 < s1; p0 += PT) {
            const int pp = p0 + col / G;
            const int h = col % G;
            const bool valid = pp < s1;
            const int src = std::min(pp, CH - 1);
            const uint32_t slot = (uint32_t)__shfl((int)rec.y, src);
            const int64_t pr = (uint32_t)__shfl((int)rec.z, src);
            const uint32_t qrow = (uint32_t)__shfl((int)rec.w, src);
            const bf16_t *qr = (const bf16_t *)a.q + ((int64_t)qrow + h) * D;
            bf16x8 bq[KS];
#pragma unroll
            for (int s = 0; s < KH; ++s) {
                const int i0 = 8 * grp + 32 * s;
                const uint4 lo = *reinterpret_cast<const uint4 *>(qr + i0);
                const uint4 hi = *reinterpret_cast<const uint4 *>(qr + i0 + D / 2);
                const float4 *cs = reinterpret_cast<const float4 *>(t.rope + pr * (D / 2) + i0);
                turn8(lo, hi, cs, bq[s], bq[s + KH]);
            }
            if (!valid) {
#pragma unroll
                for (int s = 0; s < KS; ++s) bq[s] = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
            }
            // S^T: lane (col, grp) holds tokens 16 tt + 4 grp + i of row col
            floatx4 st[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                st[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    st[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[tt][s], bq[s], st[tt], 0, 0, 0);
            }
            float z[NT][4], mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    z[tt][i] = (16 * tt + 4 * grp + i < b) ? st[tt][i] * t.scale : -INFINITY;
                    mx = fmaxf(mx, z[tt][i]);
                }
            mx = xmax32(xmax16(mx));
            // probabilities rounded to bf16 in slot order (B operand of O^T);
            // the denominator sums the rounded values
            uint32_t pw[4];
            float ls = 0.f;
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const int tt = j >> 2, i = j & 3;
                const float pa = tt < NT ? __expf(z[tt < NT ? tt : 0][i] - mx) : 0.f;
                const float pb = tt < NT ? __expf(z[tt < NT ? tt : 0][i + 1] - mx) : 0.f;
                pw[j >> 1] = pack_bf(pa, pb);
                ls += bf2f(pw[j >> 1] & 0xffffu) + bf2f(pw[j >> 1] >> 16);
            }
            const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            const float l = xsum32(xsum16(ls));
            const float inv = 1.f / l;
            bf16_t *po = a.po + ((int64_t)slot * G + h) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 av = *reinterpret_cast<const bf16x8 *>(vl + (16 * dt + col) * kVtWords + 4 * grp);
                const floatx4 o =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pf, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                if (valid)
                    *reinterpret_cast<uint2 *>(po + 16 * dt + 4 * grp) =
                        make_uint2(pack_bf(o[0] * inv, o[1] * inv), pack_bf(o[2] * inv, o[3] * inv));
            }
            if (valid && grp == 0) {
                a.pml[((int64_t)slot * G + h) * 2 + 0] = mx;
                a.pml[((int64_t)slot * G + h) * 2 + 1] = l;
            }
        }
        wave_sync();   // the next run overwrites this wave's V^T rows
    }
}

// One wave per (unit, head) row: the traversal's state (summaries and orphan
// tokens) merged with the unit's per-node states, written back in place.  The
// pair states are read four ranks at a time (all loads of a group in flight
// together) and folded in with an online rescale.
template <int D>
__global__ __launch_bounds__(256) void k_token_merge(NodeArgs a, int64_t rows)
{
    constexpr int EPL = D / 64;
    constexpr int RG = 4;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int G = a.t.G;
    const int64_t unit = row / G;
    const int h = (int)(row - unit * G);
    const int nsel = a.nsel1[unit];
    float Mn = a.part_ml[row * 2 + 0], Lw = a.part_ml[row * 2 + 1];
    float acc[EPL];
    // (a state with nothing attended has no output row)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = Mn == -INFINITY ? 0.f : a.part_acc[row * D + lane * EPL + e];
    for (int r0 = 0; r0 < nsel; r0 += RG) {
        float m[RG], l[RG], o[RG][EPL];
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            const int r = std::min(r0 + u, nsel - 1);
            const int64_t sr = (unit * a.keff + r) * G + h;
            const float2 ml = *reinterpret_cast<const float2 *>(a.pml + sr * 2);
            m[u] = (r0 + u < nsel) ? ml.x : -INFINITY;
            l[u] = ml.y;
            const bf16_t *op = a.po + sr * D + lane * EPL;
            if constexpr (EPL == 2) {
                const uint32_t x = *reinterpret_cast<const uint32_t *>(op);
                o[u][0] = bf2f(x & 0xffffu);
                o[u][1] = bf2f(x >> 16);
            } else {
                o[u][0] = bf2f(op[0]);
            }
        }
        float mg = Mn;
#pragma unroll
        for (int u = 0; u < RG; ++u) mg = fmaxf(mg, m[u]);
        if (mg == -INFINITY) continue;
        const float al = __expf(Mn - mg);
        Lw *= al;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] *= al;
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            const float wgt = l[u] * __expf(m[u] - mg);
            Lw += wgt;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] += wgt * o[u][e];
        }
        Mn = mg;
    }
    if (nsel == 0) return;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a.part_acc[row * D + lane * EPL + e] = acc[e];
    if (lane == 0) {
        a.part_ml[row * 2 + 0] = Mn;
        a.part_ml[row * 2 + 1] = Lw;
    }
}

} // namespace

bool token_nodes_apply(const hti_tree_cfg *c, const hti_select *sel)
{
    return (!sel || sel->token_nodes) && c->levels >= 1 && c->b <= 32 && (c->d == 64 || c->d == 128);
}

hipError_t launch_token_pairs(const NodeArgs &a, int64_t units, hipStream_t s)
{
    if (a.ntrees <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_pairs_scan, dim3(a.ntrees), dim3(1024), 0, s, a.cnt, (int64_t)a.t.ncap[1], a.ptot);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = units * a.keff;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_pairs_scatter, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, n);
    return hipGetLastError();
}

hipError_t launch_token_nodes(const NodeArgs &a, hipStream_t s)
{
    const int64_t waves = (int64_t)a.ntrees * ((a.cap_t + kPairsPerWave - 1) / kPairsPerWave);
    if (waves == 0) return hipSuccess;
    const dim3 grid((unsigned)((waves + 3) / 4));
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    };
    const bool two = a.t.b > 16;
    if (a.t.D == 128) {
        switch (a.t.G) {
        case 1: return two ? go(k_token_nodes<128, 1, 2>) : go(k_token_nodes<128, 1, 1>);
        case 2: return two ? go(k_token_nodes<128, 2, 2>) : go(k_token_nodes<128, 2, 1>);
        case 4: return two ? go(k_token_nodes<128, 4, 2>) : go(k_token_nodes<128, 4, 1>);
        default: return two ? go(k_token_nodes<128, 8, 2>) : go(k_token_nodes<128, 8, 1>);
        }
    }
    switch (a.t.G) {
    case 1: return two ? go(k_token_nodes<64, 1, 2>) : go(k_token_nodes<64, 1, 1>);
    case 2: return two ? go(k_token_nodes<64, 2, 2>) : go(k_token_nodes<64, 2, 1>);
    case 4: return two ? go(k_token_nodes<64, 4, 2>) : go(k_token_nodes<64, 4, 1>);
    default: return two ? go(k_token_nodes<64, 8, 2>) : go(k_token_nodes<64, 8, 1>);
    }
}

hipError_t launch_token_merge(const NodeArgs &a, int64_t units, hipStream_t s)
{
    const int64_t rows = units * a.t.G;
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (a.t.D == 128) hipLaunchKernelGGL(k_token_merge<128>, grid, dim3(256), 0, s, a, rows);
    else hipLaunchKernelGGL(k_token_merge<64>, grid, dim3(256), 0, s, a, rows);
    return hipGetLastError();
}

} // namespace hti
