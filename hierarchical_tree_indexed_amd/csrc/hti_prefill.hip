// hti_prefill.hip -- dense parts of a prefill block on the matrix cores.
//
// "Recursive Sparse Attention", abstract: the tree's summaries and the exact
// tokens share one softmax.  For a prefill block the exact tokens of query t
// are the reached prefix tokens followed by block tokens 0..t; the block part
// is plain causal attention.  RoPE is relative, so rotating the block's
// queries and keys by their block-local index gives the same logits as the
// candidate indices (prefix candidates + local index) -- the in-block product
// is then one causal attention per KV-head group, computed here on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation) and seeded with the partial
// softmax state (max, denominator, unnormalised output) left by the traversal
// of the prefix tree, so the merge is a single online softmax.
#include "hti_device.h"
#include "hti_internal.h"

namespace hti {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float floatx4;

// ----------------------------------------------------------------------------
// Rotate the block's q and k by their block-local index and store them as
// bf16 in head-major layout: qr [B, Hq, T, D], kr [B, Hkv, T, D].
// ----------------------------------------------------------------------------
template <typename T, int D>
__global__ void k_rotate_block(PrefillArgs a)
{
    const TreeArgs &t = a.t;
    const int H = t.Hq + t.Hkv;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)t.B * a.T * H * (D / 2);
    if (idx >= total) return;
    const int j = (int)(idx % (D / 2));
    int64_t r = idx / (D / 2);
    const int hh = (int)(r % H);
    r /= H;
    const int tt = (int)(r % a.T);
    const int bi = (int)(r / a.T);
    const bool isq = hh < t.Hq;
    const int h = isq ? hh : hh - t.Hq;
    const int nh = isq ? t.Hq : t.Hkv;
    const T *src = (const T *)(isq ? a.q : a.k) + (((int64_t)bi * a.T + tt) * nh + h) * D;
    bf16_t *dst = (bf16_t *)(isq ? a.qr : a.kr) + (((int64_t)bi * nh + h) * a.T + tt) * D;
    float x0, x1;
    load_vec<T, 1>(src + j, &x0);
    load_vec<T, 1>(src + j + D / 2, &x1);
    const float2 cs = t.rope[(int64_t)tt * (D / 2) + j];
    dst[j] = f2bf(x0 * cs.x - x1 * cs.y);
    dst[j + D / 2] = f2bf(x0 * cs.y + x1 * cs.x);
}

hipError_t launch_rotate_block(const PrefillArgs &a, hipStream_t s)
{
    const int64_t total = (int64_t)a.t.B * a.T * (a.t.Hq + a.t.Hkv) * (a.t.D / 2);
    if (total == 0) return hipSuccess;
    dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (a.t.dtype == HTI_BF16) {
        if (a.t.D == 128) hipLaunchKernelGGL((k_rotate_block<bf16_t, 128>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_rotate_block<bf16_t, 64>), grid, block, 0, s, a);
    } else {
        if (a.t.D == 128) hipLaunchKernelGGL((k_rotate_block<float, 128>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_rotate_block<float, 64>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// In-block causal attention (flash style) merged with the prefix partials.
//
// Work split: a workgroup owns QB*16 consecutive queries of every head of one
// KV group; wave w handles head g*G + (w % G) and queries q0 + 16*(w / G) ..
// +15.  Keys advance in tiles of 32 staged through LDS (K row-major, V
// transposed), shared by all the waves of the group.  Scores are computed
// transposed, S^T = K Q^T, so a lane's accumulator column is one query: the
// row statistics of the online softmax need only two cross-lane steps, and the
// probabilities already sit in the B-operand layout of O^T += V^T P^T.
// ----------------------------------------------------------------------------
namespace {
constexpr int KT = 32;          // keys per tile
constexpr int KPAD = 8;         // bf16 padding of a K row in LDS
constexpr int VPAD = 4;         // bf16 padding of a V^T row in LDS
}

template <int D, int G, int NWV>
__global__ __launch_bounds__(NWV * 64) void k_inblock(PrefillArgs a)
{
    constexpr int NTH = NWV * 64;
    constexpr int QB = NWV / G;              // 16-query sub-blocks per workgroup
    constexpr int KS = D / 32;               // k-steps of the QK^T product
    constexpr int DT = D / 16;               // d-tiles of the PV product
    __shared__ __attribute__((aligned(16))) bf16_t sK[KT * (D + KPAD)];
    __shared__ __attribute__((aligned(16))) bf16_t sVt[D * (KT + VPAD)];

    const TreeArgs &t = a.t;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.y, bi = blockIdx.z;
    const int T = a.T;
    const int q0blk = blockIdx.x * (QB * 16);
    const int h = g * G + (wave % G);
    const int q0 = q0blk + 16 * (wave / G);
    const int col = lane & 15, grp = lane >> 4;
    const int myq = q0 + col;                       // this lane's query (column)
    const float c2 = t.scale * 1.4426950408889634f; // scale * log2(e)

    // Q fragments (B operand of S^T = K Q^T): column = query, k-slots 8*grp..
    bf16x8 qf[KS];
    {
        const bf16_t *qb = (const bf16_t *)a.qr + (((int64_t)bi * t.Hq + h) * T) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (myq < T)
                qf[s] = *reinterpret_cast<const bf16x8 *>(qb + (int64_t)myq * D + 32 * s + 8 * grp);
            else
                qf[s] = bf16x8{};
        }
    }

    // seed the online softmax with the prefix partial state of this query
    floatx4 o[DT];
    float mrow = -INFINITY, lrow = 0.f;
    if (myq < T) {
        const int64_t row = ((int64_t)bi * T + myq) * t.Hq + h;
        const float M = a.part_ml[row * 2 + 0];
        lrow = a.part_ml[row * 2 + 1];
        mrow = (M == -INFINITY) ? -INFINITY : M * 1.4426950408889634f;
        const float *pa = a.part_acc + row * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const float4 v = *reinterpret_cast<const float4 *>(pa + 16 * dt + 4 * grp);
            o[dt] = floatx4{v.x, v.y, v.z, v.w};
        }
    } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    const int qlast = min(T - 1, q0blk + QB * 16 - 1);
    const int kend = qlast + 1;
    const bf16_t *kb = (const bf16_t *)a.kr + (((int64_t)bi * t.Hkv + g) * T) * D;
    const bf16_t *vb = (const bf16_t *)a.v;

    for (int kt0 = 0; kt0 < kend; kt0 += KT) {
        __syncthreads();
        // stage K tile (row-major) and V tile (transposed)
        for (int c = tid; c < KT * D / 8; c += NTH) {
            const int key = c / (D / 8), ch = c % (D / 8);
            uint4 kv = make_uint4(0, 0, 0, 0);
            if (kt0 + key < T)
                kv = *reinterpret_cast<const uint4 *>(kb + (int64_t)(kt0 + key) * D + 8 * ch);
            *reinterpret_cast<uint4 *>(sK + key * (D + KPAD) + 8 * ch) = kv;
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (kt0 + key < T)
                vv = *reinterpret_cast<const uint4 *>(
                    vb + (((int64_t)bi * T + kt0 + key) * t.Hkv + g) * D + 8 * ch);
            const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sVt[(8 * ch + 2 * e) * (KT + VPAD) + key] = (bf16_t)(w[e] & 0xffffu);
                sVt[(8 * ch + 2 * e + 1) * (KT + VPAD) + key] = (bf16_t)(w[e] >> 16);
            }
        }
        __syncthreads();
        if (kt0 > q0 + 15) continue;                // tile entirely in this wave's future

        // S^T tiles: keys kt0 + 16*mt + 4*grp + i, query myq
        floatx4 sc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 af = *reinterpret_cast<const bf16x8 *>(
                    sK + (16 * mt + col) * (D + KPAD) + 32 * s + 8 * grp);
                sc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[s], sc[mt], 0, 0, 0);
            }
        }
        float sv[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kt0 + 16 * mt + 4 * grp + i;
                const float x = (key <= myq) ? sc[mt][i] * c2 : -INFINITY;
                sv[mt * 4 + i] = x;
                tmax = fmaxf(tmax, x);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        const float mnew = fmaxf(mrow, tmax);
        const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(mrow - mnew);
        float psum = 0.f;
        bf16x8 pf;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float pz = (mnew == -INFINITY) ? 0.f : exp2f(sv[i] - mnew);
            psum += pz;
            pf[i] = (__bf16)pz;
        }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        lrow = lrow * alpha + psum;
        mrow = mnew;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            o[dt] *= alpha;
            // A = V^T rows d = 16*dt + col, k-slots: keys 4*grp+i (0-3), 16+4*grp+i (4-7)
            const bf16_t *vr = sVt + (16 * dt + col) * (KT + VPAD);
            const uint2 lo = *reinterpret_cast<const uint2 *>(vr + 4 * grp);
            const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16 + 4 * grp);
            uint4 pk = make_uint4(lo.x, lo.y, hi.x, hi.y);
            const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&pk);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[dt], 0, 0, 0);
        }
    }

    if (myq < T) {
        const int64_t row = ((int64_t)bi * T + myq) * t.Hq + h;
        const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
        float *op = a.out + row * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<float4 *>(op + 16 * dt + 4 * grp) =
                make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
        if (a.lse && grp == 0)
            a.lse[row] = lrow > 0.f ? mrow * 0.6931471805599453f + logf(lrow) : -INFINITY;
    }
}

template <int D>
static hipError_t inblock_d(const PrefillArgs &a, hipStream_t s)
{
    const int G = a.t.G;
    const int nwv = G == 8 ? 8 : 4;
    const int qb = nwv / G;
    dim3 grid((unsigned)((a.T + 16 * qb - 1) / (16 * qb)), (unsigned)a.t.Hkv, (unsigned)a.t.B);
    dim3 block(64 * nwv);
    switch (G) {
    case 1: hipLaunchKernelGGL((k_inblock<D, 1, 4>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_inblock<D, 2, 4>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_inblock<D, 4, 4>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_inblock<D, 8, 8>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_inblock_attention(const PrefillArgs &a, hipStream_t s)
{
    if (a.T <= 0) return hipSuccess;
    return a.t.D == 128 ? inblock_d<128>(a, s) : inblock_d<64>(a, s);
}

// ----------------------------------------------------------------------------
// Top level of the prefix tree, scored for every query of the block at once.
//
// Every query of the block sees the same candidate list at the top (all top
// nodes, node c at RoPE position c) and sits at the same position n_top, so
// the logits are one product per KV group: rows = (query, head) pairs with
// the head's query rotated by n_top, columns = (node, reference key) pairs
// with the key rotated by its node index.  The product runs on fp32 MFMA
// (v_mfma_f32_16x16x4_f32): the rotated operands are not bf16 values, and
// fp32 operands keep the logits, and so the selections, those of fp32
// arithmetic.  Each lane ends with 4 rows x 1 column of logits; the group
// score (mean over the group's heads) and the best reference key per node
// are reduced across lanes with DPP, and the winning lane writes the node's
// group score and per-head logits for the traversal to pick up.
// ----------------------------------------------------------------------------
namespace {
constexpr int kTopRows = 64;    // (query, head) rows per workgroup: 16 per wave

typedef float floatx4_t __attribute__((ext_vector_type(4)));

// (s, j) of the partner lane wins over (best, bj): larger score, then lower j
__device__ __forceinline__ void top_keep(float &best, int &bj, float s2, int j2)
{
    const bool take = (s2 > best) || (s2 == best && j2 < bj);
    best = take ? s2 : best;
    bj = take ? j2 : bj;
}
} // namespace

template <int D, int G>
__global__ __launch_bounds__(256) void k_top_scores(PrefillArgs a)
{
    const TreeArgs &t = a.t;
    const int bi = blockIdx.y / t.Hkv, g = blockIdx.y % t.Hkv;
    const int T = a.T, R = t.R;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int n = (int)t.len[bi];
    for (int l = 1; l <= t.levels; ++l) n /= t.b;
    const int ntop = n, ncol = n * R;
    if (ncol == 0) return;

    __shared__ float kr[kTopCols][D + 4];   // rotated top keys, [column][element]
    const int64_t bh = (int64_t)bi * t.Hkv + g;
    const bf16_t *kb = (const bf16_t *)t.lk[t.levels - 1] + bh * t.ncap[t.levels] * R * D;
    for (int i = tid; i < ncol * (D / 2); i += 256) {
        const int col = i / (D / 2), e = i % (D / 2);
        const int c = col / R;
        const float x0 = bf2f(kb[(int64_t)col * D + e]), x1 = bf2f(kb[(int64_t)col * D + e + D / 2]);
        const float2 cs = t.rope[(int64_t)c * (D / 2) + e];
        kr[col][e] = x0 * cs.x - x1 * cs.y;
        kr[col][e + D / 2] = x0 * cs.y + x1 * cs.x;
    }

    // A operand: lane l holds row l % 16 of the wave's tile at k = l / 16 of
    // every 4-wide k step, i.e. elements d = 4 kk + l / 16 (the rotate-half
    // partner d + D/2 has the same residue, so each lane rotates its own)
    const int kq = lane >> 4;
    const int row = blockIdx.x * kTopRows + wave * 16 + (lane & 15);
    const bool rvalid = row < T * G;
    const int tq = rvalid ? row / G : 0, hq = row % G;
    const bf16_t *qp = (const bf16_t *)a.q + (((int64_t)bi * T + tq) * t.Hq + g * G + hq) * D;
    const float2 *rq = t.rope + (int64_t)ntop * (D / 2);
    float qa[D / 4];
#pragma unroll
    for (int kk = 0; kk < D / 8; ++kk) {
        const int d = 4 * kk + kq;
        const float x0 = bf2f(qp[d]), x1 = bf2f(qp[d + D / 2]);
        const float2 cs = rq[d];
        qa[kk] = rvalid ? x0 * cs.x - x1 * cs.y : 0.f;
        qa[kk + D / 8] = rvalid ? x0 * cs.y + x1 * cs.x : 0.f;
    }
    __syncthreads();

    // the rows a lane's accumulators hold: 4 * (lane / 16) + r of the tile
    const int rbase = blockIdx.x * kTopRows + wave * 16 + 4 * kq;
    for (int c0 = 0; c0 < ncol; c0 += 16) {
        const int col = c0 + (lane & 15);
        const bool cvalid = col < ncol;
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 4; ++kk) {
            const float bv = cvalid ? kr[col][4 * kk + kq] : 0.f;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[kk], bv, acc, 0, 0, 0);
        }
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = acc[r] * t.scale;
        const int j = col % R, c = col / R;
        // queries held by this lane: G <= 4 -> 4 / G of them (rows grouped by
        // G); G == 8 -> one query spread over this lane and lane ^ 16
        constexpr int NQL = G <= 4 ? 4 / G : 1;
#pragma unroll
        for (int u = 0; u < NQL; ++u) {
            float sgrp = 0.f;
            if (G <= 4) {
#pragma unroll
                for (int h = 0; h < (G <= 4 ? G : 1); ++h) sgrp += z[u * G + h];
            } else {
                const float own = (z[0] + z[1]) + (z[2] + z[3]);
                const float oth = __shfl_xor(own, 16);
                sgrp = (kq & 1) ? oth + own : own + oth;
            }
            sgrp = sgrp / (float)G;
            float best = cvalid ? sgrp : -INFINITY;
            int bj = j;
            if (R >= 2) top_keep(best, bj, dppf<0xB1>(best), dppi<0xB1>(bj));
            if (R >= 4) top_keep(best, bj, dppf<0x4E>(best), dppi<0x4E>(bj));
            if (R >= 8) top_keep(best, bj, dppf<0x141>(best), dppi<0x141>(bj));
            const int r0 = rbase + u * (G <= 4 ? G : 4);     // first row of this query
            const bool writer = cvalid && j == bj && r0 < T * G && (G <= 4 || (kq & 1) == 0);
            if (writer) {
                const int tt = r0 / G;
                a.top_s[(((int64_t)bi * T + tt) * t.Hkv + g) * a.ntop_stride + c] = best;
                if (G <= 4) {
#pragma unroll
                    for (int h = 0; h < (G <= 4 ? G : 1); ++h)
                        a.top_z[(((int64_t)bi * T + tt) * t.Hq + g * G + h) * a.ntop_stride + c] = z[u * G + h];
                }
            }
            if (G == 8 && cvalid && j == bj && r0 - 4 * (kq & 1) < T * G) {
                // each half of the lane pair writes its own four heads
                const int tt = (r0 - 4 * (kq & 1)) / G;
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    a.top_z[(((int64_t)bi * T + tt) * t.Hq + g * G + 4 * (kq & 1) + h) * a.ntop_stride + c] =
                        z[h];
            }
        }
    }
}

template <int D>
static hipError_t top_d(const PrefillArgs &a, hipStream_t s)
{
    const int G = a.t.G;
    dim3 grid((unsigned)((a.T * G + kTopRows - 1) / kTopRows), (unsigned)(a.t.B * a.t.Hkv)), block(256);
    switch (G) {
    case 1: hipLaunchKernelGGL((k_top_scores<D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_top_scores<D, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_top_scores<D, 4>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_top_scores<D, 8>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_top_scores(const PrefillArgs &a, hipStream_t s)
{
    if (a.T <= 0 || a.t.levels < 1) return hipSuccess;
    return a.t.D == 128 ? top_d<128>(a, s) : top_d<64>(a, s);
}

} // namespace hti
