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
#include <algorithm>

#include "hti_device.h"
#include "hti_internal.h"

namespace hti {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float floatx4;

// ----------------------------------------------------------------------------
// Rotate the block's keys by their block-local index and store them as bf16
// in head-major layout: kr [B, Hkv, Tp, D] (rows T .. Tp-1 zero).  A thread
// rotates 8 consecutive pairs (j, j + D/2).  (The queries are rotated by the
// in-block kernel itself when it loads them.)
// ----------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_rotate_block(PrefillArgs a)
{
    const TreeArgs &t = a.t;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)t.B * a.Tp * t.Hkv * (D / 16);
    if (idx >= total) return;
    const int j = 8 * (int)(idx % (D / 16));
    int64_t r = idx / (D / 16);
    const int h = (int)(r % t.Hkv);
    r /= t.Hkv;
    const int tt = (int)(r % a.Tp);
    const int bi = (int)(r / a.Tp);
    bf16_t *dst = (bf16_t *)a.kr + (((int64_t)bi * t.Hkv + h) * a.Tp + tt) * D;
    if (tt >= a.T) {
        *reinterpret_cast<uint4 *>(dst + j) = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(dst + j + D / 2) = make_uint4(0, 0, 0, 0);
        return;
    }
    const T *src = (const T *)a.k + (((int64_t)bi * a.T + tt) * t.Hkv + h) * D;
    float x0[8], x1[8];
    load_vec<T, 8>(src + j, x0);
    load_vec<T, 8>(src + j + D / 2, x1);
    const float4 *cs4 = reinterpret_cast<const float4 *>(t.rope + (int64_t)tt * (D / 2) + j);
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float4 cs = cs4[e];      // (cos, sin) of pairs j + 2e, j + 2e + 1
        const float a0 = x0[2 * e] * cs.x - x1[2 * e] * cs.y;
        const float b0 = x0[2 * e] * cs.y + x1[2 * e] * cs.x;
        const float a1 = x0[2 * e + 1] * cs.z - x1[2 * e + 1] * cs.w;
        const float b1 = x0[2 * e + 1] * cs.w + x1[2 * e + 1] * cs.z;
        lo[e] = (uint32_t)f2bf(a0) | ((uint32_t)f2bf(a1) << 16);
        hi[e] = (uint32_t)f2bf(b0) | ((uint32_t)f2bf(b1) << 16);
    }
    *reinterpret_cast<uint4 *>(dst + j) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint4 *>(dst + j + D / 2) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
}

// n 32-bit words at p set to v (grid-stride).
__global__ __launch_bounds__(256) void k_fill_u32(uint32_t *p, uint32_t v, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill_u32(void *p, uint32_t v, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int blocks = (int)std::min<int64_t>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, s, (uint32_t *)p, v, n);
    return hipGetLastError();
}

hipError_t launch_rotate_block(const PrefillArgs &a, hipStream_t s)
{
    const int64_t total = (int64_t)a.t.B * a.Tp * a.t.Hkv * (a.t.D / 16);
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
// V of the block transposed per KV head for the P V product: vt [B, Hkv, D,
// Tp] bf16 with Tp = T rounded up to the key tile; keys past T are zero.
// Within each aligned group of 32 keys the columns are permuted: column
// 8*j + 4*m + i holds key 16*m + 4*j + i (j, i in 0..3, m in 0..1), the key
// that the S^T product leaves in quarter-wave j of the 16-key tile m.
// ----------------------------------------------------------------------------
namespace {
constexpr int IKT = kInblockKeys;   // keys per tile of the in-block product
}

template <int D>
__global__ __launch_bounds__(256) void k_transpose_v(PrefillArgs a)
{
    constexpr int W = D / 2 + 1;                 // padded row of 32-bit words
    __shared__ uint32_t tw[IKT * W];
    const TreeArgs &t = a.t;
    const int kt0 = blockIdx.x * IKT, g = blockIdx.y, bi = blockIdx.z;
    for (int c = threadIdx.x; c < IKT * D / 8; c += 256) {
        const int key = c / (D / 8), ch = c % (D / 8);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (kt0 + key < a.T)
            v = *reinterpret_cast<const uint4 *>(
                (const bf16_t *)a.v + (((int64_t)bi * a.T + kt0 + key) * t.Hkv + g) * D + 8 * ch);
        uint32_t *r = tw + key * W + 4 * ch;
        r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
    }
    __syncthreads();
    bf16_t *dst = (bf16_t *)a.vt + ((int64_t)bi * t.Hkv + g) * D * (int64_t)a.Tp + kt0;
    for (int c = threadIdx.x; c < D * (IKT / 8); c += 256) {
        const int d = c / (IKT / 8), k8 = c % (IKT / 8);
        // columns 8*k8 .. 8*k8+7: group k8/4, quarter j = k8%4, then (m, i)
        const int kbase = 32 * (k8 >> 2) + 4 * (k8 & 3);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key0 = kbase + 16 * (e >> 1) + 2 * (e & 1);   // columns 2e, 2e+1
            const uint32_t lo = tw[key0 * W + d / 2] >> (16 * (d & 1));
            const uint32_t hi = tw[(key0 + 1) * W + d / 2] >> (16 * (d & 1));
            w[e] = (lo & 0xffffu) | (hi << 16);
        }
        *reinterpret_cast<uint4 *>(dst + (int64_t)d * a.Tp + 8 * k8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// ----------------------------------------------------------------------------
// In-block causal attention (flash style) merged with the prefix partials.
//
// Work split: a workgroup owns QW*NW/G consecutive queries of every head of
// one KV group; wave w handles head g*G + (w % G) and the QW = 16*QT queries
// of query block w / G.  Keys advance in tiles of IKT = 64; the K tile
// (row-major) and the V^T tile are copied from global memory straight into
// LDS (global_load_lds, 16 bytes per lane, no registers), double-buffered so
// that the next tile is in flight while the current one is multiplied, with
// one barrier per tile.  LDS rows carry two 16-byte pad chunks (the copy
// lanes that map onto a pad chunk are masked off), which keeps the fragment
// reads free of bank conflicts and lets every fragment read use one base
// address plus an immediate offset.
//
// Scores are computed transposed, S^T = K Q^T, so a lane's accumulator column
// is one query: the running max needs two cross-lane steps per tile, the
// running denominator stays per lane until the end, and the probabilities
// already sit in the B-operand layout of O^T += V^T P^T (the V^T columns are
// permuted to match when V is transposed).  Workgroups are numbered so that
// one KV group's workgroups share an XCD (and its L2), and the query blocks
// with the most key tiles start first.
// ----------------------------------------------------------------------------
namespace {
typedef const __attribute__((address_space(1))) void *gvoid_t;
typedef __attribute__((address_space(3))) void *lvoid_t;
constexpr float kLazy = 8.f;    // slack of the exponent reference (log2 units)
}

template <int D, int G, int NW, int QT, int NB>
__global__ __launch_bounds__(NW * 64, QT >= 4 ? 1 : (8 / NW > 0 ? 8 / NW : 1)) void k_inblock(PrefillArgs a)
{
    constexpr int QW = 16 * QT;                  // queries per wave
    static_assert(NW >= G && NW % G == 0, "a workgroup holds whole KV groups");
    constexpr int QBW = NW / G;                  // query blocks per workgroup
    constexpr int KS = D / 32;                   // k-steps of the QK^T product
    constexpr int DT = D / 16;                   // d-tiles of the PV product
    // LDS rows carry 32 bytes of padding: measured on gfx950, 16-byte reads
    // of 16 rows (one per lane of a quarter-wave) at a stride of 256+16 or
    // 128+16 bytes stall about 4 cycles on bank conflicts, at 256+32 and
    // 128+32 bytes none
    constexpr int KPADC = 2, VPADC = 2;          // pad chunks per row
    constexpr int KCH = D / 8 + KPADC;           // chunks of a K row in LDS (incl. pad)
    constexpr int VCH = IKT / 8 + VPADC;         // chunks of a V^T row in LDS
    constexpr int KRS = 16 * KCH, VRS = 16 * VCH;
    constexpr int KCHUNKS = IKT * KCH, CHUNKS = KCHUNKS + D * VCH;
    constexpr int BUF = 16 * CHUNKS;
    constexpr int NSEG = (CHUNKS + 63) / 64;     // 1 KB wave copies per tile
    constexpr int SPW = (NSEG + NW - 1) / NW;
    static_assert(NB == 2 || NB == 3, "two or three tile buffers");
    __shared__ __attribute__((aligned(1024))) char sb0[NSEG * 1024];
    __shared__ __attribute__((aligned(1024))) char sb1[NSEG * 1024];
    __shared__ __attribute__((aligned(1024))) char sb2[NB == 3 ? NSEG * 1024 : 16];

    const TreeArgs &t = a.t;
    const int T = a.T, Tp = a.Tp;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nblk = (T + QW * QBW - 1) / (QW * QBW);
    int lin = blockIdx.x;
    const int g = lin % t.Hkv;
    lin /= t.Hkv;
    const int bi = lin % t.B;
    if (lin / t.B >= nblk) return;               // past the last query block (whole workgroup)
    const int q0blk = (nblk - 1 - lin / t.B) * (QW * QBW);
    const int h = g * G + (wave % G);
    const int q0 = q0blk + QW * (wave / G);      // this wave's first query
    const int col = lane & 15, grp = lane >> 4;
    const float c2 = t.scale * 1.4426950408889634f;   // scale * log2(e)

    // Q fragments (B operand of S^T = K Q^T): column = query, k-slots 8*grp..
    // of step s.  Each query is rotated by its block-local index here: the
    // first-half steps hold x_i c - x_{i+D/2} s, the second-half steps
    // x_i s + x_{i+D/2} c (i = 32*s + 8*grp + e), rounded to bf16.
    bf16x8 qf[QT][KS];
    {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int qq = min(q0 + 16 * qt + col, T - 1);
            const bf16_t *qrow = (const bf16_t *)a.q + (((int64_t)bi * T + qq) * t.Hq + h) * D;
#pragma unroll
            for (int s = 0; s < KS / 2; ++s) {
                const int i0 = 32 * s + 8 * grp;
                float x0[8], x1[8];
                load_vec<bf16_t, 8>(qrow + i0, x0);
                load_vec<bf16_t, 8>(qrow + i0 + D / 2, x1);
                const float4 *cs4 = reinterpret_cast<const float4 *>(t.rope + (int64_t)qq * (D / 2) + i0);
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float4 cs = cs4[e];
                    const float a0 = x0[2 * e] * cs.x - x1[2 * e] * cs.y;
                    const float b0 = x0[2 * e] * cs.y + x1[2 * e] * cs.x;
                    const float a1 = x0[2 * e + 1] * cs.z - x1[2 * e + 1] * cs.w;
                    const float b1 = x0[2 * e + 1] * cs.w + x1[2 * e + 1] * cs.z;
                    lo[e] = (uint32_t)f2bf(a0) | ((uint32_t)f2bf(a1) << 16);
                    hi[e] = (uint32_t)f2bf(b0) | ((uint32_t)f2bf(b1) << 16);
                }
                qf[qt][s] = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
                qf[qt][s + KS / 2] = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
            }
        }
    }

    // seed the online softmax with the prefix partial state of each query;
    // every element of lacc[qt] holds the query's running denominator
    floatx4 o[QT][DT], lacc[QT];
    float mrow[QT];
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int myq = q0 + 16 * qt + col;
        mrow[qt] = -INFINITY;
        lacc[qt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[qt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        // (no partial states: a tree set without prefix capacity, nothing
        // before the block)
        if (myq < T && a.part_ml != nullptr) {
            const int64_t row = ((int64_t)bi * T + myq) * t.Hq + h;
            const float M = a.part_ml[row * 2 + 0];
            const float L = a.part_ml[row * 2 + 1];
            lacc[qt] = floatx4{L, L, L, L};
            mrow[qt] = (M == -INFINITY) ? -INFINITY : M * 1.4426950408889634f;
            const float *pa = a.part_acc + row * D;
            // (a prefix with nothing to attend leaves no output row)
            if (M != -INFINITY)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const float4 v = *reinterpret_cast<const float4 *>(pa + 16 * dt + 4 * grp);
                o[qt][dt] = floatx4{v.x, v.y, v.z, v.w};
            }
        }
    }

    const int kend = min(T, q0blk + QW * QBW);
    const int ntiles = (kend + IKT - 1) / IKT;
    const bf16_t *kb = (const bf16_t *)a.kr + (((int64_t)bi * t.Hkv + g) * Tp) * D;
    const bf16_t *vtb = (const bf16_t *)a.vt + ((int64_t)bi * t.Hkv + g) * D * (int64_t)Tp;

    // copy key tile j into buf: LDS chunk c is written by lane c % 64 of the
    // copy of segment c / 64; chunks below KCHUNKS are K rows (key, D/8
    // chunks + pad), the rest V^T rows (d, IKT/8 chunks + pad).  The source
    // offsets relative to the tile are fixed per lane; pad chunks copy nothing.
    constexpr int KSEG = KCHUNKS / 64;
    static_assert(KCHUNKS % 64 == 0, "K rows end on a segment boundary");
    // (element offset, or -1 where the lane copies nothing)
    int off[SPW];
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
        const int seg = wave + NW * u;
        const int ci = seg * 64 + lane;
        if (seg < KSEG) {
            const int r = ci / KCH, p = ci % KCH;
            off[u] = p < D / 8 ? r * D + 8 * p : -1;
        } else {
            const int r = (ci - KCHUNKS) / VCH, p = (ci - KCHUNKS) % VCH;
            off[u] = (p < IKT / 8 && r < D) ? r * Tp + 8 * p : -1;
        }
    }
    // parts: 1 = the K rows, 2 = the V^T rows, 3 = both
    auto issue_parts = [&](int j, char *buf, int parts) __attribute__((always_inline)) {
        const int kt0 = j * IKT;
        const bf16_t *kt = kb + (int64_t)kt0 * D, *vt = vtb + kt0;
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            const int seg = wave + NW * u;
            if (seg >= NSEG) break;
            if (off[u] >= 0 && (parts & (seg < KSEG ? 1 : 2)))
                __builtin_amdgcn_global_load_lds((gvoid_t)((seg < KSEG ? kt : vt) + off[u]),
                                                 (lvoid_t)(buf + seg * 1024), 16, 0, 0);
        }
    };
    auto issue = [&](int j, char *buf) __attribute__((always_inline)) { issue_parts(j, buf, 3); };

    const int kbase = col * KRS + 16 * grp;                 // K row col, chunk grp
    const int vbase = KCHUNKS * 16 + col * VRS + 16 * grp;  // V^T row col, chunk grp

    // One key tile of the product in four parts: scores (S^T MFMAs), prep
    // (causal mask and the running max), expo (probabilities) and pv (O^T
    // and the row sums).  diag: some key of the tile follows some query of
    // the wave, so the causal mask applies.
    //
    // S^T: 16-key tile tm holds keys kt0 + 16*tm + 4*grp + i in lane
    // (col = query, grp), element i.  A query tile wholly before the tile's
    // keys is multiplied anyway: the mask leaves it zero weights.
    auto scores = [&](const char *buf, floatx4 (&sc)[QT][4], int q_lo, int q_hi) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                const bf16x8 af = *reinterpret_cast<const bf16x8 *>(buf + kbase + 16 * tm * KRS + 64 * s);
#pragma unroll
                for (int qt = q_lo; qt < q_hi; ++qt)
                    sc[qt][tm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af, qf[qt][s], s == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : sc[qt][tm], 0, 0, 0);
            }
    };
    // online softmax per query tile, in log2 units (c2 = scale*log2 e).  The
    // exponent reference mrow is the query's running max, raised only when a
    // score exceeds it by more than kLazy: probabilities stay below 2^kLazy
    // and the rescale of the accumulators is rare.
    auto prep = [&](int kt0, floatx4 (&sc)[QT][4], bool diag, int q_lo, int q_hi) __attribute__((always_inline)) {
        if (diag) {
            // (the empty asm keeps this a branch: as selects, the compares
            // would run on every tile)
            asm volatile("");
#pragma unroll
            for (int qt = q_lo; qt < q_hi; ++qt)
#pragma unroll
                for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (kt0 + 16 * tm + 4 * grp + i > q0 + 16 * qt + col) sc[qt][tm][i] = -INFINITY;
        }
#pragma unroll
        for (int qt = q_lo; qt < q_hi; ++qt) {
            float lmax = -INFINITY;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, sc[qt][tm][i]);
            lmax *= c2;
            if (__builtin_amdgcn_ballot_w64(lmax > mrow[qt] + kLazy)) {
                const float tmax = xmax32(xmax16(lmax));
                const float mnew = fmaxf(mrow[qt], tmax);
                const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrow[qt] - mnew);
                lacc[qt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[qt][dt] *= alpha;
                mrow[qt] = mnew;
            }
        }
    };
    // P of 32-key step kg goes to slots 4*m + i of pf[kg] (tm = 2*kg + m)
    auto expo = [&](const floatx4 (&sc)[QT][4], bf16x8 (&pf)[QT][2], int q_lo, int q_hi)
        __attribute__((always_inline)) {
#pragma unroll
        for (int qt = q_lo; qt < q_hi; ++qt) {
            const float nmu = (mrow[qt] == -INFINITY) ? 0.f : -mrow[qt];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pf[qt][tm >> 1][4 * (tm & 1) + i] =
                        (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[qt][tm][i], c2, nmu));
        }
    };
    // O^T += V^T P^T; V^T row d = 16*dt + col, k-slots 8*grp.. of step kg.
    // The row sums of P come from the same product with a ones operand.
    auto pv = [&](const char *buf, const bf16x8 (&pf)[QT][2], int q_lo, int q_hi) __attribute__((always_inline)) {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
#pragma unroll
            for (int qt = q_lo; qt < q_hi; ++qt)
                lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qt][kg], lacc[qt], 0, 0, 0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(buf + vbase + 16 * dt * VRS + 64 * kg);
#pragma unroll
                for (int qt = q_lo; qt < q_hi; ++qt)
                    o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qt][kg], o[qt][dt], 0, 0, 0);
            }
        }
    };
    auto tile = [&](int kt0, const char *buf, bool diag) __attribute__((always_inline)) {
        floatx4 sc[QT][4];
        bf16x8 pf[QT][2];
        scores(buf, sc, 0, QT);
        prep(kt0, sc, diag, 0, QT);
        expo(sc, pf, 0, QT);
        pv(buf, pf, 0, QT);
    };
    auto compute = [&](int j, const char *buf) __attribute__((always_inline)) {
        const int kt0 = j * IKT;
        if (kt0 > q0 + QW - 1) return;           // tile entirely in this wave's future
        tile(kt0, buf, kt0 + IKT - 1 > q0);
    };
    static_assert(BUF <= NSEG * 1024, "tile fits its buffer");

    if constexpr (NB == 2) {
        // copies run one tile ahead of the product
        if (ntiles > 0) issue(0, sb0);
        for (int j = 0; j < ntiles; j += 2) {
            __builtin_amdgcn_s_waitcnt(0);       // this wave's copies of tile j landed
            __syncthreads();                     // everyone's did; tile j-1 is consumed
            if (j + 1 < ntiles) issue(j + 1, sb1);
            compute(j, sb0);
            if (j + 1 < ntiles) {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (j + 2 < ntiles) issue(j + 2, sb0);
                compute(j + 1, sb1);
            }
        }
    } else {
        // copies run two tiles ahead: at the wait for tile j only the copies
        // of tile j+1 (issued after those of j; vector memory counts retire
        // in order) may still be in flight -- at least NSEG/NW of them
        constexpr int VM = NSEG / NW;
        static_assert(VM < 64, "vmcnt field");
        constexpr int kWaitNext = (VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14);
        // A plain s_barrier: __syncthreads() adds a workgroup release fence,
        // which would wait for every copy in flight (LDS writes), tile j+1's
        // included.  The explicit count wait orders this wave's copies; the
        // fragment reads of tile j-1 were consumed before the barrier, and
        // the empty asm keeps the compiler from moving LDS accesses across it.
        auto wait_tile = [&](int j) __attribute__((always_inline)) {
            if (j + 1 < ntiles) __builtin_amdgcn_s_waitcnt(kWaitNext);
            else __builtin_amdgcn_s_waitcnt(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();       // everyone's copies landed; tile j-1 is consumed
            asm volatile("" ::: "memory");
        };
        if (ntiles > 0) issue(0, sb0);
        if (ntiles > 1) issue(1, sb1);
        for (int j = 0; j < ntiles; j += 3) {
            wait_tile(j);
            if (j + 2 < ntiles) issue(j + 2, sb2);
            compute(j, sb0);
            if (j + 1 >= ntiles) break;
            wait_tile(j + 1);
            if (j + 3 < ntiles) issue(j + 3, sb0);
            compute(j + 1, sb1);
            if (j + 2 >= ntiles) break;
            wait_tile(j + 2);
            if (j + 4 < ntiles) issue(j + 4, sb1);
            compute(j + 2, sb2);
        }
    }

#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const float l = lacc[qt][0];
        const int myq = q0 + 16 * qt + col;
        if (myq < T) {
            const int64_t row = ((int64_t)bi * T + myq) * t.Hq + h;
            const float inv = l > 0.f ? 1.f / l : 0.f;
            float *op = a.out + row * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *reinterpret_cast<float4 *>(op + 16 * dt + 4 * grp) =
                    make_float4(o[qt][dt][0] * inv, o[qt][dt][1] * inv, o[qt][dt][2] * inv, o[qt][dt][3] * inv);
            if (a.lse && grp == 0)
                a.lse[row] = l > 0.f ? mrow[qt] * 0.6931471805599453f + logf(l) : -INFINITY;
        }
    }
}

// One wave per (head, 16*QT-query block); NW/G query blocks per workgroup.
// The grid is derived from the same constants as the kernel's own split.
template <int D, int G, int NW, int QT, int NB>
static hipError_t inblock_launch(const PrefillArgs &a, hipStream_t s)
{
    static_assert(NW >= G && NW % G == 0, "a workgroup holds whole KV groups");
    constexpr int q = 16 * QT * (NW / G);        // queries per workgroup
    const int64_t nblk = ((int64_t)a.T + q - 1) / q;
    hipLaunchKernelGGL((k_inblock<D, G, NW, QT, NB>), dim3((unsigned)(nblk * a.t.Hkv * a.t.B)),
                       dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t inblock_d(const PrefillArgs &a, hipStream_t s)
{
    dim3 tgrid((unsigned)(a.Tp / IKT), (unsigned)a.t.Hkv, (unsigned)a.t.B);
    hipLaunchKernelGGL((k_transpose_v<D>), tgrid, dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
#ifndef HTI_IB_QT
#define HTI_IB_QT 2
#endif
    constexpr int QT = HTI_IB_QT;
#ifndef HTI_IB_NW
#define HTI_IB_NW 4
#define HTI_IB_NB 2
#endif
    constexpr int NW = HTI_IB_NW, NB = HTI_IB_NB;
    switch (a.t.G) {
    case 1: return inblock_launch<D, 1, NW, QT, NB>(a, s);
    case 2: return inblock_launch<D, 2, NW, QT, NB>(a, s);
    case 4: return inblock_launch<D, 4, NW, QT, NB>(a, s);
    default: return inblock_launch<D, 8, (NW > 8 ? NW : 8), QT, NB>(a, s);
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
    for (int l = 1; l <= t.levels; ++l) n /= fan_in(t, l);
    const int ntop = n, ncol = n * R;
    if (ncol == 0) return;

    // rotated top keys, [column][element]; the row pitch D + 1 puts the 64
    // (column, k group) reads of one MFMA step in distinct banks
    __shared__ float kr[kTopCols][D + 1];
    const int64_t bh = (int64_t)bi * (t.Hkv / t.hdiv) + g / t.hdiv;   // tree slot of routing head g
    const bf16_t *kb = (const bf16_t *)t.lk[t.levels - 1] + bh * t.ncap[t.levels] * R * D;
    // (8-bit router keys: E4M3 codes times the row scale)
    const uint8_t *k8 = t.rfp8 ? t.lkq[t.levels - 1] + bh * t.ncap[t.levels] * R * D : nullptr;
    const float *s8 = t.rfp8 ? t.lks[t.levels - 1] + bh * t.ncap[t.levels] * R : nullptr;
    for (int i = tid; i < ncol * (D / 2); i += 256) {
        const int col = i / (D / 2), e = i % (D / 2);
        const int c = col / R;
        float x0, x1;
        if (t.rfp8) {
            const float sc = s8[col];
            x0 = __builtin_amdgcn_cvt_f32_fp8((int)k8[(int64_t)col * D + e], 0) * sc;
            x1 = __builtin_amdgcn_cvt_f32_fp8((int)k8[(int64_t)col * D + e + D / 2], 0) * sc;
        } else {
            x0 = bf2f(kb[(int64_t)col * D + e]);
            x1 = bf2f(kb[(int64_t)col * D + e + D / 2]);
        }
        const float2 cs = t.rope[(int64_t)c * (D / 2) + e];
        kr[col][e] = x0 * cs.x - x1 * cs.y;
        kr[col][e + D / 2] = x0 * cs.y + x1 * cs.x;
    }

    // A operand: lane l holds row l % 16 of the wave's tile at k = l / 16 of
    // every 4-wide k step.  Step kk < D/8 takes element d = (l / 16) * D/8 +
    // kk of the first half, step kk + D/8 its rotate-half partner d + D/2, so
    // each lane reads two contiguous runs of D/8 elements and rotates its own
    // pairs.
    constexpr int RUN = D / 8;
    const int kq = lane >> 4;
    const int row = blockIdx.x * kTopRows + wave * 16 + (lane & 15);
    const bool rvalid = row < T * G;
    const int tq = rvalid ? row / G : 0, hq = row % G;
    const bf16_t *qp = (const bf16_t *)a.q + (((int64_t)bi * T + tq) * t.Hq + g * G + hq) * D + kq * RUN;
    const float2 *rq = t.rope + (int64_t)ntop * (D / 2) + kq * RUN;
    float qa[D / 4];
#pragma unroll
    for (int w8 = 0; w8 < RUN / 8; ++w8) {
        const uint4 v0 = *reinterpret_cast<const uint4 *>(qp + 8 * w8);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(qp + D / 2 + 8 * w8);
        const uint32_t lo[4] = {v0.x, v0.y, v0.z, v0.w}, hi[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kk = 8 * w8 + i;
            const float x0 = bf2f((i & 1) ? lo[i >> 1] >> 16 : lo[i >> 1] & 0xffffu);
            const float x1 = bf2f((i & 1) ? hi[i >> 1] >> 16 : hi[i >> 1] & 0xffffu);
            const float2 cs = rq[kk];
            qa[kk] = rvalid ? x0 * cs.x - x1 * cs.y : 0.f;
            qa[kk + RUN] = rvalid ? x0 * cs.y + x1 * cs.x : 0.f;
        }
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
            const float bv = cvalid ? kr[col][(kk < RUN ? 0 : D / 2) + kq * RUN + kk % RUN] : 0.f;
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
                sgrp = xsum16(own);   // the same sum, in the same order, in both lanes
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
