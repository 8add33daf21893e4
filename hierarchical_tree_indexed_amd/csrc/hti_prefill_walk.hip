// hti_prefill_walk.hip -- tree traversal of a prefill block, one wave per
// (query, KV group) unit.
//
// The method ("Recursive Sparse Attention", abstract; "Subquadratic Attention
// with a Hierarchical Tree-Structured Indexer", Figure 3 caption) is the one
// the decode kernels run: per level, score the candidates (children of the
// kept nodes of the level above, then the level's orphans; candidate i at
// RoPE position i, the query at |C|), keep the top-k or top-p set, and let
// every other candidate join the query's softmax with its pooled key and mean
// value; at the token level every candidate joins it.  For a prefill block
// the query of block row t sits after all prefix candidates of the token
// level, at position |C_0| + t.
//
// A block has tens of thousands of units, so this kernel is built for
// throughput: each wave walks its own unit with wave-level operations only
// (no workgroup barriers), every gather is issued in branch-free batches (row
// ids derived once per lane and handed out by DPP row broadcasts), the
// selection runs in registers with DPP reductions, and the per-wave LDS is
// sized per launch so that many units share a compute unit and hide each
// other's memory latency.  It leaves the unit's partial softmax state
// (unnormalised output, running max, denominator) for the in-block kernel.
#include <algorithm>
#include <type_traits>

#include "hti_device.h"
#include "hti_internal.h"
#include "hti_trav_common.h"

namespace hti {

namespace {

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Buffer resource over `base` (raw, unswizzled; reads past `bytes` return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename R> __device__ __forceinline__ R bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <> __device__ __forceinline__ uint16_t bload<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)v, (int)s, 0);
}
template <> __device__ __forceinline__ uint32_t bload<uint32_t>(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)v, (int)s, 0);
}
template <> __device__ __forceinline__ uint2 bload<uint2>(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s)
{
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)v, (int)s, 0);
    return make_uint2(x[0], x[1]);
}
template <> __device__ __forceinline__ uint4 bload<uint4>(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s)
{
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)v, (int)s, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// acc + a.lo * b.lo + a.hi * b.hi over bf16 pairs, fp32 accumulation
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                           false);
}

} // namespace

// Per-wave LDS (4-byte words): qraw [G*D], probability pairs [MC/2 * G],
// s [MC + 64] (the last 64 words take discarded stores), z [MC * G],
// kept-node lists [2][kMaxSel]
__host__ __device__ constexpr size_t pw_wave_words(int G, int D, int MC)
{
    return (size_t)G * D + (size_t)(MC / 2) * G + MC + 64 + (size_t)MC * G + 2 * kMaxSel;
}

template <int D, int G, int MJ, bool F8>
__global__ __launch_bounds__(256, 3) void k_prefill_walk(TravArgs a, int MC)
{
    using T = bf16_t;
    constexpr int PPL = D / 32;           // rotate-half pairs per lane (16-lane row per key)
    using KR = typename Raw<T, PPL>::type;
    constexpr int KB = 8;                 // key items per quarter per batch (>= HTI_MAX_R)
    static_assert(KB >= HTI_MAX_R, "a batch holds one candidate's reference keys");
    constexpr int DPL = D / 64;           // value elements per lane (the wave holds one row)
    using VR = typename Raw<T, DPL>::type;
    constexpr int VB = 16;                // value rows per batch (even: rows go in pairs)
    constexpr int LPH = 16 / G;           // lanes per head after row_sums
    constexpr int RB = D / 2 * 8;         // bytes per RoPE table row
    static_assert(MJ <= 32, "kept bits fit one word");
    extern __shared__ __attribute__((aligned(16))) unsigned char pw_lds[];

    const TreeArgs &t = a.t;
    // the wave index is uniform in the wave: say so, so that everything the
    // unit derives from it lives in scalar registers
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane & 15, quarter = lane >> 4;
    const int64_t unit = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    const int64_t units = (int64_t)t.B * a.Nq * t.Hkv;
    if (unit >= units) return;
    // consecutive waves take consecutive queries of one KV group
    const int64_t bg = unit / a.Nq;
    const int qi = (int)(unit % a.Nq);
    const int g = (int)(bg % t.Hkv);
    const int bi = (int)(bg / t.Hkv);
    const int64_t uidx = ((int64_t)bi * a.Nq + qi) * t.Hkv + g;   // unit index of the outputs
    const int64_t bh = (int64_t)bi * (t.Hkv / t.hdiv) + g / t.hdiv;   // tree slot of routing head g
    const int b = t.b, levels = t.levels, R = t.R;
    const int keff = (a.mode == HTI_TOPK) ? a.k : a.cap;

    float *lds = reinterpret_cast<float *>(pw_lds) + (size_t)wave * pw_wave_words(G, D, MC);
    float *qraw = lds;
    uint32_t *sP = reinterpret_cast<uint32_t *>(qraw + G * D);
    float *sS = reinterpret_cast<float *>(sP + (size_t)(MC / 2) * G);
    float *sZ = sS + MC + 64;
    int *selbuf = reinterpret_cast<int *>(sZ + (size_t)MC * G);

    // node counts of the prefix tree
    int nlev[HTI_MAX_LEVELS + 1];
    {
        int n = (int)t.len[bi];
        nlev[0] = n;
#pragma unroll
        for (int l = 1; l <= HTI_MAX_LEVELS; ++l) {
            n = (l <= levels) ? n / (l == 1 ? b : t.fan) : 0;
            nlev[l] = n;
        }
    }
    const int L = nlev[0];
    // query of the unit (un-rotated) into LDS, 8 elements per lane and load;
    // an empty prefix never reads it
    if (L > 0) {
        const T *qp = (const T *)a.q + (((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G) * D;
        for (int i = lane * 8; i < G * D; i += 64 * 8) {
            const uint4 v = *reinterpret_cast<const uint4 *>(qp + i);
            *reinterpret_cast<float4 *>(qraw + i) =
                make_float4(bf2f(v.x & 0xffffu), bf2f(v.x >> 16), bf2f(v.y & 0xffffu), bf2f(v.y >> 16));
            *reinterpret_cast<float4 *>(qraw + i + 4) =
                make_float4(bf2f(v.z & 0xffffu), bf2f(v.z >> 16), bf2f(v.w & 0xffffu), bf2f(v.w >> 16));
        }
    }
    float M[G], lt[G], acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        M[h] = -INFINITY;
        lt[h] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
    }
    // RoPE table as a buffer: rows past its end read as zeros
    const __amdgpu_buffer_rsrc_t rope_rs =
        rsrc(t.rope, (uint32_t)std::min<int64_t>((int64_t)t.rope_npos * RB, 0xffffffffll));
    wave_sync();

    // ---- logits of candidates c0 .. c0 + m - 1 of a list (RoPE positions
    // c0 + i; keys at kb + (id * nref + j) * D; the query at qpos) into sZ,
    // and their group scores into sS when WGS, both indexed from 0.  Quarter
    // q scores a contiguous run of the list, KB key items per batch; the
    // query is turned to its position and scaled by 1/sqrt(d) once, every key
    // is turned to its candidate's position, and one transposed butterfly
    // sums the G heads' partial dot products, leaving head sub / LPH in lane
    // sub.
    auto score = [&](auto wgs, auto f8, const Cands &cs, const void *kb, const float *ks, int nref, int c0, int m,
                     int qpos) __attribute__((always_inline)) {
        constexpr bool WGS = decltype(wgs)::value;
        // E4M3 router keys (one byte per element) with a scale per key row
        constexpr bool Q8 = decltype(f8)::value;
        using KL = std::conditional_t<Q8, typename Raw8<PPL>::type, KR>;
        constexpr uint32_t ES = Q8 ? 1 : 2;              // bytes per key element
        constexpr int RSH = D == 128 ? 5 : 4;            // key row bytes -> scale bytes (E4M3 rows)
        float qa[G][PPL], qb[G][PPL];
        {
            const float2 *rq = t.rope + (int64_t)qpos * (D / 2) + sub * PPL;
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                const float2 cq = rq[e];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float x0 = qraw[h * D + sub * PPL + e], x1 = qraw[h * D + D / 2 + sub * PPL + e];
                    qa[h][e] = (x0 * cq.x - x1 * cq.y) * t.scale;
                    qb[h][e] = (x0 * cq.y + x1 * cq.x) * t.scale;
                }
            }
        }
        const __amdgpu_buffer_rsrc_t krs = rsrc(kb, 0xffffffffu);
        const __amdgpu_buffer_rsrc_t srs = rsrc(ks, 0xffffffffu);
        const uint32_t klane = sub * PPL * ES;     // bytes: the lane's pairs within a key half
        const int cpq = (m + 3) / 4;
        const int cb = min(m, quarter * cpq);
        const int ce = min(m, cb + cpq);
        const int nitems = (ce - cb) * nref;
        const int hsel = sub / LPH;
        const bool wz = (sub % LPH) == 0;          // lanes that store a head's logit
        const bool ws = WGS && sub == 1;           // the lane that stores the group score
        // z of one key item: the key turned by (c, s), dotted with the G heads
        auto logits = [&](const KL &kx0, const KL &kx1, const float (&c)[PPL], const float (&sn)[PPL], float sc)
            __attribute__((always_inline)) {
            float x0[PPL], x1[PPL];
            if constexpr (Q8) {
                cvt8<PPL>(kx0, x0);
                cvt8<PPL>(kx1, x1);
            } else {
                cvt(kx0, x0);
                cvt(kx1, x1);
            }
            float z[G];
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                const float r0 = x0[e] * c[e] - x1[e] * sn[e];
                const float r1 = x0[e] * sn[e] + x1[e] * c[e];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    z[h] = (e == 0) ? qa[h][0] * r0 : fmaf(qa[h][e], r0, z[h]);
                    z[h] = fmaf(qb[h][e], r1, z[h]);
                }
            }
            const float zs = row_sums<G>(z, sub);
            return Q8 ? zs * sc : zs;
        };
        if (nref == 1) {
            // every item is a candidate: no reference-key maximum.  The items
            // of a quarter's batch sit at consecutive positions p0, p0 + 1, ..:
            // the batch reads (cos, sin) of p0 and p0 + 1 and steps on with
            // cos((p+1)t) = 2 cos(t) cos(pt) - cos((p-1)t) (likewise sin).
            float tc[PPL];   // 2 cos(t) of the lane's pairs
#pragma unroll
            for (int w = 0; w < PPL / 2; ++w) {
                const uint4 st4 = bload<uint4>(rope_rs, RB + sub * PPL * 8 + w * 16, 0);
                tc[2 * w] = 2.f * __uint_as_float(st4.x);
                tc[2 * w + 1] = 2.f * __uint_as_float(st4.z);
            }
            const int nbatch = (cpq + KB - 1) / KB;   // the same in every quarter
            for (int bt = 0; bt < nbatch; ++bt) {
                const int it0 = bt * KB;
                const int nb = min(nitems - it0, KB);  // <= 0 for a short quarter
                // lane `sub` derives the row of item it0 + sub (clamped into
                // the batch); row u reaches the quarter by a DPP row broadcast
                const int cand = max(0, min(cb + it0 + (nb > 0 ? min(sub, nb - 1) : 0), m - 1));
                const uint32_t roff = (uint32_t)cs.id(c0 + cand) * (D * ES);
                KL k0[KB], k1[KB];
                float sc[KB];
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                    const uint32_t rb = (uint32_t)row_bcast((int)roff, u);
                    k0[u] = bload<KL>(krs, rb + klane, 0);
                    k1[u] = bload<KL>(krs, rb + klane + D * ES / 2, 0);
                    sc[u] = Q8 ? __uint_as_float(bload<uint32_t>(srs, rb >> RSH, 0)) : 1.f;
                }
                const uint32_t rbase = (uint32_t)(c0 + cb + it0) * RB + sub * PPL * 8;
                float c[PPL], sn[PPL], cq[PPL], sq[PPL];   // position p and p - 1 (or p + 1 before the first step)
#pragma unroll
                for (int w = 0; w < PPL / 2; ++w) {
                    const uint4 a4 = bload<uint4>(rope_rs, rbase + w * 16, 0);
                    c[2 * w] = __uint_as_float(a4.x);
                    sn[2 * w] = __uint_as_float(a4.y);
                    c[2 * w + 1] = __uint_as_float(a4.z);
                    sn[2 * w + 1] = __uint_as_float(a4.w);
                    const uint4 b4 = bload<uint4>(rope_rs, rbase + RB + w * 16, 0);
                    cq[2 * w] = __uint_as_float(b4.x);
                    sq[2 * w] = __uint_as_float(b4.y);
                    cq[2 * w + 1] = __uint_as_float(b4.z);
                    sq[2 * w + 1] = __uint_as_float(b4.w);
                }
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                    if (u == 1) {
#pragma unroll
                        for (int e = 0; e < PPL; ++e) {
                            const float c2 = cq[e], s2 = sq[e];
                            cq[e] = c[e];
                            sq[e] = sn[e];
                            c[e] = c2;
                            sn[e] = s2;
                        }
                    } else if (u > 1) {
#pragma unroll
                        for (int e = 0; e < PPL; ++e) {
                            const float c2 = fmaf(tc[e], c[e], -cq[e]);
                            const float s2 = fmaf(tc[e], sn[e], -sq[e]);
                            cq[e] = c[e];
                            sq[e] = sn[e];
                            c[e] = c2;
                            sn[e] = s2;
                        }
                    }
                    const float zh = logits(k0[u], k1[u], c, sn, sc[u]);
                    float gs = 0.f;
                    if constexpr (WGS) gs = head_total<G>(zh) * (1.f / G);
                    // every lane stores (the others into the spare words past
                    // sS[MC]), so that the batch stays one basic block
                    const int ci = cb + it0 + u;
                    float *dst = (u < nb && (wz || ws)) ? (ws ? &sS[ci] : &sZ[ci * G + hsel]) : &sS[MC + lane];
                    *dst = ws ? gs : zh;
                }
            }
        } else {
            // nref reference keys per candidate: its group score is the best
            // over them, with that key's per-head logits
            float st_c[PPL], st_s[PPL];
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                const float2 c2 = t.rope[(D / 2) + sub * PPL + e];
                st_c[e] = c2.x;
                st_s[e] = c2.y;
            }
            const int KBR = (KB / nref) * nref;
            const int nbatch = (cpq * nref + KBR - 1) / KBR;
            for (int bt = 0; bt < nbatch; ++bt) {
                const int it0 = bt * KBR;
                const int nb = min(nitems - it0, KBR);
                const int itl = it0 + (nb > 0 ? min(sub, nb - 1) : 0);
                const int cl = itl / nref;
                const int cand = max(0, min(cb + cl, m - 1));
                const uint32_t roff = ((uint32_t)cs.id(c0 + cand) * nref + (itl - cl * nref)) * (D * ES);
                KL k0[KB], k1[KB];
                float sc[KB];
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                    const uint32_t rb = (uint32_t)row_bcast((int)roff, u);
                    k0[u] = bload<KL>(krs, rb + klane, 0);
                    k1[u] = bload<KL>(krs, rb + klane + D * ES / 2, 0);
                    sc[u] = Q8 ? __uint_as_float(bload<uint32_t>(srs, rb >> RSH, 0)) : 1.f;
                }
                float cc[PPL], ss[PPL];
                {
                    const int pos = c0 + max(0, min(cb + it0 / nref, m - 1));
                    const float2 *rp = t.rope + (int64_t)pos * (D / 2) + sub * PPL;
#pragma unroll
                    for (int e = 0; e < PPL; ++e) {
                        const float2 c2 = rp[e];
                        cc[e] = c2.x;
                        ss[e] = c2.y;
                    }
                }
                int ci = cb + it0 / nref, j = 0;
                float best = -INFINITY, zbst = 0.f;
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                    if (u < nb) {
                        const float zh = logits(k0[u], k1[u], cc, ss, sc[u]);
                        const float gs = head_total<G>(zh) * (1.f / G);
                        if (gs > best) {
                            best = gs;
                            zbst = zh;
                        }
                        if (++j == nref) {
                            if (sub == 1) sS[ci] = best;
                            else if (wz) sZ[ci * G + hsel] = zbst;
                            j = 0;
                            ++ci;
                            best = -INFINITY;
#pragma unroll
                            for (int e = 0; e < PPL; ++e) {
                                const float c2 = cc[e] * st_c[e] - ss[e] * st_s[e];
                                const float s2 = cc[e] * st_s[e] + ss[e] * st_c[e];
                                cc[e] = c2;
                                ss[e] = s2;
                            }
                        }
                    }
                }
            }
        }
        wave_sync();
    };

    // ---- softmax update over candidates [0, m) of sZ; kept ones (bit jj of
    // `kept` for candidate lane + 64 jj) drop out: new running max, rescale,
    // probabilities rounded to bf16 and stored in pairs of consecutive
    // candidates (zeros up to the next multiple of VB), partial denominators
    // of the rounded values
    auto softmax_step = [&](int m, uint32_t kept) __attribute__((always_inline)) {
        float mx[G];
#pragma unroll
        for (int h = 0; h < G; ++h) mx[h] = -INFINITY;
        for (int jj = 0; jj * 64 < m; ++jj) {
            const int c = jj * 64 + lane;
            if (c < m && !((kept >> jj) & 1u)) {
#pragma unroll
                for (int h = 0; h < G; ++h) mx[h] = fmaxf(mx[h], sZ[c * G + h]);
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mn = fmaxf(M[h], wave_max(mx[h]));
            const float alpha = (mn == -INFINITY) ? 1.f : __expf(M[h] - mn);
            M[h] = mn;
            lt[h] *= alpha;
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] *= alpha;
        }
        const int mp = (m + VB - 1) / VB * VB;
        for (int jj = 0; jj * 64 < mp; ++jj) {
            const int c = jj * 64 + lane;
            const bool use = c < m && !((kept >> jj) & 1u);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = use ? __expf(sZ[c * G + h] - M[h]) : 0.f;
                const float po = dppf<0xB1>(p);   // candidate c ^ 1
                // even lanes: candidates (c, c + 1) rounded to bf16 (to
                // nearest even) as one word, and their rounded sum
                const bf16x2_t w2 = {(__bf16)p, (__bf16)po};
                const uint32_t w = __builtin_bit_cast(uint32_t, w2);
                const float both = __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
                lt[h] += (lane & 1) ? 0.f : both;
                if (!(lane & 1) && c < mp) sP[(c >> 1) * G + h] = w;
            }
        }
        wave_sync();
    };

    // ---- p * v over candidates [0, m) (values at vb + id * D): the whole
    // wave takes one row per load (lane l holds elements l*DPL ..), VB rows
    // per batch, row ids derived by lanes 0..VB-1 and handed out by readlane;
    // two rows at a time go through bf16 dot products with the probability
    // pairs (rows past m have probability 0)
    auto fold = [&](const Cands &cs, const T *vb, int c0, int m) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t vrs = rsrc(vb, 0xffffffffu);
        const uint32_t vlane = lane * DPL * 2;
        auto issue = [&](int r0, VR (&vr)[VB]) __attribute__((always_inline)) {
            const int nb = min(m - r0, VB);
            const uint32_t rl = (uint32_t)cs.id(c0 + r0 + min(lane & (VB - 1), nb - 1)) * (D * 2);
#pragma unroll
            for (int u = 0; u < VB; ++u)
                vr[u] = bload<VR>(vrs, vlane, (uint32_t)__builtin_amdgcn_readlane((int)rl, u));
        };
        auto consume = [&](int r0, const VR (&vr)[VB]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < VB; u += 2) {
                uint32_t pw[G];
                const uint32_t *pp = &sP[((r0 + u) >> 1) * G];
                if constexpr (G % 4 == 0) {
#pragma unroll
                    for (int h = 0; h < G; h += 4) {
                        const uint4 x = *reinterpret_cast<const uint4 *>(pp + h);
                        pw[h] = x.x;
                        pw[h + 1] = x.y;
                        pw[h + 2] = x.z;
                        pw[h + 3] = x.w;
                    }
                } else if constexpr (G == 2) {
                    const uint2 x = *reinterpret_cast<const uint2 *>(pp);
                    pw[0] = x.x;
                    pw[1] = x.y;
                } else {
                    pw[0] = pp[0];
                }
                if constexpr (DPL == 2) {
                    // (row u, row u+1) of element 0, then of element 1
                    const uint32_t lo = __builtin_amdgcn_perm(vr[u + 1], vr[u], 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(vr[u + 1], vr[u], 0x07060302u);
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        acc[h][0] = dot2bf(lo, pw[h], acc[h][0]);
                        acc[h][1] = dot2bf(hi, pw[h], acc[h][1]);
                    }
                } else {
                    const uint32_t pr = (uint32_t)vr[u] | ((uint32_t)vr[u + 1] << 16);
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[h][0] = dot2bf(pr, pw[h], acc[h][0]);
                }
            }
        };
        // two register sets: the next batch's gathers in flight while the
        // current one is folded
        VR va[VB], vbb[VB];
        if (m > 0) issue(0, va);
        for (int r0 = 0; r0 < m; r0 += 2 * VB) {
            if (r0 + VB < m) issue(r0 + VB, vbb);
            consume(r0, va);
            if (r0 + VB < m) {
                if (r0 + 2 * VB < m) issue(r0 + 2 * VB, va);
                consume(r0 + VB, vbb);
            }
        }
        wave_sync();
    };

    // ---- summary levels
    int cur = 0, nsel = 0;
    for (int lvl = levels; lvl >= 1; --lvl) {
        Cands cs;
        const bool top = (lvl == levels);
        cs.selp = selbuf + cur * kMaxSel;
        cs.nprev = top ? 0 : nsel;
        // (children per parent above level 1: the fan)
        const int fb = t.fan;
        cs.b = fb;
        cs.binv = a.finv;
        cs.top = top;
        const int orph0 = top ? 0 : fb * nlev[lvl + 1];
        cs.orph0 = orph0;
        const int m = top ? nlev[lvl] : nsel * fb + (nlev[lvl] - orph0);
        const T *kb = (const T *)t.lk[lvl - 1] + bh * t.ncap[lvl] * R * D;
        const T *vb = (const T *)t.lv[lvl - 1] + bh * t.ncap[lvl] * D;
        const bool take_all = (a.mode == HTI_TOPK) ? (m <= a.k) : (m <= 1);
        uint32_t kept = 0u;
        if (!take_all) {
            if (top && a.top_s != nullptr) {
                // scored for the whole block on the matrix cores
                const float *tsrc = a.top_s + uidx * a.ntop_stride;
                const float *zsrc = a.top_z + (((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G) * a.ntop_stride;
                for (int c = lane; c < m; c += 64) {
                    sS[c] = tsrc[c];
#pragma unroll
                    for (int h = 0; h < G; ++h) sZ[c * G + h] = zsrc[(int64_t)h * a.ntop_stride + c];
                }
                wave_sync();
            } else {
                if constexpr (F8)
                    score(std::true_type{}, std::true_type{}, cs, t.lkq[lvl - 1] + bh * t.ncap[lvl] * R * D,
                          t.lks[lvl - 1] + bh * t.ncap[lvl] * R, R, 0, m, m);
                else
                    score(std::true_type{}, std::false_type{}, cs, kb, nullptr, R, 0, m, m);
            }
            // selection (score desc, then lower index): the lane holds
            // candidates lane + 64 jj
            float sv[MJ];
#pragma unroll
            for (int jj = 0; jj < MJ; ++jj) {
                const int c = jj * 64 + lane;
                sv[jj] = (c < m) ? sS[c] : -INFINITY;
            }
            float gmax = 0.f, den = 1.f;
            if (a.mode == HTI_TOPP) {
                float mx = -INFINITY;
#pragma unroll
                for (int jj = 0; jj < MJ; ++jj) mx = fmaxf(mx, sv[jj]);
                gmax = wave_max(mx);
                float sm_ = 0.f;
#pragma unroll
                for (int jj = 0; jj < MJ; ++jj)
                    if (jj * 64 + lane < m) sm_ += __expf(sv[jj] - gmax);
                den = wave_sum(sm_);
            }
            const int nmax = min(keff, m);
            float cum = 0.f;
            for (int r = 0; r < nmax; ++r) {
                // the lane's best open candidate (candidates are visited in
                // index order, so the strict > keeps the lower index on ties;
                // kept ones and those past m hold -inf)
                float bv = -INFINITY;
                int bj = 0;
#pragma unroll
                for (int jj = 0; jj < MJ; ++jj) {
                    const bool bt = sv[jj] > bv;
                    bv = bt ? sv[jj] : bv;
                    bj = bt ? jj : bj;
                }
                // the wave's best score, then the lowest candidate index that
                // holds it
                float gm = bv;
                gm = fmaxf(gm, dppf<0xB1>(gm));
                gm = fmaxf(gm, dppf<0x4E>(gm));
                gm = fmaxf(gm, dppf<0x141>(gm));
                gm = fmaxf(gm, dppf<0x140>(gm));
                gm = fmaxf(fmaxf(rlane(gm, 0), rlane(gm, 16)), fmaxf(rlane(gm, 32), rlane(gm, 48)));
                const uint64_t hit = __ballot(bv == gm);
                int win;
                if (__popcll(hit) == 1) {
                    const int wl = __ffsll((unsigned long long)hit) - 1;
                    win = __builtin_amdgcn_readlane(bj, wl) * 64 + wl;
                } else {
                    win = wave_min_i(bv == gm ? bj * 64 + lane : 0x7fffffff);
                }
                if ((win & 63) == lane) {
                    kept |= 1u << (win >> 6);
#pragma unroll
                    for (int jj = 0; jj < MJ; ++jj) sv[jj] = (jj == (win >> 6)) ? -INFINITY : sv[jj];
                }
                if (a.mode == HTI_TOPP) {
                    cum += __expf(gm - gmax) / den;
                    if (cum >= a.p) break;
                }
            }
        }
        // kept set in candidate (= node) order -> the next level's parents
        int *nsl = selbuf + (cur ^ 1) * kMaxSel;
        int nn = 0;
        for (int jj = 0; jj * 64 < m; ++jj) {
            const int c = jj * 64 + lane;
            const bool k = c < m && (take_all || ((kept >> jj) & 1u));
            const uint64_t bal = __ballot(k);
            const int pos = nn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (k) nsl[pos] = (int)cs.id(c);
            nn += __popcll(bal);
        }
        wave_sync();
        if (a.sel) {
            int *o = a.sel + (uidx * levels + (lvl - 1)) * a.sel_stride;
            for (int r = lane; r < a.sel_stride; r += 64) o[r] = (r < nn) ? nsl[r] : -1;
        }
        if (lvl == 1 && a.kept1) {
            // the node-inverted token level takes the kept nodes' tokens
            for (int r = lane; r < nn; r += 64) {
                a.kept1[uidx * keff + r] = nsl[r];
                atomicAdd(&a.node_cnt[bh * t.ncap[1] + nsl[r]], 1u);
            }
            if (lane == 0) a.nsel1[uidx] = nn;
        }
        if (!take_all && !a.leaf_only) {
            softmax_step(m, kept);
            fold(cs, vb, 0, m);     // ids through cs, i.e. the parents' list
        }
        cur ^= 1;
        nsel = nn;
    }

    // ---- token level: reached prefix tokens, then orphan prefix tokens; the
    // block tokens follow them (handled by the in-block kernel), so query t
    // sits at |C_0| + t.  With the node-inverted token level (kept1) only the
    // orphan tokens are attended here.
    {
        Cands cs;
        const bool top = (levels == 0);
        cs.selp = selbuf + cur * kMaxSel;
        cs.nprev = top ? 0 : nsel;
        cs.b = b;
        cs.binv = a.binv;
        cs.top = top;
        const int orph0 = top ? 0 : b * nlev[1];
        cs.orph0 = orph0;
        const int m0 = top ? L : nsel * b + (L - orph0);
        const int qpos = m0 + qi;
        const T *kc = (const T *)t.kc + bh * t.ncap[0] * D;
        const T *vc = (const T *)t.vc + bh * t.ncap[0] * D;
        for (int c0 = a.kept1 ? nsel * b : 0; c0 < m0; c0 += MC) {
            const int mc = min(MC, m0 - c0);
            score(std::false_type{}, std::false_type{}, cs, kc, nullptr, 1, c0, mc, qpos);
            softmax_step(mc, 0u);
            fold(cs, vc, c0, mc);
        }
    }

    // ---- partial state
    const int64_t row0 = ((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float l = wave_sum(lt[h]);
        // a head with nothing attended (M = -inf: an empty prefix) leaves no
        // output row; its readers take it as zero
        if (M[h] != -INFINITY)
#pragma unroll
            for (int e = 0; e < DPL; ++e) a.part_acc[(row0 + h) * D + lane * DPL + e] = acc[h][e];
        if (lane == 0) {
            a.part_ml[(row0 + h) * 2 + 0] = M[h];
            a.part_ml[(row0 + h) * 2 + 1] = l;
        }
    }
}

template <int D, int G, int MJ, bool F8>
static hipError_t pw_launch(const TravArgs &a, int MC, int64_t units, hipStream_t s)
{
    auto kern = k_prefill_walk<D, G, MJ, F8>;
    // up to four units per workgroup, as many as fit the LDS
    const size_t per_wave = pw_wave_words(G, D, MC) * 4;
    int nw = (int)std::min<size_t>(4, (size_t)(160 * 1024) / per_wave);
    if (nw < 1) return hipErrorInvalidValue;
    const size_t dyn = (size_t)nw * per_wave;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)((units + nw - 1) / nw)), dim3(64 * nw), dyn, s, a, MC);
    return hipGetLastError();
}

template <int D, int G>
static hipError_t pw_mj(const TravArgs &a, int MC, int64_t max_summary, int64_t units, hipStream_t s)
{
    if (a.t.rfp8)
        return max_summary <= 320 ? pw_launch<D, G, 5, true>(a, MC, units, s)
                                  : pw_launch<D, G, 17, true>(a, MC, units, s);
    return max_summary <= 320 ? pw_launch<D, G, 5, false>(a, MC, units, s)
                              : pw_launch<D, G, 17, false>(a, MC, units, s);
}

template <int D>
static hipError_t pw_g(const TravArgs &a, int MC, int64_t max_summary, int64_t units, hipStream_t s)
{
    switch (a.t.G) {
    case 1: return pw_mj<D, 1>(a, MC, max_summary, units, s);
    case 2: return pw_mj<D, 2>(a, MC, max_summary, units, s);
    case 4: return pw_mj<D, 4>(a, MC, max_summary, units, s);
    default: return pw_mj<D, 8>(a, MC, max_summary, units, s);
    }
}

int prefill_walk_chunk(int64_t max_summary)
{
    const int64_t m = max_summary < 64 ? 64 : max_summary;
    return (int)((m + 63) / 64 * 64);
}

hipError_t launch_prefill_walk(const TravArgs &a, int64_t max_summary, int64_t units, hipStream_t s)
{
    if (units <= 0) return hipSuccess;
    const int MC = prefill_walk_chunk(max_summary);
    return a.t.D == 128 ? pw_g<128>(a, MC, max_summary, units, s) : pw_g<64>(a, MC, max_summary, units, s);
}

} // namespace hti
