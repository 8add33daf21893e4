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

// (v, i) of the best candidate over the wave, in every lane: larger v, then
// lower i
__device__ __forceinline__ void wave_best(float &v, int &i)
{
    auto take = [&](float v2, int i2) __attribute__((always_inline)) {
        const bool t = (v2 > v) || (v2 == v && i2 < i);
        v = t ? v2 : v;
        i = t ? i2 : i;
    };
    take(dppf<0xB1>(v), dppi<0xB1>(i));
    take(dppf<0x4E>(v), dppi<0x4E>(i));
    take(dppf<0x141>(v), dppi<0x141>(i));
    take(dppf<0x140>(v), dppi<0x140>(i));
    float v0 = rlane(v, 0);
    int i0 = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const float v2 = rlane(v, r);
        const int i2 = __builtin_amdgcn_readlane(i, r);
        const bool t = (v2 > v0) || (v2 == v0 && i2 < i0);
        v0 = t ? v2 : v0;
        i0 = t ? i2 : i0;
    }
    v = v0;
    i = i0;
}

} // namespace

// Per-wave LDS (4-byte words): qraw [G*D], s [MC + 64], z [MC * G],
// kept-node lists [2][kMaxSel]
__host__ __device__ constexpr size_t pw_wave_words(int G, int D, int MC)
{
    return (size_t)G * D + MC + 64 + (size_t)MC * G + 2 * kMaxSel;
}

template <int D, int G, int MJ>
__global__ __launch_bounds__(256, 3) void k_prefill_walk(TravArgs a, int MC)
{
    using T = bf16_t;
    constexpr int PPL = D / 32;           // rotate-half pairs per lane (16-lane row per key)
    using KR = typename Raw<T, PPL>::type;
    constexpr int KB = 8;                 // key items per quarter per batch (>= HTI_MAX_R)
    static_assert(KB >= HTI_MAX_R, "a batch holds one candidate's reference keys");
    constexpr int DPL = D / 64;           // value elements per lane (the wave holds one row)
    using VR = typename Raw<T, DPL>::type;
    constexpr int VB = 16;                // value rows per batch
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
    const int64_t bh = (int64_t)bi * t.Hkv + g;
    const int b = t.b, levels = t.levels, R = t.R;
    const int keff = (a.mode == HTI_TOPK) ? a.k : a.cap;

    float *lds = reinterpret_cast<float *>(pw_lds) + (size_t)wave * pw_wave_words(G, D, MC);
    float *qraw = lds;
    float *sS = qraw + G * D;
    float *sZ = sS + MC + 64;
    int *selbuf = reinterpret_cast<int *>(sZ + (size_t)MC * G);

    // query of the unit (un-rotated) into LDS
    const T *qp = (const T *)a.q + (((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G) * D;
    for (int i = lane; i < G * D; i += 64) qraw[i] = bf2f(*reinterpret_cast<const uint16_t *>(qp + i));
    // node counts of the prefix tree
    int nlev[HTI_MAX_LEVELS + 1];
    {
        int n = (int)t.len[bi];
        nlev[0] = n;
#pragma unroll
        for (int l = 1; l <= HTI_MAX_LEVELS; ++l) {
            n = (l <= levels) ? n / b : 0;
            nlev[l] = n;
        }
    }
    const int L = nlev[0];
    float st_c[PPL], st_s[PPL];
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        const float2 c2 = t.rope[(D / 2) + sub * PPL + e];
        st_c[e] = c2.x;
        st_s[e] = c2.y;
    }
    float M[G], lt[G], acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        M[h] = -INFINITY;
        lt[h] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
    }
    wave_sync();

    // ---- logits of candidates c0 .. c0 + m - 1 of a list (RoPE positions
    // c0 + i; keys at kb + (id * nref + j) * D; the query at qpos) into sZ,
    // group scores into sS, both indexed from 0.  Quarter q scores a
    // contiguous run of the list, KB key items per batch.
    auto score = [&](const Cands &cs, const T *kb, int nref, int c0, int m, int qpos)
        __attribute__((always_inline)) {
        float qa[G][PPL], qb[G][PPL];
        {
            const float2 *rq = t.rope + (int64_t)qpos * (D / 2) + sub * PPL;
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                const float2 cq = rq[e];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float x0 = qraw[h * D + sub * PPL + e], x1 = qraw[h * D + D / 2 + sub * PPL + e];
                    qa[h][e] = x0 * cq.x - x1 * cq.y;
                    qb[h][e] = x0 * cq.y + x1 * cq.x;
                }
            }
        }
        const int cpq = (m + 3) / 4;
        const int cb = min(m, quarter * cpq);
        const int ce = min(m, cb + cpq);
        const int nitems = (ce - cb) * nref;
        const int KBR = (KB / nref) * nref;
        const int nbatch = (cpq * nref + KBR - 1) / KBR;   // the same in every quarter
        for (int bt = 0; bt < nbatch; ++bt) {
            const int it0 = bt * KBR;
            const int nb = min(nitems - it0, KBR);         // <= 0 for a short quarter
            // lane `sub` derives the row of item it0 + sub (clamped into the
            // batch); row u reaches the quarter by a DPP row broadcast
            const int itl = it0 + (nb > 0 ? min(sub, nb - 1) : 0);
            const int cl = itl / nref;
            const int cand = max(0, min(cb + cl, m - 1));
            const uint32_t row = (uint32_t)(cs.id(c0 + cand) * nref + (itl - cl * nref));
            KR k0[KB], k1[KB];
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const uint32_t ru = (uint32_t)row_bcast((int)row, u);
                const T *kp = kb + (size_t)ru * D;
                k0[u] = *reinterpret_cast<const KR *>(kp + sub * PPL);
                k1[u] = *reinterpret_cast<const KR *>(kp + D / 2 + sub * PPL);
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
            float best = -INFINITY;
            float zbst[G];
#pragma unroll
            for (int h = 0; h < G; ++h) zbst[h] = 0.f;
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                if (u < nb) {
                    float x0[PPL], x1[PPL];
                    cvt(k0[u], x0);
                    cvt(k1[u], x1);
                    float z[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) z[h] = 0.f;
#pragma unroll
                    for (int e = 0; e < PPL; ++e) {
                        const float r0 = x0[e] * cc[e] - x1[e] * ss[e];
                        const float r1 = x0[e] * ss[e] + x1[e] * cc[e];
#pragma unroll
                        for (int h = 0; h < G; ++h) z[h] += qa[h][e] * r0 + qb[h][e] * r1;
                    }
                    float gs = 0.f;
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        z[h] = sum16(z[h]) * t.scale;
                        gs += z[h];
                    }
                    gs = gs / (float)G;
                    if (gs > best) {
                        best = gs;
#pragma unroll
                        for (int h = 0; h < G; ++h) zbst[h] = z[h];
                    }
                    if (++j == nref) {
                        if (sub == 0) {
                            sS[ci] = best;
#pragma unroll
                            for (int h = 0; h < G; ++h) sZ[ci * G + h] = zbst[h];
                        }
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
        wave_sync();
    };

    // ---- softmax update over candidates [0, m) of sZ; kept ones (bit jj of
    // `kept` for candidate lane + 64 jj) drop out: new running max, rescale,
    // probabilities back into sZ, partial denominators
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
        for (int jj = 0; jj * 64 < m; ++jj) {
            const int c = jj * 64 + lane;
            if (c < m) {
                const bool use = !((kept >> jj) & 1u);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float p = use ? __expf(sZ[c * G + h] - M[h]) : 0.f;
                    sZ[c * G + h] = p;
                    lt[h] += p;
                }
            }
        }
        wave_sync();
    };

    // ---- p * v over candidates [0, m) (values at vb + id * D): the whole
    // wave takes one row per load (lane l holds elements l*DPL ..), VB rows
    // per batch, row ids derived by lanes 0..VB-1 and handed out by readlane
    auto fold = [&](const Cands &cs, const T *vb, int c0, int m) __attribute__((always_inline)) {
        for (int r0 = 0; r0 < m; r0 += VB) {
            const int nb = min(m - r0, VB);
            const int rl = (int)cs.id(c0 + r0 + min(lane & (VB - 1), nb - 1));
            VR vr[VB];
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const uint32_t ru = (uint32_t)__builtin_amdgcn_readlane(rl, u);
                vr[u] = *reinterpret_cast<const VR *>(vb + (size_t)ru * D + lane * DPL);
            }
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                if (u < nb) {
                    float v[DPL];
                    cvt(vr[u], v);
                    const float *pz = &sZ[(r0 + u) * G];
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float p = pz[h];
#pragma unroll
                        for (int e = 0; e < DPL; ++e) acc[h][e] += p * v[e];
                    }
                }
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
        cs.b = b;
        cs.binv = a.binv;
        cs.top = top;
        const int orph0 = top ? 0 : b * nlev[lvl + 1];
        cs.orph0 = orph0;
        const int m = top ? nlev[lvl] : nsel * b + (nlev[lvl] - orph0);
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
                score(cs, kb, R, 0, m, m);
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
                float bv = -INFINITY;
                int bidx = 0x7fffffff;
#pragma unroll
                for (int jj = 0; jj < MJ; ++jj) {
                    const int c = jj * 64 + lane;
                    const bool fr = c < m && !((kept >> jj) & 1u);
                    const bool bt = fr && (sv[jj] > bv || (sv[jj] == bv && c < bidx));
                    bv = bt ? sv[jj] : bv;
                    bidx = bt ? c : bidx;
                }
                wave_best(bv, bidx);
                if ((bidx & 63) == lane) kept |= 1u << (bidx >> 6);
                if (a.mode == HTI_TOPP) {
                    cum += __expf(bv - gmax) / den;
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
        if (!take_all) {
            softmax_step(m, kept);
            fold(cs, vb, 0, m);     // ids through cs, i.e. the parents' list
        }
        cur ^= 1;
        nsel = nn;
    }

    // ---- token level: reached prefix tokens, then orphan prefix tokens; the
    // block tokens follow them (handled by the in-block kernel), so query t
    // sits at |C_0| + t
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
        for (int c0 = 0; c0 < m0; c0 += MC) {
            const int mc = min(MC, m0 - c0);
            score(cs, kc, 1, c0, mc, qpos);
            softmax_step(mc, 0u);
            fold(cs, vc, c0, mc);
        }
    }

    // ---- partial state
    const int64_t row0 = ((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float l = wave_sum(lt[h]);
#pragma unroll
        for (int e = 0; e < DPL; ++e) a.part_acc[(row0 + h) * D + lane * DPL + e] = acc[h][e];
        if (lane == 0) {
            a.part_ml[(row0 + h) * 2 + 0] = M[h];
            a.part_ml[(row0 + h) * 2 + 1] = l;
        }
    }
}

template <int D, int G, int MJ>
static hipError_t pw_launch(const TravArgs &a, int MC, int64_t units, hipStream_t s)
{
    auto kern = k_prefill_walk<D, G, MJ>;
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
    return max_summary <= 320 ? pw_launch<D, G, 5>(a, MC, units, s) : pw_launch<D, G, 17>(a, MC, units, s);
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
