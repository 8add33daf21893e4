// hti_traverse.hip -- fused tree traversal + shared online softmax.
//
// One workgroup (256 threads, 4 wavefronts) owns one (query token, KV-head
// group) unit and walks the tree from the top level to the tokens:
//   "Recursive Sparse Attention", abstract: each level above the tokens keeps
//   at most k candidates; the summaries of the candidates not kept share one
//   softmax with the exact tokens finally reached; an entry's RoPE position is
//   its index among its level's candidates.
//   "Subquadratic Attention with a Hierarchical Tree-Structured Indexer",
//   Figure 3 caption: routing scores the top level by dot products, keeps a
//   top-p set and descends recursively to the leaves.
// Readings (where the pages are silent): one selection per (query, KV group)
// scored by the mean over the group's heads of the per-head logits; with R
// reference keys a node scores the largest group mean and uses that key in the
// softmax; candidates = children of the kept nodes in node order, then the
// level's orphans (full nodes without a full parent); the query sits at
// position |C_l| on a summary level and after the tokens before it on the
// token level; ties keep the lower candidate index.
//
// Per level:
//   1. score: a quarter-wave (16 lanes) per candidate; each lane holds d/32
//      rotate-half pairs of the key (two 4..16-byte loads), rotates them with
//      the RoPE table row of the candidate's index, and dots them with the G
//      rotated query heads; 16-lane butterfly sums give the G logits;
//   2. select: wave 0 runs k (or <= cap) rounds of a wavefront arg-max over
//      the scores held in registers (ties -> lower index), then compacts the
//      kept positions in ascending order with ballots;
//   3. accumulate: the unselected candidates update the per-head online
//      softmax (block max -> rescale -> exp -> per-wave partial sums of the
//      values, each lane owning d/64 output dims of every head).
// The token level streams its candidates in chunks of HTI_MAX_CAND.
#include "hti_device.h"
#include "hti_internal.h"

namespace hti {

namespace {

constexpr int NT = 256;
constexpr int NW = NT / kWave;
constexpr int NQ = NT / 16;     // quarter-waves per block

template <int G>
struct Smem {
    float z[G * kMaxCand];       // per-head logits, then probabilities
    float s[kMaxCand];           // group scores
    uint8_t flag[kMaxCand];      // 1 = kept (selected)
    float qraw[G * HTI_MAX_LEVELS * 0 + G * 128];
    float q[G * 128];            // rotated query heads
    int sel[2][kMaxSel];
    int nsel[2];
    float M[G], l[G], alpha[G];
    float red[NW * G];
};

} // namespace

template <typename T, int D, int G, bool PREFILL>
__global__ __launch_bounds__(NT) void k_traverse(TravArgs a)
{
    constexpr int PPL = D / 32;   // rotate-half pairs per lane when scoring
    constexpr int DPL = D / 64;   // output dims per lane when accumulating
    __shared__ Smem<G> sm;

    const TreeArgs &t = a.t;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane & 15, quarter = tid >> 4;
    const int64_t unit = blockIdx.x;
    const int g = (int)(unit % t.Hkv);
    const int64_t rest = unit / t.Hkv;
    const int qi = (int)(rest % a.Nq);
    const int bi = (int)(rest / a.Nq);
    const int64_t bh = (int64_t)bi * t.Hkv + g;
    const int b = t.b, levels = t.levels, R = t.R;
    const int64_t L = t.len[bi];

    int64_t n[HTI_MAX_LEVELS + 1];
    n[0] = L;
    for (int l = 1; l <= levels; ++l) n[l] = n[l - 1] / b;

    // load the G query heads of this group (un-rotated)
    const T *qp = (const T *)a.q + (((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G) * D;
    for (int i = tid; i < G * D; i += NT) {
        float v;
        load_vec<T, 1>(qp + i, &v);
        sm.qraw[i] = v;
    }
    if (tid < G) {
        sm.M[tid] = -INFINITY;
        sm.l[tid] = 0.f;
    }
    if (tid == 0) sm.nsel[0] = 0;

    float acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
    __syncthreads();

    // rotate every query head to RoPE position `pos` (into sm.q)
    auto rotate_query = [&](int64_t pos) {
        const float2 *rp = t.rope + pos * (D / 2);
        for (int i = tid; i < G * (D / 2); i += NT) {
            const int h = i / (D / 2), j = i % (D / 2);
            const float2 cs = rp[j];
            const float x0 = sm.qraw[h * D + j], x1 = sm.qraw[h * D + j + D / 2];
            sm.q[h * D + j] = x0 * cs.x - x1 * cs.y;
            sm.q[h * D + j + D / 2] = x0 * cs.y + x1 * cs.x;
        }
    };

    // score candidates [0, m) whose key for reference j is keyptr(i, j),
    // RoPE position pos0 + i; writes sm.s (group score) and sm.z (per head)
    auto score = [&](int m, int nref, int64_t pos0, auto keyptr) {
        float qa[G][PPL], qb[G][PPL];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                qa[h][e] = sm.q[h * D + sub * PPL + e];
                qb[h][e] = sm.q[h * D + D / 2 + sub * PPL + e];
            }
        for (int i = quarter; i < m; i += NQ) {
            const float2 *rp = t.rope + (pos0 + i) * (D / 2) + sub * PPL;
            float cs_c[PPL], cs_s[PPL];
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                const float2 cs = rp[e];
                cs_c[e] = cs.x;
                cs_s[e] = cs.y;
            }
            float best = -INFINITY;
            float zb[G];
#pragma unroll
            for (int h = 0; h < G; ++h) zb[h] = 0.f;
            for (int j = 0; j < nref; ++j) {
                const T *kp = keyptr(i, j);
                float k0[PPL], k1[PPL];
                load_vec<T, PPL>(kp + sub * PPL, k0);
                load_vec<T, PPL>(kp + D / 2 + sub * PPL, k1);
                float z[G];
#pragma unroll
                for (int h = 0; h < G; ++h) z[h] = 0.f;
#pragma unroll
                for (int e = 0; e < PPL; ++e) {
                    const float r0 = k0[e] * cs_c[e] - k1[e] * cs_s[e];
                    const float r1 = k0[e] * cs_s[e] + k1[e] * cs_c[e];
#pragma unroll
                    for (int h = 0; h < G; ++h) z[h] += qa[h][e] * r0 + qb[h][e] * r1;
                }
                float gs = 0.f;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    z[h] = group_sum<16>(z[h]) * t.scale;
                    gs += z[h];
                }
                gs = gs / (float)G;
                if (gs > best) {
                    best = gs;
#pragma unroll
                    for (int h = 0; h < G; ++h) zb[h] = z[h];
                }
            }
            if (sub == 0) {
                sm.s[i] = best;
#pragma unroll
                for (int h = 0; h < G; ++h) sm.z[h * kMaxCand + i] = zb[h];
            }
        }
    };

    // online-softmax update with the candidates of [0, m) whose flag is 0;
    // value of candidate i at valptr(i)
    auto accumulate = [&](int m, auto valptr) {
        float lm[G];
#pragma unroll
        for (int h = 0; h < G; ++h) lm[h] = -INFINITY;
        for (int i = tid; i < m; i += NT)
            if (!sm.flag[i])
#pragma unroll
                for (int h = 0; h < G; ++h) lm[h] = fmaxf(lm[h], sm.z[h * kMaxCand + i]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            lm[h] = group_max<kWave>(lm[h]);
            if (lane == 0) sm.red[wave * G + h] = lm[h];
        }
        __syncthreads();
        if (tid < G) {
            float mm = sm.red[tid];
            for (int w = 1; w < NW; ++w) mm = fmaxf(mm, sm.red[w * G + tid]);
            const float Mo = sm.M[tid];
            const float Mn = fmaxf(Mo, mm);
            sm.alpha[tid] = (Mn == -INFINITY) ? 1.f : expf(Mo - Mn);
            sm.M[tid] = Mn;
        }
        __syncthreads();
        float ls[G];
#pragma unroll
        for (int h = 0; h < G; ++h) ls[h] = 0.f;
        for (int i = tid; i < m; i += NT) {
            const bool kept = sm.flag[i];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pz = kept ? 0.f : expf(sm.z[h * kMaxCand + i] - sm.M[h]);
                sm.z[h * kMaxCand + i] = pz;
                ls[h] += pz;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            ls[h] = group_sum<kWave>(ls[h]);
            if (lane == 0) sm.red[wave * G + h] = ls[h];
        }
        __syncthreads();
        if (tid < G) {
            float sum = 0.f;
            for (int w = 0; w < NW; ++w) sum += sm.red[w * G + tid];
            sm.l[tid] = sm.l[tid] * sm.alpha[tid] + sum;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float al = sm.alpha[h];
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] *= al;
        }
        for (int i = wave; i < m; i += NW) {
            if (sm.flag[i]) continue;                       // wave-uniform
            const T *vp = valptr(i);
            float v[DPL];
            load_vec<T, DPL>(vp + lane * DPL, v);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pz = sm.z[h * kMaxCand + i];
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] += pz * v[e];
            }
        }
        __syncthreads();
    };

    auto write_sel = [&](int lvl, int buf) {
        if (!a.sel) return;
        const int nsel = sm.nsel[buf];
        int *o = a.sel + ((int64_t)unit * levels + (lvl - 1)) * a.sel_stride;
        for (int r = tid; r < a.sel_stride; r += NT) o[r] = (r < nsel) ? sm.sel[buf][r] : -1;
    };

    int cur = 0;
    for (int lvl = levels; lvl >= 1; --lvl) {
        const int nprev = sm.nsel[cur];
        const bool top = (lvl == levels);
        const int64_t orph0 = top ? 0 : (int64_t)b * n[lvl + 1];
        const int m = (int)(top ? n[lvl] : (int64_t)nprev * b + (n[lvl] - orph0));
        const int *selp = sm.sel[cur];
        auto cand = [&](int i) -> int64_t {
            if (top) return i;
            if (i < nprev * b) return (int64_t)selp[i / b] * b + (i % b);
            return orph0 + (i - nprev * b);
        };
        const int nxt = cur ^ 1;
        const bool take_all = (a.mode == HTI_TOPK) ? (m <= a.k) : (m <= 1);
        if (take_all) {
            for (int i = tid; i < m; i += NT) sm.sel[nxt][i] = (int)cand(i);
            if (tid == 0) sm.nsel[nxt] = m;
            __syncthreads();
            write_sel(lvl, nxt);
            cur = nxt;
            continue;
        }

        rotate_query(m);
        for (int i = tid; i < m; i += NT) sm.flag[i] = 0;
        __syncthreads();

        const T *lk = (const T *)t.lk[lvl - 1];
        const int64_t ncap = t.ncap[lvl];
        if (PREFILL && top && a.top_s) {
            const int64_t srow = (((int64_t)bi * a.Nq + qi) * t.Hkv + g) * a.ntop_stride;
            for (int i = tid; i < m; i += NT) sm.s[i] = a.top_s[srow + i];
            for (int i = tid; i < G * m; i += NT) {
                const int h = i / m, c = i % m;
                sm.z[h * kMaxCand + c] =
                    a.top_z[(((int64_t)bi * a.Nq + qi) * t.Hq + g * G + h) * a.ntop_stride + c];
            }
        } else {
            score(m, R, 0, [&](int i, int j) -> const T * {
                return lk + ((bh * ncap + cand(i)) * R + j) * D;
            });
        }
        __syncthreads();

        // selection by wave 0: rounds of wavefront arg-max (ties -> lower index)
        if (wave == 0) {
            constexpr int RPL = kMaxCand / kWave;
            float v[RPL];
            uint32_t kept_bits = 0;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int i = lane + kWave * r;
                v[r] = (i < m) ? sm.s[i] : -INFINITY;
            }
            float mx = 0.f, den = 1.f;
            int rounds;
            if (a.mode == HTI_TOPK) {
                rounds = a.k;
            } else {
                rounds = a.cap < m ? a.cap : m;
                float lmx = -INFINITY;
#pragma unroll
                for (int r = 0; r < RPL; ++r) lmx = fmaxf(lmx, v[r]);
                mx = group_max<kWave>(lmx);
                float ld = 0.f;
#pragma unroll
                for (int r = 0; r < RPL; ++r)
                    if (lane + kWave * r < m) ld += expf(v[r] - mx);
                den = group_sum<kWave>(ld);
            }
            float cum = 0.f;
            for (int r = 0; r < rounds; ++r) {
                float bv = -INFINITY;
                int bix = 0x7fffffff;
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr)
                    if (v[rr] > bv) {
                        bv = v[rr];
                        bix = lane + kWave * rr;
                    }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    const float ov = __shfl_xor(bv, off, kWave);
                    const int oi = __shfl_xor(bix, off, kWave);
                    if (ov > bv || (ov == bv && oi < bix)) {
                        bv = ov;
                        bix = oi;
                    }
                }
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr)
                    if (lane + kWave * rr == bix) {
                        v[rr] = -INFINITY;
                        kept_bits |= 1u << rr;
                    }
                if (a.mode == HTI_TOPP) {
                    cum += expf(bv - mx) / den;
                    if (cum >= a.p) break;
                }
            }
            // ascending compaction of the kept positions
            int base = 0;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                if (r * kWave >= m) break;
                const int i = r * kWave + lane;
                const bool f = (kept_bits >> r) & 1u;
                const uint64_t mask = __ballot(f);
                const int off = __popcll(mask & ((1ull << lane) - 1ull));
                if (f) sm.sel[nxt][base + off] = (int)cand(i);
                if (i < m) sm.flag[i] = f ? 1 : 0;
                base += __popcll(mask);
            }
            if (lane == 0) sm.nsel[nxt] = base;
        }
        __syncthreads();

        const T *lv = (const T *)t.lv[lvl - 1];
        accumulate(m, [&](int i) -> const T * { return lv + (bh * ncap + cand(i)) * D; });
        write_sel(lvl, nxt);
        cur = nxt;
    }

    // token level: children of the kept level-1 nodes, then the orphan tokens
    {
        const int nsel1 = levels > 0 ? sm.nsel[cur] : 0;
        const int *selp = sm.sel[cur];
        const int64_t orph0 = levels > 0 ? (int64_t)b * n[1] : 0;
        const int64_t m0 = levels > 0 ? (int64_t)nsel1 * b + (L - orph0) : L;
        auto cand0 = [&](int64_t i) -> int64_t {
            if (levels == 0) return i;
            if (i < (int64_t)nsel1 * b) return (int64_t)selp[i / b] * b + (i % b);
            return orph0 + (i - (int64_t)nsel1 * b);
        };
        int64_t qpos;
        if (PREFILL) {
            qpos = m0 + qi;
        } else {
            // the query token (L - 1) is a candidate iff it is an orphan token
            // or its level-1 parent was kept
            bool in = (levels == 0) || (L - 1 >= orph0);
            if (!in)
                for (int r = 0; r < nsel1; ++r) in |= ((int64_t)selp[r] == (L - 1) / b);
            qpos = m0 - (in ? 1 : 0);
        }
        rotate_query(qpos);
        __syncthreads();
        const T *kc = (const T *)t.kc + bh * t.ncap[0] * D;
        const T *vc = (const T *)t.vc + bh * t.ncap[0] * D;
        for (int64_t c0 = 0; c0 < m0; c0 += kMaxCand) {
            const int mc = (int)((m0 - c0) < kMaxCand ? (m0 - c0) : kMaxCand);
            for (int i = tid; i < mc; i += NT) sm.flag[i] = 0;
            score(mc, 1, c0, [&](int i, int) -> const T * { return kc + cand0(c0 + i) * D; });
            __syncthreads();
            accumulate(mc, [&](int i) -> const T * { return vc + cand0(c0 + i) * D; });
        }
    }

    // combine the per-wave partial sums (reusing the logit buffer)
    float *red = sm.z;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) red[(wave * G + h) * D + lane * DPL + e] = acc[h][e];
    __syncthreads();
    const int64_t row = ((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G;
    for (int i = tid; i < G * D; i += NT) {
        const int h = i / D, e = i % D;
        float s = 0.f;
        for (int w = 0; w < NW; ++w) s += red[(w * G + h) * D + e];
        if (PREFILL) {
            a.part_acc[(row + h) * D + e] = s;
        } else {
            const float lh = sm.l[h];
            a.out[(row + h) * D + e] = lh > 0.f ? s / lh : 0.f;
        }
    }
    if (tid < G) {
        if (PREFILL) {
            a.part_ml[(row + tid) * 2 + 0] = sm.M[tid];
            a.part_ml[(row + tid) * 2 + 1] = sm.l[tid];
        } else if (a.lse) {
            a.lse[row + tid] = sm.l[tid] > 0.f ? sm.M[tid] + logf(sm.l[tid]) : -INFINITY;
        }
    }
}

template <typename T, int D, bool PF>
static hipError_t trav_g(const TravArgs &a, int64_t units, hipStream_t s)
{
    dim3 grid((unsigned)units), block(NT);
    switch (a.t.G) {
    case 1: hipLaunchKernelGGL((k_traverse<T, D, 1, PF>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_traverse<T, D, 2, PF>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_traverse<T, D, 4, PF>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_traverse<T, D, 8, PF>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t trav_pf(const TravArgs &a, bool prefill, int64_t units, hipStream_t s)
{
    return prefill ? trav_g<T, D, true>(a, units, s) : trav_g<T, D, false>(a, units, s);
}

hipError_t launch_traverse(const TravArgs &a, bool prefill, int64_t units, hipStream_t s)
{
    if (units <= 0) return hipSuccess;
    if (a.t.dtype == HTI_BF16)
        return a.t.D == 128 ? trav_pf<bf16_t, 128>(a, prefill, units, s)
                            : trav_pf<bf16_t, 64>(a, prefill, units, s);
    return a.t.D == 128 ? trav_pf<float, 128>(a, prefill, units, s)
                        : trav_pf<float, 64>(a, prefill, units, s);
}

} // namespace hti
