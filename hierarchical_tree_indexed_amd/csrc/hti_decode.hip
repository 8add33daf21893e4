// hti_decode.hip -- decode traversal split across workgroups.
//
// The method is the one of hti_traverse.hip ("Recursive Sparse Attention",
// abstract: per-level top-k over a tree of pooled summaries, unselected
// summaries sharing one softmax with the exact tokens, candidate-index RoPE;
// "Subquadratic Attention with a Hierarchical Tree-Structured Indexer",
// Figure 3 caption: top-p routing, reference-query keys).  Decode has few
// (query, KV group) units -- 32 at batch 4 with 8 KV heads -- and one compute
// unit can keep only a few dozen cache lines in flight, so one workgroup per
// unit would use an eighth of the chip and wait on its own gathers.  Here each
// unit is split over W workgroups (W * units ~ the CU count):
//
//   * every workgroup derives the level's candidate list (identical in all of
//     them) and takes a contiguous slice of it: it gathers the slice's keys
//     and values into registers, scores the keys and ranks them inside the
//     slice;
//   * it publishes its slice's best k (score, index) as 64-bit words carrying
//     a per-launch tag, written and read with agent-scope atomics, so a word
//     is valid exactly when its tag matches -- no fences, no counters;
//   * while the other slices' lists arrive it updates its own online softmax
//     over the whole slice (the running max may include candidates that turn
//     out to be kept; any upper bound is a valid reference point);
//   * every workgroup merges the same W lists into the same kept set, drops
//     the kept candidates' probabilities and folds its values in;
//   * the token level is sliced the same way, without an exchange;
//   * each workgroup publishes its partial state (max, denominator,
//     unnormalised output per head) the same way, and every workgroup merges
//     all of them for a slice of the output columns.
//
// The workgroups of a launch wait on each other, so they must be resident
// together: the grid is kept within one workgroup per compute unit, and every
// wait is bounded -- on timeout the unit's output is NaN.
#include <algorithm>

#include "hti_device.h"
#include "hti_internal.h"
#include "hti_trav_common.h"

namespace hti {

namespace {

constexpr int DNT = 256;              // threads per workgroup
constexpr int DNW = DNT / 64;         // waves
constexpr int DNQ = DNT / 16;         // quarter-waves (16-lane rows)
constexpr int kSlice = 128;           // largest slice of a summary level
constexpr int kMaxW = 16;             // workgroups per unit
constexpr int kSlots = kMaxSel + 2;   // words per (level, workgroup): k entries + (max, sum)
constexpr long kSpin = 1L << 22;      // bound on polling for one word

template <int G>
struct DSmem {
    float z[kSlice * G];              // [candidate][head]: logits, then probabilities
    float s[kSlice] __attribute__((aligned(16)));   // group scores of the slice
    uint8_t flag[kSlice];             // 1 = kept
    float qraw[G * 128];
    float q[G * 128];
    int sel[2][kMaxSel];
    int nsel[2];
    float M[G], l[G], alpha[G];
    float red[DNW * G];
    float xv[kMaxW * kMaxSel + 4] __attribute__((aligned(16)));   // merged lists: score, index
    int xi[kMaxW * kMaxSel + 4] __attribute__((aligned(16)));
    float xm[kMaxW], xs[kMaxW];       // per-slice max and exp-sum (top-p)
    int byrank[kMaxSel] __attribute__((aligned(16)));   // kept entries by rank: index, score
    float byv[kMaxSel];
    int nkeep;
    int64_t n[HTI_MAX_LEVELS + 1];
    uint32_t tag;
    int bad;                          // a wait of this workgroup timed out
};

__device__ __forceinline__ uint64_t pack_word(uint32_t tag, uint32_t idx, float v)
{
    return ((uint64_t)tag << 44) | ((uint64_t)(idx & 0xfffu) << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> 44); }
__device__ __forceinline__ uint32_t word_idx(uint64_t w) { return (uint32_t)(w >> 32) & 0xfffu; }
__device__ __forceinline__ float word_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

} // namespace

template <typename T, int D, int G>
__global__ __launch_bounds__(DNT) void k_decode_split(TravArgs a, DecodeWs ws)
{
    constexpr int PPL = D / 32;
    constexpr int DPL = D / 64;
    using KR = typename Raw<T, PPL>::type;
    constexpr int KRW = sizeof(KR) / 4 > 0 ? (int)sizeof(KR) / 4 : 1;
    constexpr int KB = 40 / (2 * KRW);                 // key rows per quarter per batch
    using VR = typename Raw<T, DPL>::type;
    constexpr int VBS = 8;                             // value rows per wave held in registers
    __shared__ DSmem<G> sm;
    extern __shared__ __attribute__((aligned(16))) unsigned char hti_dec_lds[];

    const TreeArgs &t = a.t;
    const int W = ws.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane & 15, quarter = tid >> 4;
    const int64_t unit = blockIdx.x / W;
    const int wg = (int)(blockIdx.x % W);
    const int g = (int)(unit % t.Hkv);
    const int64_t rest = unit / t.Hkv;
    const int qi = (int)(rest % a.Nq);
    const int bi = (int)(rest / a.Nq);
    const int64_t bh = (int64_t)bi * t.Hkv + g;
    const int b = t.b, levels = t.levels, R = t.R;
    const int64_t L = t.len[bi];
    const int keff = (a.mode == HTI_TOPK) ? a.k : a.cap;
    const int nslot = keff + (a.mode == HTI_TOPP ? 2 : 0);
    uint64_t *xw = ws.words + (int64_t)unit * levels * W * kSlots;

    if (tid == 0) {
        int64_t n = L;
        sm.n[0] = n;
        for (int l = 1; l <= levels; ++l) {
            n /= b;
            sm.n[l] = n;
        }
        sm.tag = (ws.epoch[unit] % 0xffffeu) + 1u;
        sm.nsel[0] = 0;
        sm.bad = 0;
    }
    const T *qp = (const T *)a.q + (((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G) * D;
    for (int i = tid; i < G * D; i += DNT) {
        float v;
        load_vec<T, 1>(qp + i, &v);
        sm.qraw[i] = v;
    }
    if (tid < G) {
        sm.M[tid] = -INFINITY;
        sm.l[tid] = 0.f;
        sm.alpha[tid] = 1.f;
    }
    float st_c[PPL], st_s[PPL];
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        const float2 cs = t.rope[(D / 2) + sub * PPL + e];
        st_c[e] = cs.x;
        st_s[e] = cs.y;
    }
    float acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
    __syncthreads();
    const uint32_t tag = sm.tag;

    const T *kc = (const T *)t.kc + bh * t.ncap[0] * D;
    const T *vc = (const T *)t.vc + bh * t.ncap[0] * D;

    auto rotate_query = [&](int64_t pos) __attribute__((always_inline)) {
        const float2 *rp = t.rope + pos * (D / 2);
        for (int i = tid; i < G * (D / 2); i += DNT) {
            const int h = i / (D / 2), j = i % (D / 2);
            const float2 c2 = rp[j];
            const float x0 = sm.qraw[h * D + j], x1 = sm.qraw[h * D + j + D / 2];
            sm.q[h * D + j] = x0 * c2.x - x1 * c2.y;
            sm.q[h * D + j + D / 2] = x0 * c2.y + x1 * c2.x;
        }
    };

    // Score slice candidates [0, ms) (global index s0 + i, RoPE position
    // pos0 + s0 + i): keys gathered by quarter-waves in batches, best of the
    // nref reference keys kept.  Writes sm.s, sm.z.
    // one batch of a quarter-wave's keys (items it0.., item = candidate x
    // reference key) plus the RoPE row of its first candidate
    auto load_batch = [&](int ms, int s0, int64_t pos0, int nref, auto key_row, int it0,
                          KR (&k0)[KB], KR (&k1)[KB], float (&rb_c)[PPL],
                          float (&rb_s)[PPL]) __attribute__((always_inline)) {
        const int cpq = (ms + DNQ - 1) / DNQ;
        const int c_beg = min(ms, quarter * cpq);
        const int c_end = min(ms, c_beg + cpq);
        const int nitems = (c_end - c_beg) * nref;
        const int KBR = (KB / nref) * nref;
        const int nb = min(nitems - it0, KBR);
        int ci = c_beg + it0 / nref, j = 0;
#pragma unroll
        for (int u = 0; u < KB; ++u)
            if (u < nb) {
                const T *kp = key_row(s0 + ci, j);
                k0[u] = *reinterpret_cast<const KR *>(kp + sub * PPL);
                k1[u] = *reinterpret_cast<const KR *>(kp + D / 2 + sub * PPL);
                if (++j == nref) {
                    j = 0;
                    ++ci;
                }
            }
        if (nb > 0) {
            const float2 *rp = t.rope + (pos0 + s0 + c_beg + it0 / nref) * (D / 2) + sub * PPL;
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                const float2 c2 = rp[e];
                rb_c[e] = c2.x;
                rb_s[e] = c2.y;
            }
        }
    };
    auto score_slice = [&](int ms, int s0, int64_t pos0, int nref, auto key_row,
                           bool keys_issued, KR (&k0)[KB], KR (&k1)[KB], float (&rb_c)[PPL],
                           float (&rb_s)[PPL]) __attribute__((always_inline)) {
        const int cpq = (ms + DNQ - 1) / DNQ;
        const int c_beg = min(ms, quarter * cpq);
        const int c_end = min(ms, c_beg + cpq);
        const int nitems = (c_end - c_beg) * nref;
        const int KBR = (KB / nref) * nref;
        float qa[G][PPL], qb[G][PPL];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                qa[h][e] = sm.q[h * D + sub * PPL + e];
                qb[h][e] = sm.q[h * D + D / 2 + sub * PPL + e];
            }
        for (int it0 = 0; it0 < nitems; it0 += KBR) {
            const int nb = min(nitems - it0, KBR);
            if (it0 > 0 || !keys_issued) load_batch(ms, s0, pos0, nref, key_row, it0, k0, k1, rb_c, rb_s);
            int ci = c_beg + it0 / nref, j = 0;
            float best = -INFINITY;
            float zb[G];
#pragma unroll
            for (int h = 0; h < G; ++h) zb[h] = 0.f;
            float cc[PPL], ss[PPL];
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                cc[e] = rb_c[e];
                ss[e] = rb_s[e];
            }
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
                        for (int h = 0; h < G; ++h) zb[h] = z[h];
                    }
                    if (++j == nref) {
                        if (sub == 0) {
                            sm.s[ci] = best;
#pragma unroll
                            for (int h = 0; h < G; ++h) sm.z[ci * G + h] = zb[h];
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
    };

    // value rows of the slice's candidates, wave w owning rows w, w + DNW, ...:
    // the first VBS per wave are loaded with the keys and held in registers
    // (every load is issued, rows past the slice re-reading its last row, so
    // that each writes its register unconditionally and none waits on another)
    auto issue_values = [&](int ms, auto val_row, VR (&vr)[VBS]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < VBS; ++u) {
            const int i = min(wave + DNW * u, ms - 1);
            vr[u] = *reinterpret_cast<const VR *>(val_row(i) + lane * DPL);
        }
    };

    // online-softmax reference update over the slice: running max (over every
    // slice candidate), rescale factor, probabilities over the logits
    auto softmax_ref = [&](int ms) __attribute__((always_inline)) {
        float lm[G];
#pragma unroll
        for (int h = 0; h < G; ++h) lm[h] = -INFINITY;
        for (int i = tid; i < ms; i += DNT)
#pragma unroll
            for (int h = 0; h < G; ++h) lm[h] = fmaxf(lm[h], sm.z[i * G + h]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            lm[h] = wave_max(lm[h]);
            if (lane == 0) sm.red[wave * G + h] = lm[h];
        }
        __syncthreads();
        if (tid < G) {
            float mm = sm.red[tid];
            for (int w = 1; w < DNW; ++w) mm = fmaxf(mm, sm.red[w * G + tid]);
            const float Mo = sm.M[tid];
            const float Mn = fmaxf(Mo, mm);
            sm.alpha[tid] = (Mn == -INFINITY) ? 1.f : expf(Mo - Mn);
            sm.M[tid] = Mn;
        }
        __syncthreads();
        for (int i = tid; i < ms * G; i += DNT) {
            const int h = i % G;
            sm.z[i] = expf(sm.z[i] - sm.M[h]);
        }
    };
    // denominators over the slice's entries (kept candidates' probabilities
    // zeroed first), then the values staged in LDS
    auto softmax_fold = [&](int ms, auto val_row, VR (&vr)[VBS]) __attribute__((always_inline)) {
        float ls[G];
#pragma unroll
        for (int h = 0; h < G; ++h) ls[h] = 0.f;
        for (int i = tid; i < ms; i += DNT) {
            const bool kept = sm.flag[i];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float pz = sm.z[i * G + h];
                if (kept) {
                    pz = 0.f;
                    sm.z[i * G + h] = 0.f;
                }
                ls[h] += pz;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            ls[h] = wave_sum(ls[h]);
            if (lane == 0) sm.red[wave * G + h] = ls[h];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float al = sm.alpha[h];
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] *= al;
        }
        __syncthreads();
        if (tid < G) {
            float sum = 0.f;
            for (int w = 0; w < DNW; ++w) sum += sm.red[w * G + tid];
            sm.l[tid] = sm.l[tid] * sm.alpha[tid] + sum;
        }
        auto add_row = [&](int i, const float *v) __attribute__((always_inline)) {
            const float *pz = &sm.z[i * G];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] += pz[h] * v[e];
        };
#pragma unroll
        for (int u = 0; u < VBS; ++u) {
            const int i = wave + DNW * u;
            if (i < ms) {
                float v[DPL];
                cvt(vr[u], v);
                add_row(i, v);
            }
        }
        for (int i = wave + DNW * VBS; i < ms; i += DNW) {     // rows beyond the batch
            float v[DPL];
            load_vec<T, DPL>(val_row(i) + lane * DPL, v);
            add_row(i, v);
        }
        __syncthreads();
    };

    auto better = [](float va, int ia, float vb, int ib) __attribute__((always_inline)) -> int {
        return (int)(va > vb) | ((int)(va == vb) & (int)(ia < ib));
    };

    int cur = 0;
    for (int lvl = levels; lvl >= 1; --lvl) {
        const int nprev = (lvl == levels) ? 0 : sm.nsel[cur];
        Cands cs;
        cs.selp = sm.sel[cur];
        cs.nprev = nprev;
        cs.b = b;
        cs.binv = a.binv;
        cs.top = (lvl == levels);
        cs.orph0 = cs.top ? 0 : (int64_t)b * sm.n[lvl + 1];
        const int m = (int)(cs.top ? sm.n[lvl] : (int64_t)nprev * b + (sm.n[lvl] - cs.orph0));
        const int nxt = cur ^ 1;
        const bool take_all = (a.mode == HTI_TOPK) ? (m <= a.k) : (m <= 1);
        if (take_all) {
            for (int i = tid; i < m; i += DNT) sm.sel[nxt][i] = (int)cs.id(i);
            if (tid == 0) sm.nsel[nxt] = m;
            __syncthreads();
        } else {
            const int cpw = (m + W - 1) / W;
            const int s0 = min(m, wg * cpw);
            const int ms = min(m, s0 + cpw) - s0;
            const T *lk = (const T *)t.lk[lvl - 1];
            const T *lv = (const T *)t.lv[lvl - 1];
            const int64_t ncap = t.ncap[lvl];
            auto key_row = [&](int i, int j) __attribute__((always_inline)) -> const T * {
                return lk + ((bh * ncap + cs.id(i)) * R + j) * D;
            };
            auto val_row = [&](int i) __attribute__((always_inline)) -> const T * {
                return lv + (bh * ncap + cs.id(s0 + i)) * D;
            };
            // gathers first (they depend only on the candidate list), then the
            // query rotation while they are in flight
            KR k0[KB], k1[KB];
            float rb_c[PPL], rb_s[PPL];
            load_batch(ms, s0, 0, R, key_row, 0, k0, k1, rb_c, rb_s);
            VR vr[VBS];
            if (ms > 0) issue_values(ms, val_row, vr);
            rotate_query(m);
            for (int i = tid; i < ms; i += DNT) sm.flag[i] = 0;
            __syncthreads();
            score_slice(ms, s0, 0, R, key_row, true, k0, k1, rb_c, rb_s);
            __syncthreads();

            // rank inside the slice and publish the best keff
            uint64_t *mine = xw + ((int64_t)(lvl - 1) * W + wg) * kSlots;
            for (int i = tid; i < ms; i += DNT) {
                const float si = sm.s[i];
                int rank = 0;
                int j = 0;
                for (; j + 4 <= ms; j += 4) {
                    const float4 v4 = *reinterpret_cast<const float4 *>(&sm.s[j]);
                    rank += better(v4.x, j, si, i) + better(v4.y, j + 1, si, i) +
                            better(v4.z, j + 2, si, i) + better(v4.w, j + 3, si, i);
                }
                for (; j < ms; ++j) rank += better(sm.s[j], j, si, i);
                if (rank < keff)
                    __hip_atomic_store(&mine[rank], pack_word(tag, (uint32_t)(s0 + i), si),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            for (int r = ms + tid; r < keff; r += DNT)
                __hip_atomic_store(&mine[r], pack_word(tag, 0xfffu, -INFINITY), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if (a.mode == HTI_TOPP) {
                // slice max and exp-sum of the group scores
                float lmx = -INFINITY;
                for (int i = tid; i < ms; i += DNT) lmx = fmaxf(lmx, sm.s[i]);
                lmx = wave_max(lmx);
                if (lane == 0) sm.red[wave * G] = lmx;
                __syncthreads();
                float smx = sm.red[0];
                for (int w = 1; w < DNW; ++w) smx = fmaxf(smx, sm.red[w * G]);
                float ld = 0.f;
                for (int i = tid; i < ms; i += DNT) ld += expf(sm.s[i] - smx);
                ld = wave_sum(ld);
                __syncthreads();
                if (lane == 0) sm.red[wave * G] = ld;
                __syncthreads();
                if (tid == 0) {
                    float sum = 0.f;
                    for (int w = 0; w < DNW; ++w) sum += sm.red[w * G];
                    __hip_atomic_store(&mine[keff], pack_word(tag, 0, smx), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&mine[keff + 1], pack_word(tag, 0, sum), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }

            // own softmax reference while the other slices' lists arrive
            softmax_ref(ms);

            // collect every slice's list (bounded polling on the tag)
            for (int e = tid; e < W * nslot; e += DNT) {
                const int w = e / nslot, r = e % nslot;
                const uint64_t *src = xw + ((int64_t)(lvl - 1) * W + w) * kSlots + r;
                uint64_t word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                long spins = 0;
                while (word_tag(word) != tag && ++spins < kSpin) {
                    __builtin_amdgcn_s_sleep(1);
                    word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                const bool okw = word_tag(word) == tag;
                if (!okw) {
                    __hip_atomic_store(&ws.err[unit], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    sm.bad = 1;
                }
                if (r < keff) {
                    const uint32_t ix = okw ? word_idx(word) : 0xfffu;
                    sm.xv[w * keff + r] = (okw && ix != 0xfffu) ? word_val(word) : -INFINITY;
                    sm.xi[w * keff + r] = (ix == 0xfffu) ? 0x7fffffff : (int)ix;
                } else if (r == keff) {
                    sm.xm[w] = okw ? word_val(word) : -INFINITY;
                } else {
                    sm.xs[w] = okw ? word_val(word) : 0.f;
                }
            }
            __syncthreads();

            // merge: rank every listed entry against all of them
            const int ne = W * keff;
            int nkeep = min(keff, m);
            float gmax = 0.f, den = 1.f;
            if (a.mode == HTI_TOPP) {
                gmax = -INFINITY;
                for (int w = 0; w < W; ++w) gmax = fmaxf(gmax, sm.xm[w]);
                den = 0.f;
                for (int w = 0; w < W; ++w)
                    if (sm.xm[w] > -INFINITY) den += sm.xs[w] * expf(sm.xm[w] - gmax);
            }
            // Every list is sorted (slot r holds its slice's rank-r entry), so an
            // entry's global rank is its slot plus, for every other list, the
            // number of that list's entries ranking before it.  A group of P
            // lanes (P = W rounded up to a power of two) takes an entry, lane j
            // binary-searches list j and the group sums the counts with DPP.
            {
                int P = 1;
                while (P < W) P <<= 1;
                const int lg = tid & (P - 1);
                const int ngr = DNT / P;
                int nsteps = 0;
                while ((1 << nsteps) <= keff) ++nsteps;
                const uint32_t kinv = (65536u + keff - 1) / keff;   // e / keff for e < 2^10
                const int lw = min(lg, W - 1) * keff;
                for (int e = tid / P; e - tid / P < ne; e += ngr) {
                    const bool valid = e < ne;
                    const float ve = valid ? sm.xv[e] : -INFINITY;
                    const int ie = valid ? sm.xi[e] : 0x7fffffff;
                    const int wo = (int)(((uint32_t)e * kinv) >> 16);
                    int lo = 0;
                    int hi = (lg < W && lg != wo && ie != 0x7fffffff) ? keff : 0;
                    for (int step = 0; step < nsteps; ++step) {
                        const int mid = (lo + hi) >> 1;
                        const int f = lw + min(mid, keff - 1);
                        const bool active = lo < hi;
                        const bool bt = better(sm.xv[f], sm.xi[f], ve, ie);
                        lo = (active && bt) ? mid + 1 : lo;
                        hi = (active && !bt) ? mid : hi;
                    }
                    int cnt = lo;
                    if (P >= 2) cnt += dppi<0xB1>(cnt);
                    if (P >= 4) cnt += dppi<0x4E>(cnt);
                    if (P >= 8) cnt += dppi<0x141>(cnt);
                    if (P >= 16) cnt += dppi<0x140>(cnt);
                    const int rank = cnt + (e - wo * keff);
                    if (lg == 0 && valid && ie != 0x7fffffff && rank < nkeep) {
                        sm.byrank[rank] = ie;
                        sm.byv[rank] = ve;
                    }
                }
            }
            __syncthreads();
            if (tid == 0) {
                int ns = nkeep;
                if (a.mode == HTI_TOPP) {
                    // shortest sorted prefix whose softmax mass reaches p
                    float cum = 0.f;
                    for (int r = 0; r < nkeep; ++r) {
                        cum += expf(sm.byv[r] - gmax) / den;
                        if (cum >= a.p) {
                            ns = r + 1;
                            break;
                        }
                    }
                }
                sm.nkeep = ns;
            }
            __syncthreads();
            nkeep = sm.nkeep;
            if (tid < nkeep) {
                const int ix = sm.byrank[tid];
                int pos = 0;
                int r = 0;
                for (; r + 4 <= nkeep; r += 4) {
                    const int4 b4 = *reinterpret_cast<const int4 *>(&sm.byrank[r]);
                    pos += (b4.x < ix) + (b4.y < ix) + (b4.z < ix) + (b4.w < ix);
                }
                for (; r < nkeep; ++r) pos += sm.byrank[r] < ix;
                sm.sel[nxt][pos] = (int)cs.id(ix);
                if (ix >= s0 && ix < s0 + ms) sm.flag[ix - s0] = 1;
            }
            if (tid == 0) sm.nsel[nxt] = nkeep;
            __syncthreads();
            softmax_fold(ms, val_row, vr);
        }
        if (wg == 0 && a.sel) {
            const int nsel = sm.nsel[nxt];
            int *o = a.sel + ((int64_t)unit * levels + (lvl - 1)) * a.sel_stride;
            for (int r = tid; r < a.sel_stride; r += DNT) o[r] = (r < nsel) ? sm.sel[nxt][r] : -1;
        }
        cur = nxt;
        // Every gather of this level has been consumed: say so to the
        // compiler, whose wait analysis cannot see through the predicated
        // loads and would otherwise wait for all memory before each gather of
        // the next level.
        __builtin_amdgcn_s_waitcnt(0);
    }

    // token level: children of the kept level-1 nodes, then the orphan tokens
    {
        const int nprev = levels > 0 ? sm.nsel[cur] : 0;
        Cands cs;
        cs.selp = sm.sel[cur];
        cs.nprev = nprev;
        cs.b = b;
        cs.binv = a.binv;
        cs.top = (levels == 0);
        cs.orph0 = levels > 0 ? (int64_t)b * sm.n[1] : 0;
        const int64_t m0 = levels > 0 ? (int64_t)nprev * b + (L - cs.orph0) : L;
        bool in = (levels == 0) || (L - 1 >= cs.orph0);
        if (!in)
            for (int r = 0; r < nprev; ++r) in |= ((int64_t)cs.selp[r] == (L - 1) / b);
        const int64_t qpos = m0 - (in ? 1 : 0);
        const int64_t cpw = (m0 + W - 1) / W;
        const int64_t t0 = min(m0, (int64_t)wg * cpw);
        const int64_t t1 = min(m0, t0 + cpw);
        for (int64_t c0 = t0; c0 < t1; c0 += kSlice) {
            const int ms = (int)min((int64_t)kSlice, t1 - c0);
            auto key_row = [&](int i, int) __attribute__((always_inline)) -> const T * {
                return kc + cs.id((int)(i)) * D;
            };
            auto val_row = [&](int i) __attribute__((always_inline)) -> const T * {
                return vc + cs.id((int)(c0 + i)) * D;
            };
            KR k0[KB], k1[KB];
            float rb_c[PPL], rb_s[PPL];
            load_batch(ms, (int)c0, 0, 1, key_row, 0, k0, k1, rb_c, rb_s);
            VR vr[VBS];
            issue_values(ms, val_row, vr);
            if (c0 == t0) rotate_query(qpos);
            for (int i = tid; i < ms; i += DNT) sm.flag[i] = 0;
            __syncthreads();
            score_slice(ms, (int)c0, 0, 1, key_row, true, k0, k1, rb_c, rb_s);
            __syncthreads();
            softmax_ref(ms);
            __syncthreads();
            softmax_fold(ms, val_row, vr);
            __builtin_amdgcn_s_waitcnt(0);
        }
    }

    // Partial state of this slice -> tagged words in the workspace; then every
    // workgroup merges a slice of the output columns from all W partials
    // (same exchange as the levels: a word is valid when its tag matches).
    uint64_t *pw_unit = ws.part + unit * (int64_t)W * G * (D + 2);
    {
        float *red = reinterpret_cast<float *>(hti_dec_lds);     // [DNW][G][D]
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < DPL; ++e) red[(wave * G + h) * D + lane * DPL + e] = acc[h][e];
        __syncthreads();
        uint64_t *mine = pw_unit + (int64_t)wg * G * (D + 2);
        for (int i = tid; i < G * (D + 2); i += DNT) {
            const int h = i / (D + 2), e = i % (D + 2);
            float v;
            if (e < D) {
                v = 0.f;
                for (int w = 0; w < DNW; ++w) v += red[(w * G + h) * D + e];
            } else {
                v = (e == D) ? sm.M[h] : sm.l[h];
            }
            __hip_atomic_store(&mine[i], ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // Gather n tagged words (word i at src(i)) into LDS dst[i]: every load is
    // issued first, then only words whose tag is not yet current are polled.
    auto gather_words = [&](int n, auto src, auto dst) __attribute__((always_inline)) {
        for (int i0 = 0; i0 < n; i0 += 4 * DNT) {
            uint64_t wv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * DNT + tid;
                wv[u] = (i < n) ? __hip_atomic_load(src(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : ((uint64_t)tag << 32);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * DNT + tid;
                if (i >= n) continue;
                long spins = 0;
                while ((uint32_t)(wv[u] >> 32) != tag && ++spins < kSpin) {
                    __builtin_amdgcn_s_sleep(1);
                    wv[u] = __hip_atomic_load(src(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if ((uint32_t)(wv[u] >> 32) != tag) {
                    __hip_atomic_store(&ws.err[unit], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    wv[u] = 0x7fc00000u;          // NaN: the result is visibly invalid
                }
                *dst(i) = __uint_as_float((uint32_t)wv[u]);
            }
        }
    };
    // (max, denominator) of every slice per head, and this workgroup's output
    // columns of every slice's unnormalised output, into LDS
    const int cols = (D + W - 1) / W;
    const int d0 = min(D, wg * cols), d1 = min(D, d0 + cols);
    const int nc = d1 - d0;
    float *mw = sm.z;                                                    // [W][G][2]
    float *aw = reinterpret_cast<float *>(hti_dec_lds) + DNW * G * D;    // [W][G][nc]
    __syncthreads();
    // one round: the (max, denominator) words first, then the columns
    const int nmw = W * G * 2;
    gather_words(nmw + W * G * nc, [&](int i) __attribute__((always_inline)) {
        if (i < nmw) {
            const int w = i / (G * 2), r = i % (G * 2);
            return pw_unit + ((int64_t)w * G + r / 2) * (D + 2) + D + (r % 2);
        }
        i -= nmw;
        const int w = i / (G * nc), r = i % (G * nc);
        return pw_unit + ((int64_t)w * G + r / nc) * (D + 2) + d0 + (r % nc);
    }, [&](int i) __attribute__((always_inline)) { return i < nmw ? mw + i : aw + (i - nmw); });
    __syncthreads();
    // a wait that timed out anywhere in this unit (a workgroup that was not
    // resident in time) makes its output NaN rather than silently wrong
    const bool failed = sm.bad != 0 ||
        __hip_atomic_load(&ws.err[unit], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
    const int64_t row = ((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G;
    for (int i = tid; i < G * nc; i += DNT) {
        const int h = i / nc, c = i % nc;
        float Mx = -INFINITY;
        for (int w = 0; w < W; ++w) Mx = fmaxf(Mx, mw[(w * G + h) * 2]);
        float num = 0.f, den = 0.f;
        for (int w = 0; w < W; ++w) {
            const float Mw = mw[(w * G + h) * 2];
            if (Mw == -INFINITY) continue;
            const float f = expf(Mw - Mx);
            num += aw[(w * G + h) * nc + c] * f;
            den += mw[(w * G + h) * 2 + 1] * f;
        }
        a.out[(row + h) * D + d0 + c] = failed ? __uint_as_float(0x7fc00000u) : den > 0.f ? num / den : 0.f;
    }
    if (wg == 0 && tid < G && a.lse) {
        const int h = tid;
        float Mx = -INFINITY;
        for (int w = 0; w < W; ++w) Mx = fmaxf(Mx, mw[(w * G + h) * 2]);
        float den = 0.f;
        for (int w = 0; w < W; ++w) {
            const float Mw = mw[(w * G + h) * 2];
            if (Mw != -INFINITY) den += mw[(w * G + h) * 2 + 1] * expf(Mw - Mx);
        }
        a.lse[row + h] = den > 0.f ? Mx + logf(den) : -INFINITY;
    }
    // every workgroup of this unit has read the launch tag (they all published
    // their partial state above), so the next launch may move it on
    if (wg == 0 && tid == 0) ws.epoch[unit] = ws.epoch[unit] + 1u;
}

template <typename T, int D, int G>
static hipError_t dec_launch(const TravArgs &a, const DecodeWs &ws, int64_t units, hipStream_t s)
{
    auto kern = k_decode_split<T, D, G>;
    // value stage; also holds the final per-wave partial sums
    // the per-wave partial sums and the gathered output columns of every slice
    const size_t dyn = (size_t)(DNW * G * D + G * D + kMaxW * G) * sizeof(float);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    TravArgs aa = a;
    DecodeWs ww = ws;
    void *args[] = {&aa, &ww};
    // A plain launch: the workgroups of a unit wait for each other, which
    // needs them resident together.  The plan keeps the grid within one
    // workgroup per compute unit, so they all are whenever the device is not
    // held by other work; every wait is bounded and a timeout shows as NaN
    // output (a cooperative launch would guarantee residency but costs more
    // than the whole kernel to dispatch).
    return hipLaunchKernel((const void *)kern, dim3((unsigned)(units * ws.W)), dim3(DNT), args, dyn, s);
}

template <typename T, int D>
static hipError_t dec_g(const TravArgs &a, const DecodeWs &ws, int64_t units, hipStream_t s)
{
    switch (a.t.G) {
    case 1: return dec_launch<T, D, 1>(a, ws, units, s);
    case 2: return dec_launch<T, D, 2>(a, ws, units, s);
    case 4: return dec_launch<T, D, 4>(a, ws, units, s);
    default: return dec_launch<T, D, 8>(a, ws, units, s);
    }
}

hipError_t launch_decode_split(const TravArgs &a, const DecodeWs &ws, int64_t units, hipStream_t s)
{
    if (units <= 0) return hipSuccess;
    if (a.t.dtype == HTI_BF16)
        return a.t.D == 128 ? dec_g<bf16_t, 128>(a, ws, units, s) : dec_g<bf16_t, 64>(a, ws, units, s);
    return a.t.D == 128 ? dec_g<float, 128>(a, ws, units, s) : dec_g<float, 64>(a, ws, units, s);
}

template <typename T, int D, int G>
static hipError_t dec_capacity(int *blocks_per_cu)
{
    const size_t dyn = (size_t)(DNW * G * D + G * D + kMaxW * G) * sizeof(float);
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k_decode_split<T, D, G>, DNT, dyn);
}

hipError_t decode_split_plan(const TravArgs &a, int64_t units, int64_t max_summary, int *W)
{
    static int cached_key = -1, cached_cap = 0;
    const int key = a.t.dtype * 1000 + a.t.D * 10 + a.t.G;
    if (key != cached_key) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (a.t.dtype == HTI_BF16) {
            if (a.t.D == 128) {
                e = a.t.G == 1 ? dec_capacity<bf16_t, 128, 1>(&per_cu) : a.t.G == 2 ? dec_capacity<bf16_t, 128, 2>(&per_cu)
                  : a.t.G == 4 ? dec_capacity<bf16_t, 128, 4>(&per_cu) : dec_capacity<bf16_t, 128, 8>(&per_cu);
            } else {
                e = a.t.G == 1 ? dec_capacity<bf16_t, 64, 1>(&per_cu) : a.t.G == 2 ? dec_capacity<bf16_t, 64, 2>(&per_cu)
                  : a.t.G == 4 ? dec_capacity<bf16_t, 64, 4>(&per_cu) : dec_capacity<bf16_t, 64, 8>(&per_cu);
            }
        } else {
            if (a.t.D == 128) {
                e = a.t.G == 1 ? dec_capacity<float, 128, 1>(&per_cu) : a.t.G == 2 ? dec_capacity<float, 128, 2>(&per_cu)
                  : a.t.G == 4 ? dec_capacity<float, 128, 4>(&per_cu) : dec_capacity<float, 128, 8>(&per_cu);
            } else {
                e = a.t.G == 1 ? dec_capacity<float, 64, 1>(&per_cu) : a.t.G == 2 ? dec_capacity<float, 64, 2>(&per_cu)
                  : a.t.G == 4 ? dec_capacity<float, 64, 4>(&per_cu) : dec_capacity<float, 64, 8>(&per_cu);
            }
        }
        if (e != hipSuccess) return e;
        cached_key = key;
        // one workgroup per CU keeps every unit's slices on distinct CUs
        cached_cap = cus * (per_cu < 1 ? 0 : 1);
    }
    const int64_t need = (max_summary + kSlice - 1) / kSlice;
    int64_t w = cached_cap / (units > 0 ? units : 1);
    if (w > kMaxW) w = kMaxW;
    *W = (w >= need && w >= 1 && need <= kMaxW) ? (int)w : 0;
    return hipSuccess;
}

size_t decode_ws_bytes(int64_t units, int W, int levels, int G, int D)
{
    size_t off = 0;
    off += ((size_t)units * 4 + 255) / 256 * 256;                 // epoch
    off += ((size_t)units * 4 + 255) / 256 * 256;                 // err
    off += ((size_t)units * (levels > 0 ? levels : 1) * W * kSlots * 8 + 255) / 256 * 256;
    off += ((size_t)units * W * G * (D + 2) * 8 + 255) / 256 * 256;
    return off;
}

DecodeWs decode_ws_layout(void *base, int64_t units, int W, int levels, int G, int D)
{
    DecodeWs w{};
    char *p = (char *)base;
    w.W = W;
    w.epoch = (uint32_t *)p;
    p += ((size_t)units * 4 + 255) / 256 * 256;
    w.err = (uint32_t *)p;
    p += ((size_t)units * 4 + 255) / 256 * 256;
    w.words = (uint64_t *)p;
    p += ((size_t)units * (levels > 0 ? levels : 1) * W * kSlots * 8 + 255) / 256 * 256;
    w.part = (uint64_t *)p;
    return w;
}

} // namespace hti
