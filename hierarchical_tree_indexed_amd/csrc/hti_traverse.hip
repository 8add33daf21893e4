// hti_traverse.hip -- fused tree traversal + shared online softmax.
//
// One workgroup owns one (query token, KV-head group) unit (decode: 8
// wavefronts, the level's value rows gathered straight into LDS; prefill: 2
// wavefronts, many units per compute unit, values through registers) and walks the tree from the top level to the tokens:
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
// Latency structure.  Each level costs one dependent trip to HBM.  Decode
// issues, at the start of a level, the key loads of every candidate (into
// registers) and the value rows of every candidate (straight into LDS with
// global_load_lds_dwordx4, no registers held), then scores, selects and
// updates the softmax while the values arrive; the values of the few kept
// candidates are fetched but not used (about k / |C_l| of the value bytes).
// Prefill, which runs many units per CU, folds a level's unselected values
// in with the next level's key loads instead.
//
// Per level:
//   score:  a quarter-wave (16 lanes) per candidate; each lane holds d/32
//           rotate-half pairs of the key, rotates them (RoPE row of the
//           candidate's index: exact table row at the start of each batch,
//           then an angle-step recurrence over consecutive candidates) and
//           dots them with the G rotated query heads; 16-lane butterflies
//           give the G logits;
//   select: two-level tournament: every wave runs up to k rounds of
//           wavefront arg-max (DPP max, then the lowest index holding it)
//           over its contiguous slice of candidates; wave 0 merges the
//           per-wave lists the same way (top-p: until the running softmax mass
//           reaches p, at most cap) and compacts the kept positions in
//           ascending order with ballots;
//   update: block max over the unselected logits -> rescale -> exp ->
//           denominators; the values are folded in on the next pass, each
//           lane owning d/64 output dims of every head.
#include "hti_device.h"
#include "hti_internal.h"
#include "hti_trav_common.h"

namespace hti {

namespace {

constexpr int kVStageBytes = 72 * 1024;   // LDS for one level's value rows (decode)

template <int G, int NWV>
struct Smem {
    float z[kMaxCand * G];       // [candidate][head]: logits, then probabilities
    float s[kMaxCand];           // group scores
    uint8_t flag[kMaxCand];      // 1 = kept (not an entry)
    float qraw[G * 128];
    float q[G * 128];            // rotated query heads
    int sel[2][kMaxSel];
    int nsel[2];
    float M[G], l[G], alpha[G];
    float red[NWV * G];
    float wl_v[NWV][kMaxSel];    // per-wave selection lists (score, index)
    int wl_i[NWV][kMaxSel];
    int wl_n[NWV];
    float gden;
    int64_t n[HTI_MAX_LEVELS + 1];
};


} // namespace

template <typename T, int D, int G, bool PREFILL, int NWV, bool STAGE, bool F8>
__global__ __launch_bounds__(NWV * 64, STAGE ? 1 : 4) void k_traverse(TravArgs a)
{
    constexpr int NT = NWV * 64;
    constexpr int NQ = NT / 16;                       // quarter-waves (16-lane rows)
    constexpr int PPL = D / 32;                       // rotate-half pairs per lane
    constexpr int DPL = D / 64;                       // output dims per lane
    using KR = typename Raw<T, PPL>::type;
    using VR = typename Raw<T, DPL>::type;
    constexpr int KRW = sizeof(KR) / 4 > 0 ? (int)sizeof(KR) / 4 : 1;
    constexpr int VRW = sizeof(VR) / 4 > 0 ? (int)sizeof(VR) / 4 : 1;
    // register budget of the in-flight batches: decode keeps a whole level in
    // flight; prefill keeps them small so that many units share a CU
    // key rows per quarter per batch; a batch holds at least one candidate's
    // HTI_MAX_R reference keys (it never splits a candidate)
    constexpr int KB0 = (STAGE ? 40 : 24) / (2 * KRW);
    constexpr int KB = KB0 < HTI_MAX_R ? HTI_MAX_R : KB0;
    static_assert(KB >= HTI_MAX_R, "key batch");
    constexpr int VB = 16 / VRW;                      // value rows per wave per batch
    constexpr int RB = D * (int)sizeof(T);            // bytes of one row
    constexpr int LPR = RB / 16;                      // lanes per row in a 16-byte gather
    constexpr int RPI = 64 / LPR;                     // rows per wave gather
    constexpr int VROWS = STAGE ? kVStageBytes / RB : 1;
    constexpr int SPL = ceil_div(kMaxCand, 64 * NWV); // selection scores per lane
    constexpr int MSL = ceil_div(NWV * kMaxSel, 64);  // merge slots per lane
    __shared__ Smem<G, NWV> sm;
    extern __shared__ __attribute__((aligned(16))) unsigned char hti_dyn_lds[];
    T *vst = reinterpret_cast<T *>(hti_dyn_lds);

    const TreeArgs &t = a.t;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane & 15, quarter = tid >> 4;
    const int64_t unit = blockIdx.x;
    const int g = (int)(unit % t.Hkv);
    const int64_t rest = unit / t.Hkv;
    const int qi = (int)(rest % a.Nq);
    const int bi = (int)(rest / a.Nq);
    const int64_t bh = (int64_t)bi * (t.Hkv / t.hdiv) + g / t.hdiv;   // tree slot of routing head g
    const int b = t.b, levels = t.levels, R = t.R;
    int64_t L = t.len[bi];
    if (!PREFILL && a.q_pos) {
        // a decode query at position q_pos attends to the tree of tokens 0..q_pos
        const int64_t ql = a.q_pos[(int64_t)bi * a.Nq + qi];
        if (ql < L - 1) L = ql < 0 ? 0 : ql + 1;
    }
    const int keff = (a.mode == HTI_TOPK) ? a.k : a.cap;

    if (tid == 0) {
        int64_t n = L;
        sm.n[0] = n;
        for (int l = 1; l <= levels; ++l) {
            n /= fan_in(t, l);
            sm.n[l] = n;
        }
    }
    const T *qp = (const T *)a.q + (((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G) * D;
    for (int i = tid; i < G * D; i += NT) {
        float v;
        load_vec<T, 1>(qp + i, &v);
        sm.qraw[i] = v;
    }
    if (tid < G) {
        sm.M[tid] = -INFINITY;
        sm.l[tid] = 0.f;
        sm.alpha[tid] = 1.f;
    }
    if (tid == 0) sm.nsel[0] = 0;

    // angle step of one position for this lane's pairs (RoPE table row 1)
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

    const T *kc = (const T *)t.kc + bh * t.ncap[0] * D;
    const T *vc = (const T *)t.vc + bh * t.ncap[0] * D;

    // value row of candidate i of a stage (token chunk offset ch, or level)
    struct StageRef {
        bool tok;
        int lvl;
        int64_t ch;
        Cands c;
    };
    auto val_row = [&](const StageRef &sr, int i) __attribute__((always_inline)) -> const T * {
        if (sr.tok) return vc + sr.c.id((int)(sr.ch + i)) * D;
        return (const T *)t.lv[sr.lvl - 1] + (bh * t.ncap[sr.lvl] + sr.c.id(i)) * D;
    };

    auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float al = sm.alpha[h];
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] *= al;
        }
    };
    auto add_entry = [&](int i, const float *v) __attribute__((always_inline)) {
        const float *pz = &sm.z[i * G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float p = pz[h];
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] += p * v[e];
        }
    };

    // ---- values through registers (prefill): entries of a finished stage
    int pend_m = 0;
    bool pend_flags = false;
    StageRef pend{false, 0, 0, {nullptr, 0, b, 0, 0, true}};
    auto fold_pending = [&]() __attribute__((always_inline)) {
        if (pend_m == 0) return;
        rescale();
        for (int u0 = 0; wave + NWV * u0 < pend_m; u0 += VB) {
            VR vr[VB];
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int i = wave + NWV * (u0 + u);
                if (i < pend_m && !(pend_flags && sm.flag[i]))
                    vr[u] = *reinterpret_cast<const VR *>(val_row(pend, i) + lane * DPL);
            }
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int i = wave + NWV * (u0 + u);
                if (i < pend_m && !(pend_flags && sm.flag[i])) {
                    float v[DPL];
                    cvt(vr[u], v);
                    add_entry(i, v);
                }
            }
        }
        pend_m = 0;
    };

    // ---- values through LDS (decode): rows [r0, r0 + nrows) of a stage
    constexpr int SIPW = ceil_div(VROWS, RPI * NWV);   // gathers per wave for a full stage
    auto stage_values = [&](const StageRef &sr, int r0, int nrows) __attribute__((always_inline)) {
        const int ninst = (nrows + RPI - 1) / RPI;
        const T *src[SIPW];
#pragma unroll
        for (int u = 0; u < SIPW; ++u) {
            const int row = (wave + u * NWV) * RPI + lane / LPR;
            src[u] = (row < nrows) ? val_row(sr, r0 + row) + (lane % LPR) * (16 / (int)sizeof(T))
                                   : nullptr;
        }
#pragma unroll
        for (int u = 0; u < SIPW; ++u) {
            const int ins = wave + u * NWV;
            if (ins < ninst && src[u] != nullptr) gather16_to_lds(src[u], vst + (size_t)ins * RPI * D);
        }
    };
    // kept candidates carry probability 0, so every staged row is folded in
    // without a branch
    auto fold_staged = [&](int r0, int nrows) __attribute__((always_inline)) {
        int i = r0 + wave;
        for (; i + 3 * NWV < r0 + nrows; i += 4 * NWV) {
            float v[4][DPL];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                load_vec<T, DPL>(vst + (size_t)(i + u * NWV - r0) * D + lane * DPL, v[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) add_entry(i + u * NWV, v[u]);
        }
        for (; i < r0 + nrows; i += NWV) {
            float v[DPL];
            load_vec<T, DPL>(vst + (size_t)(i - r0) * D + lane * DPL, v);
            add_entry(i, v);
        }
    };

    // softmax update for the entries of a stage (flag 0): new max, rescale
    // factor, probabilities written over the logits, denominators
    auto softmax_update = [&](int m, bool use_flags) __attribute__((always_inline)) {
        float lm[G];
#pragma unroll
        for (int h = 0; h < G; ++h) lm[h] = -INFINITY;
        for (int i = tid; i < m; i += NT)
            if (!(use_flags && sm.flag[i]))
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
            for (int w = 1; w < NWV; ++w) mm = fmaxf(mm, sm.red[w * G + tid]);
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
            const bool kept = use_flags && sm.flag[i];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pz = kept ? 0.f : expf(sm.z[i * G + h] - sm.M[h]);
                sm.z[i * G + h] = pz;
                ls[h] += pz;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            ls[h] = wave_sum(ls[h]);
            if (lane == 0) sm.red[wave * G + h] = ls[h];
        }
        __syncthreads();
        if (tid < G) {
            float sum = 0.f;
            for (int w = 0; w < NWV; ++w) sum += sm.red[w * G + tid];
            sm.l[tid] = sm.l[tid] * sm.alpha[tid] + sum;
        }
        __syncthreads();
    };

    auto write_sel = [&](int lvl, int buf) __attribute__((always_inline)) {
        if (!a.sel) return;
        const int nsel = sm.nsel[buf];
        int *o = a.sel + ((int64_t)unit * levels + (lvl - 1)) * a.sel_stride;
        for (int r = tid; r < a.sel_stride; r += NT) o[r] = (r < nsel) ? sm.sel[buf][r] : -1;
    };

    // selection over candidates [0, m) (scores in sm.s): sets sm.flag for the
    // kept ones and writes their ids, ascending, to sm.sel[nxt].  Order: higher
    // score first, lower index on ties.  Every wave ranks the candidates of
    // its contiguous slice against the slice (the global top set lies in the
    // union of the slices' top sets); wave 0 ranks that union.
    auto better = [](float va, int ia, float vb, int ib) __attribute__((always_inline)) {
        return va > vb || (va == vb && ia < ib);
    };
    auto select = [&](int m, const Cands &cs, int nxt) __attribute__((always_inline)) {
        {
            const int cpw = (m + NWV - 1) / NWV;
            const int w0 = min(m, wave * cpw), w1 = min(m, w0 + cpw);
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const int i = w0 + lane + 64 * r;
                if (r * 64 >= w1 - w0) break;
                const float si = (i < w1) ? sm.s[i] : -INFINITY;
                int rank = 0;
                int j = w0;
                for (; j + 4 <= w1; j += 4) {
                    const float4 v4 = *reinterpret_cast<const float4 *>(&sm.s[j]);
                    rank += better(v4.x, j, si, i) + better(v4.y, j + 1, si, i) +
                            better(v4.z, j + 2, si, i) + better(v4.w, j + 3, si, i);
                }
                for (; j < w1; ++j) rank += better(sm.s[j], j, si, i);
                if (i < w1 && rank < keff) {
                    sm.wl_v[wave][rank] = si;
                    sm.wl_i[wave][rank] = i;
                }
            }
            if (lane == 0) sm.wl_n[wave] = min(keff, w1 - w0);
        }
        __syncthreads();
        float gmax = 0.f;
        if (a.mode == HTI_TOPP) {
            // softmax of the group scores over all candidates
            gmax = -INFINITY;
            for (int w = 0; w < NWV; ++w)
                if (sm.wl_n[w] > 0) gmax = fmaxf(gmax, sm.wl_v[w][0]);
            float ld = 0.f;
            for (int i = tid; i < m; i += NT) ld += expf(sm.s[i] - gmax);
            ld = wave_sum(ld);
            if (lane == 0) sm.red[wave * G] = ld;
            __syncthreads();
            if (tid == 0) {
                float den = 0.f;
                for (int w = 0; w < NWV; ++w) den += sm.red[w * G];
                sm.gden = den;
            }
            __syncthreads();
        }
        if (wave == 0) {
            // rank every listed entry against the union of the lists
            int myrank[MSL];
            float myv[MSL];
            int myi[MSL];
#pragma unroll
            for (int q = 0; q < MSL; ++q) {
                const int slot = lane + 64 * q;
                const int w = slot / kMaxSel, r = slot % kMaxSel;
                const bool ok = (w < NWV) && (r < sm.wl_n[w]);
                myv[q] = ok ? sm.wl_v[w][r] : -INFINITY;
                myi[q] = ok ? sm.wl_i[w][r] : -1;
                myrank[q] = 0;
            }
            for (int w = 0; w < NWV; ++w) {
                const int nw = sm.wl_n[w];
                for (int r = 0; r < nw; ++r) {
                    const float v = sm.wl_v[w][r];
                    const int ix = sm.wl_i[w][r];
#pragma unroll
                    for (int q = 0; q < MSL; ++q) myrank[q] += better(v, ix, myv[q], myi[q]);
                }
            }
            int nsel = min(keff, m);
#pragma unroll
            for (int q = 0; q < MSL; ++q)
                if (myi[q] < 0) myrank[q] = 0x7fffffff;      // empty slot
            if (a.mode == HTI_TOPP) {
                // shortest prefix of the sorted softmax whose running sum reaches p
                float *sp = sm.wl_v[NWV - 1];            // reuse: sorted probabilities
#pragma unroll
                for (int q = 0; q < MSL; ++q)
                    if (myrank[q] < nsel) sp[myrank[q]] = expf(myv[q] - gmax) / sm.gden;
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                int ns = nsel;
                if (lane == 0) {
                    float cum = 0.f;
                    for (int r = 0; r < nsel; ++r) {
                        cum += sp[r];
                        if (cum >= a.p) {
                            ns = r + 1;
                            break;
                        }
                    }
                }
                nsel = __builtin_amdgcn_readfirstlane(ns);
            }
            // kept entries: their indices by rank, then ascending positions
            int *byrank = sm.wl_i[NWV - 1];              // reuse as scratch (rank -> index)
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < MSL; ++q)
                if (myrank[q] < nsel) byrank[myrank[q]] = myi[q];
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            if (lane < nsel) {
                const int ix = byrank[lane];
                int pos = 0;
                for (int r = 0; r < nsel; ++r) pos += byrank[r] < ix;
                sm.sel[nxt][pos] = (int)cs.id(ix);
                sm.flag[ix] = 1;
            }
            if (lane == 0) sm.nsel[nxt] = nsel;
        }
        __syncthreads();
    };

    int cur = 0;
    int lvl = levels;
    int64_t ch = 0;                 // token chunk offset
    int64_t qpos_tok = 0;
    while (true) {
        const bool tok = (lvl == 0);
        const int nprev = (lvl == levels) ? 0 : sm.nsel[cur];
        Cands cs;
        cs.selp = sm.sel[cur];
        cs.nprev = nprev;
        // children per parent: b tokens under a level-1 node, fan nodes above
        const int fb = tok ? b : t.fan;
        cs.b = fb;
        cs.binv = tok ? a.binv : a.finv;
        cs.top = (lvl == levels);
        cs.orph0 = cs.top ? 0 : (int64_t)fb * sm.n[lvl + 1];
        const int64_t mfull = cs.top ? sm.n[lvl] : (int64_t)nprev * fb + (sm.n[lvl] - cs.orph0);
        const int nxt = cur ^ 1;

        int m;
        bool take_all = false, pre = false;
        int64_t qpos;
        if (!tok) {
            m = (int)mfull;
            take_all = (a.mode == HTI_TOPK) ? (m <= a.k) : (m <= 1);
            pre = PREFILL && cs.top && a.top_s != nullptr;
            qpos = m;
        } else {
            if (ch == 0) {
                if (PREFILL) {
                    qpos_tok = mfull + qi;
                } else {
                    // the query token (L - 1) is a candidate iff it is an
                    // orphan token or its level-1 parent was kept
                    bool in = (levels == 0) || (L - 1 >= cs.orph0);
                    if (!in)
                        for (int r = 0; r < nprev; ++r) in |= ((int64_t)cs.selp[r] == (L - 1) / b);
                    qpos_tok = mfull - (in ? 1 : 0);
                }
            }
            m = (int)((mfull - ch) < kMaxCand ? (mfull - ch) : kMaxCand);
            qpos = qpos_tok;
        }
        const bool entries = tok ? (m > 0) : !take_all;
        const bool score_now = entries && !pre;
        const int nref = tok ? 1 : R;
        const StageRef sref{tok, lvl, ch, cs};

        if (score_now && (!tok || ch == 0)) {
            const float2 *rp = t.rope + qpos * (D / 2);
            for (int i = tid; i < G * (D / 2); i += NT) {
                const int h = i / (D / 2), j = i % (D / 2);
                const float2 c2 = rp[j];
                const float x0 = sm.qraw[h * D + j], x1 = sm.qraw[h * D + j + D / 2];
                sm.q[h * D + j] = x0 * c2.x - x1 * c2.y;
                sm.q[h * D + j + D / 2] = x0 * c2.y + x1 * c2.x;
            }
        }
        const int cpq = (m + NQ - 1) / NQ;
        const int c_beg = min(m, quarter * cpq);
        const int c_end = min(m, c_beg + cpq);
        const int nitems = score_now ? (c_end - c_beg) * nref : 0;
        const int KBR = (KB / nref) * nref;
        const T *lk = tok ? nullptr : (const T *)t.lk[lvl - 1];
        const int64_t ncap = tok ? 0 : t.ncap[lvl];
        const int64_t pos0 = tok ? ch : 0;
        auto key_row = [&](int ci, int j) __attribute__((always_inline)) -> const T * {
            if (tok) return kc + cs.id((int)(ch + ci)) * D;
            return lk + ((bh * ncap + cs.id(ci)) * R + j) * D;
        };
        // 8-bit router keys at the summary levels: E4M3 codes (in the low
        // bytes of the key registers) and a scale per key row
        const bool q8 = F8 && !tok;
        using K8 = typename Raw8<PPL>::type;

        KR k0[KB], k1[KB];
        float sc[KB];
        float rb_c[PPL], rb_s[PPL];
        auto issue_keys = [&](int item0, int nb) __attribute__((always_inline)) {
            int ci = c_beg + item0 / nref, j = 0;
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                if (u < nb) {
                    if (q8) {
                        const int64_t r = (bh * ncap + cs.id(ci)) * R + j;
                        const uint8_t *kp = t.lkq[lvl - 1] + r * D;
                        put8(k0[u], *reinterpret_cast<const K8 *>(kp + sub * PPL));
                        put8(k1[u], *reinterpret_cast<const K8 *>(kp + D / 2 + sub * PPL));
                        sc[u] = t.lks[lvl - 1][r];
                    } else {
                        const T *kp = key_row(ci, j);
                        k0[u] = *reinterpret_cast<const KR *>(kp + sub * PPL);
                        k1[u] = *reinterpret_cast<const KR *>(kp + D / 2 + sub * PPL);
                    }
                    if (++j == nref) {
                        j = 0;
                        ++ci;
                    }
                }
            }
            if (nb > 0) {
                const float2 *rp = t.rope + (pos0 + c_beg + item0 / nref) * (D / 2) + sub * PPL;
#pragma unroll
                for (int e = 0; e < PPL; ++e) {
                    const float2 c2 = rp[e];
                    rb_c[e] = c2.x;
                    rb_s[e] = c2.y;
                }
            }
        };
        issue_keys(0, min(nitems, KBR));
        const int vfirst = min(m, VROWS);
        if (STAGE && entries) stage_values(sref, 0, vfirst);
        if (!STAGE) fold_pending();
        __syncthreads();

        if (!tok && take_all) {
            for (int i = tid; i < m; i += NT) sm.sel[nxt][i] = (int)cs.id(i);
            if (tid == 0) sm.nsel[nxt] = m;
            __syncthreads();
            write_sel(lvl, nxt);
            cur = nxt;
            --lvl;
            continue;
        }
        if (tok && m <= 0) break;

        // ---- score
        if (pre) {
            const int64_t srow = (((int64_t)bi * a.Nq + qi) * t.Hkv + g) * a.ntop_stride;
            for (int i = tid; i < m; i += NT) sm.s[i] = a.top_s[srow + i];
            for (int i = tid; i < G * m; i += NT) {
                const int h = i / m, c = i % m;
                sm.z[c * G + h] =
                    a.top_z[(((int64_t)bi * a.Nq + qi) * t.Hq + g * G + h) * a.ntop_stride + c];
            }
        } else {
            float qa[G][PPL], qb[G][PPL];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < PPL; ++e) {
                    qa[h][e] = sm.q[h * D + sub * PPL + e] * t.scale;
                    qb[h][e] = sm.q[h * D + D / 2 + sub * PPL + e] * t.scale;
                }
            constexpr int LPH = 16 / G;        // lanes per head after row_sums
            const int hsel = sub / LPH;
            const bool wz = (sub % LPH) == 0;
            for (int it0 = 0; it0 < nitems; it0 += KBR) {
                const int nb = min(nitems - it0, KBR);
                if (it0 > 0) issue_keys(it0, nb);
                int ci = c_beg + it0 / nref, j = 0;
                float best = -INFINITY, zbh = 0.f;
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
                        if (q8) {
                            cvt8<PPL>(get8(k0[u]), x0);
                            cvt8<PPL>(get8(k1[u]), x1);
                        } else {
                            cvt(k0[u], x0);
                            cvt(k1[u], x1);
                        }
                        float z[G];
#pragma unroll
                        for (int e = 0; e < PPL; ++e) {
                            const float r0 = x0[e] * cc[e] - x1[e] * ss[e];
                            const float r1 = x0[e] * ss[e] + x1[e] * cc[e];
#pragma unroll
                            for (int h = 0; h < G; ++h) {
                                z[h] = (e == 0) ? qa[h][0] * r0 : fmaf(qa[h][e], r0, z[h]);
                                z[h] = fmaf(qb[h][e], r1, z[h]);
                            }
                        }
                        // all heads' row sums at once: lane sub holds head sub / LPH
                        float zh = row_sums<G>(z, sub);
                        if (q8) zh *= sc[u];
                        const float gs = head_total<G>(zh) * (1.f / G);
                        if (gs > best) {
                            best = gs;
                            zbh = zh;
                        }
                        if (++j == nref) {
                            if (sub == 0) sm.s[ci] = best;
                            if (wz) sm.z[ci * G + hsel] = zbh;
                            j = 0;
                            ++ci;
                            best = -INFINITY;
#pragma unroll
                            for (int e = 0; e < PPL; ++e) {   // advance one position
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
        for (int i = tid; i < m; i += NT) sm.flag[i] = 0;
        __syncthreads();

        if (!tok) select(m, cs, nxt);
        // leaf_only: a summary level routes and is not attended
        const bool attend = tok || !a.leaf_only;
        if (attend) softmax_update(m, !tok);

        if (STAGE) {
            __builtin_amdgcn_s_waitcnt(0);       // the staged values landed (attended or not)
            if (attend) {
                rescale();
                __syncthreads();
                fold_staged(0, vfirst);
                for (int r0 = VROWS; r0 < m; r0 += VROWS) {
                    const int nr = min(VROWS, m - r0);
                    __syncthreads();
                    stage_values(sref, r0, nr);
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
                    fold_staged(r0, nr);
                }
            }
            __syncthreads();
        } else {
            pend_m = attend ? m : 0;
            pend_flags = !tok;
            pend = sref;
        }

        if (tok) {
            ch += kMaxCand;
            if (ch >= mfull) break;
            continue;
        }
        write_sel(lvl, nxt);
        cur = nxt;
        --lvl;
    }
    if (!STAGE) fold_pending();

    // combine the per-wave partial sums (reusing the logit buffer)
    __syncthreads();
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
        for (int w = 0; w < NWV; ++w) s += red[(w * G + h) * D + e];
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

// decode: 8 waves per unit, value rows staged in LDS; prefill: 2 waves per
// unit, values through registers
template <typename T, int D, int G, bool PF, bool F8>
static hipError_t trav_launch_k(const TravArgs &a, int64_t units, hipStream_t s)
{
    constexpr int NWV = PF ? 2 : 8;
    constexpr bool STAGE = !PF;
    auto kern = k_traverse<T, D, G, PF, NWV, STAGE, F8>;
    const size_t dyn = STAGE ? kVStageBytes : 0;
    if (dyn > 0) {
        hipError_t e = set_dyn_lds_once((const void *)kern, dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)units), dim3(NWV * 64), dyn, s, a);
    return hipGetLastError();
}

// 8-bit router keys: bf16 caches, decode
template <typename T, int D, int G, bool PF>
static hipError_t trav_launch(const TravArgs &a, int64_t units, hipStream_t s)
{
    if constexpr (std::is_same<T, bf16_t>::value && !PF)
        if (a.t.rfp8) return trav_launch_k<T, D, G, PF, true>(a, units, s);
    if (a.t.rfp8) return hipErrorInvalidValue;
    return trav_launch_k<T, D, G, PF, false>(a, units, s);
}

template <typename T, int D, bool PF>
static hipError_t trav_g(const TravArgs &a, int64_t units, hipStream_t s)
{
    switch (a.t.G) {
    case 1: return trav_launch<T, D, 1, PF>(a, units, s);
    case 2: return trav_launch<T, D, 2, PF>(a, units, s);
    case 4: return trav_launch<T, D, 4, PF>(a, units, s);
    default: return trav_launch<T, D, 8, PF>(a, units, s);
    }
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
