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
//   * every workgroup merges the same W lists into the same kept set; as soon
//     as the kept set is known the next level's gathers are issued, and the
//     level's own softmax contribution (unkept candidates) is folded in while
//     they are in flight;
//   * the token level is sliced the same way, without an exchange;
//   * each workgroup publishes its partial state (max, denominator,
//     unnormalised output per head) the same way, and every workgroup merges
//     all of them for a slice of the output columns.
//
// Softmax state: the running max M is kept identical in every thread (each
// computes it from the same per-wave maxima); the denominator is kept as a
// per-thread partial sum and the output as per-wave partial sums, both
// rescaled by the same factors and reduced once at the end.
//
// The workgroups of a launch wait on each other, so they must be resident
// together: the grid is kept within one workgroup per compute unit, and every
// wait is bounded -- on timeout the unit's output is NaN.
#include <algorithm>

#include "hti_device.h"
#include "hti_internal.h"
#include "hti_pool.h"
#include "hti_trav_common.h"

namespace hti {

namespace {

constexpr int DNT = 256;              // threads per workgroup
constexpr int DNW = DNT / 64;         // waves
constexpr int DNQ = DNT / 16;         // quarter-waves (16-lane rows)
constexpr int kSlice = 128;           // largest slice of a summary level / token chunk
constexpr int kMaxW = 16;             // workgroups per unit
constexpr int kSlots = kMaxSel + 2 * DNW;   // words per (level, workgroup): k entries + per-wave (max, sum)
constexpr long kSpin = 1L << 22;      // bound on polling for one word

template <int G>
struct DSmem {
    float z[2][kSlice * G];           // [candidate][head]: logits, then probabilities (by step parity)
    float s[kSlice + 68] __attribute__((aligned(16)));   // group scores of the slice, -inf padded
    uint8_t flag[kSlice];             // 1 = kept
    float qraw[G * 128] __attribute__((aligned(16)));
    int sel[2][kMaxSel];
    int nsel[2];
    float redz[DNW][G];               // per-wave maxima of the logits
    float xv[kMaxW * kMaxSel] __attribute__((aligned(16)));   // collected lists: score, index
    int xi[kMaxW * kMaxSel] __attribute__((aligned(16)));
    float xm[kMaxW * DNW], xs[kMaxW * DNW];    // per-wave max and exp-sum (top-p)
    int byrank[kMaxSel] __attribute__((aligned(16)));   // kept entries by rank: index, score
    float byv[kMaxSel];
    int nkeep;
    int in_last;                      // the query's own leaf was kept (level 1)
    int n[HTI_MAX_LEVELS + 1];        // nodes per level (n[0] = tokens; all < 2^31)
    const void *lkp[HTI_MAX_LEVELS];  // this unit's level keys / values
    const void *lvp[HTI_MAX_LEVELS];
    const uint8_t *lkq[HTI_MAX_LEVELS];   // 8-bit router keys and their row scales
    const float *lks[HTI_MAX_LEVELS];
    uint32_t tag;
    int bad;                          // a wait of this workgroup timed out
    int app;                          // decode step: the new token goes in at position lold
    int lold;                         // sequence length before the step
};

__device__ __forceinline__ uint64_t pack_word(uint32_t tag, uint32_t idx, float v)
{
    return ((uint64_t)tag << 44) | ((uint64_t)(idx & 0xfffu) << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> 44); }
__device__ __forceinline__ uint32_t word_idx(uint64_t w) { return (uint32_t)(w >> 32) & 0xfffu; }
__device__ __forceinline__ float word_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

__device__ __forceinline__ int better(float va, int ia, float vb, int ib)
{
    return (int)(va > vb) | ((int)(va == vb) & (int)(ia < ib));
}

// Candidates of one step (a summary level or the token level) as seen by one
// workgroup: the list, where its keys and values live, and this workgroup's
// slice of it.
template <typename T>
struct Step {
    Cands cs;
    gptr<T> kb, vb;      // key / value rows of this unit: row r at kb + (r * nref + j) * D
    gptr<uint8_t> kq;    // summary levels with 8-bit router keys: the E4M3 rows, likewise,
    gptr<float> ks;      // and their scales, row r * nref + j
    int nref;            // keys per row (R at summary levels, 1 at tokens)
    int m;               // candidates
    int s0, ms;          // candidates this workgroup scores (first chunk at the token level)
    int t1;              // token level: end of this workgroup's range
    int fs0, fms;        // candidates whose values this workgroup folds (its own slice)
    int qpos;            // RoPE position of the query
    bool take_all;       // every candidate is kept (no scoring)
    bool local;          // the level fits one slice: every workgroup scores all of it and
                         // selects on its own, without exchanging lists
    bool tok;            // the token level
};

} // namespace

template <typename T, int D, int G, bool F8>
__global__ __launch_bounds__(DNT) void k_decode_split(TravArgs a, DecodeWs ws)
{
    constexpr int PPL = D / 32;
    constexpr int DPL = D / 64;
    using KR = typename Raw<T, PPL>::type;
    constexpr int KRW = sizeof(KR) / 4 > 0 ? (int)sizeof(KR) / 4 : 1;
    // key rows per quarter per batch: at least one candidate's HTI_MAX_R
    // reference keys (a batch never splits a candidate), at most 16 (DPP row)
    constexpr int KB0 = 40 / (2 * KRW);
    constexpr int KB = KB0 < HTI_MAX_R ? HTI_MAX_R : (KB0 > 16 ? 16 : KB0);
    static_assert(KB >= HTI_MAX_R && KB <= 16, "key batch");
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
    const int64_t bh = (int64_t)bi * (t.Hkv / t.hdiv) + g / t.hdiv;   // tree slot of routing head g
    const int b = t.b, levels = t.levels, R = t.R;
    const int keff = (a.mode == HTI_TOPK) ? a.k : a.cap;
    const bool topp = a.mode == HTI_TOPP;
    uint64_t *xw = ws.words + (int64_t)unit * levels * W * kSlots;

    if (tid == 0) {
        // the length and the launch epoch: both loads go out before either
        // is used
        const int64_t len0 = t.len[bi];
        const uint32_t epoch = ws.epoch[unit];
        int n = (int)len0;
        // decode step: this workgroup appends the new token itself (every
        // workgroup of every query of the sequence writes the same bytes) and
        // walks the tree with the new length; it counts itself as having read
        // the old length, which one workgroup replaces at the end
        const bool app = a.k_new != nullptr && (int64_t)n < t.ncap[0];
        sm.app = app ? 1 : 0;
        sm.lold = n;
        if (a.k_new != nullptr)
            __hip_atomic_fetch_add(&ws.seqcnt[bi], n >= 0 ? 1u : 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (app) ++n;
        sm.n[0] = n;
        const int bs = __builtin_ctz((unsigned)b);
        const bool pow2 = (b & (b - 1)) == 0;
        for (int l = 1; l <= levels; ++l) {
            n = pow2 ? (n >> bs) : n / b;
            sm.n[l] = n;
        }
        sm.tag = (epoch % 0xffffeu) + 1u;
        sm.nsel[0] = 0;
        sm.bad = 0;
        sm.in_last = 0;
    }
    if (tid == 64) {
        // this unit's level arrays, by another wave than the length's chain
        // (constant indices into the argument block, so scalar loads, all
        // issued together; entries past `levels` are never read)
#pragma unroll
        for (int l = 0; l < HTI_MAX_LEVELS; ++l) {
            sm.lkp[l] = (const T *)t.lk[l] + bh * t.ncap[l + 1] * R * D;
            sm.lvp[l] = (const T *)t.lv[l] + bh * t.ncap[l + 1] * D;
            if constexpr (F8) {
                sm.lkq[l] = t.lkq[l] + bh * t.ncap[l + 1] * R * D;
                sm.lks[l] = t.lks[l] + bh * t.ncap[l + 1] * R;
            }
        }
    }
    const gptr<float2> rope = to_global<float2>(t.rope);
    const gptr<T> qp = to_global<T>(a.q) + (((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G) * D;
    // the query into LDS, one 16-byte load per thread
    constexpr int EPC = 16 / (int)sizeof(T);           // elements per 16-byte chunk
    static_assert(G * D / EPC <= DNT, "one chunk of the query per thread");
    if (tid < G * D / EPC) {
        const uint4 x = gload<uint4>(qp + tid * EPC);
        float *qd = sm.qraw + tid * EPC;
        if constexpr (sizeof(T) == 2) {
            cvt(make_uint2(x.x, x.y), qd);
            cvt(make_uint2(x.z, x.w), qd + 4);
        } else {
            qd[0] = __uint_as_float(x.x);
            qd[1] = __uint_as_float(x.y);
            qd[2] = __uint_as_float(x.z);
            qd[3] = __uint_as_float(x.w);
        }
    }
    // angle step of each of this lane's RoPE frequencies (row 1 of the table)
    float st_c[PPL], st_s[PPL];
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        const float2 c2 = gload<float2>(rope + (D / 2) + sub * PPL + e);
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
    __syncthreads();
    if (sm.app) {
        // the new row of this unit's KV head at position lold, then every
        // node it completes, level by level (one wave pools)
        const int64_t Lold = sm.lold;
        const T *kn = (const T *)a.k_new + bh * D, *vn = (const T *)a.v_new + bh * D;
        T *kw = (T *)t.kc + (bh * t.ncap[0] + Lold) * D;
        T *vw = (T *)t.vc + (bh * t.ncap[0] + Lold) * D;
        if (tid < D / EPC) {
            const uint4 kx = *reinterpret_cast<const uint4 *>(kn + tid * EPC);
            const uint4 vx = *reinterpret_cast<const uint4 *>(vn + tid * EPC);
            *reinterpret_cast<uint4 *>(kw + tid * EPC) = kx;
            *reinterpret_cast<uint4 *>(vw + tid * EPC) = vx;
        }
        __syncthreads();
        // (lengths are below 2^31 here: 32-bit index arithmetic, a mask and
        // a shift when b is a power of two)
        uint32_t idx = (uint32_t)Lold + 1u;
        const bool pow2 = (b & (b - 1)) == 0;
        const int bs = __builtin_ctz((unsigned)b);
        for (int l = 1; l <= levels; ++l) {
            if (pow2 ? (idx & (uint32_t)(b - 1)) != 0u : idx % (uint32_t)b != 0u) break;
            idx = pow2 ? idx >> bs : idx / (uint32_t)b;
            if (wave == 0) pool_node<T, D, 8>(t, l, bh, g / t.hdiv, (int64_t)idx - 1, lane);
            __syncthreads();
        }
    }
    const uint32_t tag = sm.tag;
    const int L = sm.n[0];
    const int last_leaf = L > 0 ? (L - 1) / b : -1;   // level-1 node of the query token

    const gptr<T> kc = to_global<T>(t.kc) + bh * t.ncap[0] * D;
    const gptr<T> vc = to_global<T>(t.vc) + bh * t.ncap[0] * D;

    // ---- the candidates of a step ----
    // level lvl >= 1 (parents in sm.sel[cur]) or the token level (lvl == 0)
    auto make_step = [&](int lvl, int cur) __attribute__((always_inline)) -> Step<T> {
        Step<T> st;
        st.tok = lvl == 0;
        const bool top = (lvl == levels);
        const int nprev = top ? 0 : sm.nsel[cur];
        st.cs.selp = sm.sel[cur];
        st.cs.nprev = nprev;
        st.cs.b = b;
        st.cs.binv = a.binv;
        st.cs.top = top;
        const int orph0 = top ? 0 : b * sm.n[lvl + 1];
        st.cs.orph0 = orph0;
        if (lvl >= 1) {
            st.m = top ? sm.n[lvl] : nprev * b + (sm.n[lvl] - orph0);
            st.kb = to_global<T>(sm.lkp[lvl - 1]);
            st.vb = to_global<T>(sm.lvp[lvl - 1]);
            if constexpr (F8) {
                st.kq = to_global<uint8_t>(sm.lkq[lvl - 1]);
                st.ks = to_global<float>(sm.lks[lvl - 1]);
            }
            st.nref = R;
            st.take_all = (a.mode == HTI_TOPK) ? (st.m <= a.k) : (st.m <= 1);
            const int cpw = (st.m + W - 1) / W;
            st.fs0 = min(st.m, wg * cpw);
            st.fms = min(st.m, st.fs0 + cpw) - st.fs0;
            st.local = !st.take_all && st.m <= kSlice;
            st.s0 = st.local ? 0 : st.fs0;
            st.ms = st.local ? st.m : st.fms;
            st.t1 = st.s0 + st.ms;
            st.qpos = st.m;
        } else {
            // the query token is a candidate when its leaf was kept or it is
            // an orphan; it then sits last
            const int m0 = top ? L : nprev * b + (L - orph0);
            const bool in = top || (L - 1 >= orph0) || sm.in_last != 0;
            st.m = m0;
            st.kb = kc;
            st.vb = vc;
            st.nref = 1;
            st.take_all = false;
            const int cpw = (m0 + W - 1) / W;
            const int t0 = min(m0, wg * cpw);
            st.t1 = min(m0, t0 + cpw);
            st.s0 = t0;
            st.ms = min(kSlice, (int)st.t1 - t0);
            st.fs0 = st.s0;
            st.fms = st.ms;
            st.local = false;
            st.qpos = m0 - (in ? 1 : 0);
        }
        return st;
    };

    // ---- gathers ----
    // One batch of a quarter-wave's keys: its items it0.. (item = candidate x
    // reference key), at most KB of them.  Lane `sub` derives the row of item
    // it0 + sub (clamped into the batch, so surplus loads re-read a row of
    // it) and DPP row broadcasts hand row u to the whole quarter: the
    // address arithmetic is done once per lane instead of once per row, and
    // every load is issued back to back.  Also the RoPE row of the batch's
    // first candidate.
    // With go == false every load reads the (always valid) RoPE table
    // instead, so that loads never sit behind a branch.
    auto load_batch = [&](const Step<T> &st, int s0, int ms, int it0, bool go, KR (&k0)[KB], KR (&k1)[KB],
                          float (&sc)[KB], float (&rb)[2 * PPL]) __attribute__((always_inline)) {
        const int nref = st.nref;
        const int cpq = (ms + DNQ - 1) / DNQ;
        const int c_beg = min(ms, quarter * cpq);
        const int c_end = min(ms, c_beg + cpq);
        const int nitems = (c_end - c_beg) * nref;
        const int KBR = (KB / nref) * nref;
        const int nb = min(nitems - it0, KBR);
        const int itl = it0 + (nb > 0 ? min(sub, nb - 1) : 0);
        const int cl = itl / nref;
        const int cand = min(c_beg + cl, ms - 1);
        const uint32_t row = go ? (uint32_t)(st.cs.id(s0 + max(cand, 0)) * nref + (itl - cl * nref)) : 0u;
        if (F8 && !st.tok) {
            // E4M3 codes into the low bytes of the key registers, and the row scales
            using K8 = typename Raw8<PPL>::type;
            const gptr<uint8_t> k8 = go ? st.kq : to_global<uint8_t>(t.rope);
            const gptr<float> s8 = go ? st.ks : to_global<float>(t.rope);
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const uint32_t ru = (uint32_t)row_bcast((int)row, u);
                const gptr<uint8_t> kp = k8 + (size_t)ru * D;
                put8(k0[u], gload<K8>(kp + sub * PPL));
                put8(k1[u], gload<K8>(kp + D / 2 + sub * PPL));
                sc[u] = gload<float>(s8 + ru);
            }
        } else {
            const gptr<T> kbase = go ? st.kb : to_global<T>(t.rope);
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const uint32_t ru = (uint32_t)row_bcast((int)row, u);
                const gptr<T> kp = kbase + (size_t)ru * D;
                k0[u] = gload<KR>(kp + sub * PPL);
                k1[u] = gload<KR>(kp + D / 2 + sub * PPL);
            }
        }
        const gptr<float4> rp = (gptr<float4>)(
            rope + (int64_t)max(0, s0 + min(c_beg + it0 / nref, ms - 1)) * (D / 2) + sub * PPL);
#pragma unroll
        for (int e = 0; e < PPL / 2; ++e) {
            const float4 c4 = gload<float4>(rp + e);
            rb[4 * e] = c4.x;
            rb[4 * e + 1] = c4.y;
            rb[4 * e + 2] = c4.z;
            rb[4 * e + 3] = c4.w;
        }
    };
    // value rows of the slice, wave w owning rows w, w + DNW, ...: the first
    // VBS per wave go to registers.  Lane u of the wave derives the row of its
    // u-th row (rows past the slice re-read its last row) and hands it to the
    // wave through a readlane, so the loads go out back to back.
    auto issue_values = [&](const Step<T> &st, int s0, int ms, bool go, VR (&vr)[VBS]) __attribute__((always_inline)) {
        const int rl = go ? (int)st.cs.id(s0 + max(0, min(wave + DNW * (lane & (VBS - 1)), ms - 1))) : 0;
        const gptr<T> vbase = go ? st.vb : to_global<T>(t.rope);
#pragma unroll
        for (int u = 0; u < VBS; ++u) {
            const uint32_t ru = (uint32_t)__builtin_amdgcn_readlane(rl, u);
            vr[u] = gload<VR>(vbase + (size_t)ru * D + lane * DPL);
        }
    };
    // (RoPE rows stay as loaded, (cos, sin) pairs: splitting them would copy
    // registers still being loaded and so wait for the gathers right here)
    // Every load is unconditional (a step with nothing to gather reads the
    // RoPE table instead): a register that kept its old value on some path
    // would have to be copied at the loop edge, which waits for its load.
    auto issue_step = [&](const Step<T> &st, KR (&k0)[KB], KR (&k1)[KB], float (&sc)[KB], float (&rb)[2 * PPL],
                          VR (&vr)[VBS],
                          float (&qcs)[2 * PPL]) __attribute__((always_inline)) {
        const bool go = !st.take_all && st.ms > 0;
        load_batch(st, st.s0, st.ms, 0, go, k0, k1, sc, rb);
        // (the token level's values, or a summary level's when its unkept
        // candidates are attended)
        issue_values(st, st.fs0, st.fms, !st.take_all && st.fms > 0 && (st.tok || !a.leaf_only), vr);
        const gptr<float4> rp = (gptr<float4>)(rope + st.qpos * (D / 2) + sub * PPL);
#pragma unroll
        for (int e = 0; e < PPL / 2; ++e) {
            const float4 c4 = gload<float4>(rp + e);
            qcs[4 * e] = c4.x;
            qcs[4 * e + 1] = c4.y;
            qcs[4 * e + 2] = c4.z;
            qcs[4 * e + 3] = c4.w;
        }
    };

    // ---- scoring ----
    // Rotated query of this lane's elements (sub*PPL.., and the rotate-half
    // partners), then the slice's keys in quarter-wave batches: logits per
    // head into sm.z[zb], group scores into sm.s (with -inf padding), kept
    // flags cleared, per-wave maxima of the logits into sm.redz.
    auto score = [&](const Step<T> &st, int s0, int ms, int zb, KR (&k0)[KB], KR (&k1)[KB], float (&sc)[KB],
                     float (&rb)[2 * PPL], const float (&qcs)[2 * PPL]) __attribute__((always_inline)) {
        const bool q8 = F8 && !st.tok;
        float qa[G][PPL], qb[G][PPL];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                const float x0 = sm.qraw[h * D + sub * PPL + e];
                const float x1 = sm.qraw[h * D + D / 2 + sub * PPL + e];
                qa[h][e] = (x0 * qcs[2 * e] - x1 * qcs[2 * e + 1]) * t.scale;
                qb[h][e] = (x0 * qcs[2 * e + 1] + x1 * qcs[2 * e]) * t.scale;
            }
        const int nref = st.nref;
        constexpr int LPH = 16 / G;            // lanes per head after row_sums
        const int hsel = sub / LPH;
        const bool wz = (sub % LPH) == 0;
        const int cpq = (ms + DNQ - 1) / DNQ;
        const int c_beg = min(ms, quarter * cpq);
        const int c_end = min(ms, c_beg + cpq);
        const int nitems = (c_end - c_beg) * nref;
        const int KBR = (KB / nref) * nref;
        float zmaxh = -INFINITY;               // of the lane's head
        float *zz = sm.z[zb];
        for (int it0 = 0; it0 < nitems; it0 += KBR) {
            const int nb = min(nitems - it0, KBR);
            if (it0 > 0) load_batch(st, s0, ms, it0, true, k0, k1, sc, rb);
            int ci = c_beg + it0 / nref, j = 0;
            float best = -INFINITY, zbh = 0.f;
            float cc[PPL], ss[PPL];
#pragma unroll
            for (int e = 0; e < PPL; ++e) {
                cc[e] = rb[2 * e];
                ss[e] = rb[2 * e + 1];
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
                        if (sub == 0) {
                            sm.s[ci] = best;
                            sm.flag[ci] = 0;
                        }
                        if (wz) zz[ci * G + hsel] = zbh;
                        zmaxh = fmaxf(zmaxh, zbh);
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
        if (tid < 68) sm.s[ms + tid] = -INFINITY;
        // lane h * LPH of each quarter holds that quarter's maximum of head
        // h: combine the wave's four quarters
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m4 = fmaxf(fmaxf(rlane(zmaxh, h * LPH), rlane(zmaxh, 16 + h * LPH)),
                                   fmaxf(rlane(zmaxh, 32 + h * LPH), rlane(zmaxh, 48 + h * LPH)));
            if (lane == 0) sm.redz[wave][h] = m4;
        }
    };

    // new running max from the per-wave maxima (same in every thread), and
    // the factor that rescales what was accumulated under the old one
    auto new_max = [&](float (&Mn)[G], float (&alpha)[G]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mm = M[h];
#pragma unroll
            for (int w = 0; w < DNW; ++w) mm = fmaxf(mm, sm.redz[w][h]);
            Mn[h] = mm;
            alpha[h] = (mm == -INFINITY) ? 1.f : __expf(M[h] - mm);
        }
    };
    // probabilities of this thread's candidate tid in [lo, hi) (kept ones drop
    // out), the rescaled partial denominator and output
    auto probs = [&](int lo, int hi, int zb, bool use_flags, const float (&Mn)[G], const float (&alpha)[G])
        __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            lt[h] *= alpha[h];
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] *= alpha[h];
        }
        if (tid >= lo && tid < hi) {
            const bool kept = use_flags && sm.flag[tid];
            float *zp = &sm.z[zb][tid * G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = kept ? 0.f : __expf(zp[h] - Mn[h]);
                zp[h] = p;
                lt[h] += p;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) M[h] = Mn[h];
    };
    // p * v over the slice's rows: the register batch, then any further rows
    // (zo: the z row of the range's first candidate)
    auto fold = [&](const Step<T> &st, int s0, int ms, int zb, const VR (&vr)[VBS], int zo) __attribute__((always_inline)) {
        auto add_row = [&](int i, const float *v) __attribute__((always_inline)) {
            const float *pz = &sm.z[zb][(zo + i) * G];
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
        for (int i = wave + DNW * VBS; i < ms; i += DNW) {
            float v[DPL];
            cvt(gload<VR>(st.vb + st.cs.id(s0 + i) * D + lane * DPL), v);
            add_row(i, v);
        }
    };

    // ---- the steps ----
    int cur = 0, zb = 0;
    KR k0[KB], k1[KB];
    float sc[KB];   // row scales of 8-bit router keys
    float rb[2 * PPL], qcs[2 * PPL];
    VR vr[VBS];
    // Upper levels that keep every candidate need no gathers: their kept
    // lists follow from the node counts alone, so they are taken here and the
    // first gathers are those of the first scored level.
    int lvl = levels;
    Step<T> st = make_step(lvl, 0);
    while (lvl >= 1 && st.take_all) {
        const int nxt = cur ^ 1;
        for (int i = tid; i < st.m; i += DNT) sm.sel[nxt][i] = (int)st.cs.id(i);
        if (tid == 0) sm.nsel[nxt] = st.m;
        if (lvl == 1 && tid < st.m && st.cs.id(tid) == last_leaf) sm.in_last = 1;
        __syncthreads();
        if (wg == 0 && a.sel) {
            int *o = a.sel + ((int64_t)unit * levels + (lvl - 1)) * a.sel_stride;
            for (int r = tid; r < a.sel_stride; r += DNT) o[r] = (r < st.m) ? sm.sel[nxt][r] : -1;
        }
        cur = nxt;
        --lvl;
        st = make_step(lvl, cur);
    }
    issue_step(st, k0, k1, sc, rb, vr, qcs);

    for (; lvl >= 1; --lvl) {
        const int nxt = cur ^ 1;
        const bool scored = !st.take_all;
        const int s0 = st.s0, ms = st.ms;
        float Mn[G], alpha[G];
        if (!scored) {
            for (int i = tid; i < st.m; i += DNT) sm.sel[nxt][i] = (int)st.cs.id(i);
            if (tid == 0) sm.nsel[nxt] = st.m;
            if (lvl == 1 && tid < st.m && st.cs.id(tid) == last_leaf) sm.in_last = 1;
            __syncthreads();
            if (wg == 0 && a.sel) {
                int *o = a.sel + ((int64_t)unit * levels + (lvl - 1)) * a.sel_stride;
                for (int r = tid; r < a.sel_stride; r += DNT) o[r] = (r < st.m) ? sm.sel[nxt][r] : -1;
            }
        } else {
        score(st, s0, ms, zb, k0, k1, sc, rb, qcs);
        __syncthreads();                                                   // B1
        new_max(Mn, alpha);

        // rank inside the slice: Gr threads per candidate, each comparing it
        // with a run of the (padded) slice, counts summed with DPP
        uint64_t *lw_words = xw + (int64_t)(lvl - 1) * W * kSlots;
        uint64_t *mine = lw_words + (int64_t)wg * kSlots;
        {
            int Gr = 16;
            while (Gr > 1 && Gr * ms > DNT) Gr >>= 1;
            const int ci = tid / Gr, cc = tid & (Gr - 1);
            const int ch = (((ms + Gr - 1) / Gr) + 3) & ~3;
            const bool valid = ci < ms;
            const float si = valid ? sm.s[ci] : -INFINITY;
            int rank = 0;
            for (int j = cc * ch; j < cc * ch + ch; j += 4) {
                const float4 v4 = *reinterpret_cast<const float4 *>(&sm.s[j]);
                rank += better(v4.x, j, si, ci) + better(v4.y, j + 1, si, ci) +
                        better(v4.z, j + 2, si, ci) + better(v4.w, j + 3, si, ci);
            }
            if (Gr >= 2) rank += dppi<0xB1>(rank);
            if (Gr >= 4) rank += dppi<0x4E>(rank);
            if (Gr >= 8) rank += dppi<0x141>(rank);
            if (Gr >= 16) rank += dppi<0x140>(rank);
            if (st.local) {
                // the whole level: the rank is the global rank
                if (valid && cc == 0 && rank < keff) {
                    sm.byrank[rank] = ci;
                    sm.byv[rank] = si;
                }
            } else {
            if (valid && cc == 0 && rank < keff)
                __hip_atomic_store(&mine[rank], pack_word(tag, (uint32_t)(s0 + ci), si), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if (tid >= ms && tid < keff)
                __hip_atomic_store(&mine[tid], pack_word(tag, 0xfffu, -INFINITY), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            if (topp && !st.local) {
                // this wave's (max, exp-sum) of the group scores it holds
                const bool own = valid && cc == 0;
                const float wmax = wave_max(own ? si : -INFINITY);
                const float wsum = wave_sum(own ? __expf(si - wmax) : 0.f);
                if (lane == 0) {
                    __hip_atomic_store(&mine[keff + 2 * wave], pack_word(tag, 0, wmax), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&mine[keff + 2 * wave + 1], pack_word(tag, 0, wsum), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }

        const int kp4 = (keff + 3) & ~3;
        int nkeep = min(keff, st.m);
        if (!st.local) {
        // collect every slice's words (bounded polling on the tag); list w
        // lands at xv/xi[w * kp4 ..], padded to a multiple of 4 entries
        const int nrow = kp4 + (topp ? 2 * DNW : 0);
        for (int e = tid; e < W * nrow; e += DNT) {
            const int w = e / nrow, r = e % nrow;
            if (r >= keff && r < kp4) {
                sm.xv[w * kp4 + r] = -INFINITY;
                sm.xi[w * kp4 + r] = 0x7fffffff;
                continue;
            }
            const int slot = r < keff ? r : r - kp4 + keff;
            const uint64_t *src = lw_words + (int64_t)w * kSlots + slot;
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
                sm.xv[w * kp4 + r] = (okw && ix != 0xfffu) ? word_val(word) : -INFINITY;
                sm.xi[w * kp4 + r] = (ix == 0xfffu) ? 0x7fffffff : (int)ix;
            } else {
                const int q = w * DNW + (slot - keff) / 2;
                if (((slot - keff) & 1) == 0) sm.xm[q] = okw ? word_val(word) : -INFINITY;
                else sm.xs[q] = okw ? word_val(word) : 0.f;
            }
        }
        __syncthreads();                                                   // B2

        // Merge.  Every list is sorted (slot r holds its slice's rank-r
        // entry), so an entry's global rank is its slot plus, for every other
        // list, the number of that list's entries ranking before it.  A group
        // of P lanes (P = W rounded up to a power of two) takes an entry and
        // lane j counts in list j -- by comparing with all of it for short
        // lists, by binary search otherwise -- and the group sums the counts
        // with DPP.
        const int ne = W * kp4;
        {
            int P = 1;
            while (P < W) P <<= 1;
            const int lg = tid & (P - 1);
            const int ngr = DNT / P;
            const uint32_t kinv = (65536u + kp4 - 1) / kp4;   // e / kp4 for e < 2^10
            const int lwo = min(lg, W - 1) * kp4;
            for (int e0 = tid / P; e0 - tid / P < ne; e0 += 2 * ngr) {
                float ve[2];
                int ie[2], cnt[2], wo[2];
                bool act[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = e0 + u * ngr;
                    const bool valid = e < ne;
                    ve[u] = valid ? sm.xv[e] : -INFINITY;
                    ie[u] = valid ? sm.xi[e] : 0x7fffffff;
                    wo[u] = (int)(((uint32_t)e * kinv) >> 16);
                    act[u] = lg < W && lg != wo[u] && ie[u] != 0x7fffffff;
                    cnt[u] = 0;
                }
                if (kp4 <= 16) {
                    for (int r = 0; r < kp4; r += 4) {
                        const float4 v4 = *reinterpret_cast<const float4 *>(&sm.xv[lwo + r]);
                        const int4 i4 = *reinterpret_cast<const int4 *>(&sm.xi[lwo + r]);
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            cnt[u] += better(v4.x, i4.x, ve[u], ie[u]) + better(v4.y, i4.y, ve[u], ie[u]) +
                                      better(v4.z, i4.z, ve[u], ie[u]) + better(v4.w, i4.w, ve[u], ie[u]);
                    }
                } else {
                    int lo[2] = {0, 0}, hi[2] = {kp4, kp4};
                    int nsteps = 0;
                    while ((1 << nsteps) <= kp4) ++nsteps;
                    for (int step = 0; step < nsteps; ++step) {
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int mid = (lo[u] + hi[u]) >> 1;
                            const int f = lwo + min(mid, kp4 - 1);
                            const bool active = lo[u] < hi[u];
                            const bool bt = better(sm.xv[f], sm.xi[f], ve[u], ie[u]);
                            lo[u] = (active && bt) ? mid + 1 : lo[u];
                            hi[u] = (active && !bt) ? mid : hi[u];
                        }
                    }
                    cnt[0] = lo[0];
                    cnt[1] = lo[1];
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = e0 + u * ngr;
                    int c = act[u] ? cnt[u] : 0;
                    if (P >= 2) c += dppi<0xB1>(c);
                    if (P >= 4) c += dppi<0x4E>(c);
                    if (P >= 8) c += dppi<0x141>(c);
                    if (P >= 16) c += dppi<0x140>(c);
                    const int rank = c + (e - wo[u] * kp4);
                    if (lg == 0 && e < ne && ie[u] != 0x7fffffff && rank < nkeep) {
                        sm.byrank[rank] = ie[u];
                        sm.byv[rank] = ve[u];
                    }
                }
            }
        }
        }
        __syncthreads();                                                   // B3
        if (topp) {
            // shortest prefix of the sorted kept entries whose softmax mass
            // (over every candidate of the level) reaches p
            if (wave == 0) {
                float gmax = -INFINITY, den = 0.f;
                if (st.local) {
                    for (int i = lane; i < st.m; i += 64) gmax = fmaxf(gmax, sm.s[i]);
                    gmax = wave_max(gmax);
                    for (int i = lane; i < st.m; i += 64) den += __expf(sm.s[i] - gmax);
                } else {
                    const int nw = W * DNW;
                    for (int i = lane; i < nw; i += 64) gmax = fmaxf(gmax, sm.xm[i]);
                    gmax = wave_max(gmax);
                    for (int i = lane; i < nw; i += 64)
                        if (sm.xm[i] > -INFINITY) den += sm.xs[i] * __expf(sm.xm[i] - gmax);
                }
                den = wave_sum(den);
                if (lane == 0) {
                    int ns = nkeep;
                    float cum = 0.f;
                    for (int r = 0; r < nkeep; ++r) {
                        cum += __expf(sm.byv[r] - gmax) / den;
                        if (cum >= a.p) {
                            ns = r + 1;
                            break;
                        }
                    }
                    sm.nkeep = ns;
                }
            }
            __syncthreads();
            nkeep = sm.nkeep;
        }
        // kept set in node order -> next candidate list, kept flags
        if (tid < nkeep) {
            const int ix = sm.byrank[tid];
            int pos = 0;
            int r = 0;
            for (; r + 4 <= nkeep; r += 4) {
                const int4 b4 = *reinterpret_cast<const int4 *>(&sm.byrank[r]);
                pos += (b4.x < ix) + (b4.y < ix) + (b4.z < ix) + (b4.w < ix);
            }
            for (; r < nkeep; ++r) pos += sm.byrank[r] < ix;
            const int64_t node = st.cs.id(ix);
            sm.sel[nxt][pos] = (int)node;
            if (ix >= s0 && ix < s0 + ms) sm.flag[ix - s0] = 1;
            if (lvl == 1 && node == last_leaf) sm.in_last = 1;
        }
        if (tid == 0) sm.nsel[nxt] = nkeep;
        __syncthreads();                                                   // B4
        if (wg == 0 && a.sel) {
            int *o = a.sel + ((int64_t)unit * levels + (lvl - 1)) * a.sel_stride;
            for (int r = tid; r < a.sel_stride; r += DNT) o[r] = (r < nkeep) ? sm.sel[nxt][r] : -1;
        }

        }
        // the next step's gathers go out now (one issue point for both paths,
        // so the loaded registers carry into the next iteration as they are);
        // this level's unkept candidates are folded while they are in flight
        const Step<T> stc = st;
        VR vrc[VBS];
#pragma unroll
        for (int u = 0; u < VBS; ++u) vrc[u] = vr[u];
        cur = nxt;
        st = make_step(lvl - 1, cur);
        issue_step(st, k0, k1, sc, rb, vr, qcs);
        if (scored && !a.leaf_only) {
            // this workgroup's own candidates only (a local level was scored
            // whole by every workgroup)
            const int zo = stc.local ? stc.fs0 : 0;
            probs(zo, zo + stc.fms, zb, true, Mn, alpha);
            __syncthreads();                                               // B5
            fold(stc, stc.fs0, stc.fms, zb, vrc, zo);
            zb ^= 1;
        }
    }

    // token level: this workgroup's range of the candidates, in chunks (the
    // first chunk's gathers were issued with the last level's)
    for (int c0 = st.s0; c0 < st.t1; c0 += kSlice) {
        const int ms = min(kSlice, st.t1 - c0);
        if (c0 != st.s0) {
            load_batch(st, c0, ms, 0, true, k0, k1, sc, rb);
            issue_values(st, c0, ms, true, vr);
        }
        score(st, c0, ms, zb, k0, k1, sc, rb, qcs);
        __syncthreads();
        float Mn[G], alpha[G];
        new_max(Mn, alpha);
        probs(0, ms, zb, false, Mn, alpha);
        __syncthreads();
        fold(st, c0, ms, zb, vr, 0);
        zb ^= 1;
    }

    // Partial state of this slice -> tagged words in the workspace; then every
    // workgroup merges a slice of the output columns from all W partials
    // (same exchange as the levels: a word is valid when its tag matches).
    uint64_t *pw_unit = ws.part + unit * (int64_t)W * G * (D + 2);
    {
        float *red = reinterpret_cast<float *>(hti_dec_lds);     // [DNW][G][D]
        float lsum[G];
#pragma unroll
        for (int h = 0; h < G; ++h) lsum[h] = wave_sum(lt[h]);
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < DPL; ++e) red[(wave * G + h) * D + lane * DPL + e] = acc[h][e];
            if (lane == 0) sm.redz[wave][h] = lsum[h];
        }
        __syncthreads();
        uint64_t *mine = pw_unit + (int64_t)wg * G * (D + 2);
        for (int i = tid; i < G * (D + 2); i += DNT) {
            const int h = i / (D + 2), e = i % (D + 2);
            float v = 0.f;
            if (e < D) {
                for (int w = 0; w < DNW; ++w) v += red[(w * G + h) * D + e];
            } else if (e == D) {
#pragma unroll
                for (int hh = 0; hh < G; ++hh) v = (hh == h) ? M[hh] : v;
            } else {
                for (int w = 0; w < DNW; ++w) v += sm.redz[w][h];
            }
            __hip_atomic_store(&mine[i], ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // Gather n tagged words (word i at src(i)) into LDS at dst(i): every load
    // is issued first, then only words whose tag is not yet current are polled.
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
    // columns of every slice's unnormalised output, into LDS (one round)
    const int cols = (D + W - 1) / W;
    const int d0 = min(D, wg * cols), d1 = min(D, d0 + cols);
    const int nc = d1 - d0;
    float *mw = reinterpret_cast<float *>(hti_dec_lds) + DNW * G * D;   // [W][G][2]
    float *aw = mw + kMaxW * G * 2;                                      // [W][G][nc]
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
            const float f = __expf(Mw - Mx);
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
            if (Mw != -INFINITY) den += mw[(w * G + h) * 2 + 1] * __expf(Mw - Mx);
        }
        a.lse[row + h] = den > 0.f ? Mx + logf(den) : -INFINITY;
    }
    // every workgroup of this unit has read the launch tag (they all published
    // their partial state above), so the next launch may move it on
    if (wg == 0 && tid == 0) ws.epoch[unit] = ws.epoch[unit] + 1u;
    // decode step: once every workgroup of the sequence has read the old
    // length (bounded wait), the first workgroup of its first unit stores the
    // new one and clears the count for the next step
    if (a.k_new != nullptr && wg == 0 && g == 0 && qi == 0 && tid == 0) {
        const uint32_t need = (uint32_t)W * (uint32_t)t.Hkv * (uint32_t)a.Nq;
        long spins = 0;
        while (__hip_atomic_load(&ws.seqcnt[bi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need &&
               ++spins < kSpin)
            __builtin_amdgcn_s_sleep(1);
        if (spins >= kSpin) __hip_atomic_store(&ws.err[unit], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (sm.app) __hip_atomic_store(&t.len[bi], (int64_t)sm.lold + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ws.seqcnt[bi], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int G, int D>
constexpr size_t dec_dyn_bytes()
{
    // per-wave partial outputs, then the gathered (max, denominator) and
    // output columns of every slice
    return (size_t)(DNW * G * D + kMaxW * G * 2 + kMaxW * G * ((D + kMaxW - 1) / kMaxW) + G * D) *
           sizeof(float);
}

template <typename T, int D, int G, bool F8>
static hipError_t dec_launch_k(const TravArgs &a, const DecodeWs &ws, int64_t units, hipStream_t s)
{
    auto kern = k_decode_split<T, D, G, F8>;
    const size_t dyn = dec_dyn_bytes<G, D>();
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
    // needs them resident together.  The plan keeps the grid within what the
    // device holds at once (one workgroup per compute unit, or as many as the
    // occupancy admits), so they all are whenever the device is not held by
    // other work; every wait is bounded and a timeout shows as NaN
    // output (a cooperative launch would guarantee residency but costs more
    // than the whole kernel to dispatch).
    return hipLaunchKernel((const void *)kern, dim3((unsigned)(units * ws.W)), dim3(DNT), args, dyn, s);
}

// 8-bit router keys: bf16 caches only
template <typename T, int D, int G>
static hipError_t dec_launch(const TravArgs &a, const DecodeWs &ws, int64_t units, hipStream_t s)
{
    if constexpr (std::is_same<T, bf16_t>::value)
        if (a.t.rfp8) return dec_launch_k<T, D, G, true>(a, ws, units, s);
    if (a.t.rfp8) return hipErrorInvalidValue;
    return dec_launch_k<T, D, G, false>(a, ws, units, s);
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
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k_decode_split<T, D, G, false>, DNT,
                                                        dec_dyn_bytes<G, D>());
}

template <typename T, int D>
static hipError_t dec_capacity_g(int G, int *per_cu)
{
    switch (G) {
    case 1: return dec_capacity<T, D, 1>(per_cu);
    case 2: return dec_capacity<T, D, 2>(per_cu);
    case 4: return dec_capacity<T, D, 4>(per_cu);
    default: return dec_capacity<T, D, 8>(per_cu);
    }
}

hipError_t decode_split_plan(const TravArgs &a, int64_t units, int64_t max_summary, int *W)
{
    static int cached_key = -1, cached_cus = 0, cached_per_cu = 0;
    const int key = a.t.dtype * 1000 + a.t.D * 10 + a.t.G;
    if (key != cached_key) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (a.t.dtype == HTI_BF16)
            e = a.t.D == 128 ? dec_capacity_g<bf16_t, 128>(a.t.G, &per_cu) : dec_capacity_g<bf16_t, 64>(a.t.G, &per_cu);
        else
            e = a.t.D == 128 ? dec_capacity_g<float, 128>(a.t.G, &per_cu) : dec_capacity_g<float, 64>(a.t.G, &per_cu);
        if (e != hipSuccess) return e;
        cached_key = key;
        cached_cus = cus;
        cached_per_cu = per_cu;
    }
    // one workgroup per CU keeps every unit's slices on distinct CUs; more
    // per CU (as many as fit, at most four) only where fewer leave a unit
    // short of its slices or of eight workgroups (measured at 1M tokens:
    // eight per unit beat four and sixteen)
    const int64_t need = (max_summary + kSlice - 1) / kSlice;
    const int64_t want = std::max<int64_t>(need, 8);
    int64_t w = 0;
    for (int per = 1; per <= std::min(cached_per_cu, 4); ++per) {
        w = (int64_t)cached_cus * per / (units > 0 ? units : 1);
        if (w >= want) break;
    }
    if (w > kMaxW) w = kMaxW;
    *W = (w >= need && w >= 1 && need <= kMaxW) ? (int)w : 0;
    return hipSuccess;
}

size_t decode_ws_bytes(int B, int64_t units, int W, int levels, int G, int D)
{
    size_t off = 0;
    off += ((size_t)units * 4 + 255) / 256 * 256;                 // epoch
    off += ((size_t)units * 4 + 255) / 256 * 256;                 // err
    off += ((size_t)units * (levels > 0 ? levels : 1) * W * kSlots * 8 + 255) / 256 * 256;
    off += ((size_t)units * W * G * (D + 2) * 8 + 255) / 256 * 256;
    off += ((size_t)B * 4 + 255) / 256 * 256;                     // seqcnt
    return off;
}
DecodeWs decode_ws_layout(void *base, int B, int64_t units, int W, int levels, int G, int D)
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
    p += ((size_t)units * W * G * (D + 2) * 8 + 255) / 256 * 256;
    w.seqcnt = (uint32_t *)p;
    (void)B;
    return w;
}

} // namespace hti
