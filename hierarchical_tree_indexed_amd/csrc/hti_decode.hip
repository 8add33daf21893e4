// hti_decode.hip -- decode traversal split across workgroups.
//
// The method is the one of hti_traverse.hip ("Recursive Sparse Attention",
// abstract: per-level top-k over a tree of pooled summaries, unselected
// summaries sharing one softmax with the exact tokens, candidate-index RoPE;
// "Subquadratic Attention with a Hierarchical Tree-Structured Indexer",
// Figure 3 caption: top-p routing, reference-query keys).  Decode has few
// (query, KV group) units -- 32 at batch 4 with 8 KV heads -- so each unit
// is split over W workgroups (W * units ~ the CU count) that each take a
// contiguous slice of every level's candidate list:
//
//   * the slice's key rows go straight into registers (16 lanes per row, a
//     few rows per 16-lane group) and its value rows likewise, all loads of a
//     level issued back to back as soon as the previous level's kept set is
//     known;
//   * scores become 64-bit selection keys (order-preserving score bits over
//     the complemented candidate index, so that one unsigned comparison is
//     the tie rule: higher score, then lower index) and ranks are counted,
//     every wave against its share of the keys, the shares summed in LDS;
//   * a workgroup publishes its slice's best k as 64-bit words carrying a
//     per-launch tag (agent-scope atomics: a word is valid exactly when its
//     tag matches), reads every slice's words, and ranks those the same way;
//     a level of at most kSlice candidates is scored whole by every
//     workgroup, which selects on its own;
//   * every wave derives the kept set in candidate order itself (no further
//     barrier), issues the next level's loads, and folds the level's unkept
//     candidates of its own slice while they are in flight;
//   * each workgroup publishes its partial softmax state the same way and
//     merges a slice of the output columns from all W of them.
//
// Softmax state: one running maximum per head, identical in every thread of
// the workgroup (taken from per-wave maxima after the scoring barrier); the
// denominators and outputs are per-thread partial sums rescaled by the same
// factors and reduced once at the end.
//
// The workgroups of a launch wait on each other, so they must be resident
// together: the grid is kept within what the device holds at once, and every
// wait is bounded.  A wait that runs out sets the workspace's status word:
// the outputs of that launch and of every later launch with the same
// workspace are NaN (and no length advances) until the caller zeroes the
// workspace again; hti_decode_status reads the word.
#include <algorithm>
#include <mutex>
#include <vector>

#include "hti_device.h"
#include "hti_internal.h"
#include "hti_pool.h"
#include "hti_trav_common.h"

namespace hti {

namespace {

constexpr int DNT = 256;              // threads per workgroup (one wave per SIMD)
constexpr int DNW = DNT / 64;         // waves
constexpr int DNQ = DNT / 16;         // 16-lane rows ("quarters")
constexpr int kSlice = 128;           // candidates one workgroup scores at once
constexpr int kMaxW = HTI_DECODE_MAX_SPLIT;
constexpr int kSlots = kMaxSel + 2;   // words per (level, workgroup): k entries, top-p (max, exp-sum)
constexpr int kMaxEnt = kMaxW * kMaxSel;   // entries of one exchange
constexpr int kSelN = kSlice + kMaxEnt;    // selection entries of one level: slice, then exchange
constexpr int KB = 4;                 // key rows per quarter per batch
constexpr int VB = 3;                 // value rows per quarter held in registers (more are loaded at the fold)
constexpr long kSpin = 1L << 22;      // polls of one word before a wait gives up



// Phase timeline (a separate build of this file with HTI_DECODE_TIMELINE
// defined, for measurement only): thread 0 of every workgroup notes the
// constant-rate clock at each phase boundary in LDS and copies the list to
// the workspace at the end (kTlEvents words per workgroup, after the status
// word).  Event word: phase << 52 | level << 48 | clock.
constexpr int kTlEvents = 64;
constexpr int kTlMaxBlocks = 8192;
#ifdef HTI_DECODE_TIMELINE
#define DTL(ph, lv)                                                                                  \
    do {                                                                                             \
        if (tid == 0 && tln < kTlEvents)                                                             \
            sm.tl[tln] = ((uint64_t)(ph) << 52) | ((uint64_t)((lv) & 15) << 48) |                     \
                         (__builtin_amdgcn_s_memrealtime() & 0xffffffffffffull);                      \
        ++tln;                                                                                       \
    } while (0)
constexpr size_t kTlBytes = (size_t)kTlMaxBlocks * kTlEvents * 8;
#else
#define DTL(ph, lv) do {} while (0)
constexpr size_t kTlBytes = 0;
#endif

template <int G>
struct DSmem {
    // selection entries of the two most recent levels (by parity): keys,
    // group scores, candidate indices and per-wave partial ranks; entries
    // [0, kSlice) are the scored slice, [kSlice, kSelN) the exchange
    uint64_t key[2][kSelN] __attribute__((aligned(16)));
    float esc[2][kSelN];
    int16_t eix[2][kSelN];
    uint8_t prt[2][DNW][kSelN];
    float z[2][kSlice * G];           // [candidate][head] logits of the scored slice / chunk
    float qraw[G * 128] __attribute__((aligned(16)));
    float redz[2][DNW][G];            // per-wave maxima of the logits (by the parity of sm.z)
    // per wave: the kept set in candidate order (node ids, candidate
    // indices) by level parity, and the kept entries by rank
    int wsel[2][DNW][kMaxSel];
    int wcix[2][DNW][kMaxSel];
    int wrix[DNW][kMaxSel];
    float wrsc[DNW][kMaxSel];
    uint8_t wflag[2][DNW][kSlice] __attribute__((aligned(4)));   // per wave: kept flags of its fold slice
    uint64_t wkx[DNW][128] __attribute__((aligned(16)));   // per wave: the exchange keys it read
    float xm[kMaxW], xs[kMaxW];       // top-p: each slice's (max, exp-sum) of group scores
    int n[HTI_MAX_LEVELS + 1];        // nodes per level (n[0] = tokens)
    const void *lkp[HTI_MAX_LEVELS];  // this unit's level keys / values
    const void *lvp[HTI_MAX_LEVELS];
    const uint8_t *lkq[HTI_MAX_LEVELS];   // 8-bit router keys and their row scales
    const float *lks[HTI_MAX_LEVELS];
    uint32_t tag;                     // this launch's tag of the exchange words
    uint32_t st0;                     // the workspace status at the start
    int app;                          // decode step: the new token goes in at position lold
    int lold;                         // sequence length before the step
    int bad;                          // a wait of this workgroup ran out
    int last;                         // this workgroup arrived last at the unit's final merge
#ifdef HTI_DECODE_TIMELINE
    uint64_t tl[kTlEvents];
#endif
};

__device__ __forceinline__ uint64_t pack_word(uint32_t tag, uint32_t idx, float v)
{
    return ((uint64_t)tag << 44) | ((uint64_t)(idx & 0xfffu) << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> 44); }
__device__ __forceinline__ uint32_t word_idx(uint64_t w) { return (uint32_t)(w >> 32) & 0xfffu; }
__device__ __forceinline__ float word_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Selection key: larger means kept first (higher score, then lower index);
// -0 counts as +0, as in a float comparison.
__device__ __forceinline__ uint64_t sel_key(float s, int ix)
{
    uint32_t u = __float_as_uint(s + 0.f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - (uint32_t)ix);
}

// Order this wave's LDS accesses (lanes read what other lanes of the same
// wave wrote just before): the LDS executes one wave's accesses in order, so
// only the compiler must be kept from moving them.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Value row slice of one lane: EPL consecutive elements.
template <typename T, int EPL> struct VRow;
template <> struct VRow<bf16_t, 8> {
    uint4 r;
    __device__ __forceinline__ void load(gptr<bf16_t> p) { r = gload<uint4>(p); }
    __device__ __forceinline__ void get(float *o) const
    {
        cvt(make_uint2(r.x, r.y), o);
        cvt(make_uint2(r.z, r.w), o + 4);
    }
};
template <> struct VRow<bf16_t, 4> {
    uint2 r;
    __device__ __forceinline__ void load(gptr<bf16_t> p) { r = gload<uint2>(p); }
    __device__ __forceinline__ void get(float *o) const { cvt(r, o); }
};
template <> struct VRow<float, 8> {
    float4 a, b;
    __device__ __forceinline__ void load(gptr<float> p)
    {
        a = gload<float4>(p);
        b = gload<float4>(p + 4);
    }
    __device__ __forceinline__ void get(float *o) const
    {
        cvt(a, o);
        cvt(b, o + 4);
    }
};
template <> struct VRow<float, 4> {
    float4 a;
    __device__ __forceinline__ void load(gptr<float> p) { a = gload<float4>(p); }
    __device__ __forceinline__ void get(float *o) const { cvt(a, o); }
};

// Candidates of one step (a summary level or the token level) as seen by one
// workgroup: the list, where its keys and values live, and this workgroup's
// slices of it.
template <typename T>
struct Step {
    Cands cs;
    gptr<T> kb, vb;      // key / value rows of this unit: row r at kb + (r * nref + j) * D
    gptr<uint8_t> kq;    // summary levels with 8-bit router keys: the E4M3 rows, likewise,
    gptr<float> ks;      // and their scales, row r * nref + j
    int nref;            // keys per row (R at summary levels, 1 at tokens)
    int m;               // candidates
    int s0, ms;          // candidates this workgroup scores (the first chunk at the token level)
    int t1;              // token level: end of this workgroup's range
    int fs0, fms;        // candidates whose values this workgroup folds (its own slice)
    int qpos;            // RoPE position of the query
    bool take_all;       // every candidate is kept (no scoring)
    bool local;          // the level fits one slice: every workgroup scores all of it and
                         // selects on its own, without exchanging lists
    bool tok;            // the token level
};

} // namespace

// x is a multiple of f (a mask when f is a power of two)
__device__ __forceinline__ bool completes(uint32_t x, int f)
{
    return (f & (f - 1)) == 0 ? (x & (uint32_t)(f - 1)) == 0u : x % (uint32_t)f == 0u;
}

// OCC: the waves per SIMD the instance is built for.  OCC = 2 caps it at 256
// registers per lane (at some spill cost), so that the plan can place two
// workgroups per CU where one per CU leaves a unit short of workgroups.  At
// 1M tokens, batch 16 ran W = 2 at 74 us per step and W = 4 at two per CU
// 47 us.  The plan uses OCC = 1 wherever one workgroup per CU suffices.
template <typename T, int D, int G, bool F8, int OCC>
__global__ __launch_bounds__(DNT, OCC) void k_decode_split(TravArgs a, DecodeWs ws)
{
    constexpr int PPL = D / 32;                        // rotate-half pairs per lane of a key row
    constexpr int EPL = D / 16;                        // elements per lane of a value row
    using KR = typename Raw<T, PPL>::type;
    using VR = VRow<T, EPL>;
    __shared__ DSmem<G> sm;
    extern __shared__ __attribute__((aligned(16))) unsigned char hti_dec_lds[];

    const TreeArgs &t = a.t;
    // Every 64-byte line of the argument block goes into the scalar cache in
    // one round trip, before the first field is used: each launch's arguments
    // are fresh memory, and fields read later, one line at a time as the code
    // first needs them, would each wait for their own miss.
    // (Written out as one block of scalar loads and a single wait: left to
    // the compiler, the loads went out in two batches with a wait between,
    // two round trips.)  The segment also holds the hidden arguments after
    // the explicit ones, so the fourteenth line is inside it.
    int W = ws.W;
    {
        const auto kp = __builtin_amdgcn_kernarg_segment_ptr();
        static_assert((sizeof(TravArgs) + sizeof(DecodeWs) + 63) / 64 + 1 == 14, "argument block lines");
        uint32_t x[14];
        asm volatile("s_load_dword %0, %14, 0x0\n\t"
                     "s_load_dword %1, %14, 0x40\n\t"
                     "s_load_dword %2, %14, 0x80\n\t"
                     "s_load_dword %3, %14, 0xc0\n\t"
                     "s_load_dword %4, %14, 0x100\n\t"
                     "s_load_dword %5, %14, 0x140\n\t"
                     "s_load_dword %6, %14, 0x180\n\t"
                     "s_load_dword %7, %14, 0x1c0\n\t"
                     "s_load_dword %8, %14, 0x200\n\t"
                     "s_load_dword %9, %14, 0x240\n\t"
                     "s_load_dword %10, %14, 0x280\n\t"
                     "s_load_dword %11, %14, 0x2c0\n\t"
                     "s_load_dword %12, %14, 0x300\n\t"
                     "s_load_dword %13, %14, 0x340\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&s"(x[0]), "=&s"(x[1]), "=&s"(x[2]), "=&s"(x[3]), "=&s"(x[4]), "=&s"(x[5]),
                       "=&s"(x[6]), "=&s"(x[7]), "=&s"(x[8]), "=&s"(x[9]), "=&s"(x[10]), "=&s"(x[11]),
                       "=&s"(x[12]), "=&s"(x[13])
                     : "s"(kp)
                     : "memory");
        uint32_t touch = 0;
#pragma unroll
        for (int i = 0; i < 14; ++i) touch ^= x[i];
        asm volatile("" : "+s"(W) : "s"(touch));
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sub = lane & 15, quarter = tid >> 4;
    // grid: (workgroup of the unit, routing head, sequence x query)
    const int wg = (int)blockIdx.x;
    const int g = (int)blockIdx.y;
    const int qi = a.Nq == 1 ? 0 : (int)(blockIdx.z % (uint32_t)a.Nq);
    const int bi = a.Nq == 1 ? (int)blockIdx.z : (int)(blockIdx.z / (uint32_t)a.Nq);
    const int64_t unit = (int64_t)blockIdx.z * t.Hkv + g;
    const int64_t bh = (int64_t)bi * (t.Hkv / t.hdiv) + g / t.hdiv;   // tree slot of routing head g
    const int b = t.b, levels = t.levels, R = t.R;
    const int fan = __builtin_amdgcn_readfirstlane(t.fan);
    const uint32_t binv = __builtin_amdgcn_readfirstlane(a.binv), finv = __builtin_amdgcn_readfirstlane(a.finv);
    const int keff = (a.mode == HTI_TOPK) ? a.k : a.cap;
    const bool topp = a.mode == HTI_TOPP;
    uint64_t *xw = ws.words + (int64_t)unit * levels * W * kSlots;
    const int64_t orow = ((int64_t)bi * a.Nq + qi) * t.Hq + (int64_t)g * G;
    int tln = 0;
    (void)tln;
    DTL(1, 0);

    // ---- start: every load that does not depend on the length goes out
    // first (the query, the decode step's new row of this unit's KV head,
    // the RoPE angle steps; unconditional, so the compiler's wait counts
    // stay exact), then the length, the launch epoch and the workspace
    // status: one round trip for all of them ----
    constexpr int EPC = 16 / (int)sizeof(T);           // elements per 16-byte chunk
    static_assert(G * D / EPC <= DNT, "one chunk of the query per thread");
    static_assert(D / EPC <= 64, "the new row in one wave");
    const gptr<T> qsrc = to_global<T>(a.q) + orow * D;
    const uint4 qx = gload<uint4>(qsrc + (tid < G * D / EPC ? tid : 0) * EPC);
    // (without a new row, the query stands in as the source: read, not used)
    const int nl = tid & (D / EPC - 1);
    const uint4 knx = gload<uint4>((a.k_new ? to_global<T>(a.k_new) + bh * D : qsrc) + nl * EPC);
    const uint4 vnx = gload<uint4>((a.k_new ? to_global<T>(a.v_new) + bh * D : qsrc) + nl * EPC);
    const gptr<float2> rope = to_global<float2>(t.rope);
    // angle step of each of this lane's RoPE frequencies (row 1 of the table)
    float st_c[PPL], st_s[PPL];
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        const float2 c2 = gload<float2>(rope + (D / 2) + sub * PPL + e);
        st_c[e] = c2.x;
        st_s[e] = c2.y;
    }
    if (tid == 0) {
        const int64_t len0 = t.len[bi];
        const uint32_t epoch = ws.epoch[unit];
        const uint32_t st0 = __hip_atomic_load(ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.tag = (epoch % 0xffffeu) + 1u;
        sm.st0 = st0;
        DTL(20, 0);
        int n = (int)len0;
        // decode step: this workgroup appends the new token itself (every
        // workgroup of every query of the sequence writes the same bytes) and
        // walks the tree with the new length; it counts itself as having read
        // the old length, which one workgroup replaces at the end
        const bool app = st0 == 0u && a.k_new != nullptr && (int64_t)n < t.ncap[0];
        sm.app = app ? 1 : 0;
        sm.lold = n;
        sm.bad = 0;
        if (a.k_new != nullptr && st0 == 0u)
            __hip_atomic_fetch_add(&ws.seqcnt[bi], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (app) ++n;
        // a query at position q_pos attends to the tree of tokens 0..q_pos
        if (a.q_pos) {
            const int64_t ql = a.q_pos[(int64_t)bi * a.Nq + qi];
            if (ql < (int64_t)n - 1) n = ql < 0 ? 0 : (int)(ql + 1);
        }
        sm.n[0] = n;
        for (int l = 1; l <= levels; ++l) {
            const int f = l == 1 ? b : fan;           // children per node of level l
            n = (f & (f - 1)) == 0 ? (n >> __builtin_ctz((unsigned)f)) : n / f;
            sm.n[l] = n;
        }
    }
    if (tid == 64) {
        // this unit's level arrays (constant indices into the argument block,
        // so scalar loads, all issued together; entries past `levels` are
        // never read)
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
    // the query into LDS
    if (tid < G * D / EPC) {
        float *qd = sm.qraw + tid * EPC;
        if constexpr (sizeof(T) == 2) {
            cvt(make_uint2(qx.x, qx.y), qd);
            cvt(make_uint2(qx.z, qx.w), qd + 4);
        } else {
            qd[0] = __uint_as_float(qx.x);
            qd[1] = __uint_as_float(qx.y);
            qd[2] = __uint_as_float(qx.z);
            qd[3] = __uint_as_float(qx.w);
        }
        DTL(21, 0);
    }
    float M[G], lt[G], acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        M[h] = -INFINITY;
        lt[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }
    __syncthreads();
    DTL(2, 0);
    const uint32_t tag = sm.tag;
    if (__builtin_expect(sm.st0 != 0u, 0)) {
        // an earlier launch with this workspace ran out of a wait: NaN, no
        // other effect, until the workspace is zeroed
        const int cols = (D + W - 1) / W;
        const int d0 = min(D, wg * cols), d1 = min(D, d0 + cols);
        for (int i = tid; i < G * (d1 - d0); i += DNT)
            a.out[(orow + i / (d1 - d0)) * D + d0 + i % (d1 - d0)] = __uint_as_float(0x7fc00000u);
        if (wg == 0 && tid < G && a.lse) a.lse[orow + tid] = __uint_as_float(0x7fc00000u);
        return;
    }
    if (sm.app) {
        // the new row of this unit's KV head at position lold, then every
        // node it completes, level by level (one wave pools)
        const int64_t Lold = sm.lold;
        T *kw = (T *)t.kc + (bh * t.ncap[0] + Lold) * D;
        T *vw = (T *)t.vc + (bh * t.ncap[0] + Lold) * D;
        if (tid < D / EPC) {
            *reinterpret_cast<uint4 *>(kw + tid * EPC) = knx;
            *reinterpret_cast<uint4 *>(vw + tid * EPC) = vnx;
        }
        DTL(22, 0);
        // (lengths are below 2^31 here: 32-bit index arithmetic, a mask and
        // a shift when a fan-in is a power of two)
        uint32_t idx = (uint32_t)Lold + 1u;
        // Only a token that completes a node needs the row in place before
        // anything else (its pooling reads it): otherwise the stores complete
        // in the background, long before the token level reads the row.
        if (__builtin_expect(levels > 0 && completes(idx, b), 0)) {
            __syncthreads();
            for (int l = 1; l <= levels; ++l) {
                const int f = l == 1 ? b : fan;       // children per node of level l
                if (!completes(idx, f)) break;
                idx = (f & (f - 1)) == 0 ? idx >> __builtin_ctz((unsigned)f) : idx / (uint32_t)f;
                if (wave == 0) pool_node<T, D, 8>(t, l, bh, g / t.hdiv, (int64_t)idx - 1, lane);
                __syncthreads();
            }
        }
    }
    const int L = sm.n[0];
    const int last_leaf = L > 0 ? (L - 1) / b : -1;   // level-1 node of the query token
    DTL(19, 0);

    const gptr<T> kc = to_global<T>(t.kc) + bh * t.ncap[0] * D;
    const gptr<T> vc = to_global<T>(t.vc) + bh * t.ncap[0] * D;

    // ---- the candidates of a step ----
    // level lvl >= 1 (parents: this wave's kept list of parity cur, nprev of
    // them) or the token level (lvl == 0)
    auto make_step = [&](int lvl, int cur, int nprev) __attribute__((always_inline)) -> Step<T> {
        Step<T> st;
        st.tok = lvl == 0;
        const bool top = (lvl == levels);
        st.cs.selp = sm.wsel[cur][wave];
        st.cs.nprev = top ? 0 : nprev;
        // children per parent: b tokens under a level-1 node, fan nodes above
        // (values read once below: a select between two argument fields
        // would become a load through a selected argument address, which
        // puts part of the argument block in scratch)
        const int fb = lvl == 0 ? b : fan;
        st.cs.b = fb;
        st.cs.binv = lvl == 0 ? binv : finv;
        st.cs.top = top;
        const int orph0 = top ? 0 : fb * sm.n[lvl + 1];
        st.cs.orph0 = orph0;
        if (lvl >= 1) {
            st.m = top ? sm.n[lvl] : nprev * fb + (sm.n[lvl] - orph0);
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
            bool in = top || (L - 1 >= orph0);
            for (int r = 0; r < nprev && !in; ++r) in = sm.wsel[cur][wave][r] == last_leaf;
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
    // One batch of a quarter's keys: its items it0.. (item = candidate x
    // reference key), at most KB of them.  Lane `sub` derives the row of item
    // it0 + sub (clamped into the batch, so surplus loads re-read a row of
    // it) and DPP row broadcasts hand row u to the whole quarter, so the
    // loads go out back to back.  Also the RoPE row of the batch's first
    // candidate.  The number of loads is fixed (go == false reads the RoPE
    // table instead): the compiler then knows exactly how many loads each
    // later wait may leave in flight.
    auto load_batch = [&](const Step<T> &st, int s0, int ms, int it0, bool go, KR (&k0)[KB], KR (&k1)[KB],
                          float (&sc)[KB], float (&rb)[2 * PPL]) __attribute__((always_inline)) {
        const int nref = st.nref;
        const int cpq = (ms + DNQ - 1) / DNQ;
        const int c_beg = min(ms, quarter * cpq);
        const int c_end = min(ms, c_beg + cpq);
        const int nitems = (c_end - c_beg) * nref;
        const int nb = min(nitems - it0, KB);
        const int itl = it0 + (nb > 0 ? min(sub, nb - 1) : 0);
        const int cl = itl / nref;
        const int cand = min(c_beg + cl, ms - 1);
        const uint32_t row = go ? (uint32_t)(st.cs.id(s0 + max(cand, 0)) * nref + (itl - cl * nref)) : 0u;
        if (F8 && !st.tok) {
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
    // value rows of the fold slice: quarter q owns rows q, q + DNQ, ...
    // (rows past the slice re-read its last row)
    // (a fixed number of loads: rows past the slice re-read its last row, and
    // go == false reads the RoPE table)
    auto issue_values = [&](const Step<T> &st, int s0, int ms, bool go, VR (&vr)[VB]) __attribute__((always_inline)) {
        int64_t rid[VB];
#pragma unroll
        for (int u = 0; u < VB; ++u) rid[u] = go ? st.cs.id(s0 + max(0, min(quarter + DNQ * u, ms - 1))) : 0;
        const gptr<T> vbase = go ? st.vb : to_global<T>(t.rope);
#pragma unroll
        for (int u = 0; u < VB; ++u) vr[u].load(vbase + (size_t)rid[u] * D + sub * EPL);
    };
    // the loads of a step: its first key batch and the query's RoPE row
    // (its value rows go out separately, once the previous step's are folded)
    auto issue_step = [&](const Step<T> &st, KR (&k0)[KB], KR (&k1)[KB], float (&sc)[KB],
                          float (&rb)[2 * PPL], float (&qcs)[2 * PPL]) __attribute__((always_inline)) {
        load_batch(st, st.s0, st.ms, 0, !st.take_all && st.ms > 0, k0, k1, sc, rb);
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

    // (the token level's values, or a summary level's when its unkept
    // candidates are attended)
    auto step_values = [&](const Step<T> &st, VR (&vr)[VB]) __attribute__((always_inline)) {
        issue_values(st, st.fs0, st.fms, !st.take_all && st.fms > 0 && (st.tok || !a.leaf_only), vr);
    };

    // ---- scoring ----
    // Rotated query of this lane's elements (sub*PPL.., and the rotate-half
    // partners), then the slice's keys in quarter batches: per-head logits
    // into sm.z[zb], selection entries (key, score, index) into the level's
    // slice entries, per-wave maxima of the logits into sm.redz.
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
        float zmaxh = -INFINITY;               // of the lane's head
        float *zz = sm.z[zb];
        uint64_t *ek = sm.key[zb];
        float *es = sm.esc[zb];
        int16_t *ei = sm.eix[zb];
        // slots [ms, 64) hold zero keys, which beat nothing (rank_le64 reads
        // whole 16-key batches)
        if (tid >= ms && tid < 64) ek[tid] = 0ull;
        // the running best over a candidate's reference keys carries across
        // batches (a batch may end inside a candidate)
        int ci = c_beg, j = 0;
        float best = -INFINITY, zbh = 0.f;
        float cc[PPL], ss[PPL];
        for (int it0 = 0; it0 < nitems; it0 += KB) {
            const int nb = min(nitems - it0, KB);
            if (it0 > 0) load_batch(st, s0, ms, it0, true, k0, k1, sc, rb);
            if (it0 == 0 || j == 0) {
                // (a batch that starts a candidate starts at the RoPE row
                // just loaded; one that continues a candidate keeps its row)
#pragma unroll
                for (int e = 0; e < PPL; ++e) {
                    cc[e] = rb[2 * e];
                    ss[e] = rb[2 * e + 1];
                }
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
                            ek[ci] = sel_key(best, s0 + ci);
                            es[ci] = best;
                            ei[ci] = (int16_t)(s0 + ci);
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
        // lane h * LPH of each quarter holds that quarter's maximum of head
        // h: combine the wave's four quarters
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m4 = fmaxf(fmaxf(rlane(zmaxh, h * LPH), rlane(zmaxh, 16 + h * LPH)),
                                   fmaxf(rlane(zmaxh, 32 + h * LPH), rlane(zmaxh, 48 + h * LPH)));
            if (lane == 0) sm.redz[zb][wave][h] = m4;
        }
    };

    // ---- selection ----
    // Partial ranks: entry e (of the n from `base` in the parity-zb arrays)
    // counted against this wave's share of the same entries; after a barrier
    // rank(e) = the sum over waves.
    auto partial_ranks = [&](int zb, int base, int n) __attribute__((always_inline)) {
        const int j0 = base + n * wave / DNW, j1 = base + n * (wave + 1) / DNW;
        const uint64_t *kk = sm.key[zb];
        for (int e = base + lane; e < base + n; e += 64) {
            const uint64_t ke = kk[e];
            int c = 0;
            for (int j = j0; j < j1; ++j) c += (int)(kk[j] > ke);
            sm.prt[zb][wave][e] = (uint8_t)c;
        }
    };
    auto rank_of = [&](int zb, int e) __attribute__((always_inline)) -> int {
        int r = 0;
#pragma unroll
        for (int w = 0; w < DNW; ++w) r += sm.prt[zb][w][e];
        return r;
    };
    // Entries held in registers, two per lane (entry lane and lane + 64): up
    // to 128 of them, compared by readlane broadcasts with no LDS round trip.
    struct Ents {
        uint64_t k[2];
        int ix[2];
        float sc[2];
    };
    auto ents_from_slice = [&](int zb, int n, Ents &E) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int e = lane + 64 * t;
            const bool v = e < n;
            E.k[t] = v ? sm.key[zb][e] : 0ull;
            E.ix[t] = v ? (int)sm.eix[zb][e] : 0;
            E.sc[t] = v ? sm.esc[zb][e] : -INFINITY;
        }
    };
    // how many of the keys kk[j0 .. j1) (uniform bounds; LDS, read by every
    // lane at the same address) beat each entry; eight reads go out before
    // the first comparison
    auto count_range = [&](const uint64_t *kk, const Ents &E, int j0, int j1, int (&c)[2])
        __attribute__((always_inline)) {
        c[0] = c[1] = 0;
        j0 = __builtin_amdgcn_readfirstlane(j0);
        j1 = __builtin_amdgcn_readfirstlane(j1);
        for (int jb = j0; jb < j1; jb += 8) {
            uint64_t kj[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) kj[u] = kk[min(jb + u, j1 - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const bool in = jb + u < j1;
                c[0] += (int)(in && kj[u] > E.k[0]);
                c[1] += (int)(in && kj[u] > E.k[1]);
            }
        }
    };
    // Rank of one entry per lane among n <= 64 selection keys kk[0 .. n) in
    // LDS (how many of them beat it), the slots [n, 64) holding zero keys,
    // which beat nothing.  Keys are read two per 16-byte LDS access, a batch
    // of 16 per round trip, with no bounds to test.  With n <= 32 the entry
    // is lane & 31 and each half of the wave counts 16 of the slots (lanes
    // 0-31 slots 0-15, lanes 32-63 slots 16-31), the halves summed by one
    // lane swap; otherwise the entry is `lane` and every lane counts the
    // first ceil(n / 16) batches.  Lanes past the n entries get a rank of no
    // meaning.
    auto rank_le64 = [&](const uint64_t *kk, int n) __attribute__((always_inline)) -> int {
        n = __builtin_amdgcn_readfirstlane(n);
        const bool split = n <= 32;
        const int e = split ? (lane & 31) : lane;
        const uint64_t ke = kk[max(0, min(e, n - 1))];
        const int j0 = split ? ((lane & 32) >> 1) : 0;
        const int nb = split ? 1 : (n + 15) >> 4;
        int c = 0;
        for (int bt = 0; bt < nb; ++bt) {
            const ulonglong2 *kp = reinterpret_cast<const ulonglong2 *>(kk + j0 + 16 * bt);
            ulonglong2 kj[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) kj[u] = kp[u];
#pragma unroll
            for (int u = 0; u < 8; ++u) c += (int)(kj[u].x > ke) + (int)(kj[u].y > ke);
        }
        if (split) {
            const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)c, (uint32_t)c, false, false);
            c = (int)(r[0] + r[1]);
        }
        return c;
    };
    // Kept set from the ranks of the n entries held in registers, which run
    // in increasing candidate order over (t, lane): the first nav by rank
    // (top-p: the shortest prefix reaching mass p), in candidate order, into
    // this wave's lists of parity nxt.  Returns the kept count.
    auto finalize_regs = [&](const Ents &E, const int (&rank)[2], int n, int m, const Cands &cs, int nxt,
                             float gmax, float den, int fs0, int fms) __attribute__((always_inline)) -> int {
        const int nav = min(keff, m);
        uint32_t *fw = reinterpret_cast<uint32_t *>(sm.wflag[nxt][wave]);
        if (lane < kSlice / 4) fw[lane] = 0u;
        int nkeep = nav;
        if (topp) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (lane + 64 * t < n && rank[t] < nav) sm.wrsc[wave][rank[t]] = E.sc[t];
            wave_sync();
            int ns = nav;
            if (lane == 0) {
                float cum = 0.f;
                for (int r = 0; r < nav; ++r) {
                    cum += __expf(sm.wrsc[wave][r] - gmax) / den;
                    if (cum >= a.p) {
                        ns = r + 1;
                        break;
                    }
                }
            }
            nkeep = max(1, min(__builtin_amdgcn_readfirstlane(ns), a.cap));
        }
        bool kept[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) kept[t] = lane + 64 * t < n && rank[t] < nkeep;
        // the entries run in candidate order over (t, lane): a kept entry's
        // place is the number of kept entries before it
        const uint64_t b0 = __ballot(kept[0]), b1 = __ballot(kept[1]);
        int pos[2];
        pos[0] = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b0, 0u));
        pos[1] = __builtin_popcountll(b0) +
                 (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b1, 0u));
        wave_sync();
#pragma unroll
        for (int t = 0; t < 2; ++t)
            if (kept[t]) {
                const int ix = E.ix[t];
                sm.wcix[nxt][wave][pos[t]] = ix;
                sm.wsel[nxt][wave][pos[t]] = (int)cs.id(ix);
                if (ix >= fs0 && ix < fs0 + fms) sm.wflag[nxt][wave][ix - fs0] = 1;
            }
        wave_sync();
        return nkeep;
    };
    // Kept set from the ranks of n entries (from `base`): the first nav by
    // rank (top-p: the shortest prefix whose mass over every candidate,
    // max gmax and denominator den, reaches p), in candidate order, into
    // this wave's lists of parity nxt.  Returns the kept count.
    auto finalize = [&](int zb, int base, int n, int m, const Cands &cs, int nxt, float gmax, float den, int fs0,
                        int fms) __attribute__((always_inline)) -> int {
        const int nav = min(keff, m);
        uint32_t *fw = reinterpret_cast<uint32_t *>(sm.wflag[nxt][wave]);
        if (lane < kSlice / 4) fw[lane] = 0u;
        for (int e = base + lane; e < base + n; e += 64) {
            const int r = rank_of(zb, e);
            if (r < nav) {
                sm.wrix[wave][r] = sm.eix[zb][e];
                sm.wrsc[wave][r] = sm.esc[zb][e];
            }
        }
        wave_sync();
        int nkeep = nav;
        if (topp) {
            int ns = nav;
            if (lane == 0) {
                float cum = 0.f;
                for (int r = 0; r < nav; ++r) {
                    cum += __expf(sm.wrsc[wave][r] - gmax) / den;
                    if (cum >= a.p) {
                        ns = r + 1;
                        break;
                    }
                }
            }
            nkeep = max(1, min(__builtin_amdgcn_readfirstlane(ns), a.cap));
        }
        if (lane < nkeep) {
            const int ix = sm.wrix[wave][lane];
            int pos = 0;
            for (int r = 0; r < nkeep; ++r) pos += (int)(sm.wrix[wave][r] < ix);
            sm.wcix[nxt][wave][pos] = ix;
            sm.wsel[nxt][wave][pos] = (int)cs.id(ix);
            if (ix >= fs0 && ix < fs0 + fms) sm.wflag[nxt][wave][ix - fs0] = 1;
        }
        wave_sync();
        return nkeep;
    };

    // the running max takes in this step's per-wave maxima (the same in
    // every thread) and what was accumulated under the old one is rescaled;
    // folds at any later point then take their terms against the current max
    auto new_max = [&](int zb) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mm = M[h];
#pragma unroll
            for (int w = 0; w < DNW; ++w) mm = fmaxf(mm, sm.redz[zb][w][h]);
            const float alpha = (mm == -INFINITY) ? 1.f : __expf(M[h] - mm);
            lt[h] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
            M[h] = mm;
        }
    };
    // softmax terms of this quarter's fold rows (candidates fs0 + quarter +
    // DNQ u; logits at z index c - zo) times their value rows; kept ones
    // (flags of parity nxt, when `kept` is set) drop out.  Each lane takes
    // the exponential of its own head (head sub / (16 / G)) and the quarter
    // hands the G of them round by DPP row broadcasts.
    auto fold = [&](int fs0, int fms, int zo, int zb, int nxt, bool kept, const VR (&vr)[VB], gptr<T> vsrc,
                    const Cands &vcs) __attribute__((always_inline)) {
        constexpr int LPH = 16 / G;
        const int hsel = sub / LPH;
        // this lane's head's running max, by masks (an indexed pick would put
        // M in private memory)
        uint32_t mb = 0u;
#pragma unroll
        for (int h = 0; h < G; ++h) mb |= (0u - (uint32_t)(hsel == h)) & __float_as_uint(M[h]);
        const float Mh = __uint_as_float(mb);
        auto add_row = [&](int i, const VR &row) __attribute__((always_inline)) {
            const int c = fs0 + i;
            const bool k = kept && sm.wflag[nxt][wave][i] != 0;
            const float pl = k ? 0.f : __expf(sm.z[zb][(c - zo) * G + hsel] - Mh);
            float v[EPL];
            row.get(v);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = __int_as_float(row_bcast(__float_as_int(pl), h * LPH));
                lt[h] += p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
            }
        };
#pragma unroll
        for (int u = 0; u < VB; ++u)
            if (quarter + DNQ * u < fms) add_row(quarter + DNQ * u, vr[u]);
        for (int i = quarter + DNQ * VB; i < fms; i += DNQ) {
            VR row;
            row.load(vsrc + (size_t)vcs.id(fs0 + i) * D + sub * EPL);
            add_row(i, row);
        }
    };
    auto write_sel = [&](int lvl, int nxt, int nkeep) __attribute__((always_inline)) {
        if (wg == 0 && wave == 0 && a.sel) {
            int *o = a.sel + ((int64_t)unit * levels + (lvl - 1)) * a.sel_stride;
            for (int r = lane; r < a.sel_stride; r += 64) o[r] = (r < nkeep) ? sm.wsel[nxt][0][r] : -1;
        }
    };

    // ---- the steps ----
    int cur = 0, zb = 0, nsel = 0;
    KR k0[KB], k1[KB];
    float sc[KB];   // row scales of 8-bit router keys
    float rb[2 * PPL], qcs[2 * PPL];
    VR vr[VB];
    // Upper levels that keep every candidate need no gathers: their kept
    // lists follow from the node counts alone (every wave takes them itself).
    int lvl = levels;
    Step<T> st = make_step(lvl, 0, 0);
    while (lvl >= 1 && st.take_all) {
        const int nxt = cur ^ 1;
        for (int i = lane; i < st.m; i += 64) {
            sm.wsel[nxt][wave][i] = (int)st.cs.id(i);
            sm.wcix[nxt][wave][i] = i;
        }
        wave_sync();
        nsel = st.m;
        write_sel(lvl, nxt, nsel);
        cur = nxt;
        --lvl;
        st = make_step(lvl, cur, nsel);
    }
    DTL(17, lvl);
    issue_step(st, k0, k1, sc, rb, qcs);
    DTL(18, lvl);
    step_values(st, vr);
    DTL(3, lvl);

    // A summary level's unkept candidates are folded one level later, while
    // the next level's exchange is in flight (or before the token level's
    // fold): the pending level's slice, logits, kept flags and value rows.
    bool pend = false;
    int p_fs0 = 0, p_fms = 0, p_zo = 0, p_zb = 0, p_par = 0;
    Step<T> p_st = st;
    VR vrp[VB];
    auto fold_pending = [&]() __attribute__((always_inline)) {
        if (pend) fold(p_fs0, p_fms, p_zo, p_zb, p_par, true, vrp, p_st.vb, p_st.cs);
        pend = false;
    };
    for (; lvl >= 1; --lvl) {
        const int nxt = cur ^ 1;
        const int s0 = st.s0, ms = st.ms;
        int nkeep;
        if (st.take_all) {
            // (a lower level can keep everything when an upper one kept few)
            for (int i = lane; i < st.m; i += 64) {
                sm.wsel[nxt][wave][i] = (int)st.cs.id(i);
                sm.wcix[nxt][wave][i] = i;
            }
            wave_sync();
            nkeep = st.m;
        } else {
            score(st, s0, ms, zb, k0, k1, sc, rb, qcs);
            __syncthreads();                                           // B1: slice entries, logits
            DTL(4, lvl);
            if (!a.leaf_only) new_max(zb);
            DTL(23, lvl);
            const int ne = W * keff;                                   // exchanged entries
            if (st.local) {
                fold_pending();
                // the whole level: ranks among all of it (every wave counts
                // against its share of the keys), selected locally
                Ents E;
                ents_from_slice(zb, ms, E);
                int rk[2];
                if (ms <= 64) {
                    // (every wave ranks all of them itself: no barrier)
                    rk[0] = rank_le64(sm.key[zb], ms);
                    rk[1] = 1 << 20;
                    DTL(5, lvl);
                } else {
                    int c[2];
                    count_range(sm.key[zb], E, ms * wave / DNW, ms * (wave + 1) / DNW, c);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        if (lane + 64 * t < ms) sm.prt[zb][wave][lane + 64 * t] = (uint8_t)c[t];
                    __syncthreads();                                   // B2
                    DTL(5, lvl);
#pragma unroll
                    for (int t = 0; t < 2; ++t) rk[t] = lane + 64 * t < ms ? rank_of(zb, lane + 64 * t) : 1 << 20;
                }
                float gmax = -INFINITY, den = 0.f;
                if (topp) {
                    gmax = wave_max(fmaxf(E.sc[0], E.sc[1]));
                    den = wave_sum((E.sc[0] > -INFINITY ? __expf(E.sc[0] - gmax) : 0.f) +
                                   (E.sc[1] > -INFINITY ? __expf(E.sc[1] - gmax) : 0.f));
                }
                nkeep = finalize_regs(E, rk, ms, st.m, st.cs, nxt, gmax, den, st.fs0, st.fms);
            } else if (ne <= 128) {
                uint64_t *lw_words = xw + (int64_t)(lvl - 1) * W * kSlots;
                if (wave == 0) {
                    // this slice's ranks (wave 0 alone) and its best keff as
                    // words
                    Ents S;
                    ents_from_slice(zb, ms, S);
                    DTL(25, lvl);
#ifdef HTI_DECODE_TIMELINE
                    __builtin_amdgcn_s_waitcnt(0x0f70);   // (vector memory drained: measurement only)
                    DTL(26, lvl);
#endif
                    int c[2];
                    if (ms <= 64) {
                        c[0] = rank_le64(sm.key[zb], ms);
                        c[1] = 1 << 20;
                    } else {
                        count_range(sm.key[zb], S, 0, ms, c);
                    }
                    DTL(24, lvl);
                    uint64_t *mine = lw_words + (int64_t)wg * kSlots;
                    // the best keff go out in candidate order (slot = the
                    // number of them before it in the slice), so that the
                    // W lists read back run in candidate order too
                    const bool pub0 = lane < ms && c[0] < keff, pub1 = lane + 64 < ms && c[1] < keff;
                    const uint64_t q0 = __ballot(pub0), q1 = __ballot(pub1);
                    const int slot0 =
                        (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(q0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)q0, 0u));
                    const int slot1 = __builtin_popcountll(q0) + (int)__builtin_amdgcn_mbcnt_hi(
                                                                     (uint32_t)(q1 >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)q1, 0u));
                    if (pub0)
                        __hip_atomic_store(&mine[slot0], pack_word(tag, (uint32_t)S.ix[0], S.sc[0]), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    if (pub1)
                        __hip_atomic_store(&mine[slot1], pack_word(tag, (uint32_t)S.ix[1], S.sc[1]), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    if (lane >= ms && lane < keff)
                        __hip_atomic_store(&mine[lane], pack_word(tag, 0xfffu, -INFINITY), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    if (topp) {
                        const float wmax = wave_max(fmaxf(S.sc[0], S.sc[1]));
                        const float wsum = wave_sum((S.sc[0] > -INFINITY ? __expf(S.sc[0] - wmax) : 0.f) +
                                                    (S.sc[1] > -INFINITY ? __expf(S.sc[1] - wmax) : 0.f));
                        if (lane == 0) {
                            __hip_atomic_store(&mine[keff], pack_word(tag, 0, wmax), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                            __hip_atomic_store(&mine[keff + 1], pack_word(tag, 0, wsum), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                    DTL(6, lvl);
                }
                // the previous level's fold, while the other slices' words
                // are on their way
                fold_pending();
                // every wave reads all W * keff words itself (lane e: entry
                // e and e + 64; bounded polling on the tag)
                auto poll = [&](const uint64_t *src, bool &okw) __attribute__((always_inline)) -> uint64_t {
                    uint64_t word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    long spins = 0;
                    while (word_tag(word) != tag && ++spins < kSpin) {
                        __builtin_amdgcn_s_sleep(1);
                        word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    okw = word_tag(word) == tag;
                    if (!okw) sm.bad = 1;
                    return word;
                };
                Ents X;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int e = lane + 64 * t;
                    X.k[t] = 0ull;
                    X.ix[t] = 0;
                    X.sc[t] = -INFINITY;
                    if (e < ne) {
                        const int w = e / keff;
                        bool okw;
                        const uint64_t word = poll(lw_words + (int64_t)w * kSlots + (e - w * keff), okw);
                        const uint32_t ix = okw ? word_idx(word) : 0xfffu;
                        if (ix != 0xfffu) {
                            X.k[t] = sel_key(word_val(word), (int)ix);
                            X.ix[t] = (int)ix;
                            X.sc[t] = word_val(word);
                        }
                    }
                }
                float gmax = -INFINITY, den = 0.f;
                if (topp) {
                    float xm = -INFINITY, xs = 0.f;
                    if (lane < W) {
                        bool ok1, ok2;
                        const uint64_t w1 = poll(lw_words + (int64_t)lane * kSlots + keff, ok1);
                        const uint64_t w2 = poll(lw_words + (int64_t)lane * kSlots + keff + 1, ok2);
                        xm = ok1 ? word_val(w1) : -INFINITY;
                        xs = ok2 ? word_val(w2) : 0.f;
                    }
                    gmax = wave_max(xm);
                    den = wave_sum(xm > -INFINITY ? xs * __expf(xm - gmax) : 0.f);
                }
                DTL(7, lvl);
                int rk[2];
                if (ne <= 64) {
                    // (X.k is zero past the entries: the slots [ne, 64) are
                    // zero keys; every wave ranks all of them itself)
                    sm.wkx[wave][lane] = X.k[0];
                    wave_sync();
                    rk[0] = rank_le64(sm.wkx[wave], ne);
                    rk[1] = 1 << 20;
                    DTL(8, lvl);
                } else {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        if (lane + 64 * t < ne) sm.wkx[wave][lane + 64 * t] = X.k[t];
                    wave_sync();
                    int c[2];
                    count_range(sm.wkx[wave], X, ne * wave / DNW, ne * (wave + 1) / DNW, c);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        if (lane + 64 * t < ne) sm.prt[zb][wave][kSlice + lane + 64 * t] = (uint8_t)c[t];
                    __syncthreads();                                   // B2
                    DTL(8, lvl);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        rk[t] = lane + 64 * t < ne ? rank_of(zb, kSlice + lane + 64 * t) : 1 << 20;
                }
                nkeep = finalize_regs(X, rk, ne, st.m, st.cs, nxt, gmax, den, st.fs0, st.fms);
            } else {
                uint64_t *lw_words = xw + (int64_t)(lvl - 1) * W * kSlots;
                partial_ranks(zb, 0, ms);
                __syncthreads();                                       // B2
                DTL(5, lvl);
                if (wave == 0) {
                    // this slice's best keff, as words at slot = rank
                    uint64_t *mine = lw_words + (int64_t)wg * kSlots;
                    for (int e = lane; e < ms; e += 64) {
                        const int r = rank_of(zb, e);
                        if (r < keff)
                            __hip_atomic_store(&mine[r], pack_word(tag, (uint32_t)sm.eix[zb][e], sm.esc[zb][e]),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    for (int r = ms + lane; r < keff; r += 64)
                        __hip_atomic_store(&mine[r], pack_word(tag, 0xfffu, -INFINITY), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    if (topp) {
                        float wmax = -INFINITY, wsum = 0.f;
                        for (int i = lane; i < ms; i += 64) wmax = fmaxf(wmax, sm.esc[zb][i]);
                        wmax = wave_max(wmax);
                        for (int i = lane; i < ms; i += 64) wsum += __expf(sm.esc[zb][i] - wmax);
                        wsum = wave_sum(wsum);
                        if (lane == 0) {
                            __hip_atomic_store(&mine[keff], pack_word(tag, 0, wmax), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                            __hip_atomic_store(&mine[keff + 1], pack_word(tag, 0, wsum), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
                DTL(6, lvl);
                fold_pending();
                // every slice's words (bounded polling on the tag) -> the
                // exchange entries at [kSlice, kSlice + W * keff)
                const int ne = W * keff;
                const int nw = ne + (topp ? 2 * W : 0);
                for (int i = tid; i < nw; i += DNT) {
                    const int w = i < ne ? i / keff : (i - ne) >> 1;
                    const int slot = i < ne ? i - w * keff : keff + ((i - ne) & 1);
                    const uint64_t *src = lw_words + (int64_t)w * kSlots + slot;
                    uint64_t word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    long spins = 0;
                    while (word_tag(word) != tag && ++spins < kSpin) {
                        __builtin_amdgcn_s_sleep(1);
                        word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    const bool okw = word_tag(word) == tag;
                    if (!okw) sm.bad = 1;
                    if (i < ne) {
                        const uint32_t ix = okw ? word_idx(word) : 0xfffu;
                        const bool real = ix != 0xfffu;
                        sm.key[zb][kSlice + i] = real ? sel_key(word_val(word), (int)ix) : 0ull;
                        sm.esc[zb][kSlice + i] = real ? word_val(word) : -INFINITY;
                        sm.eix[zb][kSlice + i] = (int16_t)(real ? ix : 0);
                    } else if (slot == keff) {
                        sm.xm[w] = okw ? word_val(word) : -INFINITY;
                    } else {
                        sm.xs[w] = okw ? word_val(word) : 0.f;
                    }
                }
                __syncthreads();                                       // B3
                DTL(7, lvl);
                partial_ranks(zb, kSlice, ne);
                __syncthreads();                                       // B4
                DTL(8, lvl);
                float gmax = -INFINITY, den = 0.f;
                if (topp) {
                    for (int w = lane; w < W; w += 64) gmax = fmaxf(gmax, sm.xm[w]);
                    gmax = wave_max(gmax);
                    for (int w = lane; w < W; w += 64)
                        if (sm.xm[w] > -INFINITY) den += sm.xs[w] * __expf(sm.xm[w] - gmax);
                    den = wave_sum(den);
                }
                nkeep = finalize(zb, kSlice, ne, st.m, st.cs, nxt, gmax, den, st.fs0, st.fms);
            }
        }
        DTL(9, lvl);
        write_sel(lvl, nxt, nkeep);

        // this level's fold becomes pending (its own candidates only; a
        // local level was scored whole by every workgroup, so its logits sit
        // at the candidate index), and the next step's keys and value rows
        // go out
        if (!st.take_all && !a.leaf_only) {
            pend = true;
            p_fs0 = st.fs0;
            p_fms = st.fms;
            p_zo = st.local ? 0 : st.s0;
            p_zb = zb;
            p_par = nxt;
            p_st = st;
#pragma unroll
            for (int u = 0; u < VB; ++u) vrp[u] = vr[u];
        }
        const bool scored = !st.take_all;
        st = make_step(lvl - 1, nxt, nkeep);
        issue_step(st, k0, k1, sc, rb, qcs);
        step_values(st, vr);
        DTL(10, lvl);
        if (scored) zb ^= 1;
        cur = nxt;
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
        DTL(12, 0);
        new_max(zb);
        fold_pending();
        fold(c0, ms, c0, zb, cur, false, vr, st.vb, st.cs);
        DTL(13, 0);
        zb ^= 1;
    }
    fold_pending();     // (a token level with no candidates for this workgroup)

    // Partial state of this workgroup: the quarters' sums within each wave by
    // lane swaps, then across waves in LDS; stored (fp32) in the workspace and
    // released before one arrival count per unit.  The workgroup that arrives
    // last acquires, merges every output column from all W partial states and
    // writes the outputs; the others are done.
    float *pf_unit = ws.part + unit * (int64_t)W * G * (D + 2);
    {
        float *red = reinterpret_cast<float *>(hti_dec_lds);     // [DNW][G][D], then [DNW][G] sums
        float *redl = red + DNW * G * D;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float l4 = xsum32(xsum16(lt[h]));
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = xsum32(xsum16(acc[h][e]));
            if (lane < 16) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) red[(wave * G + h) * D + sub * EPL + e] = acc[h][e];
            }
            if (lane == 0) redl[wave * G + h] = l4;
        }
        __syncthreads();
        float *mine = pf_unit + (int64_t)wg * G * (D + 2);
        for (int i = tid; i < G * (D + 2); i += DNT) {
            const int h = i / (D + 2), e = i % (D + 2);
            float v = 0.f;
            if (e < D) {
#pragma unroll
                for (int w = 0; w < DNW; ++w) v += red[(w * G + h) * D + e];
            } else if (e == D) {
#pragma unroll
                for (int hh = 0; hh < G; ++hh) v = (hh == h) ? M[hh] : v;
            } else {
#pragma unroll
                for (int w = 0; w < DNW; ++w) v += redl[w * G + h];
            }
            // (agent-scope stores reach the point where every XCD sees them;
            // an agent-scope release fence would write back the whole L2)
            __hip_atomic_store(reinterpret_cast<uint32_t *>(mine + i), __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // a wait that ran out in this workgroup goes to the status word before
    // the arrival, so the merging workgroup sees it
    if (tid == 0 && sm.bad) __hip_atomic_store(ws.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every store of this workgroup has completed before its arrival is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    DTL(14, 0);
    if (tid == 0) {
        const uint32_t n = __hip_atomic_fetch_add(&ws.arrive[unit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.last = (n == (uint32_t)W - 1u);
    }
    __syncthreads();
    DTL(15, 0);
    bool failed;
    if (sm.last) {
        // a wait that ran out in any workgroup of this launch, or before (the
        // status word), leaves NaN
        failed = sm.bad != 0 || __hip_atomic_load(ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
        auto ld = [](const float *p) __attribute__((always_inline)) {
            return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
        };
        for (int i = tid; i < G * D; i += DNT) {
            const int h = i / D, c = i % D;
            // (all W slices' values read first, then combined in slice order)
            float Mw[kMaxW], Lw[kMaxW], Aw[kMaxW];
#pragma unroll
            for (int w = 0; w < kMaxW; ++w) {
                const float *pw = pf_unit + ((int64_t)w * G + h) * (D + 2);
                Mw[w] = w < W ? ld(pw + D) : -INFINITY;
                Lw[w] = w < W ? ld(pw + D + 1) : 0.f;
                Aw[w] = w < W ? ld(pw + c) : 0.f;
            }
            float Mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kMaxW; ++w) Mx = fmaxf(Mx, Mw[w]);
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int w = 0; w < kMaxW; ++w) {
                const float f = Mw[w] == -INFINITY ? 0.f : __expf(Mw[w] - Mx);
                num += Aw[w] * f;
                den += Lw[w] * f;
            }
            a.out[(orow + h) * D + c] = failed ? __uint_as_float(0x7fc00000u) : den > 0.f ? num / den : 0.f;
            if (c == 0 && a.lse)
                a.lse[orow + h] = failed ? __uint_as_float(0x7fc00000u) : den > 0.f ? Mx + logf(den) : -INFINITY;
        }
        // every workgroup of this unit has read the launch tag (each read it
        // on entry, before its arrival), so the next launch may move it on;
        // the count starts from zero again
        if (tid == 0) {
            ws.epoch[unit] = ws.epoch[unit] + 1u;
            __hip_atomic_store(&ws.arrive[unit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        failed = sm.bad != 0 || __hip_atomic_load(ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    }
    DTL(16, 0);
#ifdef HTI_DECODE_TIMELINE
    const int64_t lin = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    if (tid == 0 && lin < kTlMaxBlocks) {
        uint64_t *tr = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(ws.status) + 256) + lin * kTlEvents;
        for (int i = 0; i < kTlEvents; ++i) tr[i] = i < tln ? sm.tl[i] : 0ull;
    }
#endif
    // decode step: once every workgroup of the sequence has read the old
    // length (bounded wait), the first workgroup of its first unit stores the
    // new one and clears the count for the next step; if the wait runs out,
    // the length stays and the status word is set
    if (a.k_new != nullptr && wg == 0 && g == 0 && qi == 0 && tid == 0) {
        const uint32_t need = (uint32_t)W * (uint32_t)t.Hkv * (uint32_t)a.Nq;
        long spins = 0;
        while (__hip_atomic_load(&ws.seqcnt[bi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need &&
               ++spins < kSpin)
            __builtin_amdgcn_s_sleep(1);
        if (spins >= kSpin || failed) {
            __hip_atomic_store(ws.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (sm.app)
                __hip_atomic_store(&t.len[bi], (int64_t)sm.lold + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ws.seqcnt[bi], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int G, int D>
constexpr size_t dec_dyn_bytes()
{
    // per-wave partial outputs and sums
    return (size_t)(DNW * G * D + DNW * G) * sizeof(float);
}

namespace {

// Per-device, per-instance facts the host side caches: whether the dynamic
// LDS attribute was set and how many workgroups of the instance one CU holds.
struct DecInstInfo {
    bool attr = false;
    int per_cu = 0;
};
std::mutex g_dec_mu;
std::vector<std::pair<std::pair<int, const void *>, DecInstInfo>> g_dec_info;   // (device, kernel) -> info
std::vector<std::pair<int, int>> g_dev_cus;                                       // device -> CU count

DecInstInfo &dec_info_locked(int dev, const void *kern)
{
    for (auto &p : g_dec_info)
        if (p.first.first == dev && p.first.second == kern) return p.second;
    g_dec_info.push_back({{dev, kern}, DecInstInfo{}});
    return g_dec_info.back().second;
}

template <typename T, int D, int G, bool F8, int OCC>
hipError_t dec_prepare(int dev, DecInstInfo *out)
{
    auto kern = k_decode_split<T, D, G, F8, OCC>;
    const size_t dyn = dec_dyn_bytes<G, D>();
    std::lock_guard<std::mutex> lk(g_dec_mu);
    DecInstInfo &info = dec_info_locked(dev, (const void *)kern);
    if (!info.attr) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, DNT, dyn);
        if (e != hipSuccess) return e;
        info.per_cu = per_cu;
        info.attr = true;
    }
    *out = info;
    return hipSuccess;
}

template <typename T, int D, int G, bool F8, int OCC>
hipError_t dec_launch_k(const TravArgs &a, const DecodeWs &ws, int64_t units, hipStream_t s)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    DecInstInfo info;
    if ((e = dec_prepare<T, D, G, F8, OCC>(dev, &info)) != hipSuccess) return e;
    TravArgs aa = a;
    DecodeWs ww = ws;
    void *args[] = {&aa, &ww};
    // A plain launch: the workgroups of a unit wait for each other, which
    // needs them resident together.  The plan keeps the grid within what the
    // device holds at once, so they all are whenever the device is not held
    // by other work; every wait is bounded and a timeout sets the status
    // word (a cooperative launch would guarantee residency but costs more
    // than the whole kernel to dispatch).
    const unsigned heads = (unsigned)a.t.Hkv;
    return hipLaunchKernel((const void *)k_decode_split<T, D, G, F8, OCC>,
                           dim3((unsigned)ws.W, heads, (unsigned)(units / heads)), dim3(DNT), args,
                           dec_dyn_bytes<G, D>(), s);
}

// Dispatch over the instances: 8-bit router keys with bf16 caches only.
template <typename T, int D, int G, typename Fn>
hipError_t dec_dispatch_f8(bool rfp8, Fn &&fn)
{
    if constexpr (std::is_same<T, bf16_t>::value)
        if (rfp8) return fn(std::integral_constant<bool, true>{});
    if (rfp8) return hipErrorInvalidValue;
    return fn(std::integral_constant<bool, false>{});
}

template <typename T, int D, typename Fn>
hipError_t dec_dispatch_g(int G, bool rfp8, Fn &&fn)
{
    auto go = [&](auto gc) {
        constexpr int GG = decltype(gc)::value;
        return dec_dispatch_f8<T, D, GG>(rfp8, [&](auto f8) { return fn(std::integral_constant<int, GG>{}, f8); });
    };
    switch (G) {
    case 1: return go(std::integral_constant<int, 1>{});
    case 2: return go(std::integral_constant<int, 2>{});
    case 4: return go(std::integral_constant<int, 4>{});
    default: return go(std::integral_constant<int, 8>{});
    }
}

template <typename Fn>
hipError_t dec_dispatch(const TravArgs &a, Fn &&fn)
{
    const bool r8 = a.t.rfp8 != 0;
    auto with = [&](auto tc, auto dc) {
        using TT = typename decltype(tc)::type;
        constexpr int DD = decltype(dc)::value;
        return dec_dispatch_g<TT, DD>(a.t.G, r8, [&](auto gc, auto f8) {
            return fn(tc, dc, gc, f8);
        });
    };
    struct BF { using type = bf16_t; };
    struct FP { using type = float; };
    if (a.t.dtype == HTI_BF16)
        return a.t.D == 128 ? with(BF{}, std::integral_constant<int, 128>{}) : with(BF{}, std::integral_constant<int, 64>{});
    return a.t.D == 128 ? with(FP{}, std::integral_constant<int, 128>{}) : with(FP{}, std::integral_constant<int, 64>{});
}

} // namespace

hipError_t launch_decode_split(const TravArgs &a, const DecodeWs &ws, int64_t units, int occ, hipStream_t s)
{
    if (units <= 0) return hipSuccess;
    return dec_dispatch(a, [&](auto tc, auto dc, auto gc, auto f8) {
        using TT = typename decltype(tc)::type;
        constexpr int DD = decltype(dc)::value, GG = decltype(gc)::value;
        constexpr bool FF = decltype(f8)::value;
        return occ == 2 ? dec_launch_k<TT, DD, GG, FF, 2>(a, ws, units, s)
                        : dec_launch_k<TT, DD, GG, FF, 1>(a, ws, units, s);
    });
}

hipError_t decode_split_plan(const TravArgs &a, int64_t units, int64_t max_summary, int *W, int *occ)
{
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> lk(g_dec_mu);
        for (auto &p : g_dev_cus)
            if (p.first == dev) cus = p.second;
    }
    if (cus == 0) {
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        std::lock_guard<std::mutex> lk(g_dec_mu);
        g_dev_cus.push_back({dev, cus});
    }
    // occupancy of the two instances (one and two waves per SIMD)
    int per1 = 0, per2 = 0;
    e = dec_dispatch(a, [&](auto tc, auto dc, auto gc, auto f8) {
        using TT = typename decltype(tc)::type;
        constexpr int DD = decltype(dc)::value, GG = decltype(gc)::value;
        constexpr bool FF = decltype(f8)::value;
        DecInstInfo i1, i2;
        hipError_t r = dec_prepare<TT, DD, GG, FF, 1>(dev, &i1);
        if (r == hipSuccess) r = dec_prepare<TT, DD, GG, FF, 2>(dev, &i2);
        per1 = i1.per_cu;
        per2 = i2.per_cu;
        return r;
    });
    if (e != hipSuccess) return e;
    // one workgroup per CU keeps every unit's slices on distinct CUs; more
    // per CU (as many as fit, at most four) only where fewer leave a unit
    // short of its slices or of eight workgroups
    const int64_t need = (max_summary + kSlice - 1) / kSlice;
    const int64_t want = std::max<int64_t>(need, 8);
    // the uncapped instance where one workgroup per CU gives every unit its
    // wanted width (or the capped one holds no more per CU); else the capped
    // one, with as many per CU as it holds
    const bool one_fits = (int64_t)cus / (units > 0 ? units : 1) >= want;
    const int o = (one_fits || per2 <= per1) ? 1 : 2;
    const int per_cu = o == 2 ? per2 : per1;
    *occ = o;
    int64_t w = 0;
    for (int per = 1; per <= std::min(per_cu, 4); ++per) {
        w = (int64_t)cus * per / (units > 0 ? units : 1);
        if (w >= want) break;
    }
    if (w > kMaxW) w = kMaxW;
    // (few units: no more workgroups than the wanted width)
    if (w > want) w = want;
    // every workgroup ranks all W * keff exchanged entries; up to 128 of them
    // are ranked in registers, more take the slower path through LDS: fewer
    // workgroups per unit where that still covers the level's slices
    const int keff = a.mode == HTI_TOPK ? a.k : a.cap;
    const int64_t fast = 128 / (keff > 0 ? keff : 1);
    if (fast >= need && w > fast) w = fast;
    *W = (w >= need && w >= 1 && need <= kMaxW) ? (int)w : 0;
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// The split decode's workspace for callers that cannot allocate: a static
// device array (every GPU the library runs on holds its own copy until the
// process ends).  In host code `scratch` only names the symbol; its device
// address on the current device comes from hipGetSymbolAddress, taken once
// per device and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scr_mu;
std::vector<std::pair<int, void *>> g_scr_ptr;     // device -> address of its scratch

__global__ void k_fill_zero(uint4 *p, int64_t n16)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

} // namespace

hipError_t decode_static_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_scr_mu);
    for (auto &p : g_scr_ptr)
        if (p.first == dev) {
            *ptr = p.second;
            return hipSuccess;
        }
    void *q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scr_ptr.push_back({dev, q});
    *ptr = q;
    return hipSuccess;
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s)
{
    const int64_t n16 = (int64_t)((bytes + 15) / 16);
    if (n16 == 0) return hipSuccess;
    const int blocks = (int)std::min<int64_t>(1024, (n16 + 255) / 256);
    hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, s, (uint4 *)p, n16);
    return hipGetLastError();
}

size_t decode_ws_bytes(int B, int64_t units, int W, int levels, int G, int D)
{
    size_t off = 0;
    off += 256;                                                   // status
    off += kTlBytes;                                              // phase timeline (timeline build)
    off += ((size_t)units * 4 + 255) / 256 * 256;                 // epoch
    off += ((size_t)units * 4 + 255) / 256 * 256;                 // arrival counts
    off += ((size_t)units * (levels > 0 ? levels : 1) * W * kSlots * 8 + 255) / 256 * 256;
    off += ((size_t)units * W * G * (D + 2) * 4 + 255) / 256 * 256;
    off += ((size_t)B * 4 + 255) / 256 * 256;                     // seqcnt
    return off;
}
DecodeWs decode_ws_layout(void *base, int B, int64_t units, int W, int levels, int G, int D)
{
    DecodeWs w{};
    char *p = (char *)base;
    w.W = W;
    w.status = (uint32_t *)p;
    p += 256 + kTlBytes;
    w.epoch = (uint32_t *)p;
    p += ((size_t)units * 4 + 255) / 256 * 256;
    w.arrive = (uint32_t *)p;
    p += ((size_t)units * 4 + 255) / 256 * 256;
    w.words = (uint64_t *)p;
    p += ((size_t)units * (levels > 0 ? levels : 1) * W * kSlots * 8 + 255) / 256 * 256;
    w.part = (float *)p;
    p += ((size_t)units * W * G * (D + 2) * 4 + 255) / 256 * 256;
    w.seqcnt = (uint32_t *)p;
    (void)B;
    return w;
}

} // namespace hti
