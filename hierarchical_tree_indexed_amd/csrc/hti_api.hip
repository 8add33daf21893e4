// hti_api.hip -- the C ABI: argument validation, buffer plan, launches.
// Every check happens on the host before anything is enqueued; on error the
// device state is untouched and hti_last_error() holds the reason.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "hti_internal.h"

using namespace hti;

namespace hti {

hipError_t set_dyn_lds_once(const void *kern, size_t bytes)
{
    static std::mutex mu;
    static std::vector<std::pair<int, const void *>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu);
    for (auto &p : done)
        if (p.first == dev && p.second == kern) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done.push_back({dev, kern});
    return e;
}

} // namespace hti

namespace {

thread_local std::string g_err;

hti_status fail(hti_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

hti_status ok()
{
    g_err.clear();
    return HTI_OK;
}

hti_status check_cfg(const hti_tree_cfg *c)
{
    if (!c) return fail(HTI_ERR_INVALID_ARG, "cfg is NULL");
    if (c->B < 1 || c->Hq < 1 || c->Hkv < 1) return fail(HTI_ERR_INVALID_ARG, "B, Hq, Hkv must be >= 1");
    if (c->Hq % c->Hkv) return fail(HTI_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", c->Hq, c->Hkv);
    const int G = c->Hq / c->Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(HTI_ERR_UNSUPPORTED, "group size Hq/Hkv = %d not in {1,2,4,8}", G);
    if (c->Hkv > 16) return fail(HTI_ERR_UNSUPPORTED, "Hkv = %d > 16", c->Hkv);
    if (c->d != 64 && c->d != 128) return fail(HTI_ERR_UNSUPPORTED, "head dim %d not in {64,128}", c->d);
    if (c->b < 2 || c->b > 64) return fail(HTI_ERR_UNSUPPORTED, "branching factor %d not in [2,64]", c->b);
    if (c->fan != 0 && (c->fan < 2 || c->fan > 64))
        return fail(HTI_ERR_UNSUPPORTED, "fan %d not 0 or in [2,64]", c->fan);
    if (c->levels < 0 || c->levels > HTI_MAX_LEVELS)
        return fail(HTI_ERR_INVALID_ARG, "levels %d not in [0,%d]", c->levels, HTI_MAX_LEVELS);
    if (c->R < 1 || c->R > HTI_MAX_R) return fail(HTI_ERR_UNSUPPORTED, "R = %d not in [1,%d]", c->R, HTI_MAX_R);
    if (c->dtype != HTI_F32 && c->dtype != HTI_BF16) return fail(HTI_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
    if (c->Lcap < 0 || c->Lcap >= (int64_t(1) << 31))
        return fail(HTI_ERR_UNSUPPORTED, "Lcap %lld outside [0, 2^31)", (long long)c->Lcap);
    if (!(c->rope_base > 0.f)) return fail(HTI_ERR_INVALID_ARG, "rope_base must be > 0");
    if (c->rope_npos < 1) return fail(HTI_ERR_INVALID_ARG, "rope_npos must be >= 1");
    if (c->router_fp8 != 0 && c->router_fp8 != 1) return fail(HTI_ERR_INVALID_ARG, "router_fp8 must be 0 or 1");
    if (c->router_fp8 && c->dtype != HTI_BF16)
        return fail(HTI_ERR_UNSUPPORTED, "8-bit router keys need bf16 caches");
    return HTI_OK;
}

hti_status check_select(const hti_select *s)
{
    if (!s) return fail(HTI_ERR_INVALID_ARG, "select is NULL");
    if (s->mode == HTI_TOPK) {
        if (s->k < 1 || s->k > HTI_MAX_SELECT)
            return fail(HTI_ERR_UNSUPPORTED, "k = %d not in [1,%d]", s->k, HTI_MAX_SELECT);
    } else if (s->mode == HTI_TOPP) {
        if (!(s->p > 0.f && s->p <= 1.f)) return fail(HTI_ERR_INVALID_ARG, "p must be in (0,1]");
        if (s->cap < 1 || s->cap > HTI_MAX_SELECT)
            return fail(HTI_ERR_UNSUPPORTED, "cap = %d not in [1,%d]", s->cap, HTI_MAX_SELECT);
    } else {
        return fail(HTI_ERR_INVALID_ARG, "unknown selection mode %d", s->mode);
    }
    if (s->per_head != 0 && s->per_head != 1) return fail(HTI_ERR_INVALID_ARG, "per_head must be 0 or 1");
    if (s->leaf_only != 0 && s->leaf_only != 1) return fail(HTI_ERR_INVALID_ARG, "leaf_only must be 0 or 1");
    if (s->token_nodes != 0 && s->token_nodes != 1) return fail(HTI_ERR_INVALID_ARG, "token_nodes must be 0 or 1");
    return HTI_OK;
}

int sel_size(const hti_select *s) { return s->mode == HTI_TOPK ? s->k : s->cap; }

void caps(const hti_tree_cfg *c, int64_t *ncap)
{
    ncap[0] = c->Lcap;
    for (int l = 1; l <= HTI_MAX_LEVELS; ++l) ncap[l] = (l <= c->levels) ? ncap[l - 1] / (l == 1 ? c->b : cfg_fan(c)) : 0;
}

// Largest candidate list per level for any length <= Lcap, and the largest
// RoPE row a traversal can touch (T > 0: prefill block of T tokens).
struct Bounds {
    int64_t cand[HTI_MAX_LEVELS + 1];
    int64_t max_summary;   // largest summary-level list
    int64_t rope_rows;     // rows needed
};

Bounds bounds(const hti_tree_cfg *c, const hti_select *s, int32_t T)
{
    int64_t ncap[HTI_MAX_LEVELS + 1];
    caps(c, ncap);
    Bounds r{};
    const int64_t keff = s ? sel_size(s) : 1;
    const int Lv = c->levels;
    r.max_summary = 0;
    r.rope_rows = 2;   // row 1 is the per-position angle step
    if (Lv == 0) {
        r.cand[0] = ncap[0];
    } else {
        r.cand[Lv] = ncap[Lv];
        for (int l = Lv - 1; l >= 0; --l) {
            const int64_t kept = std::min(keff, r.cand[l + 1]);
            const int64_t f = l == 0 ? c->b : cfg_fan(c);   // children per node of level l + 1
            r.cand[l] = std::min(ncap[l], kept * f + (f - 1));
        }
        for (int l = 1; l <= Lv; ++l) {
            r.max_summary = std::max(r.max_summary, r.cand[l]);
            r.rope_rows = std::max(r.rope_rows, r.cand[l] + 1);
        }
    }
    // token level: decode query at <= |C_0|; prefill query at |C_0| + T - 1 and
    // block-local positions < T
    const int64_t tok = T > 0 ? r.cand[0] + T : r.cand[0] + 1;
    r.rope_rows = std::max(r.rope_rows, tok);
    if (T > 0) r.rope_rows = std::max<int64_t>(r.rope_rows, T);
    return r;
}

TreeArgs tree_args(const hti_tree *tr)
{
    TreeArgs a{};
    const hti_tree_cfg &c = tr->cfg;
    a.kc = tr->k_cache;
    a.vc = tr->v_cache;
    for (int l = 0; l < HTI_MAX_LEVELS; ++l) {
        a.lk[l] = tr->lvl_k[l];
        a.lv[l] = tr->lvl_v[l];
        a.lkq[l] = c.router_fp8 ? tr->lvl_kq[l] : nullptr;
        a.lks[l] = c.router_fp8 ? tr->lvl_ks[l] : nullptr;
    }
    a.rfp8 = c.router_fp8;
    caps(&c, a.ncap);
    a.refs = tr->ref_q;
    a.len = tr->len;
    a.rope = reinterpret_cast<const float2 *>(tr->rope);
    a.rope_npos = c.rope_npos;
    a.B = c.B;
    a.Hq = c.Hq;
    a.Hkv = c.Hkv;
    a.D = c.d;
    a.b = c.b;
    a.fan = cfg_fan(&c);
    a.levels = c.levels;
    a.R = c.R;
    a.G = c.Hq / c.Hkv;
    a.hdiv = 1;
    a.scale = 1.0f / sqrtf((float)c.d);
    a.dtype = c.dtype;
    return a;
}

// The tree as the traversal kernels see it: per KV group, or (per-head
// routing) one routing head per query head, a group of one
TreeArgs routing_args(const hti_tree *tr, const hti_select *sel)
{
    TreeArgs a = tree_args(tr);
    if (sel->per_head) {
        a.hdiv = a.G;
        a.Hkv = a.Hq;
        a.G = 1;
    }
    return a;
}

// routing heads per sequence and query heads per routing head
int routing_heads(const hti_tree_cfg *c, const hti_select *sel)
{
    return sel && sel->per_head ? c->Hq : c->Hkv;
}

hti_status check_tree(const hti_tree *tr, bool need_refs)
{
    if (!tr) return fail(HTI_ERR_INVALID_ARG, "tree is NULL");
    hti_status st = check_cfg(&tr->cfg);
    if (st) return st;
    if (tr->cfg.Lcap > 0 && (!tr->k_cache || !tr->v_cache))
        return fail(HTI_ERR_INVALID_ARG, "k_cache/v_cache is NULL");
    if (!tr->len) return fail(HTI_ERR_INVALID_ARG, "len is NULL");
    if (!tr->rope) return fail(HTI_ERR_INVALID_ARG, "rope is NULL");
    int64_t ncap[HTI_MAX_LEVELS + 1];
    caps(&tr->cfg, ncap);
    for (int l = 0; l < tr->cfg.levels; ++l)   // a level with no capacity is never touched
        if (ncap[l + 1] > 0 && (!tr->lvl_k[l] || !tr->lvl_v[l]))
            return fail(HTI_ERR_INVALID_ARG, "level %d buffers are NULL", l + 1);
    if (tr->cfg.router_fp8)
        for (int l = 0; l < tr->cfg.levels; ++l)
            if (ncap[l + 1] > 0 && (!tr->lvl_kq[l] || !tr->lvl_ks[l]))
                return fail(HTI_ERR_INVALID_ARG, "level %d router-key buffers are NULL", l + 1);
    if (need_refs && !tr->ref_q) return fail(HTI_ERR_INVALID_ARG, "ref_q is NULL");
    return HTI_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ceil(2^32 / b): for 0 <= i < 2^16 and 2 <= b <= 64, umulhi(i, binv) == i / b
uint32_t binv_of(int b) { return (uint32_t)(((uint64_t(1) << 32) + (uint64_t)b - 1) / (uint64_t)b); }

hti_status launched(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(HTI_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

struct PrefillWs {
    size_t part_acc, part_ml, kr, vt, top_s, top_z;
    // node-inverted token level (nodes)
    size_t kept1, nsel1, cnt, ptot, pairs, po, pml;
    size_t total;
    int64_t ntop;       // top-level capacity when the top level is scored on the matrix cores, else 0
    bool nodes;
    int keff, ntrees;
    int64_t cap_t, cnt_words;
};

size_t inblock_tp(int32_t T) { return ((size_t)T + kInblockKeys - 1) / kInblockKeys * kInblockKeys; }

// sel == NULL sizes for shared routing with the largest kept set and the
// node-inverted token level
PrefillWs prefill_ws(const hti_tree_cfg *c, const hti_select *sel, int32_t T)
{
    PrefillWs w{};
    const int hu = routing_heads(c, sel);
    const size_t rows = (size_t)c->B * (size_t)T;
    int64_t ncap[HTI_MAX_LEVELS + 1];
    caps(c, ncap);
    w.ntop = (c->levels >= 1 && ncap[c->levels] >= 1 && ncap[c->levels] * c->R <= kTopCols)
                 ? ncap[c->levels] : 0;
    size_t off = 0;
    w.part_acc = off;
    off += align256(rows * c->Hq * c->d * sizeof(float));
    w.part_ml = off;
    off += align256(rows * c->Hq * 2 * sizeof(float));
    w.kr = off;
    off += align256((size_t)c->B * inblock_tp(T) * c->Hkv * c->d * 2);
    w.vt = off;
    off += align256((size_t)c->B * inblock_tp(T) * c->Hkv * c->d * 2);
    w.top_s = off;
    off += align256(rows * (size_t)hu * (size_t)w.ntop * sizeof(float));
    w.top_z = off;
    off += align256(rows * c->Hq * (size_t)w.ntop * sizeof(float));
    w.nodes = token_nodes_apply(c, sel);
    if (w.nodes) {
        const size_t units = rows * (size_t)hu;
        const int G = c->Hq / hu;
        w.keff = sel ? sel_size(sel) : HTI_MAX_SELECT;
        w.ntrees = c->B * c->Hkv;
        w.cap_t = (int64_t)T * (hu / c->Hkv) * w.keff;
        w.cnt_words = (int64_t)w.ntrees * ncap[1];
        w.kept1 = off;
        off += align256(units * w.keff * 4);
        w.nsel1 = off;
        off += align256(units * 4);
        w.cnt = off;
        off += align256((size_t)w.cnt_words * 4);
        w.ptot = off;
        off += align256((size_t)w.ntrees * 4);
        w.pairs = off;
        off += align256((size_t)w.ntrees * w.cap_t * 16);
        w.po = off;
        off += align256(units * w.keff * G * c->d * 2);
        w.pml = off;
        off += align256(units * w.keff * G * 2 * sizeof(float));
    }
    w.total = off;
    return w;
}

} // namespace

extern "C" {

const char *hti_last_error(void) { return g_err.c_str(); }

hti_status hti_plan(const hti_tree_cfg *cfg, const hti_select *sel, int32_t T, hti_plan_out *out)
{
    hti_status st = check_cfg(cfg);
    if (st) return st;
    if (!out) return fail(HTI_ERR_INVALID_ARG, "out is NULL");
    if (sel && (st = check_select(sel))) return st;
    if (T < 0) return fail(HTI_ERR_INVALID_ARG, "T < 0");
    memset(out, 0, sizeof *out);
    caps(cfg, out->ncap);
    const size_t es = cfg->dtype == HTI_BF16 ? 2 : 4;
    const size_t bh = (size_t)cfg->B * cfg->Hkv;
    out->cache_bytes = bh * (size_t)cfg->Lcap * cfg->d * es;
    for (int l = 1; l <= cfg->levels; ++l) {
        out->lvl_k_bytes[l - 1] = bh * (size_t)out->ncap[l] * cfg->R * cfg->d * es;
        out->lvl_v_bytes[l - 1] = bh * (size_t)out->ncap[l] * cfg->d * es;
        if (cfg->router_fp8) {
            out->lvl_kq_bytes[l - 1] = bh * (size_t)out->ncap[l] * cfg->R * cfg->d;
            out->lvl_ks_bytes[l - 1] = bh * (size_t)out->ncap[l] * cfg->R * sizeof(float);
        }
    }
    out->rope_bytes = (size_t)cfg->rope_npos * cfg->d * sizeof(float);
    const Bounds bd = bounds(cfg, sel, T);
    out->rope_npos_needed = (int32_t)std::min<int64_t>(bd.rope_rows, INT32_MAX);
    return ok();
}

hti_status hti_rope_init(const hti_tree *tree, void *stream)
{
    if (!tree) return fail(HTI_ERR_INVALID_ARG, "tree is NULL");
    hti_status st = check_cfg(&tree->cfg);
    if (st) return st;
    if (!tree->rope) return fail(HTI_ERR_INVALID_ARG, "rope is NULL");
    TreeArgs a = tree_args(tree);
    return launched(launch_rope_init(a, (double)tree->cfg.rope_base, (hipStream_t)stream), "rope_init");
}

} // extern "C"

namespace hti {
__global__ void k_set_len(int64_t *len, int base, int n, int64_t v0, int64_t v1, int64_t v2, int64_t v3, int64_t v4, int64_t v5, int64_t v6,
                          int64_t v7)
{
    const int i = threadIdx.x;
    const int64_t v[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
    if (i < n) len[base + i] = v[i];
}
} // namespace hti

extern "C" {

hti_status hti_tree_build(const hti_tree *tree, const int64_t *L_host, void *stream)
{
    hti_status st = check_tree(tree, true);
    if (st) return st;
    if (!L_host) return fail(HTI_ERR_INVALID_ARG, "L_host is NULL");
    const hti_tree_cfg &c = tree->cfg;
    int64_t maxL = 0;
    for (int s = 0; s < c.B; ++s) {
        if (L_host[s] < 0 || L_host[s] > c.Lcap)
            return fail(HTI_ERR_CAPACITY, "L_host[%d] = %lld outside [0, Lcap = %lld]", s,
                        (long long)L_host[s], (long long)c.Lcap);
        maxL = std::max(maxL, L_host[s]);
    }
    hipStream_t hs = (hipStream_t)stream;
    // lengths travel as kernel arguments (no host buffer outlives the call)
    for (int s0 = 0; s0 < c.B; s0 += 8) {
        int64_t v[8] = {0};
        const int n = std::min(8, c.B - s0);
        for (int i = 0; i < n; ++i) v[i] = L_host[s0 + i];
        hipLaunchKernelGGL(k_set_len, dim3(1), dim3(64), 0, hs, tree->len, s0, n, v[0], v[1],
                           v[2], v[3], v[4], v[5], v[6], v[7]);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return launched(e, "tree_build(set_len)");
    }
    TreeArgs a = tree_args(tree);
    int64_t n = maxL;
    for (int l = 1; l <= c.levels; ++l) {
        n /= l == 1 ? c.b : cfg_fan(&c);
        hipError_t e = launch_build_level(a, l, n, hs);
        if (e != hipSuccess) return launched(e, "tree_build(level)");
    }
    return ok();
}

hti_status hti_tree_append(const hti_tree *tree, const void *k_new, const void *v_new, void *stream)
{
    hti_status st = check_tree(tree, true);
    if (st) return st;
    if (!k_new || !v_new) return fail(HTI_ERR_INVALID_ARG, "k_new/v_new is NULL");
    TreeArgs a = tree_args(tree);
    return launched(launch_append(a, k_new, v_new, (hipStream_t)stream), "tree_append");
}

hti_status hti_tree_extend(const hti_tree *tree, const void *k_blk, const void *v_blk, int32_t T,
                           void *stream)
{
    hti_status st = check_tree(tree, true);
    if (st) return st;
    if (T < 0) return fail(HTI_ERR_INVALID_ARG, "T must be >= 0");
    if (T > 0 && (!k_blk || !v_blk)) return fail(HTI_ERR_INVALID_ARG, "k_blk/v_blk is NULL");
    TreeArgs a = tree_args(tree);
    return launched(launch_extend(a, k_blk, v_blk, T, (hipStream_t)stream), "tree_extend");
}

static hti_status check_traversal(const hti_tree *tree, const hti_select *sel, int32_t T,
                                  int32_t *sel_out, int32_t sel_stride)
{
    hti_status st = check_tree(tree, false);
    if (st) return st;
    if ((st = check_select(sel))) return st;
    if (sel_out && sel_stride < sel_size(sel))
        return fail(HTI_ERR_INVALID_ARG, "sel_stride %d < selection size %d", sel_stride, sel_size(sel));
    const Bounds bd = bounds(&tree->cfg, sel, T);
    if (bd.max_summary > HTI_MAX_CAND)
        return fail(HTI_ERR_UNSUPPORTED, "a summary level can hold %lld candidates (> %d)",
                    (long long)bd.max_summary, HTI_MAX_CAND);
    if (bd.rope_rows > tree->cfg.rope_npos)
        return fail(HTI_ERR_CAPACITY, "RoPE table has %d rows, this call can need %lld",
                    tree->cfg.rope_npos, (long long)bd.rope_rows);
    return HTI_OK;
}

size_t hti_decode_workspace_bytes(const hti_tree_cfg *cfg, const hti_select *sel, int32_t Nq)
{
    if (check_cfg(cfg) || Nq < 1 || (sel && check_select(sel))) return 0;
    const int hu = routing_heads(cfg, sel);
    const int64_t units = (int64_t)cfg->B * Nq * hu;
    return decode_ws_bytes(cfg->B, units, HTI_DECODE_MAX_SPLIT, cfg->levels, cfg->Hq / hu, cfg->d);
}

} // extern "C"

namespace {

// sparse_decode, and the decode step (k_new != NULL: append, then decode);
// use_static: the split workspace is the library's static device array
// (zeroed by a fill kernel before the launch), `ws` is ignored
hti_status decode_impl(const char *what, const hti_tree *tree, const hti_select *sel, const void *k_new,
                       const void *v_new, const void *q, const int64_t *q_pos, int32_t Nq, float *out, float *lse,
                       int32_t *sel_out, int32_t sel_stride, void *ws, size_t ws_bytes, void *stream,
                       bool use_static = false)
{
    hti_status st = check_traversal(tree, sel, 0, sel_out, sel_stride);
    if (st) return st;
    if (!q || !out) return fail(HTI_ERR_INVALID_ARG, "q/out is NULL");
    if (Nq < 1) return fail(HTI_ERR_INVALID_ARG, "Nq must be >= 1");
    const int hu = routing_heads(&tree->cfg, sel);
    const int64_t units_ws = (int64_t)tree->cfg.B * Nq * hu;
    const int G = tree->cfg.Hq / hu;
    if (ws && ws_bytes < decode_ws_bytes(tree->cfg.B, units_ws, HTI_DECODE_MAX_SPLIT, tree->cfg.levels, G, tree->cfg.d))
        return fail(HTI_ERR_WORKSPACE, "decode workspace of %zu bytes is too small", ws_bytes);
    TravArgs a{};
    a.t = routing_args(tree, sel);
    a.mode = sel->mode;
    a.k = sel->k;
    a.cap = sel->cap;
    a.p = sel->p;
    a.leaf_only = sel->leaf_only;
    a.q = q;
    a.q_pos = q_pos;
    a.Nq = Nq;
    a.out = out;
    a.lse = lse;
    a.sel = sel_out;
    a.sel_stride = sel_stride;
    a.binv = binv_of(tree->cfg.b);
    a.finv = binv_of(cfg_fan(&tree->cfg));
    const int64_t units = units_ws;
    if (units >= (int64_t(1) << 31)) return fail(HTI_ERR_UNSUPPORTED, "too many (query, group) units");
    const hipStream_t hs = (hipStream_t)stream;
    int W = 0, occ = 1;
    if (ws || use_static) {
        // split each unit over W workgroups when all of them fit on the device
        // at once; otherwise one workgroup per unit
        const Bounds bd = bounds(&tree->cfg, sel, 0);
        hipError_t e = decode_split_plan(a, units, bd.max_summary, &W, &occ);
        if (e != hipSuccess) return launched(e, what);
    }
    if (use_static && W > 0) {
        // the layout of this call's W, in the static array: checked against
        // its size, zeroed, and used as the workspace
        const size_t need = decode_ws_bytes(tree->cfg.B, units, W, tree->cfg.levels, G, tree->cfg.d);
        if (need > kStaticScratchBytes)
            return fail(HTI_ERR_WORKSPACE, "%s needs %zu bytes of split workspace, above the static array's %zu",
                        what, need, kStaticScratchBytes);
        hipError_t e = decode_static_scratch(&ws);
        if (e == hipSuccess) e = launch_zero(ws, need, hs);
        if (e != hipSuccess) return launched(e, what);
    }
    if (k_new) {
        if (W > 0 && tree->cfg.b <= 32 && cfg_fan(&tree->cfg) <= 32) {
            // the split kernel appends the token itself (one launch)
            a.k_new = k_new;
            a.v_new = v_new;
        } else {
            hipError_t e = launch_append(tree_args(tree), k_new, v_new, hs);
            if (e != hipSuccess) return launched(e, what);
        }
    }
    if (W > 0) {
        const DecodeWs dw = decode_ws_layout(ws, tree->cfg.B, units, W, tree->cfg.levels, G, tree->cfg.d);
        return launched(launch_decode_split(a, dw, units, occ, hs), what);
    }
    return launched(launch_traverse(a, false, units, hs), what);
}

} // namespace

extern "C" {

hti_status hti_sparse_decode(const hti_tree *tree, const hti_select *sel, const void *q, const int64_t *q_pos,
                             int32_t Nq, float *out, float *lse, int32_t *sel_out, int32_t sel_stride, void *ws,
                             size_t ws_bytes, void *stream)
{
    return decode_impl("sparse_decode", tree, sel, nullptr, nullptr, q, q_pos, Nq, out, lse, sel_out, sel_stride,
                       ws, ws_bytes, stream);
}

hti_status hti_sparse_decode_static(const hti_tree *tree, const hti_select *sel, const void *q,
                                    const int64_t *q_pos, int32_t Nq, float *out, float *lse, int32_t *sel_out,
                                    int32_t sel_stride, void *stream)
{
    return decode_impl("sparse_decode_static", tree, sel, nullptr, nullptr, q, q_pos, Nq, out, lse, sel_out,
                       sel_stride, nullptr, 0, stream, true);
}

hti_status hti_decode_status(const void *ws, size_t ws_bytes, void *stream)
{
    if (!ws || ws_bytes < 4) return fail(HTI_ERR_INVALID_ARG, "ws is NULL or too small");
    uint32_t st = 0;
    // the status word is the first word of the workspace
    hipError_t e = hipMemcpyAsync(&st, ws, 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(HTI_ERR_LAUNCH, "decode_status: %s", hipGetErrorString(e));
    if (st != 0)
        return fail(HTI_ERR_TIMEOUT, "a decode launch with this workspace ran out of a wait between workgroups: "
                                     "its outputs and those of later launches are NaN; zero the workspace");
    return ok();
}

hti_status hti_decode_step(const hti_tree *tree, const hti_select *sel, const void *k_new, const void *v_new,
                           const void *q, int32_t Nq, float *out, float *lse, int32_t *sel_out,
                           int32_t sel_stride, void *ws, size_t ws_bytes, void *stream)
{
    if (!k_new || !v_new) return fail(HTI_ERR_INVALID_ARG, "k_new/v_new is NULL");
    if (hti_status st = check_tree(tree, true)) return st;
    return decode_impl("decode_step", tree, sel, k_new, v_new, q, nullptr, Nq, out, lse, sel_out, sel_stride, ws,
                       ws_bytes, stream);
}

size_t hti_prefill_workspace_bytes(const hti_tree_cfg *cfg, const hti_select *sel, int32_t T)
{
    if (check_cfg(cfg) || T < 0 || (sel && check_select(sel))) return 0;
    return prefill_ws(cfg, sel, T).total;
}

hti_status hti_sparse_prefill(const hti_tree *tree, const hti_select *sel, const void *q_blk,
                              const void *k_blk, const void *v_blk, int32_t T, float *out, float *lse,
                              int32_t *sel_out, int32_t sel_stride, void *ws, size_t ws_bytes,
                              void *stream)
{
    if (T < 1) return fail(HTI_ERR_INVALID_ARG, "T must be >= 1");
    hti_status st = check_traversal(tree, sel, T, sel_out, sel_stride);
    if (st) return st;
    if (tree->cfg.dtype != HTI_BF16)
        return fail(HTI_ERR_UNSUPPORTED, "prefill runs on bf16 matrix cores; dtype must be bf16");
    if (!q_blk || !k_blk || !v_blk || !out) return fail(HTI_ERR_INVALID_ARG, "q/k/v/out is NULL");
    const PrefillWs w = prefill_ws(&tree->cfg, sel, T);
    if (!ws || ws_bytes < w.total)
        return fail(HTI_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, w.total);
    const int64_t units = (int64_t)tree->cfg.B * T * routing_heads(&tree->cfg, sel);
    if (units >= (int64_t(1) << 31)) return fail(HTI_ERR_UNSUPPORTED, "too many (query, group) units");
    {
        // the traversal addresses rows by 32-bit byte offsets within one
        // (sequence, KV head) slice of the cache and of each level
        int64_t ncap[HTI_MAX_LEVELS + 1];
        caps(&tree->cfg, ncap);
        int64_t big = ncap[0];
        for (int l = 1; l <= tree->cfg.levels; ++l) big = std::max(big, ncap[l] * tree->cfg.R);
        if (big * tree->cfg.d * 2 > (int64_t)0xffffffffll)
            return fail(HTI_ERR_UNSUPPORTED, "prefill needs each (sequence, KV head) cache slice under 4 GiB");
    }
    char *wb = (char *)ws;
    hipStream_t hs = (hipStream_t)stream;

    TravArgs ta{};
    ta.t = routing_args(tree, sel);
    ta.mode = sel->mode;
    ta.k = sel->k;
    ta.cap = sel->cap;
    ta.p = sel->p;
    ta.leaf_only = sel->leaf_only;
    ta.q = q_blk;
    ta.Nq = T;
    ta.sel = sel_out;
    ta.sel_stride = sel_stride;
    ta.binv = binv_of(tree->cfg.b);
    ta.finv = binv_of(cfg_fan(&tree->cfg));
    ta.part_acc = (float *)(wb + w.part_acc);
    ta.part_ml = (float *)(wb + w.part_ml);

    PrefillArgs pa{};
    pa.t = ta.t;   // the routing view for the top-level scores; the block kernels take the KV heads
    pa.q = q_blk;
    pa.k = k_blk;
    pa.v = v_blk;
    pa.T = T;
    hipError_t e = hipSuccess;
    // A tree set without prefix capacity (the first block of a sequence) has
    // nothing before the block: no traversal, no partial states, and every
    // selection slot is empty.
    const bool no_prefix = tree->cfg.Lcap == 0;
    if (no_prefix) {
        if (sel_out) {
            e = launch_fill_u32(sel_out, 0xffffffffu, units * tree->cfg.levels * (int64_t)sel_stride,
                                hs);
            if (e != hipSuccess) return launched(e, "sparse_prefill(selections)");
        }
    }
    if (!no_prefix && w.ntop > 0) {
        // the top level of every query of the block, scored on the matrix cores
        pa.top_s = (float *)(wb + w.top_s);
        pa.top_z = (float *)(wb + w.top_z);
        pa.ntop_stride = (int)w.ntop;
        e = launch_top_scores(pa, hs);
        if (e != hipSuccess) return launched(e, "sparse_prefill(top scores)");
        ta.top_s = pa.top_s;
        ta.top_z = pa.top_z;
        ta.ntop_stride = pa.ntop_stride;
    }
    if (!no_prefix && w.nodes) {
        if ((int64_t)units * w.keff >= (int64_t(1) << 32) || (int64_t)tree->cfg.B * T * tree->cfg.Hq >= (int64_t(1) << 32))
            return fail(HTI_ERR_UNSUPPORTED, "too many (query, group, rank) pairs for the node-inverted token level");
        ta.kept1 = (int *)(wb + w.kept1);
        ta.nsel1 = (int *)(wb + w.nsel1);
        ta.node_cnt = (uint32_t *)(wb + w.cnt);
        e = launch_zero(ta.node_cnt, (size_t)w.cnt_words * 4, hs);
        if (e != hipSuccess) return launched(e, "sparse_prefill(zero counts)");
    }
    if (!no_prefix) {
        e = launch_prefill_walk(ta, bounds(&tree->cfg, sel, T).max_summary, units, hs);
        if (e != hipSuccess) return launched(e, "sparse_prefill(traverse)");
    }
    if (!no_prefix && w.nodes) {
        NodeArgs na{};
        na.t = ta.t;
        na.q = q_blk;
        na.T = T;
        na.keff = w.keff;
        na.cap_t = w.cap_t;
        na.ntrees = w.ntrees;
        na.kept1 = ta.kept1;
        na.nsel1 = ta.nsel1;
        na.cnt = ta.node_cnt;
        na.ptot = (uint32_t *)(wb + w.ptot);
        na.pairs = (uint4 *)(wb + w.pairs);
        na.po = (uint16_t *)(wb + w.po);
        na.pml = (float *)(wb + w.pml);
        na.part_acc = ta.part_acc;
        na.part_ml = ta.part_ml;
        e = launch_token_pairs(na, units, hs);
        if (e != hipSuccess) return launched(e, "sparse_prefill(token pairs)");
        e = launch_token_nodes(na, hs);
        if (e != hipSuccess) return launched(e, "sparse_prefill(token nodes)");
        e = launch_token_merge(na, units, hs);
        if (e != hipSuccess) return launched(e, "sparse_prefill(token merge)");
    }

    pa.t = tree_args(tree);
    pa.part_acc = no_prefix ? nullptr : ta.part_acc;
    pa.part_ml = no_prefix ? nullptr : ta.part_ml;
    pa.out = out;
    pa.lse = lse;
    pa.kr = wb + w.kr;
    pa.vt = wb + w.vt;
    pa.Tp = (int)inblock_tp(T);
    e = launch_rotate_block(pa, hs);
    if (e != hipSuccess) return launched(e, "sparse_prefill(rotate)");
    return launched(launch_inblock_attention(pa, hs), "sparse_prefill(inblock)");
}

} // extern "C"
