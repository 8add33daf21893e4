/*
 * hti_oracle.c -- plain, slow, single-threaded CPU oracle of tree-indexed
 * recursive sparse attention.  TEST INFRASTRUCTURE ONLY: it exists so that the
 * GPU library can be checked against an independent reading of the method.
 * Nothing in the product library links, calls or includes this file.
 *
 * Arithmetic: fp32 throughout (the method statement fixes an fp32 oracle),
 * every sum taken sequentially in the index order written below, compiled
 * without floating-point contraction or fast-math.  RoPE angles are formed in
 * double and their cosine/sine rounded once to fp32.
 *
 * Sources (cited by page title and element):
 *  [RecSA]  "Recursive Sparse Attention: Million-Token Length Extrapolation at
 *           Logarithmic Cost", abstract: tree over the KV cache, one key and one
 *           mean-pooled value per node, one pooler per layer shared by all
 *           levels, at most k candidates selected per level above the tokens,
 *           summaries of unselected candidates share one softmax with the exact
 *           tokens, RoPE position = index among the level's candidates.
 *  [ZHA-F3] "Subquadratic Attention with a Hierarchical Tree-Structured
 *           Indexer", Figure 3 caption: a chunk of contiguous key nodes is
 *           summarised by an attention-weighted sum of its keys, attention taken
 *           w.r.t. reference queries; several reference queries, key nodes
 *           stored per reference in parallel; recursive construction; routing by
 *           dot-product scores with top-p selection, descending to the leaves.
 *  [ZHA-T8] same page, Table VIII: only full nodes exist, n_l(T) = floor(T/C^l);
 *           decode maintenance is amortised over full-node completions.
 *  [ESM13]  "Efficient Sequence Modeling, Issue 13", RecSA editor's note: the
 *           shared pooler provides both the selection keys and the summary keys.
 *
 * Readings where the pages are silent (each restated where it is used):
 *  - pooler: alpha = softmax_c(r . k_c / sqrt(d)) over a node's children,
 *    pooled key = sum_c alpha_c k_c; value = arithmetic mean of the children;
 *  - tree geometry [ZHA, Figure 4 caption and Table II: chunk size C, fan F,
 *    levels L, e.g. "C4 F4 L6"]: a level-1 node pools a chunk of b = C
 *    consecutive tokens, a node above pools fan = F consecutive nodes of the
 *    level below (every geometry the page lists has C = F, the default);
 *    n_1 = floor(n_0 / C), n_l = floor(n_{l-1} / F);
 *  - nodes are stored in the cache dtype (bf16 by round-to-nearest-even), and
 *    higher levels pool the stored (rounded) children;
 *  - one selection per (query, KV-head group), scored by the mean over the
 *    group's heads of the per-head logits; the softmax stays per head;
 *  - with R reference queries a node's score is the largest group-mean logit
 *    over its R keys (first index on ties) and that key is the node's key in
 *    the softmax;
 *  - candidate order: children of the selected nodes in ascending node order,
 *    then the level's orphans (full nodes with no full parent) ascending;
 *  - query RoPE position: |C_l| at a summary level; at the token level the
 *    number of candidate tokens before the query position;
 *  - ties: higher score first, then lower candidate index;
 *  - top-p: softmax of the group scores over the candidates, candidates sorted
 *    by score, shortest prefix whose running fp32 sum reaches p, size clamped
 *    to [1, cap];
 *  - a level with no more candidates than the selection size is taken whole
 *    without scoring.
 *  - RoPE: rotate-half pairs (j, j + d/2), theta_j = base^(-2j/d).
 *  - low-precision router keys [ZHA, Figure 16 caption: router operands,
 *    reference-key cache and scoring in 4-bit floats while the KV cache and
 *    the sparse attention stay in bf16]: 8-bit floats here (OCP E4M3, the
 *    format the target's vector unit converts).  Each stored summary key row
 *    (one node, one reference) is divided by a power-of-two scale
 *    2^(e - 8), where amax = f * 2^e with f in [0.5, 1) is the row's largest
 *    magnitude (scale 1 for an all-zero row), and every element is rounded to
 *    the nearest E4M3 value, ties to the even code.  Every summary-level logit
 *    (selection score and, with summaries attended, the summary's softmax
 *    logit) comes from the dequantised row; tokens and values are untouched.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MAXLVL 32

/* fp32 -> bf16 -> fp32, round to nearest, ties to even (finite inputs). */
static float round_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    u &= 0xffff0000u;
    float y;
    memcpy(&y, &u, 4);
    return y;
}

static float dot_seq(const float *a, const float *b, int d)
{
    float acc = 0.0f;
    for (int t = 0; t < d; ++t)
        acc += a[t] * b[t];
    return acc;
}

/* OCP E4M3 magnitude of code c in 0..126 (4 exponent bits, bias 7, 3
 * mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; code 127
 * is NaN and never produced here). */
static double e4m3_value(int c)
{
    int e = (c >> 3) & 15, m = c & 7;
    return e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* Code of the E4M3 value nearest to x (|x| <= 448), ties to the even code,
 * found by trying every finite magnitude; the sign bit is x's. */
static uint8_t e4m3_encode(float x)
{
    double a = fabs((double)x), bd = INFINITY;
    int best = 0;
    for (int c = 0; c <= 126; ++c) {
        double dv = fabs(e4m3_value(c) - a);
        if (dv < bd || (dv == bd && (c & 1) == 0)) {
            bd = dv;
            best = c;
        }
    }
    return (uint8_t)((signbit(x) ? 0x80 : 0) | best);
}

/* Router copy of one key row: codes[d] and its power-of-two scale. */
void orc_router_fp8(const float *k, int d, uint8_t *codes, float *scale)
{
    float amax = 0.0f;
    for (int t = 0; t < d; ++t)
        if (fabsf(k[t]) > amax) amax = fabsf(k[t]);
    int e = 8;
    if (amax > 0.0f) frexpf(amax, &e);
    *scale = ldexpf(1.0f, e - 8);
    for (int t = 0; t < d; ++t)
        codes[t] = e4m3_encode(k[t] / *scale);
}

/* The key row as the router sees it: codes times scale. */
static void router_dequant(const float *k, int d, float *y)
{
    uint8_t codes[512];   /* d <= 512 */
    float sc;
    orc_router_fp8(k, d, codes, &sc);
    for (int t = 0; t < d; ++t) {
        double v = e4m3_value(codes[t] & 0x7f);
        y[t] = (float)((codes[t] & 0x80) ? -v : v) * sc;
    }
}

/* y = RoPE(x, pos): rotate-half, angle pos * base^(-2j/d) formed in double. */
static void rope(const float *x, int d, long pos, double base, float *y)
{
    int h = d / 2;
    for (int j = 0; j < h; ++j) {
        double theta = pow(base, -2.0 * (double)j / (double)d);
        double ang = (double)pos * theta;
        float c = (float)cos(ang), s = (float)sin(ang);
        float x0 = x[j], x1 = x[j + h];
        y[j] = x0 * c - x1 * s;
        y[j + h] = x0 * s + x1 * c;
    }
}

/* ------------------------------------------------------------------------ */
/* Tree construction [RecSA abstract; ZHA-F3; ZHA-T8].                      */
/* ------------------------------------------------------------------------ */

/*
 * Build every full node of levels 1..levels over the first L tokens of one
 * (sequence, KV head).
 *   K, V    : [L][d] token keys / values (already in their stored precision)
 *   refs    : [R][d] reference queries of this KV head
 *   lvl_k[l]: [n_{l+1}][R][d] pooled keys of level l+1
 *   lvl_v[l]: [n_{l+1}][d]    mean values of level l+1
 *   bf16    : nonzero -> every stored node is rounded to bf16
 * Returns the number of levels built.
 */
int orc_build(long L, int d, int b, int fan, int levels, int R, int bf16,
              const float *K, const float *V, const float *refs,
              float *const *lvl_k, float *const *lvl_v)
{
    float scale = 1.0f / sqrtf((float)d);
    float *a = (float *)malloc(sizeof(float) * (size_t)(b > fan ? b : fan));
    long n_prev = L;
    for (int l = 1; l <= levels; ++l) {
        const int fb = (l == 1) ? b : fan;           /* children per node of level l */
        long n = n_prev / fb;                        /* full nodes only [ZHA-T8] */
        float *Kl = lvl_k[l - 1], *Vl = lvl_v[l - 1];
        for (long i = 0; i < n; ++i) {
            for (int j = 0; j < R; ++j) {
                /* child c of node i, pooled by reference j: level 0 has a single
                 * key per token, higher levels keep one key per reference */
                const float *child0;
                long cstride;
                if (l == 1) {
                    child0 = K + (size_t)(i * fb) * d;
                    cstride = d;
                } else {
                    child0 = lvl_k[l - 2] + ((size_t)(i * fb) * R + j) * d;
                    cstride = (long)R * d;
                }
                const float *r = refs + (size_t)j * d;
                float mx = -INFINITY;
                for (int c = 0; c < fb; ++c) {
                    a[c] = dot_seq(r, child0 + c * cstride, d) * scale;
                    if (a[c] > mx) mx = a[c];
                }
                float den = 0.0f;
                for (int c = 0; c < fb; ++c) {
                    a[c] = expf(a[c] - mx);
                    den += a[c];
                }
                float *out = Kl + ((size_t)i * R + j) * d;
                for (int t = 0; t < d; ++t) {
                    float acc = 0.0f;
                    for (int c = 0; c < fb; ++c)
                        acc += (a[c] / den) * child0[c * cstride + t];
                    out[t] = bf16 ? round_bf16(acc) : acc;
                }
            }
            /* mean-pooled value [RecSA abstract] */
            const float *vc = (l == 1) ? V + (size_t)(i * fb) * d : lvl_v[l - 2] + (size_t)(i * fb) * d;
            float *vo = Vl + (size_t)i * d;
            for (int t = 0; t < d; ++t) {
                float acc = 0.0f;
                for (int c = 0; c < fb; ++c)
                    acc += vc[(size_t)c * d + t];
                acc = acc / (float)fb;
                vo[t] = bf16 ? round_bf16(acc) : acc;
            }
        }
        n_prev = n;
    }
    free(a);
    return levels;
}

/* ------------------------------------------------------------------------ */
/* Traversal and the shared softmax [RecSA abstract; ZHA-F3; ESM13].         */
/* ------------------------------------------------------------------------ */

typedef struct {
    int d, b, fan, levels, R, G;   /* b: tokens per level-1 node; fan: nodes per node above */
    int mode;            /* 0 = top-k, 1 = top-p */
    int k, cap;
    float p;
    double rope_base;
    long Ltree;          /* tokens covered by the tree */
    long qpos;           /* decode: absolute query position (<= Ltree-1); prefill: -1 */
    long t;              /* prefill: query index inside the block; decode: -1 */
    const float *K, *V;  /* [Ltree][d] */
    const float *const *lvl_k;
    const float *const *lvl_v;
    const float *blk_k, *blk_v; /* prefill block [T][d] of this KV head */
    const float *q;      /* [G][d] the group's query heads */
    const int *replay;   /* [levels][kmax] ascending node ids, -1 padded; or NULL */
    int kmax;
    int leaf_only;       /* 1: only the reached tokens are attended (the leaf
                            union the router dispatches, ZHA Figure 3 caption);
                            0: unselected summaries join the softmax too */
    int router_fp8;      /* 1: summary keys are scored through their E4M3 copy */
} orc_query_args;

typedef struct {
    float *out;          /* [G][d] */
    float *lse;          /* [G] */
    int *sel;            /* [levels][kmax] (row l-1 = level l), or NULL */
    float *gap;          /* [levels] score gap at the selection boundary, or NULL */
    float *pmargin;      /* [levels] top-p running-sum margin, or NULL */
    long *counts;        /* [2]: keys scored, values read */
    int *ent_level;      /* entry list (optional): level, node id, candidate index */
    long *ent_node;
    long *ent_pos;
    long ent_cap;
    long n_ent;
} orc_query_out;

typedef struct {
    float s;
    long pos;
} scored;

static int cmp_scored(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->pos < b->pos) ? -1 : (a->pos > b->pos);
}

static int cmp_long(const void *pa, const void *pb)
{
    long a = *(const long *)pa, b = *(const long *)pb;
    return (a < b) ? -1 : (a > b);
}

typedef struct {
    long n, cap;
    float *z;            /* [cap][G] */
    const float **v;     /* [cap] value rows */
} entry_set;

static void ent_push(entry_set *E, int G, const float *z, const float *v)
{
    if (E->n == E->cap) {
        E->cap = E->cap ? 2 * E->cap : 1024;
        E->z = (float *)realloc(E->z, sizeof(float) * (size_t)E->cap * G);
        E->v = (const float **)realloc(E->v, sizeof(float *) * (size_t)E->cap);
    }
    memcpy(E->z + (size_t)E->n * G, z, sizeof(float) * G);
    E->v[E->n] = v;
    E->n++;
}

static void rec_entry(orc_query_out *o, int level, long node, long pos)
{
    if (o->ent_level && o->n_ent < o->ent_cap) {
        o->ent_level[o->n_ent] = level;
        o->ent_node[o->n_ent] = node;
        o->ent_pos[o->n_ent] = pos;
    }
    o->n_ent++;
}

/*
 * Attention of one query token (G heads of one KV group) over one tree.
 * Decode: the tree covers tokens [0, Ltree), the query sits at qpos.
 * Prefill: the tree covers the prefix [0, Ltree); after the prefix candidates
 * the level-0 list continues with block tokens 0..t, and the query's own
 * position is (number of prefix candidates) + t.
 * Returns 0, or -1 on a malformed replay list.
 */
int orc_query(const orc_query_args *A, orc_query_out *O)
{
    const int d = A->d, G = A->G, R = A->R, Lv = A->levels;
    const float scale = 1.0f / sqrtf((float)d);
    const int prefill = A->t >= 0;
    long n[ORC_MAXLVL + 1];
    n[0] = A->Ltree;
    for (int l = 1; l <= Lv; ++l)
        n[l] = n[l - 1] / (l == 1 ? A->b : A->fan);             /* [ZHA-T8] */

    long cap_c = 1024;
    long *cand = (long *)malloc(sizeof(long) * cap_c);
    long m = n[Lv];                                   /* C_top = all top nodes */
    if (m > cap_c) { cap_c = m; cand = (long *)realloc(cand, sizeof(long) * cap_c); }
    for (long i = 0; i < m; ++i) cand[i] = i;

    float *qr = (float *)malloc(sizeof(float) * (size_t)G * d);
    float *kr = (float *)malloc(sizeof(float) * (size_t)d);
    float *kq = (float *)malloc(sizeof(float) * (size_t)d);
    float *zt = (float *)malloc(sizeof(float) * (size_t)G * (R > 0 ? R : 1));
    entry_set E = {0, 0, NULL, NULL};
    O->counts[0] = O->counts[1] = 0;
    O->n_ent = 0;
    int status = 0;

    for (int l = Lv; l >= 1; --l) {
        int row = l - 1;
        if (O->sel)
            for (int s = 0; s < A->kmax; ++s) O->sel[row * A->kmax + s] = -1;
        if (O->gap) O->gap[row] = INFINITY;
        if (O->pmargin) O->pmargin[row] = INFINITY;

        /* selection size rule: top-k keeps k; top-p keeps at most cap and
         * decides among >= 2 candidates; a replayed selection that leaves
         * candidates out needs their logits too */
        long take_all_below = (A->mode == 0) ? A->k : 1;
        const int *rp = A->replay ? A->replay + (size_t)row * A->kmax : NULL;
        long nrep = 0;
        if (rp)
            while (nrep < A->kmax && rp[nrep] >= 0) ++nrep;
        int need_scores = (m > take_all_below) || (rp && nrep < m);
        float *s = NULL, *z = NULL;
        long nsel = m;
        long *sel_pos = (long *)malloc(sizeof(long) * (size_t)(m > 0 ? m : 1));
        for (long i = 0; i < m; ++i) sel_pos[i] = i;

        if (need_scores) {
            /* score every candidate: candidate i sits at RoPE position i, the
             * query at position m = |C_l| [RecSA abstract] */
            s = (float *)malloc(sizeof(float) * (size_t)m);
            z = (float *)malloc(sizeof(float) * (size_t)m * G);
            for (int h = 0; h < G; ++h)
                rope(A->q + (size_t)h * d, d, m, A->rope_base, qr + (size_t)h * d);
            const float *Kl = A->lvl_k[l - 1];
            for (long i = 0; i < m; ++i) {
                float best = -INFINITY;
                int jbest = 0;
                for (int j = 0; j < R; ++j) {
                    const float *krow = Kl + ((size_t)cand[i] * R + j) * d;
                    if (A->router_fp8) {
                        router_dequant(krow, d, kq);
                        krow = kq;
                    }
                    rope(krow, d, i, A->rope_base, kr);
                    float gsum = 0.0f;
                    for (int h = 0; h < G; ++h) {
                        zt[j * G + h] = dot_seq(qr + (size_t)h * d, kr, d) * scale;
                        gsum += zt[j * G + h];
                    }
                    float gmean = gsum / (float)G;
                    if (gmean > best) { best = gmean; jbest = j; }
                }
                s[i] = best;
                for (int h = 0; h < G; ++h) z[i * G + h] = zt[jbest * G + h];
            }
            O->counts[0] += m * R;
        }

        if (m > take_all_below) {
            scored *srt = (scored *)malloc(sizeof(scored) * (size_t)m);
            for (long i = 0; i < m; ++i) { srt[i].s = s[i]; srt[i].pos = i; }
            qsort(srt, (size_t)m, sizeof(scored), cmp_scored);
            if (A->mode == 0) {
                nsel = A->k;
                if (O->gap) O->gap[row] = srt[nsel - 1].s - srt[nsel].s;
            } else {
                /* top-p over the softmax of the group scores (largest first) */
                float mx = srt[0].s, den = 0.0f;
                for (long i = 0; i < m; ++i) den += expf(s[i] - mx);
                float run = 0.0f, prev = 0.0f;
                long nat = m;
                for (long r = 0; r < m; ++r) {
                    prev = run;
                    run += expf(srt[r].s - mx) / den;
                    if (run >= A->p) { nat = r + 1; break; }
                }
                nsel = nat;
                if (nsel > A->cap) nsel = A->cap;
                if (nsel < 1) nsel = 1;
                if (O->pmargin && nsel == nat && nat < m) {
                    float m1 = run - A->p, m2 = A->p - prev;
                    O->pmargin[row] = (nat == 1) ? m1 : (m1 < m2 ? m1 : m2);
                }
                if (O->gap && nsel < m) O->gap[row] = srt[nsel - 1].s - srt[nsel].s;
            }
            for (long r = 0; r < nsel; ++r) sel_pos[r] = srt[r].pos;
            qsort(sel_pos, (size_t)nsel, sizeof(long), cmp_long);
            free(srt);
        }

        if (rp) {
            /* externally supplied selection of this level (ascending node ids) */
            long cnt = 0;
            for (long r = 0; r < nrep; ++r) {
                long i = 0;
                while (i < m && cand[i] != rp[r]) ++i;
                if (i == m || (cnt > 0 && i <= sel_pos[cnt - 1])) { status = -1; break; }
                sel_pos[cnt++] = i;
            }
            if (status) { free(sel_pos); free(s); free(z); break; }
            nsel = cnt;
        }

        /* unselected candidates join the shared softmax as summaries (not
         * when only the reached tokens are dispatched) */
        long r = 0;
        for (long i = 0; i < m && !A->leaf_only; ++i) {
            if (r < nsel && sel_pos[r] == i) { ++r; continue; }
            ent_push(&E, G, z + (size_t)i * G, A->lvl_v[l - 1] + (size_t)cand[i] * d);
            rec_entry(O, l, cand[i], i);
            O->counts[1] += 1;
        }
        if (O->sel)
            for (long q = 0; q < nsel && q < A->kmax; ++q)
                O->sel[row * A->kmax + q] = (int)cand[sel_pos[q]];

        /* next candidates: children of the selected nodes in node order, then
         * the orphans of level l-1 (indices fb*n_l .. n_{l-1}-1), fb being the
         * children per node of level l */
        const int fb = (l == 1) ? A->b : A->fan;
        long orph0 = (long)fb * n[l], norph = n[l - 1] - orph0;
        long m2 = nsel * fb + norph;
        long *nc = (long *)malloc(sizeof(long) * (size_t)(m2 > 0 ? m2 : 1));
        long w = 0;
        for (long q = 0; q < nsel; ++q)
            for (int c = 0; c < fb; ++c) nc[w++] = cand[sel_pos[q]] * fb + c;
        for (long i = 0; i < norph; ++i) nc[w++] = orph0 + i;
        free(cand);
        cand = nc;
        m = m2;
        free(sel_pos);
        free(s);
        free(z);
    }

    if (status == 0) {
        /* token level: every candidate is an exact entry.  Decode keeps the
         * tokens <= qpos; the query's position is the number of candidates
         * before it.  Prefill appends the block tokens 0..t after the prefix
         * candidates. */
        long m0 = 0;
        for (long i = 0; i < m; ++i)
            if (prefill || cand[i] <= A->qpos) cand[m0++] = cand[i];
        long qp;
        if (prefill) {
            qp = m0 + A->t;
        } else {
            qp = 0;
            while (qp < m0 && cand[qp] < A->qpos) ++qp;
        }
        for (int h = 0; h < G; ++h)
            rope(A->q + (size_t)h * d, d, qp, A->rope_base, qr + (size_t)h * d);
        long ntok = m0 + (prefill ? A->t + 1 : 0);
        float *zz = (float *)malloc(sizeof(float) * (size_t)G);
        for (long i = 0; i < ntok; ++i) {
            const float *kk, *vv;
            long node;
            if (i < m0) {
                kk = A->K + (size_t)cand[i] * d;
                vv = A->V + (size_t)cand[i] * d;
                node = cand[i];
            } else {
                kk = A->blk_k + (size_t)(i - m0) * d;
                vv = A->blk_v + (size_t)(i - m0) * d;
                node = A->Ltree + (i - m0);
            }
            rope(kk, d, i, A->rope_base, kr);
            for (int h = 0; h < G; ++h)
                zz[h] = dot_seq(qr + (size_t)h * d, kr, d) * scale;
            ent_push(&E, G, zz, vv);
            rec_entry(O, 0, node, i);
        }
        O->counts[0] += ntok;
        O->counts[1] += ntok;
        free(zz);

        /* one softmax per head over every entry [RecSA abstract] */
        for (int h = 0; h < G; ++h) {
            float M = -INFINITY;
            for (long e = 0; e < E.n; ++e)
                if (E.z[e * G + h] > M) M = E.z[e * G + h];
            float den = 0.0f;
            for (long e = 0; e < E.n; ++e) den += expf(E.z[e * G + h] - M);
            float *o = O->out + (size_t)h * d;
            for (int t = 0; t < d; ++t) {
                float acc = 0.0f;
                for (long e = 0; e < E.n; ++e)
                    acc += expf(E.z[e * G + h] - M) * E.v[e][t];
                o[t] = acc / den;
            }
            if (O->lse) O->lse[h] = M + logf(den);
        }
    }

    free(cand);
    free(qr);
    free(kr);
    free(kq);
    free(zt);
    free(E.z);
    free(E.v);
    return status;
}
