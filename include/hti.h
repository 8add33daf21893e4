/*
 * hti.h -- C ABI of the tree-indexed recursive sparse attention library
 * (gfx950 / MI355X).
 *
 * The method (sources cited by page title and element):
 *   "Recursive Sparse Attention: Million-Token Length Extrapolation at
 *   Logarithmic Cost", abstract -- a tree over the KV cache whose nodes hold
 *   one key (from a per-layer pooler shared by every level) and one mean-pooled
 *   value; each level above the tokens keeps at most k candidates; the
 *   summaries of the candidates that were not kept share one softmax with the
 *   exact tokens finally reached; an entry's RoPE position is its index among
 *   its level's candidates.
 *   "Subquadratic Attention with a Hierarchical Tree-Structured Indexer",
 *   Figure 3 caption -- keys of a chunk of contiguous nodes are pooled by
 *   attention w.r.t. reference queries (R of them, keys stored per reference in
 *   parallel); routing scores the top level, keeps a top-p set and descends;
 *   Table VIII -- only full nodes exist, n_l(T) = floor(T / b^l).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller, unless the
 *     argument says "host".  The library never allocates, frees or retains
 *     device memory, with one exception: the static device array that
 *     hti_sparse_decode_static uses as its workspace.  The only device state
 *     it keeps between calls is in the decode workspace the caller hands it
 *     (a status word, per-unit launch counters, per-sequence step counts).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call only enqueues work on it and returns; results are valid once the
 *     stream has reached that point.
 *   - Every call validates its arguments on the host before enqueuing
 *     anything.  On error nothing is enqueued, device memory is unchanged, a
 *     negative hti_status is returned and hti_last_error() describes it.
 *   - Element types: HTI_F32 = IEEE fp32, HTI_BF16 = bfloat16 (stored as the
 *     upper 16 bits of an fp32).  Tree nodes are stored in the cache dtype
 *     (bf16 by round-to-nearest-even); all arithmetic is fp32.
 *   - Layouts are dense, row-major, innermost dimension last.
 *   - RoPE: rotate-half pairs (j, j + d/2), angle pos * base^(-2j/d).
 *   - Pooler: for node i and reference r_j, alpha = softmax over its b
 *     children of (r_j . k_child / sqrt(d)); pooled key = sum alpha k_child
 *     (level 1 pools token keys, level l >= 2 pools the level l-1 keys of the
 *     same reference); value = mean of the children's values.
 */
#ifndef HTI_H
#define HTI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HTI_MAX_LEVELS 12   /* tree levels above the tokens */
#define HTI_MAX_SELECT 32   /* largest k (top-k) or cap (top-p) */
#define HTI_MAX_CAND 1024   /* largest candidate list of a summary level */
#define HTI_MAX_R 8         /* reference queries per KV head */
#define HTI_DECODE_MAX_SPLIT 16  /* most workgroups one decode unit is split over */

typedef enum {
    HTI_OK = 0,
    HTI_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shapes */
    HTI_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels handle (d, G, ...) */
    HTI_ERR_CAPACITY = -3,    /* a length exceeds a buffer capacity */
    HTI_ERR_WORKSPACE = -4,   /* workspace missing or too small */
    HTI_ERR_LAUNCH = -5,      /* the HIP runtime refused a launch */
    HTI_ERR_TIMEOUT = -6      /* a split decode's workgroups ran out of a wait (hti_decode_status) */
} hti_status;

typedef enum { HTI_F32 = 0, HTI_BF16 = 1 } hti_dtype;
typedef enum { HTI_TOPK = 0, HTI_TOPP = 1 } hti_select_mode;

/* Shape of one layer's tree set: B sequences x Hkv KV heads, one tree each. */
typedef struct {
    int32_t B;          /* sequences */
    int32_t Hq;         /* query heads; Hq % Hkv == 0, G = Hq / Hkv in {1,2,4,8} */
    int32_t Hkv;        /* KV heads */
    int32_t d;          /* head dim: 64 or 128 */
    int32_t b;          /* tokens per level-1 node (ZHA's chunk size C), 2..64;
                           also the children per node above level 1 unless
                           `fan` says otherwise */
    int32_t levels;     /* tree levels above the tokens, 0..HTI_MAX_LEVELS */
    int32_t R;          /* reference queries per KV head, 1..HTI_MAX_R */
    int32_t dtype;      /* hti_dtype of the caches, tree nodes and q/k/v inputs */
    int64_t Lcap;       /* token capacity of the cache per (sequence, head) */
    float rope_base;    /* RoPE base (e.g. 10000) */
    int32_t rope_npos;  /* rows of the RoPE table (largest position + 1) */
    int32_t router_fp8; /* 0: summary keys are scored as stored.  1 (bf16 caches
                           only): every summary key row also has an 8-bit float
                           copy (lvl_kq, lvl_ks) that the build, append and extend
                           calls write beside it, and the traversals score every
                           summary candidate through that copy -- its selection
                           score and, unless leaf_only, its softmax logit.  Token
                           keys and all values stay in the cache dtype.  The
                           low-precision router of ZHA Figure 16 (router operands,
                           reference-key cache and scoring in low precision, the
                           KV cache and the sparse attention in bf16), here in
                           OCP E4M3: each row is divided by the power of two
                           2^(e - 8), amax = f * 2^e with f in [0.5, 1) its
                           largest magnitude (1 for an all-zero row), and
                           rounded to the nearest E4M3 value, ties to even. */
    int32_t fan;        /* children per node above level 1 (ZHA's fan F, which
                           Figure 4 and Table II name apart from the chunk size
                           C; every geometry there has F = C), 2..64; 0 means b.
                           Level 1 has floor(L / b) nodes, level l > 1
                           floor(n_{l-1} / fan).  A decode step appends in its
                           own launch when b and fan are at most 32. */
} hti_tree_cfg;

/* Device buffers of a tree set (all caller-allocated, sizes from hti_plan). */
typedef struct {
    hti_tree_cfg cfg;
    void *k_cache;                    /* [B, Hkv, Lcap, d] un-rotated token keys */
    void *v_cache;                    /* [B, Hkv, Lcap, d] token values */
    void *lvl_k[HTI_MAX_LEVELS];      /* level l+1: [B, Hkv, ncap_{l+1}, R, d] pooled keys */
    void *lvl_v[HTI_MAX_LEVELS];      /* level l+1: [B, Hkv, ncap_{l+1}, d] mean values */
    const float *ref_q;               /* [Hkv, R, d] fp32 reference queries */
    int64_t *len;                     /* [B] device: tokens currently in each tree */
    float *rope;                      /* [rope_npos, d/2, 2] fp32 (cos, sin), see hti_rope_init */
    /* cfg.router_fp8 only (else ignored): */
    uint8_t *lvl_kq[HTI_MAX_LEVELS];  /* level l+1: [B, Hkv, ncap_{l+1}, R, d] E4M3 codes of lvl_k */
    float *lvl_ks[HTI_MAX_LEVELS];    /* level l+1: [B, Hkv, ncap_{l+1}, R] their scales */
} hti_tree;

/* Per-call selection rule (RecSA: top-k per level; ZHA: top-p per level). */
typedef struct {
    int32_t mode;       /* hti_select_mode */
    int32_t k;          /* top-k: nodes kept per level, 1..HTI_MAX_SELECT */
    float p;            /* top-p: probability mass, (0, 1] */
    int32_t cap;        /* top-p: largest kept set, 1..HTI_MAX_SELECT */
    int32_t per_head;   /* 0: the G query heads of a KV group share one selection,
                           scored by the mean of their logits; 1: every query
                           head routes on its own (a group of one) over its KV
                           head's tree.  sel_out and the units then count query
                           heads instead of KV groups. */
    int32_t leaf_only;  /* 0: the unselected candidates of every level join the
                           softmax with their summaries (RecSA); 1: only the
                           reached tokens are attended, the summaries serve the
                           routing alone (the leaf union the ZHA router
                           dispatches, ZHA Figure 3 caption) */
    int32_t token_nodes;/* prefill only.  0: every query gathers its own prefix
                           token rows in the traversal (fp32 logits).  1: the
                           token level of the prefix runs node-inverted -- the
                           block's queries are grouped by the level-1 nodes they
                           kept, and each kept node's b token rows are read once
                           per block and multiplied with all of its queries on
                           the matrix cores (bf16 operands, fp32 accumulation;
                           the token level selects nothing) -- wherever the
                           geometry allows it (levels >= 1, b <= 32; else as 0).
                           Selections are the same; outputs agree to the output
                           tolerance. */
} hti_select;

/* Sizes for a configuration (all host values). */
typedef struct {
    int64_t ncap[HTI_MAX_LEVELS + 1]; /* ncap[0] = Lcap, ncap[1] = floor(Lcap / b),
                                         ncap[l] = floor(ncap[l-1] / fan) above */
    size_t cache_bytes;               /* each of k_cache, v_cache */
    size_t lvl_k_bytes[HTI_MAX_LEVELS];
    size_t lvl_v_bytes[HTI_MAX_LEVELS];
    size_t rope_bytes;
    int32_t rope_npos_needed;         /* rows hti_sparse_decode needs for this cfg and
                                         the selection passed to hti_plan */
    size_t lvl_kq_bytes[HTI_MAX_LEVELS]; /* router copies (0 unless cfg.router_fp8) */
    size_t lvl_ks_bytes[HTI_MAX_LEVELS];
} hti_plan_out;

/*
 * hti_plan: capacity of every buffer of `cfg` (host only, no device work).
 * `sel` (nullable) lets the plan report the RoPE rows decode will need, and
 * `T` the extra rows of a prefill block (0 for decode only).
 * Errors: HTI_ERR_INVALID_ARG / HTI_ERR_UNSUPPORTED on a bad cfg.
 */
hti_status hti_plan(const hti_tree_cfg *cfg, const hti_select *sel, int32_t T,
                    hti_plan_out *out);

/*
 * hti_rope_init: fill tree->rope with cos/sin of pos * base^(-2j/d) for
 * pos < rope_npos, j < d/2, each formed in double and rounded once to fp32.
 */
hti_status hti_rope_init(const hti_tree *tree, void *stream);

/*
 * hti_tree_build: build every full node of every level over the first
 * L_host[s] cached tokens of each sequence s and set len[s] = L_host[s]
 * (a streaming pooling pass over the cache, level by level).
 *   L_host: host [B], 0 <= L_host[s] <= Lcap.
 * Source: RecSA abstract (one key, one mean value per node; shared pooler);
 * ZHA Figure 3 caption (reference-query pooling of contiguous chunks,
 * recursive); ZHA Table VIII (full nodes only, all built in prefill).
 */
hti_status hti_tree_build(const hti_tree *tree, const int64_t *L_host, void *stream);

/*
 * hti_tree_append: append one token per sequence at row len[s], build every
 * node that this token completes (level 1 when (len+1) % b == 0, level 2 when
 * (len+1) % b^2 == 0, ...), then len[s] += 1.
 *   k_new, v_new: [B, Hkv, d] in the cache dtype.
 * A sequence whose cache is full (len[s] == Lcap) is left unchanged and its
 * len is not advanced (the device checks this; callers that track lengths on
 * the host should check capacity before calling).
 * Source: ZHA Table VIII (decode maintenance amortised over full-node
 * completions).
 */
hti_status hti_tree_append(const hti_tree *tree, const void *k_new, const void *v_new,
                           void *stream);

/*
 * hti_tree_extend: append a block of T tokens to every sequence (rows
 * len[s] .. len[s] + T - 1), build every node of every level that these
 * tokens complete, then len[s] += T -- the tree that hti_tree_build over the
 * longer prefix gives, bit for bit, so that decoding can follow a prefill
 * block.  A sequence takes only the tokens its cache still holds (rows past
 * Lcap are dropped and len[s] stops at Lcap; the device checks this).
 *   k_blk, v_blk: [B, T, Hkv, d] in the cache dtype (the layout of
 *   hti_sparse_prefill's block), un-rotated; T >= 0 (0: no-op).
 * Source: ZHA Table VIII (all full nodes are built in prefill; maintenance
 * amortised over full-node completions).
 */
hti_status hti_tree_extend(const hti_tree *tree, const void *k_blk, const void *v_blk, int32_t T,
                           void *stream);

/*
 * hti_decode_workspace_bytes: size of the workspace hti_sparse_decode uses to
 * split each (query, KV group) unit over several workgroups.
 */
size_t hti_decode_workspace_bytes(const hti_tree_cfg *cfg, const hti_select *sel, int32_t Nq);

/*
 * hti_sparse_decode: attention of Nq query tokens per sequence over that
 * sequence's trees.
 *   q:     [B, Nq, Hq, d] in the cache dtype (un-rotated)
 *   q_pos: [B, Nq] int64 (nullable): query n of sequence s sits at position
 *          q_pos[s, n] and attends to the tree of tokens 0..q_pos[s, n] -- the
 *          nodes wholly inside that prefix, as a decode at length q_pos + 1
 *          would see them.  NULL puts every query at len[s] - 1.  Values at
 *          or above len[s] - 1 act as len[s] - 1; a negative value attends to
 *          nothing (output 0, lse -inf).
 *   out:   [B, Nq, Hq, d] fp32 attention output
 *   lse:   [B, Nq, Hq] fp32 log-sum-exp of the logits (nullable)
 *   sel:   [B, Nq, Hkv, levels, sel_stride] int32 (nullable): node ids kept at
 *          each level (row l-1 = level l), ascending, -1 padded;
 *          sel_stride >= k (top-k) or cap (top-p).
 * Per (query, KV group): the top level's nodes are all candidates; at each
 * level the candidates are scored by the mean over the group's heads of the
 * RoPE'd logits (candidate i at position i, the query at position |C_l|), the
 * top-k (or top-p set, capped) is kept and its children, followed by the
 * level's orphan nodes, form the next level's candidates; the others enter the
 * per-head softmax with their pooled key and mean value.  At the token level
 * every candidate enters the softmax exactly.
 * Source: RecSA abstract; ZHA Figure 3 caption (top-p routing).
 *   ws, ws_bytes: device workspace of hti_decode_workspace_bytes(cfg, sel, Nq)
 *        bytes, filled with zeros before its first use and then left to the
 *        library (it keeps a status word and per-unit launch counters there).
 *        With a workspace each unit is split over up to HTI_DECODE_MAX_SPLIT
 *        workgroups that wait on each other's partial results; the grid is
 *        kept within what the device holds at once (one workgroup per
 *        compute unit, or as many as the kernel's occupancy admits, at most
 *        four, where one per CU would leave a unit fewer than eight) so that
 *        all are resident while the device runs nothing else.  Every wait is
 *        bounded: if work on other streams keeps some workgroups from starting
 *        in time, the wait runs out, the launch's outputs are NaN and the
 *        workspace's status word is set; every later launch with that
 *        workspace then writes NaN and changes nothing else until the caller
 *        zeroes the workspace (hti_decode_status reports it).  ws = NULL runs
 *        one independent workgroup per unit (no waits).  One workspace serves
 *        one (cfg, Nq) shape and one stream at a time: calls that share it
 *        must not overlap.
 * Errors additionally: HTI_ERR_CAPACITY if rope_npos is below the positions
 * this cfg/selection can reach, HTI_ERR_UNSUPPORTED if a summary level can
 * exceed HTI_MAX_CAND candidates, HTI_ERR_WORKSPACE if ws_bytes is too small.
 */
hti_status hti_sparse_decode(const hti_tree *tree, const hti_select *sel, const void *q,
                             const int64_t *q_pos, int32_t Nq, float *out, float *lse,
                             int32_t *sel_out, int32_t sel_stride, void *ws, size_t ws_bytes,
                             void *stream);

/*
 * hti_sparse_decode_static: hti_sparse_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid hipMalloc, harnesses that own every allocation).  Same arguments,
 * results and errors as hti_sparse_decode with a workspace, except that the
 * split workspace is a static device array inside the library
 * (HTI_DECODE_STATIC_SCRATCH_BYTES, 8 MiB, held by every GPU the library runs
 * on until the process ends).  The call allocates nothing: before the
 * decode it zeroes the part of the array this call's shape uses with a fill
 * kernel on `stream`, so no state carries over between calls (a wait that
 * runs out makes that call's outputs NaN and leaves nothing sticky).  All
 * calls on one GPU share its array: calls that overlap in time on that GPU
 * (other streams, other threads) race and must not be made.
 * Returns HTI_ERR_WORKSPACE if the shape needs more split workspace than
 * the array holds (hti_decode_workspace_bytes above the limit gives a bound;
 * the exact need depends on the split the device allows).
 */
#define HTI_DECODE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
hti_status hti_sparse_decode_static(const hti_tree *tree, const hti_select *sel, const void *q,
                                    const int64_t *q_pos, int32_t Nq, float *out, float *lse,
                                    int32_t *sel_out, int32_t sel_stride, void *stream);

/*
 * hti_decode_status: whether a split decode with this workspace has run out
 * of a wait (see hti_sparse_decode).  Synchronises `stream`, reads the
 * workspace's status word (4 bytes at its start) and returns HTI_OK, or
 * HTI_ERR_TIMEOUT if the word is set: the outputs of the launch that set it
 * and of every later one with this workspace are NaN, and no decode step
 * advanced a length since; the tree itself stays consistent with its stored
 * lengths.  Zeroing the workspace clears the word.
 */
hti_status hti_decode_status(const void *ws, size_t ws_bytes, void *stream);

/*
 * hti_decode_step: one decode step of every sequence -- append the step's
 * token (as hti_tree_append) and then attend (as hti_sparse_decode, the
 * queries at position len[s] - 1 of the grown sequence).  The result, the
 * caches, the tree levels and len are those of the two calls in that order.
 *   k_new, v_new: [B, Hkv, d] in the cache dtype; the other arguments as for
 *   hti_sparse_decode (the same workspace).
 * With a workspace and b <= 32 this is one kernel launch: every workgroup of
 * a (sequence, KV group) writes the new row and pools the nodes it completes
 * itself (identical bytes), and one workgroup per sequence advances len once
 * every workgroup of that sequence has read the old value (a bounded wait; a
 * timeout sets the status word and leaves the length, as in
 * hti_sparse_decode).  The queries sit at len[s] - 1 of the grown sequence
 * (no q_pos).  Otherwise
 * it runs the two calls.  The workspace keeps a per-sequence count between
 * steps, so steps that share it must not overlap.
 * Source: RecSA abstract (decoding over the tree); ZHA Table VIII (decode
 * maintenance amortised over full-node completions).
 */
hti_status hti_decode_step(const hti_tree *tree, const hti_select *sel, const void *k_new,
                           const void *v_new, const void *q, int32_t Nq, float *out, float *lse,
                           int32_t *sel_out, int32_t sel_stride, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * hti_prefill_workspace_bytes: device workspace hti_sparse_prefill needs.
 */
size_t hti_prefill_workspace_bytes(const hti_tree_cfg *cfg, const hti_select *sel, int32_t T);

/*
 * hti_sparse_prefill: attention of a block of T new tokens per sequence,
 * at positions len[s] .. len[s] + T - 1, over the tree of the prefix
 * [0, len[s]) plus causal attention inside the block, merged in one softmax.
 * The tree is not extended by the block.
 *   q_blk: [B, T, Hq, d], k_blk, v_blk: [B, T, Hkv, d] (cache dtype, un-rotated)
 *   out:   [B, T, Hq, d] fp32;  lse: [B, T, Hq] fp32 (nullable)
 *   sel_out: [B, T, Hkv, levels, sel_stride] int32 (nullable), as in decode
 *   ws, ws_bytes: device workspace of at least hti_prefill_workspace_bytes()
 * Candidate lists and prefix positions follow decode; at the token level the
 * prefix candidates are followed by the block tokens 0..t, and query t sits
 * at position (number of prefix candidates) + t.  Attention weights are
 * rounded to bf16 before they multiply values (the denominators sum the
 * rounded weights); scores and the selection are fp32.
 * A tree set with cfg.Lcap == 0 (the first block of new sequences) holds no
 * prefix: the call then runs the causal attention inside the block alone,
 * with no traversal, and fills sel_out with -1.
 * Errors: as decode; HTI_ERR_UNSUPPORTED also for dtype other than bf16 and
 * when one (sequence, KV head) slice of the cache or of a level's keys
 * reaches 4 GiB.
 * Source: RecSA abstract (prefill with the same tree and shared softmax).
 */
hti_status hti_sparse_prefill(const hti_tree *tree, const hti_select *sel, const void *q_blk,
                              const void *k_blk, const void *v_blk, int32_t T, float *out,
                              float *lse, int32_t *sel_out, int32_t sel_stride, void *ws,
                              size_t ws_bytes, void *stream);

/* Description of the last error on the calling thread ("" if none). */
const char *hti_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HTI_H */
