// hti_internal.h -- kernel argument blocks and launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hti.h"

namespace hti {

constexpr int kMaxCand = HTI_MAX_CAND;
constexpr int kMaxSel = HTI_MAX_SELECT;

// Device view of one tree set (copied by value into kernel arguments).
struct TreeArgs {
    const void *kc, *vc;                 // [B, Hkv, Lcap, D]
    void *lk[HTI_MAX_LEVELS];            // level l+1 keys [B, Hkv, ncap, R, D]
    void *lv[HTI_MAX_LEVELS];            // level l+1 values [B, Hkv, ncap, D]
    uint8_t *lkq[HTI_MAX_LEVELS];        // level l+1 E4M3 router keys [B, Hkv, ncap, R, D] (rfp8)
    float *lks[HTI_MAX_LEVELS];          // their row scales [B, Hkv, ncap, R] (rfp8)
    int64_t ncap[HTI_MAX_LEVELS + 1];    // ncap[0] = Lcap
    const float *refs;                   // [Hkv, R, D]
    int64_t *len;                        // [B]
    const float2 *rope;                  // [rope_npos, D/2] (cos, sin)
    int rope_npos;
    int B, Hq, Hkv, D, b, levels, R, G;
    // Traversals: Hkv routing heads per sequence, G query heads each; the
    // tree arrays of routing head g are those of KV head g / hdiv, of
    // Hkv / hdiv per sequence (hdiv > 1: every query head routes on its own)
    int hdiv;
    float scale;                         // 1 / sqrt(D)
    int dtype;
    int rfp8;                            // summary keys are scored through lkq / lks
};

// Selection rule and the query-side buffers of one traversal launch.
struct TravArgs {
    TreeArgs t;
    int mode, k, cap;
    float p;
    int leaf_only;     // 1: summaries route but do not join the softmax
    uint32_t binv;     // ceil(2^32 / b), for division by b in index arithmetic
    const void *q;     // decode [B, Nq, Hq, D]; prefill [B, T, Hq, D]
    int Nq;            // queries per sequence (decode) or block length T (prefill)
    float *out;        // decode [B, Nq, Hq, D]
    float *lse;        // decode [B, Nq, Hq] (nullable)
    int *sel;          // [B, Nq, Hkv, levels, sel_stride] (nullable)
    int sel_stride;
    // decode step: the token appended to every sequence before the queries
    // attend, [B, Hkv, D] each (nullptr: plain decode)
    const void *k_new, *v_new;
    // prefill only
    const float *top_s;  // [B, T, Hkv, ntop_stride] group scores of the top level (nullable)
    const float *top_z;  // [B, T, Hq, ntop_stride] per-head logits of the top level
    int ntop_stride;
    float *part_acc;     // [B, T, Hq, D] unnormalised partial outputs
    float *part_ml;      // [B, T, Hq, 2] running max and denominator
};

// Workspace of the split decode (zeroed by the caller before first use, then
// owned by the library): per-unit launch epoch, per-unit timeout marks, the
// per-level exchange words and the per-workgroup partial states, all as words
// tagged with the launch epoch.
struct DecodeWs {
    int W;              // workgroups per (query, KV group) unit
    uint32_t *epoch;    // [units]
    uint32_t *err;      // [units]: tag of the last launch in which a wait timed out
    uint64_t *words;    // [units][levels][W][HTI_MAX_SELECT + 2]
    uint64_t *part;     // [units][W][G][D + 2]: tag << 32 | fp32 bits
    uint32_t *seqcnt;   // [B]: workgroups of a decode step that have read the sequence length
};
// W > 0: split each unit over W workgroups; W == 0: one workgroup per unit.
hipError_t decode_split_plan(const TravArgs &a, int64_t units, int64_t max_summary, int *W);
size_t decode_ws_bytes(int B, int64_t units, int W, int levels, int G, int D);
DecodeWs decode_ws_layout(void *base, int B, int64_t units, int W, int levels, int G, int D);
hipError_t launch_decode_split(const TravArgs &a, const DecodeWs &ws, int64_t units, hipStream_t s);

hipError_t launch_rope_init(const TreeArgs &t, double base, hipStream_t s);
hipError_t launch_build_level(const TreeArgs &t, int lvl, int64_t max_nodes, hipStream_t s);
hipError_t launch_append(const TreeArgs &t, const void *k_new, const void *v_new, hipStream_t s);
hipError_t launch_extend(const TreeArgs &t, const void *k_blk, const void *v_blk, int T, hipStream_t s);
hipError_t launch_traverse(const TravArgs &a, bool prefill, int64_t units, hipStream_t s);
// Prefill traversal, one wave per (query, KV group) unit; max_summary bounds
// the candidate list of every summary level.
hipError_t launch_prefill_walk(const TravArgs &a, int64_t max_summary, int64_t units, hipStream_t s);

// Prefill dense parts (MFMA).
struct PrefillArgs {
    TreeArgs t;
    const void *q, *k, *v;     // block [B, T, Hq|Hkv, D]
    int T;
    float *top_s, *top_z;      // outputs of the top-level scoring
    int ntop_stride;
    const float *part_acc, *part_ml;
    float *out, *lse;
    void *qr, *kr;             // rotated block q/k (bf16 staging) [B, Hq|Hkv, T, D]
    void *vt;                  // block v transposed (bf16 staging) [B, Hkv, D, Tp]
    int Tp;                    // T rounded up to the in-block key tile
};
// Top-level scoring of a prefill block on the matrix cores; used when the top
// level has at most kTopCols (node, reference key) columns.
constexpr int kTopCols = 64;
// Key tile of the in-block product; the transposed V rows are padded to it.
constexpr int kInblockKeys = 64;
hipError_t launch_top_scores(const PrefillArgs &a, hipStream_t s);
hipError_t launch_rotate_block(const PrefillArgs &a, hipStream_t s);
hipError_t launch_inblock_attention(const PrefillArgs &a, hipStream_t s);

} // namespace hti
