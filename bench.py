"""Benchmark of the tree-indexed sparse attention hot path on one MI355X.

Headline (value): decode queries/s at 1,048,576 context, batch 4, where one
step = tree_append of one token per sequence + sparse_decode of one query per
sequence (32 query heads over 8 KV heads, d 128, bf16, b 32, 4 levels, top-k 8);
the timed steps are captured into one HIP graph and replayed (an eager pass,
one host launch per call, is timed beside it and gives the decode kernel's
time for the roofline).  Reported beside it: achieved HBM
GB/s of the decode traversal kernel (algorithmic bytes / kernel time) and the
prefill throughput (tokens/s) of an 8192-token block over a 524,288-token
prefix including tree_build of the prefix.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import hierarchical_tree_indexed_amd as hti  # noqa: E402
import hti_workloads as W  # noqa: E402

METRIC = "decode queries/s + achieved HBM GB/s at 1M ctx; prefill tokens/s at 524K"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DEV = "cuda"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gen_kv_device(w, Lcap):
    """Seeded N(0,1) caches drawn on the device, one (sequence, head) at a time."""
    dt = W.TORCH_DTYPE[w.dtype]
    K = torch.zeros((w.B, w.Hkv, Lcap, w.d), dtype=dt, device=DEV)
    V = torch.zeros_like(K)
    g = torch.Generator(device=DEV)
    for bi in range(w.B):
        for h in range(w.Hkv):
            g.manual_seed(1_000_003 * (w.seed + 1) + 4096 * bi + h)
            K[bi, h, : w.L] = torch.randn((w.L, w.d), generator=g, device=DEV).to(dt)
            V[bi, h, : w.L] = torch.randn((w.L, w.d), generator=g, device=DEV).to(dt)
    return K, V


def treeset(w, Lcap, K, V, T=0):
    sel = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap)
    cfg = hti.make_cfg(w.B, w.Hq, w.Hkv, w.d, w.b, w.levels, w.R, w.dtype, Lcap, w.rope_base, 1, fan=w.fan)
    cfg.rope_npos = hti.plan(cfg, sel, T).rope_npos_needed
    ts = hti.TreeSet(cfg, device=DEV, k_cache=K, v_cache=V)
    ts.ref_q.copy_(W.gen_refs(w))
    ts.rope_init()
    return ts, sel


def decode_unit_bytes(w, L, router_fp8=False):
    """Algorithmic bytes one (query, KV group) unit must touch at length L:
    scored keys (x R) + unselected summary values + token keys and values,
    plus its query and output rows.  Entry = d elements of the cache dtype;
    with 8-bit router keys a summary key is d bytes and a 4-byte scale."""
    n = w.level_counts(L)
    keff = w.k if w.mode == "topk" else w.cap
    thr = w.k if w.mode == "topk" else 1
    keys = vals = 0
    m = n[w.levels]
    skeys = 0
    for lvl in range(w.levels, 0, -1):
        if m > thr:
            nsel = min(keff, m)
            skeys += m * w.R
            vals += m - nsel
        else:
            nsel = m
        f = w.b if lvl == 1 else w.F                     # children per node of level lvl
        m = nsel * f + (n[lvl - 1] - f * n[lvl])
    keys += m
    vals += m
    e = w.d * w.elem_bytes
    ek = w.d + 4 if router_fp8 else e
    return skeys * ek + (keys + vals) * e + w.G * w.d * (w.elem_bytes + 4)


def bench_decode(args):
    w = W.DEC1M
    S, Wm = args.steps, args.warmup
    Lcap = w.L + Wm + 2 * S
    log(f"[decode] generating {w.B}x{w.Hkv}x{w.L} bf16 K/V on the device")
    K, V = gen_kv_device(w, Lcap)
    q0 = W.gen_queries(w, 0, device=DEV)
    W.plant_needles(w, K, q0)
    ts, sel = treeset(w, Lcap, K, V)
    ts.tree_build([w.L] * w.B)
    torch.cuda.synchronize()
    log("[decode] tree built")
    dt = W.TORCH_DTYPE[w.dtype]
    gq = torch.Generator(device=DEV)
    gq.manual_seed(12345)
    nstep = Wm + 2 * S
    qs = torch.randn((nstep, w.B, 1, w.Hq, w.d), generator=gq, device=DEV).to(dt)
    ak = torch.randn((nstep, w.B, w.Hkv, w.d), generator=gq, device=DEV).to(dt)
    av = torch.randn((nstep, w.B, w.Hkv, w.d), generator=gq, device=DEV).to(dt)
    out = torch.empty((w.B, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, 1, w.Hq), dtype=torch.float32, device=DEV)

    def step(s):
        # append this step's token and attend: one launch (decode_step)
        ts.decode_step(sel, ak[s], av[s], qs[s], out, lse)

    for s in range(Wm):
        step(s)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(S)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for s in range(S):
        ev[s][0].record()
        step(Wm + s)
        ev[s][1].record()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_ms = e0.elapsed_time(e1)
    dec_ms = sum(a.elapsed_time(b) for a, b in ev) / S
    bytes_per_launch = sum(decode_unit_bytes(w, w.L + Wm + s + 1) for s in range(S)) / S * w.B * w.Hkv

    # The next S steps (fresh tokens and queries) captured into one HIP graph
    # and replayed once: back-to-back launches of the step kernel, so the
    # events bracket S kernels with only the dispatch gaps between them.
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            for s in range(S):
                step(Wm + S + s)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    total_ms = g0.elapsed_time(g1)
    del graph
    kern_ms = total_ms / S

    ph_ms = lf_ms = plain_ms = r8_ms = float("nan")
    if not args.no_variants:
        ph_ms, lf_ms, plain_ms, r8_ms = decode_variants(ts, w, qs, Wm, S, out, cs)
    Lr = w.L + Wm + 2 * S
    res = dict(ms_per_step=total_ms / S, eager_ms_per_step=eager_ms / S, wall_s=wall,
               decode_kernel_ms=kern_ms, decode_eager_kernel_ms=dec_ms, bytes_per_launch=bytes_per_launch,
               qps=w.B * S / (total_ms / 1e3),
               gbs=bytes_per_launch / (kern_ms / 1e3) / 1e9,
               per_head_ms=ph_ms, per_head_qps=w.B / (ph_ms / 1e3),
               per_head_gbs=decode_unit_bytes(w, w.L + Wm + 2 * S) * w.B * w.Hq / (ph_ms / 1e3) / 1e9,
               leaf_only_ms=lf_ms, leaf_only_qps=w.B / (lf_ms / 1e3),
               plain_ms=plain_ms, plain_gbs=decode_unit_bytes(w, Lr) * w.B * w.Hkv / (plain_ms / 1e3) / 1e9,
               r8_ms=r8_ms, r8_qps=w.B / (r8_ms / 1e3),
               r8_gbs=decode_unit_bytes(w, Lr, True) * w.B * w.Hkv / (r8_ms / 1e3) / 1e9,
               r8_bytes=decode_unit_bytes(w, Lr, True) * w.B * w.Hkv,
               plain_bytes=decode_unit_bytes(w, Lr) * w.B * w.Hkv)
    log(f"[decode] {res}")
    del K, V, ts
    torch.cuda.empty_cache()
    return res


def finite(x):
    """x, or None where a timing was skipped (NaN)"""
    return None if x != x else x


def decode_variants(ts, w, qs, Wm, S, out, cs):
    """Graph-timed sparse_decode per step under per-query-head routing, under
    leaf-only dispatch, plain, and with 8-bit router keys (the tree as the
    main step left it)."""
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # per-query-head routing (every query head its own selection): the same
    # queries at the reached length, sparse_decode without the append, S
    # calls in one graph
    sel_ph = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, per_head=True)
    out_ph = torch.empty_like(out)
    for s in range(4):
        ts.sparse_decode(sel_ph, qs[s], out_ph)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            for s in range(S):
                ts.sparse_decode(sel_ph, qs[Wm + s], out_ph)
    torch.cuda.synchronize()
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    ph_ms = g0.elapsed_time(g1) / S
    del graph

    # leaf-only dispatch (the summaries route, only the reached tokens are
    # attended): the same queries, timed the same way
    sel_lf = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, leaf_only=True)
    for s in range(4):
        ts.sparse_decode(sel_lf, qs[s], out_ph)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            for s in range(S):
                ts.sparse_decode(sel_lf, qs[Wm + s], out_ph)
    torch.cuda.synchronize()
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    lf_ms = g0.elapsed_time(g1) / S
    del graph

    # plain sparse_decode on the bf16 keys, then the same call on a second
    # tree set over the same caches whose summary keys carry the 8-bit router
    # copy (built at the reached length)
    def gtime(t_, sel_):
        for s in range(4):
            t_.sparse_decode(sel_, qs[s], out_ph)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cs):
            with torch.cuda.graph(gr, stream=cs):
                for s in range(S):
                    t_.sparse_decode(sel_, qs[Wm + s], out_ph)
        torch.cuda.synchronize()
        g0.record()
        gr.replay()
        g1.record()
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) / S

    sel = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap)
    plain_ms = gtime(ts, sel)
    cfg8 = hti.TreeCfg.from_buffer_copy(ts.cfg)
    cfg8.router_fp8 = 1
    ts8 = hti.TreeSet(cfg8, device=DEV, k_cache=ts.k_cache, v_cache=ts.v_cache)
    ts8.ref_q.copy_(ts.ref_q)
    ts8.rope_init()
    ts8.tree_build(ts.len.cpu().tolist())
    r8_ms = gtime(ts8, sel)
    del ts8
    return ph_ms, lf_ms, plain_ms, r8_ms


def graph_ms(fn, S, warm=4):
    """Average time of fn() over S calls captured into one HIP graph and
    replayed once (events on the replay stream)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            for _ in range(S):
                fn()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    del graph
    return g0.elapsed_time(g1) / S


def build_bytes(w, L):
    """Algorithmic bytes of tree_build over L tokens of every (sequence, KV
    head): each level reads its children's keys (one per token at level 1,
    R per node above) and values, and writes its nodes' R keys and value."""
    n = w.level_counts(L)
    row = w.d * w.elem_bytes
    tot = 0
    for lvl in range(1, w.levels + 1):
        tot += n[lvl - 1] * ((1 if lvl == 1 else w.R) + 1) * row
        tot += n[lvl] * (w.R + 1) * row
    return tot * w.B * w.Hkv


def bench_side_workloads(args):
    """The 131,072-token decode (one query, 8 KV groups, 8 planted needles),
    the 1M-token batch-4 decode on a chunk-32 / fan-8 tree, and the
    2,097,152-token top-p workload with four reference keys per node
    (tree_build of the whole context, then one top-p decode query), each
    against the HBM roofline of its algorithmic bytes."""
    res = {}
    reps = max(16, args.steps // 4)
    w = W.DEC128K
    K, V = gen_kv_device(w, w.L)
    q0 = W.gen_queries(w, 0, device=DEV)
    W.plant_needles(w, K, q0)
    ts, sel = treeset(w, w.L, K, V)
    ts.tree_build([w.L] * w.B)
    out = torch.empty((w.B, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
    ms = graph_ms(lambda: ts.sparse_decode(sel, q0, out), reps)
    by = decode_unit_bytes(w, w.L) * w.B * w.Hkv
    res["decode_128k"] = dict(ms=ms, queries_per_s=w.B / (ms / 1e3), bytes=by, gbs=by / (ms / 1e3) / 1e9,
                              frac_hbm=by / (ms / 1e3) / 1e9 / HBM_PEAK_GBS)
    log(f"[side] decode_128k {res['decode_128k']}")
    del K, V, ts
    torch.cuda.empty_cache()
    # the 1M-token, batch-4 decode on a tree with chunk size 32 at level 1 and
    # fan 8 above (five levels) instead of C = F = 32 (four levels): the
    # depth-for-width trade of the pages' tree geometries
    w = W.DEC1M.replace(name="decode_1m_b4_c32_f8", fan=8, levels=5)
    K, V = gen_kv_device(w, w.L)
    q0 = W.gen_queries(w, 0, device=DEV)
    W.plant_needles(w, K, q0)
    ts, sel = treeset(w, w.L, K, V)
    ts.tree_build([w.L] * w.B)
    out = torch.empty((w.B, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
    ms = graph_ms(lambda: ts.sparse_decode(sel, q0, out), reps)
    by = decode_unit_bytes(w, w.L) * w.B * w.Hkv
    res["decode_1m_c32_f8"] = dict(ms=ms, queries_per_s=w.B / (ms / 1e3), bytes=by, gbs=by / (ms / 1e3) / 1e9,
                                   frac_hbm=by / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, levels=w.levels, chunk=w.b,
                                   fan=w.F)
    log(f"[side] decode_1m_c32_f8 {res['decode_1m_c32_f8']}")
    del K, V, ts
    torch.cuda.empty_cache()
    w = W.ZHA2M
    K, V = gen_kv_device(w, w.L)
    ts, sel = treeset(w, w.L, K, V)
    ts.tree_build([w.L] * w.B)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bms = []
    for r in range(2 + args.prefill_reps):
        e0.record()
        ts.tree_build([w.L] * w.B)
        e1.record()
        torch.cuda.synchronize()
        if r >= 2:
            bms.append(e0.elapsed_time(e1))
    bms = sum(bms) / len(bms)
    bb = build_bytes(w, w.L)
    q = W.gen_queries(w, 0, device=DEV)
    out = torch.empty((w.B, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
    ms = graph_ms(lambda: ts.sparse_decode(sel, q, out), reps)
    by = decode_unit_bytes(w, w.L) * w.B * w.Hkv
    res["zha_topp_2m_r4"] = dict(build_ms=bms, build_bytes=bb, build_gbs=bb / (bms / 1e3) / 1e9,
                                 build_frac_hbm=bb / (bms / 1e3) / 1e9 / HBM_PEAK_GBS,
                                 decode_ms=ms, decode_queries_per_s=w.B / (ms / 1e3),
                                 decode_bytes_upper=by, decode_gbs_upper=by / (ms / 1e3) / 1e9,
                                 decode_frac_hbm_upper=by / (ms / 1e3) / 1e9 / HBM_PEAK_GBS)
    log(f"[side] zha_topp_2m_r4 {res['zha_topp_2m_r4']}")
    del K, V, ts
    torch.cuda.empty_cache()
    return res


def bench_prefill(args):
    w = W.PREFILL
    log(f"[prefill] generating prefix {w.L} and block {w.T}")
    K, V = gen_kv_device(w, w.L)
    qb, kb, vb = W.gen_block(w, device=DEV)
    ts, sel = treeset(w, w.L, K, V, T=w.T)
    # the prefix token level node-inverted (queries grouped by kept level-1
    # node, each node's token rows read once per block) instead of walked per
    # query: a variant, with the larger workspace
    sel_tw = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, token_nodes=True)
    ws = torch.empty(max(ts.prefill_workspace_bytes(sel, w.T), ts.prefill_workspace_bytes(sel_tw, w.T)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((w.B, w.T, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.T, w.Hq), dtype=torch.float32, device=DEV)

    def run():
        ts.tree_build([w.L] * w.B)
        ts.sparse_prefill(sel, qb, kb, vb, out, ws, lse)

    def timed(fn, reps):
        for _ in range(args.prefill_warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(run, args.prefill_reps)
    sel_lf = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, leaf_only=True)

    def run_lf():
        ts.tree_build([w.L] * w.B)
        ts.sparse_prefill(sel_lf, qb, kb, vb, out, ws, lse)

    ms_lf = float("nan") if args.no_variants else timed(run_lf, args.prefill_reps)
    def run_tw():
        ts.tree_build([w.L] * w.B)
        ts.sparse_prefill(sel_tw, qb, kb, vb, out, ws, lse)

    ms_tw = float("nan") if args.no_variants else timed(run_tw, args.prefill_reps)
    # 8-bit router keys: a tree set over the same prefix whose summary keys
    # carry the E4M3 copy, built and prefilled the same way
    ms_r8 = float("nan")
    if not args.no_variants:
        cfg8 = hti.TreeCfg.from_buffer_copy(ts.cfg)
        cfg8.router_fp8 = 1
        ts8 = hti.TreeSet(cfg8, device=DEV, k_cache=K, v_cache=V)
        ts8.ref_q.copy_(ts.ref_q)
        ts8.rope_init()

        def run_r8():
            ts8.tree_build([w.L] * w.B)
            ts8.sparse_prefill(sel, qb, kb, vb, out, ws, lse)

        ms_r8 = timed(run_r8, args.prefill_reps)
        del ts8
    # the dense part alone: the same block in a tree set without prefix
    # capacity (the first block of a sequence) runs only the in-block causal
    # attention on the matrix cores, plus the rotation of the block's keys
    # and the transpose of its values
    ts0, sel0 = treeset(w.replace(L=0), 0, None, None, T=w.T)
    ts0.tree_build([0] * w.B)
    ws0 = torch.empty(ts0.prefill_workspace_bytes(sel0, w.T), dtype=torch.uint8, device=DEV)
    ms_dense = timed(lambda: ts0.sparse_prefill(sel0, qb, kb, vb, out, ws0, lse), args.prefill_reps)
    pairs = w.T * (w.T + 1) // 2
    inblock_flop = pairs * w.Hq * 4 * w.d
    # the block folded into the tree (tree_extend), so that decoding can
    # follow the prefill: timed alone, each time after a rebuild of the
    # prefix tree
    del ts0, ws0
    Kx = torch.zeros((w.B, w.Hkv, w.L + w.T, w.d), dtype=K.dtype, device=DEV)
    Vx = torch.zeros_like(Kx)
    Kx[:, :, :w.L] = K
    Vx[:, :, :w.L] = V
    tsx, _ = treeset(w, w.L + w.T, Kx, Vx, T=w.T)
    kbc, vbc = kb.contiguous(), vb.contiguous()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ext = []
    for r in range(args.prefill_warmup + args.prefill_reps):
        tsx.tree_build([w.L] * w.B)
        e0.record()
        tsx.tree_extend(kbc, vbc)
        e1.record()
        torch.cuda.synchronize()
        if r >= args.prefill_warmup:
            ext.append(e0.elapsed_time(e1))
    ms_ext = sum(ext) / len(ext)
    # block K and V read, cache rows written, then read again by the pooling
    # of the nodes they complete, plus those nodes' keys (x R) and values
    row_bytes = w.B * w.T * w.Hkv * w.d * W.TORCH_DTYPE[w.dtype].itemsize
    nodes = sum(a - b for a, b in zip(w.level_counts(w.L + w.T)[1:], w.level_counts(w.L)[1:]))
    ext_bytes = 3 * 2 * row_bytes + nodes * w.B * w.Hkv * (w.R + 1) * w.d * W.TORCH_DTYPE[w.dtype].itemsize
    res = dict(ms_per_block=ms, tokens_per_s=w.T * w.B / (ms / 1e3), inblock_gflop=inblock_flop / 1e9,
               dense_ms=ms_dense, dense_tflops=inblock_flop / (ms_dense / 1e3) / 1e12,
               extend_ms=ms_ext, extend_gbs=ext_bytes / (ms_ext / 1e3) / 1e9, leaf_only_ms=ms_lf,
               r8_ms=ms_r8, token_nodes_ms=ms_tw)
    log(f"[prefill] {res}")
    del K, V, ts, ws, tsx, Kx, Vx
    torch.cuda.empty_cache()
    return res


DECODE_SOURCES = ("hierarchical_tree_indexed_amd/csrc/hti_decode.hip", "hierarchical_tree_indexed_amd/csrc/hti_pool.h",
                  "hierarchical_tree_indexed_amd/csrc/hti_device.h", "hierarchical_tree_indexed_amd/csrc/hti_internal.h",
                  "hierarchical_tree_indexed_amd/csrc/hti_trav_common.h", "include/hti.h")


def decode_source_sha():
    """sha1 over the decode kernel's source file and the headers it includes."""
    import hashlib
    h = hashlib.sha1()
    for f in DECODE_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, if it
    was taken on the decode kernel source as it is now (else None)."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        rec = json.load(open(path))
        sha = decode_source_sha()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha1") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration():
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters: 1 GiB read + 1 GiB written per launch."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=DEV).fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[copy] 5 copies of {n} bytes")


PHASES = {1: "entry", 2: "length and query read", 3: "first gathers issued", 4: "scored (B1)",
          5: "slice ranked (B2)", 6: "slice published", 7: "exchange read (B3)", 8: "exchange ranked (B4)",
          9: "kept set known", 10: "next gathers issued", 11: "level folded", 12: "tokens scored",
          13: "tokens folded", 14: "partial stored", 15: "arrival counted", 16: "output written (last arrival)",
          17: "take-all levels resolved", 18: "first keys issued", 19: "append checked",
          20: "length, epoch and status loaded", 21: "query loaded", 22: "new row stored",
          23: "running max updated", 24: "slice ranked (wave 0)", 25: "slice entries read (wave 0)",
          26: "vector memory drained (wave 0)"}


def decode_timeline(args):
    """Phase timeline of the split decode step on the headline workload, from
    the timeline build of the library (libhti_timeline.so, the kernel with
    clock readings at each phase boundary): per phase, the median over
    workgroups and launches of the time since the launch's first workgroup
    started, in microseconds.  The launches sampled are the last of a run of
    back-to-back steps in one HIP graph, as the benchmark runs them; the
    entry spread of launches made one at a time, each after a
    synchronisation, is reported beside it."""
    import numpy as np
    hti.LIB_PATH = os.path.join(ROOT, "hierarchical_tree_indexed_amd", "libhti_timeline.so")
    hti.lib()
    w = W.DEC1M
    # (17 steps per graph, 32 replays: the sampled launches append at 32
    # different positions modulo the chunk size, so that the share that
    # completes a node is the workload's own, 1 in 32)
    n_eager, n_graph, reps = 16, 17, 32
    nst = n_eager + n_graph
    Lcap = w.L + n_eager + n_graph * (reps + 1) + 8
    K, V = gen_kv_device(w, Lcap)
    q0 = W.gen_queries(w, 0, device=DEV)
    W.plant_needles(w, K, q0)
    ts, sel = treeset(w, Lcap, K, V)
    ts.tree_build([w.L] * w.B)
    dt = W.TORCH_DTYPE[w.dtype]
    gq = torch.Generator(device=DEV)
    gq.manual_seed(12345)
    qs = torch.randn((nst, w.B, 1, w.Hq, w.d), generator=gq, device=DEV).to(dt)
    ak = torch.randn((nst, w.B, w.Hkv, w.d), generator=gq, device=DEV).to(dt)
    av = torch.randn((nst, w.B, w.Hkv, w.d), generator=gq, device=DEV).to(dt)
    out = torch.empty((w.B, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
    ws = ts.decode_workspace(sel, 1)
    tl = ws[256: 256 + 8192 * 64 * 8].view(torch.int64).view(8192, 64)
    mask48 = (1 << 48) - 1

    def launch_events():
        # the stamps of the most recent launch: [blocks, events], zero-padded
        ev = tl.cpu().numpy()
        return ev[(ev[:, 0] != 0)]

    eager_spread = []
    for s in range(n_eager):
        ts.decode_step(sel, ak[s], av[s], qs[s], out)
        torch.cuda.synchronize()
        if s >= 4:
            ent = launch_events()[:, 0] & mask48
            eager_spread.append(float(np.percentile(ent - ent.min(), 90)) * 0.01)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            for s in range(n_eager, nst):
                ts.decode_step(sel, ak[s], av[s], qs[s], out)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    samples = {}
    ends = []
    for _ in range(reps):
        graph.replay()
        torch.cuda.synchronize()
        used = launch_events()
        t0 = (used[:, 0] & mask48).min()
        for row in used:
            for e in row:
                if e == 0:
                    break
                ph, lv, tk = int(e >> 52), int((e >> 48) & 15), int(e & mask48)
                samples.setdefault((ph, lv), []).append((tk - t0) * 0.01)      # 100 MHz ticks -> us
        ends.append(((used & mask48).max() - t0) * 0.01)
    del graph
    rows = []
    for (ph, lv), v in sorted(samples.items(), key=lambda kv: np.median(kv[1])):
        rows.append(dict(phase=PHASES.get(ph, str(ph)), level=lv, median_us=float(np.median(v)),
                         p10_us=float(np.percentile(v, 10)), p90_us=float(np.percentile(v, 90)), n=len(v)))
    res = dict(workload=w.name, launches="last of %d back-to-back steps in a HIP graph, %d replays" % (n_graph, reps),
               kernel_span_us_median=float(np.median(ends)),
               eager_entry_spread_p90_us_median=float(np.median(eager_spread)), phases=rows)
    for r in rows:
        log(f"[timeline] {r['median_us']:7.2f} us (p10 {r['p10_us']:6.2f}, p90 {r['p90_us']:6.2f})  "
            f"level {r['level']}  {r['phase']}")
    log(f"[timeline] kernel span (first entry to last event) median {res['kernel_span_us_median']:.2f} us")
    log(f"[timeline] entry spread (p90) of launches made one at a time after a synchronisation: "
        f"median {res['eager_entry_spread_p90_us_median']:.2f} us")
    return res


def measure_floors():
    """On-device floors from the probe library (hti_probe.hip): dependent-load
    latency in L2, in the memory-side cache and in HBM; the one-way latency of
    an exchange between two workgroups through agent-scope atomics (same and
    different XCD); streaming read and copy bandwidth; bf16 matrix-core
    throughput.  These are the measured peaks the roofline fractions are also
    given against."""
    import ctypes as C
    path = os.path.join(ROOT, "hierarchical_tree_indexed_amd", "libhti_probe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python hierarchical_tree_indexed_amd/build.py`")
    P = C.CDLL(path)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    P.hti_probe_wallclock_khz.argtypes = [vp]
    P.hti_probe_chase.argtypes = [vp, C.c_uint32, i32, i32, vp, vp]
    P.hti_probe_pingpong.argtypes = [vp, i32, i32, vp, vp]
    P.hti_probe_read.argtypes = [vp, i64, vp, i32, vp]
    P.hti_probe_mfma.argtypes = [vp, i32, i32, vp]
    khz = C.c_int(0)
    assert P.hti_probe_wallclock_khz(C.byref(khz)) == 0 and khz.value > 0
    tick_ns = 1e6 / khz.value
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(2, dtype=torch.int64, device=DEV)
    res = {"wallclock_khz": khz.value, "cus": cus}

    def chain(nbytes):
        lines = nbytes // 128
        perm = torch.randperm(lines, device=DEV)
        buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
        buf.view(lines, 32)[perm, 0] = (torch.roll(perm, -1) * 32).to(torch.int32)
        return buf, int(perm[0].item()) * 32, lines

    def chase(buf, start, steps, coherent=0):
        assert P.hti_probe_chase(buf.data_ptr(), start, steps, coherent, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        return out[0].item() * tick_ns / steps

    steps = 20000
    for name, nbytes, warm in (("l2_hit", 1 << 20, True), ("mall_hit", 64 << 20, True),
                               ("hbm_1gib", 1 << 30, False), ("hbm_8gib", 8 << 30, False)):
        buf, start, lines = chain(nbytes)
        if warm:
            chase(buf, start, lines)
        res[f"chase_ns_{name}"] = chase(buf, start, steps)
        if name == "l2_hit":
            res["chase_ns_l2_agent_scope"] = chase(buf, start, steps, coherent=1)
        del buf
        torch.cuda.empty_cache()
    log(f"[floors] dependent loads (ns): " + ", ".join(f"{k[9:]} {v:.0f}" for k, v in res.items()
                                                       if k.startswith("chase_ns_")))
    flags = torch.zeros(64, dtype=torch.int32, device=DEV)
    for name, other in (("same_xcd", 8), ("other_xcd", 1)):
        flags.zero_()
        iters = 2000
        assert P.hti_probe_pingpong(flags.data_ptr(), iters, other, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        assert out[1].item() == 0, "ping-pong poll ran out"
        res[f"exchange_ns_{name}"] = out[0].item() * tick_ns / iters / 2
    log(f"[floors] one-way exchange (ns): same XCD {res['exchange_ns_same_xcd']:.0f}, "
        f"other XCD {res['exchange_ns_other_xcd']:.0f}")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nbytes = 8 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device=DEV).fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    best = float("inf")
    for _ in range(4):
        e0.record()
        assert P.hti_probe_read(a.data_ptr(), nbytes, sink.data_ptr(), cus * 8, stream) == 0
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    res["read_gbs"] = nbytes / (best / 1e3) / 1e9
    half = nbytes // 2
    best = float("inf")
    for _ in range(4):
        e0.record()
        a[half:].copy_(a[:half])
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    res["copy_gbs"] = 2 * half / (best / 1e3) / 1e9
    del a
    torch.cuda.empty_cache()
    fsink = torch.zeros(1, dtype=torch.float32, device=DEV)
    blocks, iters = cus * 8, 20000
    best = float("inf")
    for _ in range(3):
        e0.record()
        assert P.hti_probe_mfma(fsink.data_ptr(), blocks, iters, stream) == 0
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    flop = blocks * 4 * iters * 4 * 2 * 32 * 32 * 16
    res["mfma_bf16_tflops"] = flop / (best / 1e3) / 1e12
    log(f"[floors] read {res['read_gbs']:.0f} GB/s, copy {res['copy_gbs']:.0f} GB/s, "
        f"bf16 MFMA {res['mfma_bf16_tflops']:.0f} TFLOP/s")
    # launch ramp: entry-time spread of 256 workgroups (the split decode's
    # grid) at several workgroup sizes, 40 KB of LDS each
    P.hti_probe_entry.argtypes = [vp, i32, i32, i32, vp]
    stamps = torch.zeros(256, dtype=torch.int64, device=DEV)
    ramp = {}
    for threads in (64, 128, 256, 512):
        p90 = []
        for _ in range(9):
            assert P.hti_probe_entry(stamps.data_ptr(), 256, threads, 40 * 1024, stream) == 0
            torch.cuda.synchronize()
            t = (stamps - stamps.min()).double() * tick_ns / 1e3
            p90.append(float(torch.quantile(t, 0.9)))
        ramp[threads] = sorted(p90)[len(p90) // 2]
        res[f"launch_ramp_us_p90_256wg_{threads}t"] = ramp[threads]
    log("[floors] launch ramp, p90 of 256 workgroup entries (us): " +
        ", ".join(f"{k} threads {v:.2f}" for k, v in ramp.items()))
    return res


def host_info():
    """CPU model and the cores this process may use."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return dict(cpu_model=model, nproc=usable, cpu_count=os.cpu_count())


def cpu_baseline(args):
    """The oracle, as it stands, on bounded samples of the timed workloads.

    Decode (the headline unit): queries of one 1,048,576-token sequence over
    2 of its 8 KV groups, timed single-threaded and then with one oracle call
    per (query, group) on a pool of threads (the oracle's C calls release the
    interpreter lock), each scaled to all 8 groups.  Also the oracle's tree
    build over one (sequence, KV head), and rows of the 8192-token prefill
    block over the 524,288-token prefix (tree build untimed there)."""
    import concurrent.futures as cf

    import oracle
    hinfo = host_info()
    threads = max(1, min(16, hinfo["nproc"]))
    w = W.DEC1M
    groups = (0, 1)
    log("[cpu] oracle trees for 2 KV heads of one 1M-token sequence")
    K, V = gen_kv_device(w.replace(B=1), w.L)
    refs = W.gen_refs(w)
    trees, data = {}, {}
    build_s = []
    for g in groups:
        Kh = K[0, g].float().cpu().numpy()
        Vh = V[0, g].float().cpu().numpy()
        t0 = time.perf_counter()
        trees[g] = oracle.build_tree(Kh, Vh, refs[g], w.b, w.levels, bf16=True)
        build_s.append(time.perf_counter() - t0)
        data[g] = (Kh, Vh)
    del K, V
    gen = torch.Generator().manual_seed(7)

    def one(q, g):
        oracle.query(trees[g], data[g][0], data[g][1], q[g * w.G:(g + 1) * w.G], k=w.k)

    # single thread: as many queries as fit about eight seconds (at least four)
    budget_s, nq1, el1 = 8.0, 0, 0.0
    while nq1 < 4 or (el1 < budget_s and nq1 < 100000):
        q = torch.randn((w.Hq, w.d), generator=gen).to(torch.bfloat16).float().numpy()
        t0 = time.perf_counter()
        for g in groups:
            one(q, g)
        el1 += time.perf_counter() - t0
        nq1 += 1
    qps1 = nq1 / el1 / (w.Hkv / len(groups))
    # a pool of threads over (query, group) units, for about eight seconds
    nqt = max(4, int(round(qps1 * (w.Hkv / len(groups)) * budget_s * threads * 0.8)))
    qs = [torch.randn((w.Hq, w.d), generator=gen).to(torch.bfloat16).float().numpy() for _ in range(nqt)]
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda u: one(qs[u[0]], u[1]), [(i, g) for i in range(nqt) for g in groups]))
    elt = time.perf_counter() - t0
    qpst = nqt / elt / (w.Hkv / len(groups))
    # prefill block rows over the 524,288-token prefix (two groups)
    wp = W.PREFILL
    Kp, Vp = gen_kv_device(wp, wp.L)
    qb, kb, vb = W.gen_block(wp)
    rows = [0, wp.T // 2, wp.T - 1]
    refsp = W.gen_refs(wp)
    pre_el, pre_n = 0.0, 0
    for g in groups:
        Kh = Kp[0, g].float().cpu().numpy()
        Vh = Vp[0, g].float().cpu().numpy()
        tr = oracle.build_tree(Kh, Vh, refsp[g], wp.b, wp.levels, bf16=True)
        bk, bv = kb[0, :, g].float().numpy(), vb[0, :, g].float().numpy()
        for t in rows:
            t0 = time.perf_counter()
            oracle.query(tr, Kh, Vh, qb[0, t, g * wp.G:(g + 1) * wp.G], k=wp.k, t=t, blk_k=bk, blk_v=bv)
            pre_el += time.perf_counter() - t0
            pre_n += 1
    del Kp, Vp
    pre_row_s = pre_el / pre_n                                     # one (row, group)
    pre_block_s_1t = pre_row_s * wp.T * wp.Hkv
    return dict(value=qpst, unit="queries/s", cores=threads, kind="oracle",
                sample=(f"decode: {nqt} queries x {len(groups)} of {w.Hkv} KV groups of one 1,048,576-token "
                        f"sequence on {threads} threads ({elt:.1f} s) and {nq1} queries on one thread "
                        f"({el1:.1f} s), each scaled x{w.Hkv // len(groups)} to all groups; tree build "
                        f"timed apart; prefill: {pre_n} (row, group) units of the 8192-token block, "
                        f"scaled to the block"),
                single_thread_qps=qps1, threads=threads,
                build_s_per_head_1m=sum(build_s) / len(build_s),
                build_s_all_heads_1m_b4_est=sum(build_s) / len(build_s) * w.B * w.Hkv,
                prefill_s_per_row_group=pre_row_s,
                prefill_block_s_one_thread_est=pre_block_s_1t,
                prefill_block_tokens_per_s_one_thread_est=wp.T / pre_block_s_1t,
                **hinfo)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "side", "all"], default="all")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the per-head-routing and leaf-only timings (profiled runs of the main step)")
    ap.add_argument("--floors", action="store_true",
                    help="only measure the on-device floors (latency, exchange, bandwidth, matrix-core peak)")
    ap.add_argument("--no-floors", action="store_true")
    ap.add_argument("--timeline", action="store_true",
                    help="only the phase timeline of the decode step (timeline build of the library)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the method's sequences and KV heads are independent, "
              "so a multi-GPU run would shard them with no communication; --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.floors:
        print(json.dumps(measure_floors()), flush=True)
        return
    if args.timeline:
        print(json.dumps(decode_timeline(args)), flush=True)
        return
    hti.lib()
    dec = bench_decode(args) if args.only in ("decode", "all") else None
    pre = bench_prefill(args) if args.only in ("prefill", "all") else None
    side = bench_side_workloads(args) if args.only in ("all", "side") and not args.no_variants else None
    floors = None
    if not args.no_floors and args.only == "all":
        floors = measure_floors()
    cpu = None if args.no_cpu_baseline else cpu_baseline(args)
    w = W.DEC1M
    line = {
        "metric": METRIC,
        "value": dec["qps"] if dec else None,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"] if dec else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "context": w.L, "Hq": w.Hq, "Hkv": w.Hkv,
                   "d": w.d, "b": w.b, "levels": w.levels, "k": w.k,
                   "step": "decode_step (tree_append + sparse_decode in one launch), steps captured in one HIP graph",
                   "prefill_workload": W.PREFILL.name},
        "hbm_gbs": dec["gbs"] if dec else None,
        "decode_eager_ms_per_step": dec["eager_ms_per_step"] if dec else None,
        "decode_per_head_routing_ms": finite(dec["per_head_ms"]) if dec else None,
        "decode_per_head_routing_qps": finite(dec["per_head_qps"]) if dec else None,
        "decode_per_head_routing_gbs": finite(dec["per_head_gbs"]) if dec else None,
        "decode_leaf_only_ms": finite(dec["leaf_only_ms"]) if dec else None,
        "decode_leaf_only_qps": finite(dec["leaf_only_qps"]) if dec else None,
        "prefill_leaf_only_ms_per_block": finite(pre["leaf_only_ms"]) if pre else None,
        "prefill_token_nodes_ms_per_block": finite(pre["token_nodes_ms"]) if pre else None,
        "decode_plain_ms": finite(dec["plain_ms"]) if dec else None,
        "decode_plain_gbs": finite(dec["plain_gbs"]) if dec else None,
        "decode_router_fp8_ms": finite(dec["r8_ms"]) if dec else None,
        "decode_router_fp8_qps": finite(dec["r8_qps"]) if dec else None,
        "decode_router_fp8_gbs": finite(dec["r8_gbs"]) if dec else None,
        "decode_router_fp8_bytes_per_launch": dec["r8_bytes"] if dec else None,
        "decode_plain_bytes_per_launch": dec["plain_bytes"] if dec else None,
        "prefill_router_fp8_ms_per_block": finite(pre["r8_ms"]) if pre else None,
        "prefill_tokens_per_s": pre["tokens_per_s"] if pre else None,
        "prefill_ms_per_block": pre["ms_per_block"] if pre else None,
        "prefill_extend_ms": pre["extend_ms"] if pre else None,
        "prefill_extend_gbs": pre["extend_gbs"] if pre else None,
        "roofline": ({"bound": "hbm", "achieved": dec["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": dec["gbs"] / HBM_PEAK_GBS, "traffic": measured_traffic(),
                      "kernel": "k_decode_split",
                      "kernel_ms": dec["decode_kernel_ms"],
                      "bytes_per_launch": dec["bytes_per_launch"]} if dec else None),
        "prefill_roofline": ({"bound": "mfma", "achieved": pre["dense_tflops"], "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": pre["dense_tflops"] / BF16_PEAK_TFLOPS,
                              "kernel": "k_inblock (causal in-block attention, bf16 MFMA)",
                              "dense_ms": pre["dense_ms"], "gflop": pre["inblock_gflop"]} if pre else None),
        "cpu_baseline": cpu,
        "side_workloads": side,
        "measured_floors": floors,
    }
    if floors and dec:
        line["roofline"]["frac_of_measured_read_bw"] = dec["gbs"] / floors["read_gbs"]
    if floors and pre:
        line["prefill_roofline"]["frac_of_measured_mfma"] = pre["dense_tflops"] / floors["mfma_bf16_tflops"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
