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
    cfg = hti.make_cfg(w.B, w.Hq, w.Hkv, w.d, w.b, w.levels, w.R, w.dtype, Lcap, w.rope_base, 1)
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
        m = nsel * w.b + (n[lvl - 1] - w.b * n[lvl])
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


def bench_prefill(args):
    w = W.PREFILL
    log(f"[prefill] generating prefix {w.L} and block {w.T}")
    K, V = gen_kv_device(w, w.L)
    qb, kb, vb = W.gen_block(w, device=DEV)
    ts, sel = treeset(w, w.L, K, V, T=w.T)
    ws = torch.empty(ts.prefill_workspace_bytes(sel, w.T), dtype=torch.uint8, device=DEV)
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
    # the dense part alone: the same block over an empty prefix leaves only
    # the in-block causal attention on the matrix cores (plus the rotation
    # of the block and an empty traversal)
    ts0, sel0 = treeset(w.replace(L=0), w.L, K, V, T=w.T)
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
    nodes = sum((w.L + w.T) // w.b ** l - w.L // w.b ** l for l in range(1, w.levels + 1))
    ext_bytes = 3 * 2 * row_bytes + nodes * w.B * w.Hkv * (w.R + 1) * w.d * W.TORCH_DTYPE[w.dtype].itemsize
    res = dict(ms_per_block=ms, tokens_per_s=w.T * w.B / (ms / 1e3), inblock_gflop=inblock_flop / 1e9,
               dense_ms=ms_dense, dense_tflops=inblock_flop / (ms_dense / 1e3) / 1e12,
               extend_ms=ms_ext, extend_gbs=ext_bytes / (ms_ext / 1e3) / 1e9, leaf_only_ms=ms_lf,
               r8_ms=ms_r8)
    log(f"[prefill] {res}")
    del K, V, ts, ws, tsx, Kx, Vx
    torch.cuda.empty_cache()
    return res


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, if it
    was taken on the decode kernel source as it is now (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    src = os.path.join(ROOT, "hierarchical_tree_indexed_amd", "csrc", "hti_decode.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha1(open(src, "rb").read()).hexdigest()
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


def cpu_baseline(args):
    """The oracle, as it stands, on a bounded sample of the decode workload."""
    import numpy as np

    import oracle
    w = W.DEC1M
    groups = (0, 1)
    nq = 4
    log("[cpu] building oracle trees for 2 KV heads of one 1M-token sequence (untimed)")
    K, V = gen_kv_device(w.replace(B=1), w.L)
    refs = W.gen_refs(w)
    trees = {}
    data = {}
    for g in groups:
        Kh = K[0, g].float().cpu().numpy()
        Vh = V[0, g].float().cpu().numpy()
        trees[g] = oracle.build_tree(Kh, Vh, refs[g], w.b, w.levels, bf16=True)
        data[g] = (Kh, Vh)
    del K, V
    # as many queries as fit about ten seconds (at least four)
    gen = torch.Generator().manual_seed(7)
    budget_s, nq, el = 10.0, 0, 0.0
    while nq < 4 or (el < budget_s and nq < 100000):
        q = torch.randn((w.Hq, w.d), generator=gen).to(torch.bfloat16).float().numpy()
        t0 = time.perf_counter()
        for g in groups:
            oracle.query(trees[g], data[g][0], data[g][1], q[g * w.G:(g + 1) * w.G], k=w.k)
        el += time.perf_counter() - t0
        nq += 1
    per_query = el / nq * (w.Hkv / len(groups))       # all 8 groups of one query
    return dict(value=1.0 / per_query, unit="queries/s", cores=1, kind="oracle",
                sample=f"{nq} decode queries x {len(groups)} of {w.Hkv} KV groups of one "
                       f"1,048,576-token sequence ({el:.1f} s), time scaled x{w.Hkv // len(groups)} "
                       f"to all groups; tree build untimed; single thread")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "all"], default="all")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the per-head-routing and leaf-only timings (profiled runs of the main step)")
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
    hti.lib()
    dec = bench_decode(args) if args.only in ("decode", "all") else None
    pre = bench_prefill(args) if args.only in ("prefill", "all") else None
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
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
