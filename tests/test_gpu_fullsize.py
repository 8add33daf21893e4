"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: the 131,072-token decode, the 1,048,576-token decode at
batch 4 (with one appended token), the 2,097,152-token top-p decode with four
reference keys per node, and the 8192-token prefill block over a
524,288-token prefix (the 4096-token fp32 workload is checked whole with the
other decode tests).

The caches are drawn on the device (seeded per sequence and head), the whole
batch runs through the C ABI, and sampled (sequence, KV group) units -- and,
for the prefill, sampled block rows -- are checked one by one against the
oracle, which builds its own tree from the same cache rows copied to the
host."""
import numpy as np
import pytest
import torch

import hierarchical_tree_indexed_amd as hti
import hti_workloads as W
from gpu_helpers import (accept, kmax_of, log, make_treeset, oracle_tree, oracle_tree_from_device,
                         router_copy_matches, select_of)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _host(x):
    return x.cpu()


def _decode_full(w, units, Lcap, append_steps=0, leaf_only=False, per_head=False, router_fp8=False):
    """Build the tree over the full context, append `append_steps` tokens,
    decode one query per sequence with the split kernel, and accept the
    sampled units against the oracle (leaf_only / per_head: the selection
    variants; per_head checks every query head of the sampled KV groups as a
    group of one; router_fp8: routing through the 8-bit key copy, checked
    bit for bit at the sampled units, the oracle on the stored levels)."""
    log(f"full-size decode {w.name}: B={w.B} L={w.L} Hkv={w.Hkv} levels={w.levels} R={w.R} {w.mode}")
    K, V = W.gen_kv(w, Lcap=Lcap, device=DEV)
    q0 = W.gen_queries(w)
    if w.needles:
        W.plant_needles(w, K, q0)
    refs = W.gen_refs(w)
    ts = make_treeset(w, Lcap, K, V, refs.to(DEV), router_fp8=router_fp8)
    ts.tree_build([w.L] * w.B)
    for s in range(append_steps):
        kn, vn = W.gen_append(w, s, device=DEV)
        ts.tree_append(kn, vn)
    L = w.L + append_steps
    q = q0                     # the query whose direction the needles copy
    out = torch.empty((w.B, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, 1, w.Hq), dtype=torch.float32, device=DEV)
    hu = w.Hq if per_head else w.Hkv
    sel = torch.empty((w.B, 1, hu, w.levels, kmax_of(w)), dtype=torch.int32, device=DEV)
    rule = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, per_head=per_head, leaf_only=leaf_only)
    ts.sparse_decode(rule, q.to(DEV).contiguous(), out, lse, sel, split=True)
    torch.cuda.synchronize()
    assert ts.len.cpu().tolist() == [L] * w.B
    out, lse, sel = out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()
    nex, emax = 0, 0.0
    for bi, g in units:
        Kh, Vh = _host(K[bi, g, :L]), _host(V[bi, g, :L])
        if router_fp8:
            rows = router_copy_matches(ts, w, bi, g, L)
            log(f"  unit (seq {bi}, group {g}): {rows} router rows identical")
            tree = oracle_tree_from_device(ts, w, bi, g, L)
        else:
            tree = oracle_tree(w, Kh, Vh, refs[g], L)
        heads = [slice(h, h + 1) for h in range(g * w.G, (g + 1) * w.G)] if per_head else \
            [slice(g * w.G, (g + 1) * w.G)]
        for hs in heads:
            srow = sel[bi, 0, hs.start] if per_head else sel[bi, 0, g]
            ex, err = accept(w, tree, Kh, Vh, q[bi, 0, hs], out[bi, 0, hs], lse[bi, 0, hs], srow,
                             leaf_only=leaf_only, router_fp8=router_fp8)
            nex += ex
            emax = max(emax, err)
        log(f"  unit (seq {bi}, group {g}): exempt so far {nex}, max_err {emax:.2e}")
    assert np.isfinite(out).all()
    return nex, emax


def test_decode_128k_all_units():
    """131,072 tokens, 32 query heads on 8 KV heads, 8 planted needles: every
    unit checked."""
    w = W.DEC128K
    _decode_full(w, [(0, g) for g in range(w.Hkv)], Lcap=w.L)


def test_decode_1m_batch4_sampled():
    """1,048,576 tokens x 4 sequences, 16 planted needles each, one appended
    token, then the decode step; four units sampled across sequences and
    groups."""
    w = W.DEC1M
    _decode_full(w, [(0, 0), (1, 5), (2, 2), (3, 7)], Lcap=w.L + 4, append_steps=1)


def test_decode_1m_c32_f8_sampled():
    """The 1,048,576-token decode at batch 4 on a tree with chunk size 32 at
    level 1 and fan 8 above it (five levels: 32,768 / 4,096 / 512 / 64 / 8
    nodes), the fan-out geometry the benchmark times beside the C = F = 32
    tree; one appended token, four units sampled against the oracle's own
    tree of the same geometry."""
    w = W.DEC1M.replace(name="decode_1m_b4_c32_f8", fan=8, levels=5)
    _decode_full(w, [(0, 1), (1, 6), (2, 3), (3, 4)], Lcap=w.L + 4, append_steps=1)


def test_decode_step_1m_batch4_benched_config():
    """The step the benchmark times, in its configuration: 1,048,575 cached
    tokens x 4 sequences (16 planted needles each), then two decode_step
    calls (the append and the split decode in one launch).  The first
    appended token completes a node at every level (1,048,576 = 32^4), the
    second completes none.  After each step: output, lse, selections,
    lengths, cache rows and every level bit for bit against tree_append +
    sparse_decode on a second tree set; sampled units against the oracle's
    own tree, built from the grown cache rows."""
    w = W.DEC1M
    L0 = w.L - 1
    Lcap = L0 + 2
    log(f"decode_step at the benched configuration: B={w.B} L={L0}+2 levels={w.levels}")
    K, V = W.gen_kv(w.replace(L=L0), Lcap=Lcap, device=DEV)
    q0 = W.gen_queries(w)
    W.plant_needles(w.replace(L=L0), K, q0)
    refs = W.gen_refs(w)
    ta = make_treeset(w, Lcap, K, V, refs.to(DEV))
    tb = make_treeset(w, Lcap, K.clone(), V.clone(), refs.to(DEV))
    ta.tree_build([L0] * w.B)
    tb.tree_build([L0] * w.B)
    sel = select_of(w)
    kmax = kmax_of(w)
    shape = (w.B, 1, w.Hq, w.d)
    oa, ob = (torch.empty(shape, dtype=torch.float32, device=DEV) for _ in range(2))
    la, lb = (torch.empty(shape[:3], dtype=torch.float32, device=DEV) for _ in range(2))
    sa, sb = (torch.empty((w.B, 1, w.Hkv, w.levels, kmax), dtype=torch.int32, device=DEV) for _ in range(2))
    units = [(0, 0), (1, 5), (2, 2), (3, 7)]
    for s in range(2):
        kn, vn = W.gen_append(w, s, device=DEV)
        q = (q0 if s == 0 else W.gen_queries(w, step=s)).to(DEV).contiguous()
        ta.decode_step(sel, kn.contiguous(), vn.contiguous(), q, oa, la, sa)
        tb.tree_append(kn.contiguous(), vn.contiguous())
        tb.sparse_decode(sel, q, ob, lb, sb)
        torch.cuda.synchronize()
        L = L0 + s + 1
        assert ta.len.cpu().tolist() == [L] * w.B and torch.equal(ta.len, tb.len)
        assert torch.equal(oa, ob), f"step {s}: max diff {(oa - ob).abs().max().item()}"
        assert torch.equal(la, lb) and torch.equal(sa, sb), s
        assert torch.equal(ta.k_cache[:, :, L - 1], tb.k_cache[:, :, L - 1])
        assert torch.equal(ta.v_cache[:, :, L - 1], tb.v_cache[:, :, L - 1])
        for l in range(w.levels):
            assert torch.equal(ta.lvl_k[l], tb.lvl_k[l]) and torch.equal(ta.lvl_v[l], tb.lvl_v[l]), (s, l)
        if s == 0:
            # the top node exists now: a kept top level of one node
            assert (sa[:, 0, :, w.levels - 1, 0] == 0).all()
        out, lse, so = oa.cpu().numpy(), la.cpu().numpy(), sa.cpu().numpy()
        nex, emax = 0, 0.0
        for bi, g in units:
            Kh, Vh = ta.k_cache[bi, g, :L].cpu(), ta.v_cache[bi, g, :L].cpu()
            tree = oracle_tree(w, Kh, Vh, refs[g], L)
            hs = slice(g * w.G, (g + 1) * w.G)
            ex, err = accept(w, tree, Kh, Vh, q.cpu()[bi, 0, hs], out[bi, 0, hs], lse[bi, 0, hs], so[bi, 0, g])
            nex += ex
            emax = max(emax, err)
            log(f"  step {s} unit (seq {bi}, group {g}): exempt so far {nex}, max_err {emax:.2e}")
        assert np.isfinite(out).all()


def test_decode_1m_batch4_variants_sampled():
    """The 1M-token decode at batch 4 under leaf-only dispatch and under
    per-query-head routing; sampled units (every query head of them for the
    per-head run) against the oracle's variants."""
    w = W.DEC1M
    _decode_full(w, [(1, 3), (3, 6)], Lcap=w.L, leaf_only=True)
    _decode_full(w, [(0, 2), (2, 7)], Lcap=w.L, per_head=True)


def test_decode_1m_batch4_router_fp8_sampled():
    """The 1M-token decode at batch 4 with 8-bit router keys, after one
    appended token (so the append writes the copy of the nodes it
    completes); sampled units, the copy bit for bit, routing and output
    against the oracle's 8-bit routing."""
    w = W.DEC1M
    _decode_full(w, [(0, 1), (3, 4)], Lcap=w.L + 4, append_steps=1, router_fp8=True)


def test_decode_zha_2m_topp_sampled():
    """2,097,152 tokens, b = 16, top-p 0.9 capped at 16 nodes, four reference
    keys per node; both KV groups checked."""
    w = W.ZHA2M
    _decode_full(w, [(0, 0), (0, 1)], Lcap=w.L)


def test_prefill_524k_block_sampled():
    """8192-token block over the 524,288-token prefix; block rows at both ends,
    the middle and a few seeded ones, in two KV groups."""
    _prefill_full(router_fp8=False)


def test_prefill_524k_block_router_fp8_sampled():
    """The same block with 8-bit router keys (the walk and the matrix-core top
    level score through the copy)."""
    _prefill_full(router_fp8=True)


def test_prefill_524k_block_token_nodes_sampled():
    """The same block with the node-inverted token level (the block's queries
    grouped by kept level-1 node)."""
    _prefill_full(router_fp8=False, token_nodes=True)


def _prefill_full(router_fp8, token_nodes=False):
    w = W.PREFILL
    T = w.T
    log(f"full-size prefill {w.name}: L={w.L} T={T}")
    K, V = W.gen_kv(w, Lcap=w.L, device=DEV)
    refs = W.gen_refs(w)
    ts = make_treeset(w, w.L, K, V, refs.to(DEV), T=T, router_fp8=router_fp8)
    ts.tree_build([w.L] * w.B)
    qb, kb, vb = W.gen_block(w)
    sel = select_of(w, token_nodes=token_nodes)
    ws = torch.empty(ts.prefill_workspace_bytes(sel, T), dtype=torch.uint8, device=DEV)
    out = torch.empty((w.B, T, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, T, w.Hq), dtype=torch.float32, device=DEV)
    so = torch.empty((w.B, T, w.Hkv, w.levels, kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_prefill(sel, qb.to(DEV).contiguous(), kb.to(DEV).contiguous(), vb.to(DEV).contiguous(),
                      out, ws, lse, so)
    torch.cuda.synchronize()
    out, lse, so = out.cpu().numpy(), lse.cpu().numpy(), so.cpu().numpy()
    assert np.isfinite(out).all()
    rng = np.random.default_rng(11)
    rows = sorted(set([0, 1, 63, 64, T // 2, T - 2, T - 1] + rng.integers(0, T, 5).tolist()))
    nex, emax = 0, 0.0
    for g in (0, 5):
        Kh, Vh = _host(K[0, g, :w.L]), _host(V[0, g, :w.L])
        if router_fp8:
            router_copy_matches(ts, w, 0, g, w.L)
            tree = oracle_tree_from_device(ts, w, 0, g, w.L)
        else:
            tree = oracle_tree(w, Kh, Vh, refs[g], w.L)
        bk = kb[0, :, g].float().numpy()
        bv = vb[0, :, g].float().numpy()
        hs = slice(g * w.G, (g + 1) * w.G)
        for t in rows:
            ex, err = accept(w, tree, Kh, Vh, qb[0, t, hs], out[0, t, hs], lse[0, t, hs], so[0, t, g],
                             t=t, blk_k=bk, blk_v=bv, router_fp8=router_fp8)
            nex += ex
            emax = max(emax, err)
        log(f"  group {g}: {len(rows)} block rows, exempt so far {nex}, max_err {emax:.2e}")
