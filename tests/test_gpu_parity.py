"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles, ragged tails and the degenerate cases of the method."""
import numpy as np
import pytest
import torch

import hierarchical_tree_indexed_amd as hti
import hti_workloads as W
import oracle
from gpu_helpers import accept, kmax_of, log, make_treeset, oracle_tree, select_of, tree_close

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _setup(w, Lcap=None, Ls=None):
    Lcap = Lcap or w.L
    K, V = W.gen_kv(w, Lcap=Lcap)
    refs = W.gen_refs(w)
    ts = make_treeset(w, Lcap, K.to(DEV), V.to(DEV), refs.to(DEV))
    Ls = Ls or [w.L] * w.B
    ts.tree_build(Ls)
    return ts, K, V, refs, Ls


def _decode(ts, w, q, split=True):
    out = torch.empty((w.B, q.shape[1], w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, q.shape[1], w.Hq), dtype=torch.float32, device=DEV)
    sel = torch.empty((w.B, q.shape[1], w.Hkv, max(w.levels, 1), kmax_of(w)), dtype=torch.int32,
                      device=DEV)
    ts.sparse_decode(select_of(w), q.to(DEV).contiguous(), out, lse, sel, split=split)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()


def _check_decode(ts, w, K, V, refs, Ls, q, trees=None, upload=False, split=True):
    """Decode every query of every sequence/group and accept against the oracle."""
    trees = trees or {}
    for bi in range(w.B):
        for g in range(w.Hkv):
            if (bi, g) not in trees:
                trees[(bi, g)] = oracle_tree(w, K[bi, g], V[bi, g], refs[g], Ls[bi])
            if upload:
                tr = trees[(bi, g)]
                for l in range(w.levels):
                    n = tr.lk[l].shape[0]
                    ts.lvl_k[l][bi, g, :n] = torch.from_numpy(tr.lk[l]).to(ts.lvl_k[l].dtype).to(DEV)
                    ts.lvl_v[l][bi, g, :n] = torch.from_numpy(tr.lv[l]).to(ts.lvl_v[l].dtype).to(DEV)
    out, lse, sel = _decode(ts, w, q, split=split)
    nex, emax = 0, 0.0
    for bi in range(w.B):
        for qi in range(q.shape[1]):
            for g in range(w.Hkv):
                hs = slice(g * w.G, (g + 1) * w.G)
                ex, err = accept(w, trees[(bi, g)], K[bi, g, : Ls[bi]], V[bi, g, : Ls[bi]],
                                 q[bi, qi, hs], out[bi, qi, hs], lse[bi, qi, hs], sel[bi, qi, g])
                nex += ex
                emax = max(emax, err)
    log(f"  {w.name} split={split}: units={w.B * q.shape[1] * w.Hkv} exempt={nex} max_err={emax:.2e}")
    return trees, out, sel, nex


# --------------------------------------------------------------------------- build
BUILD_CASES = [
    W.TINY,
    W.DEC128K.replace(name="bf16_b32", L=40000 + 17, B=2, needles=0),
    W.ZHA2M.replace(name="bf16_r4_b16", L=70000 + 5, levels=4),
    W.TINY.replace(name="f32_d128_b8", d=128, b=8, levels=4, L=9000 + 3, Hq=4, Hkv=2, R=2),
    W.DEC128K.replace(name="bf16_d64_b3", d=64, b=3, levels=6, L=3000, Hq=4, Hkv=4),
    # 16 children per lane row (b > 32), two references, a partial last node
    W.DEC128K.replace(name="bf16_b64_r2", b=64, levels=2, L=64 * 64 * 2 + 77, R=2, Hq=4, Hkv=2, needles=0),
    # the most references (their rows fill the staged block exactly), fp32, d = 64
    W.TINY.replace(name="f32_d64_b40_r8", d=64, b=40, levels=2, L=40 * 40 * 2 + 11, R=8, Hq=2, Hkv=2),
    # a fan above level 1 apart from the chunk size: 16 tokens per level-1
    # node, 4 nodes per node above (and the reverse, with 2 references)
    W.DEC128K.replace(name="bf16_c16_f4", b=16, fan=4, levels=3, L=16 * 4 * 4 * 5 + 77, Hq=4, Hkv=2, needles=0),
    W.TINY.replace(name="f32_c4_f16_r2", b=4, fan=16, levels=3, L=4 * 16 * 16 * 2 + 9, R=2, Hq=2, Hkv=2),
]


@pytest.mark.parametrize("w", BUILD_CASES, ids=lambda w: w.name)
def test_build_parity(w):
    log(f"build parity {w.name} L={w.L} b={w.b} levels={w.levels} R={w.R} {w.dtype}")
    ts, K, V, refs, Ls = _setup(w)
    torch.cuda.synchronize()
    assert ts.len.cpu().tolist() == Ls
    exact = []
    for bi in range(w.B):
        for g in range(w.Hkv):
            tr = oracle_tree(w, K[bi, g], V[bi, g], refs[g], w.L)
            for l in range(w.levels):
                n = tr.lk[l].shape[0]
                exact.append(tree_close(w, ts.lvl_k[l][bi, g, :n], ts.lvl_v[l][bi, g, :n],
                                        tr.lk[l], tr.lv[l], level=l + 1))
    log(f"  fraction of bit-exact node elements {np.mean(exact):.5f}")
    if w.dtype == "bf16":
        assert np.mean(exact) > 0.99


# --------------------------------------------------------------------------- decode
@pytest.mark.parametrize("split", [True, False])
def test_decode_tiny_workload(split):
    """The 4096-token fp32 workload at full size: 16 queries, top-k 4."""
    w = W.TINY
    ts, K, V, refs, Ls = _setup(w)
    q = W.gen_queries(w)
    _check_decode(ts, w, K, V, refs, Ls, q, split=split)


DECODE_CASES = [
    W.DEC128K.replace(name="gqa4_ragged", B=3, L=20000, needles=0, levels=2),
    W.DEC128K.replace(name="gqa4_orphans", L=32 * 32 * 5 + 32 * 7 + 13, levels=2, Nq=3),
    W.DEC128K.replace(name="g1_d64", Hq=2, Hkv=2, d=64, L=7777, b=8, levels=3, k=3),
    W.DEC128K.replace(name="g2_k1", Hq=4, Hkv=2, L=5000, b=16, levels=2, k=1),
    W.DEC128K.replace(name="g8", Hq=16, Hkv=2, L=6000, b=16, levels=2, k=5),
    W.DEC128K.replace(name="f32_d128", dtype="f32", Hq=8, Hkv=2, L=9000, b=16, levels=2, k=6),
    W.ZHA2M.replace(name="topp_r4", L=16 ** 4 * 2 + 300, levels=4),
    W.ZHA2M.replace(name="topp_p1_cap32", L=3000, levels=2, p=1.0, cap=32, R=2),
    W.ZHA2M.replace(name="topp_p05", L=20000, levels=3, p=0.5, cap=8, R=1),
    W.DEC128K.replace(name="k32", L=33000, b=16, levels=3, k=32),
    # eight reference keys per node in fp32 at d = 128: a key batch must hold
    # all of a candidate's keys
    W.DEC128K.replace(name="f32_d128_r8", dtype="f32", Hq=8, Hkv=2, L=6000, b=16, levels=2, k=3, R=8),
    # chunk size 32 at level 1, fan 8 above (ZHA's C and F apart), top-k and
    # top-p with two references; and fan 48 over chunks of 8
    W.DEC128K.replace(name="c32_f8", L=32 * 8 * 8 * 3 + 8 * 32 + 17, fan=8, levels=3, B=2, needles=0),
    W.ZHA2M.replace(name="topp_c16_f4_r2", L=16 * 4 ** 3 * 3 + 70, fan=4, levels=4, R=2),
    W.DEC128K.replace(name="c8_f48_d64", Hq=4, Hkv=2, d=64, b=8, fan=48, levels=2, L=8 * 48 * 4 + 100, k=3),
]


@pytest.mark.parametrize("w", DECODE_CASES, ids=lambda w: w.name)
def test_decode_parity(w):
    log(f"decode parity {w.name}")
    Ls = [w.L - 977 * i for i in range(w.B)]
    ts, K, V, refs, _ = _setup(w, Lcap=w.L, Ls=Ls)
    q = W.gen_queries(w)
    trees, _, _, _ = _check_decode(ts, w, K, V, refs, Ls, q)
    _check_decode(ts, w, K, V, refs, Ls, q, trees=trees, split=False)
    # the same decode on the oracle's own tree (decode kernels in isolation)
    _check_decode(ts, w, K, V, refs, Ls, q, trees=trees, upload=True)
    _check_decode(ts, w, K, V, refs, Ls, q, trees=trees, upload=True, split=False)


QPOS_CASES = [
    W.DEC128K.replace(name="qpos_b32", B=2, L=32 * 32 * 3 + 77, levels=2, needles=0, Nq=5),
    W.ZHA2M.replace(name="qpos_topp_r4", L=16 ** 3 * 2 + 33, levels=3, Nq=4),
    # node boundaries of a chunk-8 / fan-16 tree
    W.DEC128K.replace(name="qpos_c8_f16", B=2, b=8, fan=16, L=8 * 16 * 16 + 77, levels=3, needles=0, Nq=5),
]


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("w", QPOS_CASES, ids=lambda w: w.name)
def test_decode_q_pos(w, split):
    """Queries at their own positions (q_pos): each attends to the tree of
    tokens 0..q_pos, which the oracle builds over q_pos + 1 tokens.  The
    positions span a node boundary, an upper-level boundary, the last token,
    values past it (clamped to len - 1) and a negative one (nothing: 0 out,
    -inf lse)."""
    L = w.L
    ts, K, V, refs, Ls = _setup(w, Lcap=L, Ls=[L] * w.B)
    q = W.gen_queries(w)
    pos = np.array([[L - 1, 32 * 32 * 2 - 1, 31, L + 40, 1000][: w.Nq],
                    [L - 2, 16 ** 3 - 1, 16 ** 2 * 3 + 5, -1, 7][: w.Nq]][: w.B], np.int64)
    qp = torch.from_numpy(pos).to(DEV)
    out = torch.empty((w.B, w.Nq, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Nq, w.Hq), dtype=torch.float32, device=DEV)
    so = torch.empty((w.B, w.Nq, w.Hkv, w.levels, kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_decode(select_of(w), q.to(DEV).contiguous(), out, lse, so, split=split, q_pos=qp)
    torch.cuda.synchronize()
    out, lse, so = out.cpu().numpy(), lse.cpu().numpy(), so.cpu().numpy()
    nex = 0
    for bi in range(w.B):
        for qi in range(w.Nq):
            p = int(pos[bi, qi])
            if p < 0:
                assert (out[bi, qi] == 0).all() and np.isneginf(lse[bi, qi]).all()
                assert (so[bi, qi] == -1).all()
                continue
            Lq = min(p, L - 1) + 1
            for g in range(w.Hkv):
                tree = oracle_tree(w, K[bi, g], V[bi, g], refs[g], Lq)
                hs = slice(g * w.G, (g + 1) * w.G)
                ex, _ = accept(w, tree, K[bi, g, :Lq], V[bi, g, :Lq], q[bi, qi, hs], out[bi, qi, hs],
                               lse[bi, qi, hs], so[bi, qi, g])
                nex += ex
    log(f"  {w.name} split={split}: positions {pos.tolist()} exempt={nex}")


def test_decode_status_is_sticky():
    """The workspace's status word (set here from the host, standing in for a
    wait that ran out): the next decode and decode step write NaN, leave the
    length and the cache alone, and hti_decode_status reports the timeout;
    after the workspace is zeroed the same calls give the normal results."""
    w = W.DEC128K.replace(name="status", B=2, L=32 * 40 + 31, levels=2, needles=0)
    Lcap = w.L + 2
    ts, K, V, refs, Ls = _setup(w, Lcap=Lcap, Ls=[w.L] * w.B)
    sel = select_of(w)
    q = W.gen_queries(w).to(DEV).contiguous()
    out = torch.empty((w.B, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
    ts.sparse_decode(sel, q, out)
    ts.decode_status(sel, 1)
    good = out.clone()
    ws = ts.decode_workspace(sel, 1)
    ws[:4] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device=DEV)   # status word
    ts.sparse_decode(sel, q, out)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    with pytest.raises(hti.HTIError) as ei:
        ts.decode_status(sel, 1)
    assert ei.value.status == -6
    kn, vn = W.gen_append(w, 0, device=DEV)
    k_before = ts.k_cache[:, :, w.L].clone()
    ts.decode_step(sel, kn.contiguous(), vn.contiguous(), q, out)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    assert ts.len.cpu().tolist() == [w.L] * w.B
    assert torch.equal(ts.k_cache[:, :, w.L], k_before)
    ws.zero_()
    ts.sparse_decode(sel, q, out)
    torch.cuda.synchronize()
    assert torch.equal(out, good)
    ts.decode_step(sel, kn.contiguous(), vn.contiguous(), q, out)
    ts.decode_status(sel, 1)
    assert ts.len.cpu().tolist() == [w.L + 1] * w.B
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("split", [True, False])
def test_decode_exact_ties(split):
    """Exactly equal scores: zero keys score 0 at every position.  With all
    but three level-1 nodes zeroed most candidates tie; the kept sets must be
    the oracle's (higher score, then lower index) with no exemption."""
    w = W.DEC128K.replace(name="ties", L=32 * 32 * 4 + 70, levels=2, needles=0, Nq=2)
    K, V = W.gen_kv(w, Lcap=w.L)
    keep = torch.zeros(w.L, dtype=torch.bool)
    for n in (70, 90, 100):
        keep[n * 32:(n + 1) * 32] = True
    K[:, :, ~keep] = 0
    refs = W.gen_refs(w)
    ts = make_treeset(w, w.L, K.to(DEV), V.to(DEV), refs.to(DEV))
    ts.tree_build([w.L] * w.B)
    q = W.gen_queries(w)
    _, _, _, nex = _check_decode(ts, w, K, V, refs, [w.L] * w.B, q, split=split)
    assert nex == 0


def test_candidate_capacity_is_enforced():
    """k = 32 with b = 32 can put 32 * 32 + 31 candidates on a level: more than
    the kernel's LDS holds, so the call is refused before any launch."""
    import hierarchical_tree_indexed_amd as hti
    w = W.DEC128K.replace(name="k32b32", L=33000, levels=2, k=32)
    K, V = W.gen_kv(w, Lcap=w.L)
    ts = make_treeset(w, w.L, K.to(DEV), V.to(DEV), W.gen_refs(w).to(DEV))
    out = torch.empty((1, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
    with pytest.raises(hti.HTIError) as ei:
        ts.sparse_decode(select_of(w), W.gen_queries(w).to(DEV), out)
    assert ei.value.status == -2


@pytest.mark.parametrize("split", [True, False])
def test_decode_is_deterministic(split):
    """Repeated launches give bit-identical results (the split path also
    reuses its workspace across launches)."""
    w = DECODE_CASES[0]
    ts, K, V, refs, Ls = _setup(w)
    q = W.gen_queries(w)
    a = _decode(ts, w, q, split=split)
    for _ in range(3):
        b = _decode(ts, w, q, split=split)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    ws = ts.decode_workspace(select_of(w), 1)
    assert int(ws[0:4].view(torch.int32).item()) >= 0


def test_split_decode_matches_unsplit():
    """Both decode paths keep the same nodes and agree on the output."""
    w = W.DEC128K.replace(name="split_vs_unsplit", L=60000, levels=3, needles=0, B=2, Nq=2)
    ts, K, V, refs, Ls = _setup(w)
    q = W.gen_queries(w)
    o1, l1, s1 = _decode(ts, w, q, split=True)
    o2, l2, s2 = _decode(ts, w, q, split=False)
    assert np.array_equal(s1, s2)
    assert np.abs(o1 - o2).max() < 1e-5 and np.abs(l1 - l2).max() < 1e-5


@pytest.mark.parametrize("B,Nq", [(8, 1), (4, 4)])
def test_decode_two_workgroups_per_cu(B, Nq):
    """64 and 128 (query, group) units: one workgroup per CU would give each
    unit fewer than eight (four and two), so the plan places two per CU.
    Against the oracle, and against the one-workgroup-per-unit path."""
    w = W.DEC128K.replace(name=f"two_per_cu_b{B}_nq{Nq}", L=40000 + 17, needles=0, B=B, Nq=Nq)
    ts, K, V, refs, Ls = _setup(w)
    q = W.gen_queries(w)
    _check_decode(ts, w, K, V, refs, Ls, q, split=True)
    o1, l1, s1 = _decode(ts, w, q, split=True)
    o2, l2, s2 = _decode(ts, w, q, split=False)
    assert np.array_equal(s1, s2)
    assert np.abs(o1 - o2).max() < 1e-5 and np.abs(l1 - l2).max() < 1e-5


@pytest.mark.parametrize("L,levels", [(1, 2), (5, 2), (31, 1), (32, 1), (33, 3), (1024, 2), (700, 0)])
def test_decode_edge_lengths(L, levels):
    """Lengths below one node, exactly one node, a single top node, no tree."""
    w = W.DEC128K.replace(name=f"edge_{L}_{levels}", L=L, levels=levels, needles=0,
                          k=32 if levels == 0 else 8)
    ts, K, V, refs, Ls = _setup(w)
    q = W.gen_queries(w)
    _check_decode(ts, w, K, V, refs, Ls, q)
    _check_decode(ts, w, K, V, refs, Ls, q, split=False)


def test_dense_equivalence_on_gpu():
    """Every level keeps all its candidates -> plain causal attention."""
    from ref_f64 import dense_causal
    w = W.DEC128K.replace(name="dense", L=1024, b=32, levels=2, k=32, needles=0)
    ts, K, V, refs, Ls = _setup(w)
    q = W.gen_queries(w)
    out, _, _ = _decode(ts, w, q)
    for g in range(w.Hkv):
        hs = slice(g * w.G, (g + 1) * w.G)
        ref = dense_causal(q[0, 0, hs].float().numpy(), K[0, g].float().numpy(),
                           V[0, g].float().numpy(), w.L - 1)
        assert np.abs(out[0, 0, hs] - ref).max() < 2e-2


# --------------------------------------------------------------------------- append
def test_append_matches_build_and_oracle():
    w = W.DEC128K.replace(name="append", B=2, L=32 * 32 * 3 - 5, levels=3, steps=40, needles=0)
    Lcap = w.L + w.steps
    K, V = W.gen_kv(w, Lcap=Lcap)
    refs = W.gen_refs(w)
    Kd, Vd = K.clone().to(DEV), V.clone().to(DEV)
    ts = make_treeset(w, Lcap, Kd, Vd, refs.to(DEV))
    ts.tree_build([w.L] * w.B)
    for s in range(w.steps):
        kn, vn = W.gen_append(w, s, device=DEV)
        ts.tree_append(kn.contiguous(), vn.contiguous())
        K[:, :, w.L + s] = kn.cpu()
        V[:, :, w.L + s] = vn.cpu()
    torch.cuda.synchronize()
    Lf = w.L + w.steps
    assert ts.len.cpu().tolist() == [Lf] * w.B
    assert torch.equal(Kd.cpu(), K) and torch.equal(Vd.cpu(), V)
    # a fresh build over the final length gives bit-identical nodes
    ts2 = make_treeset(w, Lcap, K.to(DEV), V.to(DEV), refs.to(DEV))
    ts2.tree_build([Lf] * w.B)
    torch.cuda.synchronize()
    for l in range(w.levels):
        assert torch.equal(ts.lvl_k[l], ts2.lvl_k[l]) and torch.equal(ts.lvl_v[l], ts2.lvl_v[l])
    # and the oracle agrees
    for bi in range(w.B):
        for g in range(w.Hkv):
            tr = oracle_tree(w, K[bi, g], V[bi, g], refs[g], Lf)
            for l in range(w.levels):
                n = tr.lk[l].shape[0]
                tree_close(w, ts.lvl_k[l][bi, g, :n], ts.lvl_v[l][bi, g, :n], tr.lk[l], tr.lv[l],
                           level=l + 1)
    q = W.gen_queries(w)
    _check_decode(ts, w, K, V, refs, [Lf] * w.B, q)


def test_append_full_cache_is_a_no_op():
    w = W.DEC128K.replace(name="full", B=1, L=64, levels=1, needles=0)
    K, V = W.gen_kv(w, Lcap=64)
    ts = make_treeset(w, 64, K.to(DEV), V.to(DEV), W.gen_refs(w).to(DEV))
    ts.tree_build([64])
    kn, vn = W.gen_append(w, 0, device=DEV)
    before = ts.k_cache.clone()
    ts.tree_append(kn.contiguous(), vn.contiguous())
    torch.cuda.synchronize()
    assert ts.len.item() == 64 and torch.equal(before, ts.k_cache)


# --------------------------------------------------------------------------- per-head routing
def _per_head_sel(w):
    return hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, per_head=True)


def _check_per_head(w, trees, K, V, Ls, q, out, lse, so, t_of=None, blk=None):
    """Each query head against the oracle as a group of one over its KV head's tree."""
    nex, emax = 0, 0.0
    for bi in range(w.B):
        for qi in range(q.shape[1]):
            for hq in range(w.Hq):
                g = hq // w.G
                kw = {}
                if t_of is not None:
                    kw = dict(t=t_of(qi), blk_k=blk[0][bi, :, g].float().numpy(),
                              blk_v=blk[1][bi, :, g].float().numpy())
                ex, err = accept(w, trees[(bi, g)], K[bi, g, :Ls[bi]], V[bi, g, :Ls[bi]], q[bi, qi, hq:hq + 1],
                                 out[bi, qi, hq:hq + 1], lse[bi, qi, hq:hq + 1], so[bi, qi, hq], **kw)
                nex += ex
                emax = max(emax, err)
    return nex, emax


PER_HEAD_CASES = [
    W.DEC128K.replace(name="ph_gqa4", B=2, L=20000, needles=0, levels=2, Nq=2),
    W.ZHA2M.replace(name="ph_topp_r4", L=16 ** 4 + 300, levels=3, Hq=8, Hkv=2),
    W.DEC128K.replace(name="ph_c32_f4", L=32 * 4 * 4 * 4 + 99, fan=4, levels=3, needles=0, Nq=2),
]


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("w", PER_HEAD_CASES, ids=lambda w: w.name)
def test_decode_per_head_routing(w, split):
    """Every query head routes on its own over its KV head's tree (a group of
    one): selections per query head and outputs against the oracle."""
    Ls = [w.L - 977 * i for i in range(w.B)]
    ts, K, V, refs, _ = _setup(w, Lcap=w.L, Ls=Ls)
    q = W.gen_queries(w)
    trees = {(bi, g): oracle_tree(w, K[bi, g], V[bi, g], refs[g], Ls[bi]) for bi in range(w.B) for g in range(w.Hkv)}
    out = torch.empty((w.B, w.Nq, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Nq, w.Hq), dtype=torch.float32, device=DEV)
    so = torch.empty((w.B, w.Nq, w.Hq, w.levels, kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_decode(_per_head_sel(w), q.to(DEV).contiguous(), out, lse, so, split=split)
    torch.cuda.synchronize()
    nex, emax = _check_per_head(w, trees, K, V, Ls, q, out.cpu().numpy(), lse.cpu().numpy(), so.cpu().numpy())
    log(f"  {w.name} per-head split={split}: exempt={nex} max_err={emax:.2e}")


def test_decode_step_per_head_matches_append_then_decode():
    """decode_step with per-head routing (every query head a unit) equals
    tree_append followed by sparse_decode, bit for bit, over several steps."""
    w = W.DEC128K.replace(name="ph_step", B=2, L=32 * 32 * 2 + 29, needles=0, levels=2, Nq=1)
    Lcap = w.L + 8
    sel = _per_head_sel(w)
    res = []
    for fused in (True, False):
        ts, K, V, refs, _ = _setup(w, Lcap=Lcap, Ls=[w.L] * w.B)
        outs = []
        for step in range(4):
            kn, vn = W.gen_append(w, step, device=DEV)
            q = W.gen_queries(w, step=step + 1).to(DEV).contiguous()
            out = torch.empty((w.B, 1, w.Hq, w.d), dtype=torch.float32, device=DEV)
            if fused:
                ts.decode_step(sel, kn.contiguous(), vn.contiguous(), q, out)
            else:
                ts.tree_append(kn.contiguous(), vn.contiguous())
                ts.sparse_decode(sel, q, out)
            outs.append(out.cpu())
        torch.cuda.synchronize()
        res.append(outs)
    for a_, b_ in zip(*res):
        assert torch.equal(a_, b_)


def test_prefill_per_head_routing():
    """A prefill block with per-head routing (the top level scored per query
    head on the matrix cores), every query head against the oracle."""
    w = PF.replace(levels=2, k=8, Hq=8, Hkv=2)
    P0, T = 32 * 32 * 12 + 70, 40
    w = w.replace(L=P0, T=T)
    K, V = W.gen_kv(w, Lcap=P0)
    refs = W.gen_refs(w)
    ts = make_treeset(w, P0, K.to(DEV), V.to(DEV), refs.to(DEV), T=T)
    ts.tree_build([P0] * w.B)
    qb, kb, vb = W.gen_block(w)
    sel = _per_head_sel(w)
    ws = torch.empty(ts.prefill_workspace_bytes(sel, T), dtype=torch.uint8, device=DEV)
    out = torch.empty((w.B, T, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, T, w.Hq), dtype=torch.float32, device=DEV)
    so = torch.empty((w.B, T, w.Hq, w.levels, kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_prefill(sel, qb.to(DEV).contiguous(), kb.to(DEV).contiguous(), vb.to(DEV).contiguous(),
                      out, ws, lse, so)
    torch.cuda.synchronize()
    trees = {(bi, g): oracle_tree(w, K[bi, g], V[bi, g], refs[g], P0) for bi in range(w.B) for g in range(w.Hkv)}
    nex, emax = _check_per_head(w, trees, K, V, [P0] * w.B, qb, out.cpu().numpy(), lse.cpu().numpy(),
                                so.cpu().numpy(), t_of=lambda t: t, blk=(kb, vb))
    log(f"  prefill per-head: exempt={nex} max_err={emax:.2e}")


# --------------------------------------------------------------------------- leaf-only dispatch
LEAF_CASES = [
    W.DEC128K.replace(name="leaf_gqa4", B=2, L=20000, needles=0, levels=2, Nq=2),
    W.ZHA2M.replace(name="leaf_topp_r4", L=16 ** 4 + 300, levels=3, Hq=8, Hkv=2),
    W.ZHA2M.replace(name="leaf_topp_c16_f8", L=16 * 8 * 8 * 3 + 41, fan=8, levels=3, Hq=8, Hkv=2),
]


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("w", LEAF_CASES, ids=lambda w: w.name)
def test_decode_leaf_only(w, split):
    """Leaf-only dispatch: the summaries route but only the reached tokens are
    attended; selections and outputs against the oracle's leaf-only variant."""
    Ls = [w.L - 977 * i for i in range(w.B)]
    ts, K, V, refs, _ = _setup(w, Lcap=w.L, Ls=Ls)
    q = W.gen_queries(w)
    sel = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, leaf_only=True)
    out = torch.empty((w.B, w.Nq, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Nq, w.Hq), dtype=torch.float32, device=DEV)
    so = torch.empty((w.B, w.Nq, w.Hkv, w.levels, kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_decode(sel, q.to(DEV).contiguous(), out, lse, so, split=split)
    torch.cuda.synchronize()
    out, lse, so = out.cpu().numpy(), lse.cpu().numpy(), so.cpu().numpy()
    nex, emax = 0, 0.0
    for bi in range(w.B):
        for g in range(w.Hkv):
            tr = oracle_tree(w, K[bi, g], V[bi, g], refs[g], Ls[bi])
            hs = slice(g * w.G, (g + 1) * w.G)
            for qi in range(w.Nq):
                ex, err = accept(w, tr, K[bi, g, :Ls[bi]], V[bi, g, :Ls[bi]], q[bi, qi, hs], out[bi, qi, hs],
                                 lse[bi, qi, hs], so[bi, qi, g], leaf_only=True)
                nex += ex
                emax = max(emax, err)
    log(f"  {w.name} leaf-only split={split}: exempt={nex} max_err={emax:.2e}")


def test_prefill_leaf_only():
    """A prefill block with leaf-only dispatch (the prefix summaries route,
    the reached prefix tokens and the block are attended), against the oracle."""
    w = PF.replace(levels=2, k=8)
    P0, T = 32 * 32 * 12 + 70, 40
    w = w.replace(L=P0, T=T)
    K, V = W.gen_kv(w, Lcap=P0)
    refs = W.gen_refs(w)
    ts = make_treeset(w, P0, K.to(DEV), V.to(DEV), refs.to(DEV), T=T)
    ts.tree_build([P0] * w.B)
    qb, kb, vb = W.gen_block(w)
    sel = hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, leaf_only=True)
    ws = torch.empty(ts.prefill_workspace_bytes(sel, T), dtype=torch.uint8, device=DEV)
    out = torch.empty((w.B, T, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, T, w.Hq), dtype=torch.float32, device=DEV)
    so = torch.empty((w.B, T, w.Hkv, w.levels, kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_prefill(sel, qb.to(DEV).contiguous(), kb.to(DEV).contiguous(), vb.to(DEV).contiguous(),
                      out, ws, lse, so)
    torch.cuda.synchronize()
    out, lse, so = out.cpu().numpy(), lse.cpu().numpy(), so.cpu().numpy()
    nex, emax = 0, 0.0
    for g in range(w.Hkv):
        tr = oracle_tree(w, K[0, g], V[0, g], refs[g], P0)
        hs = slice(g * w.G, (g + 1) * w.G)
        bk, bv = kb[0, :, g].float().numpy(), vb[0, :, g].float().numpy()
        for t in range(T):
            ex, err = accept(w, tr, K[0, g, :P0], V[0, g, :P0], qb[0, t, hs], out[0, t, hs], lse[0, t, hs],
                             so[0, t, g], t=t, blk_k=bk, blk_v=bv, leaf_only=True)
            nex += ex
            emax = max(emax, err)
    log(f"  prefill leaf-only: exempt={nex} max_err={emax:.2e}")


# --------------------------------------------------------------------------- block extension
def _extend_pair(w, P0, T, Lcap):
    """Tree A: built over P0[s] tokens, then extended by the next T tokens of
    each sequence as one block [B, T, Hkv, d]; tree B: built over the longer
    prefix min(P0[s] + T, Lcap).  Returns both tree sets and the new lengths."""
    K, V = W.gen_kv(w.replace(L=Lcap), Lcap=Lcap)
    refs = W.gen_refs(w)
    KA, VA = K.clone(), V.clone()
    for s_ in range(w.B):
        KA[s_, :, P0[s_]:] = 0
        VA[s_, :, P0[s_]:] = 0
    ka = torch.zeros((w.B, T, w.Hkv, w.d), dtype=K.dtype)
    va = torch.zeros_like(ka)
    for s_ in range(w.B):
        n = min(T, Lcap - P0[s_])
        ka[s_, :n] = K[s_, :, P0[s_]:P0[s_] + n].permute(1, 0, 2)
        va[s_, :n] = V[s_, :, P0[s_]:P0[s_] + n].permute(1, 0, 2)
    A = make_treeset(w, Lcap, KA.to(DEV), VA.to(DEV), refs.to(DEV))
    A.tree_build(P0)
    A.tree_extend(ka.to(DEV).contiguous(), va.to(DEV).contiguous())
    L1 = [min(p + T, Lcap) for p in P0]
    B_ = make_treeset(w, Lcap, K.to(DEV), V.to(DEV), refs.to(DEV))
    B_.tree_build(L1)
    torch.cuda.synchronize()
    return A, B_, L1


def _same_tree(w, A, B_, L1):
    assert A.len.cpu().tolist() == L1
    for s_ in range(w.B):
        n = L1[s_]
        assert torch.equal(A.k_cache[s_, :, :n], B_.k_cache[s_, :, :n])
        assert torch.equal(A.v_cache[s_, :, :n], B_.v_cache[s_, :, :n])
        for l in range(w.levels):
            n //= w.b if l == 0 else w.F
            assert torch.equal(A.lvl_k[l][s_, :, :n], B_.lvl_k[l][s_, :, :n]), (s_, l)
            assert torch.equal(A.lvl_v[l][s_, :, :n], B_.lvl_v[l][s_, :, :n]), (s_, l)


EXTEND_CASES = [
    W.DEC128K.replace(name="ext_bf16_b32", B=2, Hq=8, Hkv=2, L=32 * 32 * 3 + 500, levels=3, needles=0),
    W.TINY.replace(name="ext_f32_d64_b8", B=2, Hq=2, Hkv=2, b=8, levels=4, L=3000),
    # four references: the levels above the first pool one (node, reference) per wave
    W.ZHA2M.replace(name="ext_bf16_r4_b16", B=2, L=16 * 16 * 16 + 900, levels=3),
    W.DEC128K.replace(name="ext_c32_f4", B=2, Hq=8, Hkv=2, L=32 * 4 * 4 * 3 + 500, fan=4, levels=3, needles=0),
]


@pytest.mark.parametrize("w", EXTEND_CASES, ids=lambda w: w.name)
def test_extend_matches_build(w):
    """tree_extend of a T-token block (ragged lengths; the block completes
    nodes at every level) gives the tree tree_build gives over the longer
    prefix, bit for bit; a decode on it then matches the oracle."""
    T = 1234
    P0 = [w.L, w.L - 333]
    A, B_, L1 = _extend_pair(w, P0, T, Lcap=w.L + T + 7)
    _same_tree(w, A, B_, L1)
    K = torch.stack([A.k_cache[s_].cpu() for s_ in range(w.B)])
    V = torch.stack([A.v_cache[s_].cpu() for s_ in range(w.B)])
    q = W.gen_queries(w.replace(Nq=2))
    _check_decode(A, w.replace(Nq=2), K, V, W.gen_refs(w), L1, q)


def test_extend_clamps_at_capacity():
    """A block longer than the free capacity fills the cache and stops there:
    len = Lcap, and the tree is the one built over Lcap tokens."""
    w = EXTEND_CASES[0]
    Lcap = w.L + 100
    A, B_, L1 = _extend_pair(w, [w.L, Lcap - 3], 300, Lcap)
    assert L1 == [Lcap, Lcap]
    _same_tree(w, A, B_, L1)


# --------------------------------------------------------------------------- prefill
def _prefill(ts, w, T, qb, kb, vb, token_nodes=False):
    sel = select_of(w, token_nodes=token_nodes)
    ws = torch.empty(ts.prefill_workspace_bytes(sel, T), dtype=torch.uint8, device=DEV)
    out = torch.empty((w.B, T, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, T, w.Hq), dtype=torch.float32, device=DEV)
    so = torch.empty((w.B, T, w.Hkv, max(w.levels, 1), kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_prefill(sel, qb.to(DEV).contiguous(), kb.to(DEV).contiguous(), vb.to(DEV).contiguous(),
                      out, ws, lse, so)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), so.cpu().numpy()


def _check_prefill(w, P0, T, ts_list=None, queries=None, edit_kv=None, token_nodes=False):
    w = w.replace(L=P0, T=T)
    K, V = W.gen_kv(w, Lcap=max(P0, 1))
    if edit_kv is not None:
        edit_kv(K, V)
    refs = W.gen_refs(w)
    ts = make_treeset(w, max(P0, 1), K.to(DEV), V.to(DEV), refs.to(DEV), T=T)
    ts.tree_build([P0] * w.B)
    qb, kb, vb = W.gen_block(w)
    out, lse, so = _prefill(ts, w, T, qb, kb, vb, token_nodes=token_nodes)
    queries = queries if queries is not None else range(T)
    nex, emax = 0, 0.0
    for bi in range(w.B):
        for g in range(w.Hkv):
            tr = oracle_tree(w, K[bi, g], V[bi, g], refs[g], P0)
            bk = kb[bi, :, g].float().numpy()
            bv = vb[bi, :, g].float().numpy()
            for t in queries:
                hs = slice(g * w.G, (g + 1) * w.G)
                ex, err = accept(w, tr, K[bi, g, :P0], V[bi, g, :P0], qb[bi, t, hs], out[bi, t, hs],
                                 lse[bi, t, hs], so[bi, t, g], t=t, blk_k=bk, blk_v=bv)
                nex += ex
                emax = max(emax, err)
    log(f"  prefill P0={P0} T={T} token_nodes={token_nodes}: exempt={nex} max_err={emax:.2e}")
    return out, nex


PF = W.PREFILL.replace(name="pf_small")


@pytest.mark.parametrize("token_nodes", [False, True])
@pytest.mark.parametrize("P0,T,levels", [(3000, 100, 2), (32 * 32 * 4 + 70, 77, 2), (5000, 1, 2),
                                         (0, 130, 2), (40, 64, 1), (2000, 33, 0)])
def test_prefill_parity(P0, T, levels, token_nodes):
    """token_nodes True: the prefix token level node-inverted (levels >= 1);
    False: every query gathers its own token rows."""
    _check_prefill(PF.replace(levels=levels, k=8 if levels else 32), P0, T, token_nodes=token_nodes)


@pytest.mark.parametrize("token_nodes", [False, True])
@pytest.mark.parametrize("b,fan,levels,P0,T", [(32, 4, 3, 32 * 4 * 4 * 3 + 70, 90), (8, 32, 2, 8 * 32 * 5 + 3, 40)])
def test_prefill_fanout(b, fan, levels, P0, T, token_nodes):
    """A tree whose fan above level 1 differs from its chunk size, on both
    token-level paths (the node-inverted one groups queries by level-1 node,
    whose b tokens stay contiguous)."""
    _check_prefill(PF.replace(b=b, fan=fan, levels=levels, k=6), P0, T, token_nodes=token_nodes)


@pytest.mark.parametrize("Hq,Hkv,R,k,P0", [(32, 8, 1, 8, 32 * 32 * 12 + 70), (8, 8, 1, 8, 32 * 32 * 12 + 70),
                                          (16, 8, 2, 8, 32 * 32 * 12 + 31), (64, 8, 1, 8, 32 * 32 * 9 + 3),
                                          (32, 8, 8, 4, 32 * 32 * 7 + 5)])
def test_prefill_scored_top_level(Hq, Hkv, R, k, P0):
    """The top level has more nodes than are kept, so it is scored for the
    whole block at once on the matrix cores (G = 1, 2, 4, 8; R = 1, 2, 8)."""
    w = PF.replace(Hq=Hq, Hkv=Hkv, R=R, k=k, levels=2)
    _check_prefill(w, P0, 40)


@pytest.mark.parametrize("Hq,Hkv,d,P0,T", [(32, 8, 128, 3000, 300), (8, 1, 128, 500, 200),
                                           (2, 2, 128, 700, 261), (8, 4, 64, 900, 190)])
def test_prefill_inblock_tiles(Hq, Hkv, d, P0, T):
    """The causal block product spans several 64-key tiles with a ragged
    last tile, for head groups G = 4, 8, 1, 2 and head_dim 128 / 64."""
    w = PF.replace(Hq=Hq, Hkv=Hkv, d=d, levels=2)
    _check_prefill(w, P0, T)


@pytest.mark.parametrize("token_nodes", [False, True])
def test_prefill_without_prefix_capacity(token_nodes):
    """A tree set with Lcap = 0 (the first block of new sequences) holds no
    prefix, so no traversal runs: the outputs must equal, bit for bit, those
    of the same block over an empty prefix in a tree set with capacity (the
    same in-block kernel, seeded with nothing), and the oracle's; every
    selection slot is -1."""
    w = PF.replace(levels=2, L=0, T=150)
    T = w.T
    qb, kb, vb = W.gen_block(w)
    K, V = W.gen_kv(w, Lcap=1)
    refs = W.gen_refs(w)
    res = []
    for Lcap in (0, 3000):
        ts = make_treeset(w, Lcap, refs=refs.to(DEV), T=T)
        ts.tree_build([0] * w.B)
        res.append(_prefill(ts, w, T, qb, kb, vb, token_nodes=token_nodes))
        del ts
    (o0, l0, s0), (o1, l1, s1) = res
    assert (s0 == -1).all()
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32))
    assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32))
    for bi in range(w.B):
        for g in range(w.Hkv):
            tr = oracle_tree(w, K[bi, g], V[bi, g], refs[g], 0)
            bk = kb[bi, :, g].float().numpy()
            bv = vb[bi, :, g].float().numpy()
            hs = slice(g * w.G, (g + 1) * w.G)
            for t in (0, 1, 63, 64, T - 1):
                accept(w, tr, K[bi, g, :0], V[bi, g, :0], qb[bi, t, hs], o0[bi, t, hs], l0[bi, t, hs],
                       s0[bi, t, g], t=t, blk_k=bk, blk_v=bv)
    log(f"  prefill without prefix capacity, token_nodes={token_nodes}: T={T} bit-identical")


def test_prefill_exact_ties():
    """Exactly equal scores: keys that are zero score 0 at every position, so
    with all but three level-1 nodes zeroed most candidates tie.  The kept
    sets must be those of the oracle (higher score, then lower index) with no
    exemption, and the outputs must agree."""
    w = PF.replace(levels=2, k=8)
    P0 = 32 * 32 * 4 + 70

    def zero_most(K, V):
        keep = torch.zeros(P0, dtype=torch.bool)
        for n in (70, 90, 100):
            keep[n * 32:(n + 1) * 32] = True
        K[:, :, :P0][:, :, ~keep] = 0

    _, nex = _check_prefill(w, P0, 24, edit_kv=zero_most)
    assert nex == 0


@pytest.mark.parametrize("token_nodes", [False, True])
def test_prefill_b24(token_nodes):
    """A branching factor that is not a power of two (b = 24): candidate
    positions, orphans and the division by b in the index arithmetic; in the
    node-inverted token level, tokens 24..31 of the second 16-token tile are
    masked."""
    w = PF.replace(b=24, levels=2, k=6)
    _check_prefill(w, 24 * 24 * 3 + 50, 40, token_nodes=token_nodes)


@pytest.mark.parametrize("token_nodes", [False, True])
def test_prefill_topp_r4(token_nodes):
    """Top-p with four reference keys and b = 16 (one 16-token tile per node
    in the node-inverted token level; kept sets of varying size)."""
    _check_prefill(W.ZHA2M.replace(name="pf_topp", levels=3), 16 ** 3 * 3 + 50, 48, token_nodes=token_nodes)


def test_prefill_small_b_hot_node():
    """b = 5 (one partly masked token tile) and every query keeping every
    level-1 node (take-all at level 1): each node's run spans many waves of
    the node-inverted token level."""
    w = PF.replace(b=5, levels=1, k=8)
    _check_prefill(w, 5 * 7 + 3, 200, token_nodes=True)


def test_prefill_T1_equals_decode():
    """A one-token block at P0 gives the decode result at position P0 when
    the token completes no node ((P0 + 1) % b != 0)."""
    w = PF.replace(L=4000, T=1, levels=2)
    K, V = W.gen_kv(w, Lcap=w.L + 1)
    refs = W.gen_refs(w)
    qb, kb, vb = W.gen_block(w)
    K[:, :, w.L] = kb[:, 0]
    V[:, :, w.L] = vb[:, 0]
    ts = make_treeset(w, w.L + 1, K.to(DEV), V.to(DEV), refs.to(DEV), T=1)
    ts.tree_build([w.L] * w.B)
    pout, _, psel = _prefill(ts, w, 1, qb, kb, vb)
    ts.tree_build([w.L + 1] * w.B)
    dout, _, dsel = _decode(ts, w, qb[:, :1])
    assert np.array_equal(psel[:, 0], dsel[:, 0])
    assert np.abs(pout[:, 0] - dout[:, 0]).max() < 2e-2


# --------------------------------------------------------------------------- decode step
STEP_CASES = [
    # steps 3..4 complete a level-1 and a level-2 node (b = 32)
    W.DEC128K.replace(name="step_b32", B=2, L=32 * 32 * 3 - 3, levels=2, needles=0),
    # batch 8 (64 units): one workgroup per CU would leave each unit four, so
    # the plan launches the two-waves-per-SIMD instance, two per CU; step 3
    # completes a level-1 and a level-2 node
    W.DEC128K.replace(name="step_b32_two_per_cu", B=8, L=32 * 32 * 2 - 3, levels=2, needles=0),
    # b = 16, top-p with four reference keys: a level-3 node completes
    W.ZHA2M.replace(name="step_topp_r4_b16", L=16 ** 3 * 2 - 4, levels=3),
    # G = 8, d = 64, b = 8, two queries per sequence
    W.DEC128K.replace(name="step_g8_d64_b8_nq2", Hq=16, Hkv=2, d=64, b=8, levels=3, L=8 ** 3 * 2 - 5,
                      needles=0, k=3, Nq=2),
    # b = 64: the two-launch form
    W.DEC128K.replace(name="step_b64", b=64, levels=2, L=64 * 64 - 3, k=4, needles=0),
    # chunk 16, fan 4: steps complete nodes of levels 1 to 3 in the one launch
    W.DEC128K.replace(name="step_c16_f4", b=16, fan=4, levels=3, L=16 * 4 * 4 * 3 - 3, k=4, needles=0),
    # fan 48 above chunks of 8: the two-launch form
    W.DEC128K.replace(name="step_c8_f48", b=8, fan=48, levels=2, L=8 * 48 * 2 - 4, k=3, needles=0),
]


@pytest.mark.parametrize("w", STEP_CASES, ids=lambda w: w.name)
def test_decode_step_matches_append_then_decode(w):
    """decode_step (one launch where the split kernel applies) against
    tree_append followed by sparse_decode on a second tree set: outputs,
    lse, selections, lengths, caches and every tree level bit for bit, over
    steps that complete nodes; the last step also against the oracle."""
    steps = 8
    Lcap = w.L + steps
    K, V = W.gen_kv(w, Lcap=Lcap)
    refs = W.gen_refs(w)
    ta = make_treeset(w, Lcap, K.to(DEV), V.to(DEV), refs.to(DEV))
    tb = make_treeset(w, Lcap, K.to(DEV), V.to(DEV), refs.to(DEV))
    ta.tree_build([w.L] * w.B)
    tb.tree_build([w.L] * w.B)
    sel = select_of(w)
    kmax = kmax_of(w)
    shape = (w.B, w.Nq, w.Hq, w.d)
    oa, ob = (torch.empty(shape, dtype=torch.float32, device=DEV) for _ in range(2))
    la, lb = (torch.empty(shape[:3], dtype=torch.float32, device=DEV) for _ in range(2))
    sa, sb = (torch.empty((w.B, w.Nq, w.Hkv, w.levels, kmax), dtype=torch.int32, device=DEV) for _ in range(2))
    for s in range(steps):
        kn, vn = W.gen_append(w, s, device=DEV)
        q = W.gen_queries(w, step=s + 1).to(DEV).contiguous()
        ta.decode_step(sel, kn.contiguous(), vn.contiguous(), q, oa, la, sa)
        tb.tree_append(kn.contiguous(), vn.contiguous())
        tb.sparse_decode(sel, q, ob, lb, sb)
        torch.cuda.synchronize()
        assert torch.equal(ta.len, tb.len), s
        assert torch.equal(oa, ob), f"step {s}: max diff {(oa - ob).abs().max().item()}"
        assert torch.equal(la, lb) and torch.equal(sa, sb), s
    assert ta.len.cpu().tolist() == [w.L + steps] * w.B
    assert torch.equal(ta.k_cache, tb.k_cache) and torch.equal(ta.v_cache, tb.v_cache)
    for l in range(w.levels):
        assert torch.equal(ta.lvl_k[l], tb.lvl_k[l]) and torch.equal(ta.lvl_v[l], tb.lvl_v[l]), l
    # the last step against the oracle, on the grown caches
    L = w.L + steps
    Kh, Vh = ta.k_cache.cpu(), ta.v_cache.cpu()
    out, lse, so = oa.cpu().numpy(), la.cpu().numpy(), sa.cpu().numpy()
    for bi in range(w.B):
        for g in range(w.Hkv):
            tree = oracle_tree(w, Kh[bi, g], Vh[bi, g], refs[g], L)
            hs = slice(g * w.G, (g + 1) * w.G)
            for qi in range(w.Nq):
                accept(w, tree, Kh[bi, g, :L], Vh[bi, g, :L], q.cpu()[bi, qi, hs], out[bi, qi, hs],
                       lse[bi, qi, hs], so[bi, qi, g])
    log(f"  {w.name}: {steps} steps, lengths {ta.len.cpu().tolist()}")


# --------------------------------------------------------------------------- graph capture
@pytest.mark.parametrize("mode", ["split", "unsplit", "step"])
def test_decode_graph_replay_matches_eager(mode):
    """A step of tree_append + sparse_decode (or the fused decode_step)
    captured into a HIP graph gives, on every replay, what tree_append +
    sparse_decode give eagerly: a second tree set runs those calls eagerly
    between the replays, from the same start."""
    split = mode != "unsplit"
    w = W.DEC128K.replace(name="graph", B=2, L=32 * 156 + 29, levels=2, needles=0)   # completes a node
    steps = 4
    Lcap = w.L + steps
    K, V = W.gen_kv(w, Lcap=Lcap)
    refs = W.gen_refs(w)
    tg = make_treeset(w, Lcap, K.to(DEV), V.to(DEV), refs.to(DEV))
    te = make_treeset(w, Lcap, K.to(DEV), V.to(DEV), refs.to(DEV))
    tg.tree_build([w.L] * w.B)
    te.tree_build([w.L] * w.B)
    sel = select_of(w)
    q = W.gen_queries(w).to(DEV).contiguous()
    kn, vn = W.gen_append(w, 0, device=DEV)
    kn, vn = kn.contiguous(), vn.contiguous()
    og = torch.empty((w.B, q.shape[1], w.Hq, w.d), dtype=torch.float32, device=DEV)
    oe = torch.empty_like(og)
    # workspaces exist before capture (nothing is allocated inside the graph)
    tg.decode_workspace(sel, q.shape[1])
    te.decode_workspace(sel, q.shape[1])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            if mode == "step":
                tg.decode_step(sel, kn, vn, q, og)
            else:
                tg.tree_append(kn, vn)
                tg.sparse_decode(sel, q, og, split=split)
    torch.cuda.synchronize()
    for r in range(steps):
        graph.replay()
        torch.cuda.synchronize()
        te.tree_append(kn, vn)
        te.sparse_decode(sel, q, oe, split=split)
        torch.cuda.synchronize()
        assert torch.equal(tg.len, te.len), r
        assert torch.equal(og, oe), f"replay {r}: max diff {(og - oe).abs().max().item()}"
        assert torch.equal(tg.k_cache, te.k_cache) and torch.equal(tg.lvl_k[0], te.lvl_k[0]), r
