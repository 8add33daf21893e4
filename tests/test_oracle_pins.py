"""Pins of the CPU oracle against facts the pages and mathematics fix.

Each test names the pin it implements:
  P1 every node selected  -> dense causal attention (textbook routine)
  P2 mean-pooled values    -> subtree means (closed form)
  P3 pooler closed forms   -> r = 0 gives the child mean, permutation invariance,
                              a dominant reference gives its argmax child,
                              equal children give that child; children whose
                              logits are ln 3, 0, 0, ln 2 pool with weights
                              3/7, 1/7, 1/7, 2/7 exactly (the 1/sqrt(d)
                              temperature, at three head sizes)
  P3b per-reference chains -> every level of a tree with R distinct reference
                              queries equals a float64 whole-level pooler in
                              which each reference pools its own chain
  P12 exact ties           -> top-k and top-p over exactly equal scores keep
                              the lowest node indices; a node whose R keys
                              tie takes the first reference's key
  P4 selection certificate -> brute force over all subsets / top-p mass rules
  P5 entries partition the visible tokens
  P6 entries read          -> exact count formula, linear in log_b L
  P7 exhaustive small trees (64 tokens) against the node-predicate formulation
     of E and a float64 softmax over it
  P9 prefill with T = 1 is decode; prefill over an empty prefix is causal attention
  P10 R equal references equal R = 1; top-p with cap 1 equals top-1
  bf16 node rounding matches torch's round-to-nearest-even
  P11 E4M3 router keys     -> torch's float8_e4m3fn cast (library routine), code
                              values worked out by hand from the format, and a
                              tree whose summary keys are the dequantised rows
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import hti_workloads as W
from ref_f64 import (candidates_by_predicate, covered_tokens, dense_causal,
                     entries_from_candidates, group_scores_f64, level_counts, pool_tree_f64,
                     rope_c, softmax_over_entries)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16r(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def rand_kv(L, d, seed, bf16=False):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L, d)).astype(np.float32)
    V = rng.standard_normal((L, d)).astype(np.float32)
    if bf16:
        K, V = bf16r(K), bf16r(V)
    return K, V, rng


def sel_sets(res, levels):
    s = [set() for _ in range(levels + 1)]
    for l in range(1, levels + 1):
        s[l] = {int(x) for x in res["sel"][l - 1] if x >= 0}
    return s


def eval_f64(tree, K, V, q, sel, *, base=10000.0, t=-1, blk_k=None, blk_v=None, leaf_only=False):
    """Shared softmax in float64 over the entry set implied by `sel` (only the
    reached tokens when leaf_only)."""
    L, b, lv = tree.L, tree.b, tree.levels
    cands = candidates_by_predicate(L, b, lv, sel, getattr(tree, "fan", b))
    zs, vals = [], []
    for l in range(lv, 0, -1):
        if leaf_only:
            break
        C = cands[l]
        uns = [i for i, x in enumerate(C) if x not in sel[l]]
        if not uns:
            continue
        _, z = group_scores_f64(q, tree.lk[l - 1][C], len(C), base)
        zs.append(z[:, uns])
        vals.append(tree.lv[l - 1][[C[i] for i in uns]].astype(np.float64))
    C0 = list(cands[0])
    keys0 = K[C0].astype(np.float64)
    vals0 = V[C0].astype(np.float64)
    if t >= 0:
        qp = len(C0) + t
        keys0 = np.concatenate([keys0, blk_k[: t + 1]])
        vals0 = np.concatenate([vals0, blk_v[: t + 1]])
    else:
        qp = sum(1 for x in C0 if x < L - 1)
    kr = rope_c(keys0, np.arange(len(keys0)), base)
    zs.append(rope_c(q, qp, base) @ kr.T / np.sqrt(q.shape[-1]))
    vals.append(vals0)
    return softmax_over_entries(np.concatenate(zs, axis=1), np.concatenate(vals))


# --------------------------------------------------------------------------- golden
def test_level_counts_golden():
    g = json.load(open(os.path.join(GOLDEN, "level_counts.json")))
    for name, e in g.items():
        if name.startswith("_"):
            continue
        w = W.WORKLOADS[name]
        assert (w.L, w.b, w.levels) == (e["L"], e["b"], e["levels"])
        assert w.level_counts() == e["counts"]
        # the oracle sizes its level arrays with the same rule (tiny tree per
        # workload geometry: scale the count list by the first level)
        tr = oracle.Tree(e["L"], 1, e["b"], e["levels"], 1, False)
        assert [x.shape[0] for x in tr.lk] == e["counts"][1:]


# --------------------------------------------------------------------------- P1
@pytest.mark.parametrize("mode", ["topk", "topp"])
def test_dense_equivalence_tiny_workload(mode):
    """P1 on the tiny-decode geometry.  With a per-level budget, every token is
    reached exactly when each level keeps all of its candidates; the largest
    candidate list is level 1 (n_1 = 256 nodes), so k = 256 (or top-p with
    p = 1 and cap = 256)."""
    w = W.TINY
    K, V = W.gen_kv(w, Lcap=w.L)
    refs = W.gen_refs(w)
    q = W.gen_queries(w)
    K0, V0 = K[0, 0].numpy(), V[0, 0].numpy()
    tr = oracle.build_tree(K0, V0, refs[0], w.b, w.levels, bf16=False)
    for qi in (0, 7, 15):
        qq = q[0, qi].numpy()                      # [Hq=1, d]
        if mode == "topk":
            r = oracle.query(tr, K0, V0, qq, k=256)
        else:
            r = oracle.query(tr, K0, V0, qq, mode="topp", p=1.0, cap=256)
        ref = dense_causal(qq, K0, V0, w.L - 1)
        assert np.abs(r["out"] - ref).max() < 1e-5
        # top-p still scores every summary level (16 + 256 keys) before keeping all
        scored = 0 if mode == "topk" else 16 + 256
        assert r["counts"][0] == w.L + scored and r["counts"][1] == w.L


@pytest.mark.parametrize("L,b,levels,R,G,d", [(700, 4, 3, 2, 4, 32), (1000, 8, 2, 1, 2, 128),
                                             (257, 2, 6, 3, 1, 16)])
def test_dense_equivalence_bf16_gqa(L, b, levels, R, G, d):
    K, V, rng = rand_kv(L, d, seed=L, bf16=True)
    refs = (rng.standard_normal((R, d)) / np.sqrt(d)).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, levels, bf16=True)
    q = bf16r(rng.standard_normal((G, d)))
    r = oracle.query(tr, K, V, q, k=L // b)      # n_1 = largest candidate list
    ref = dense_causal(q, K, V, L - 1)
    assert np.abs(r["out"] - ref).max() < 1e-5


# --------------------------------------------------------------------------- P2
@pytest.mark.parametrize("bf16", [False, True])
def test_values_are_subtree_means(bf16):
    L, d, b, levels = 4096 + 77, 64, 4, 5
    K, V, rng = rand_kv(L, d, seed=3, bf16=bf16)
    refs = (rng.standard_normal((2, d)) / 8).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, levels, bf16=bf16)
    for l in range(1, levels + 1):
        n = L // b ** l
        span = b ** l
        means = V[: n * span].astype(np.float64).reshape(n, span, d).mean(axis=1)
        err = np.abs(tr.lv[l - 1] - means).max()
        # fp32: sequential sums of <= b terms per level; bf16: one rounding of
        # at most half an ulp (2^-9 relative) per level on values |mean| <= 4
        bound = 2e-6 * l if not bf16 else l * 2.0 ** -9 * 4.0
        assert err < bound, (l, err, bound)


# --------------------------------------------------------------------------- P3
def test_pooler_closed_forms():
    L, d, b, levels = 512, 32, 8, 3
    K, V, rng = rand_kv(L, d, seed=5)
    # r = 0: every weight is 1/b -> pooled key = child mean (recursively: subtree mean)
    tr0 = oracle.build_tree(K, V, np.zeros((1, d), np.float32), b, levels, bf16=False)
    for l in range(1, levels + 1):
        n, span = L // b ** l, b ** l
        means = K[: n * span].astype(np.float64).reshape(n, span, d).mean(axis=1)
        assert np.abs(tr0.lk[l - 1][:, 0] - means).max() < 2e-6 * l

    # equal children: pooling a node whose children all equal u returns u
    u = rng.standard_normal(d).astype(np.float32)
    Ku = np.tile(u, (L, 1))
    refs = rng.standard_normal((2, d)).astype(np.float32)
    tru = oracle.build_tree(Ku, V, refs, b, levels, bf16=False)
    for l in range(levels):
        assert np.abs(tru.lk[l] - u).max() < 4e-6 * np.abs(u).max()

    # permutation of a node's children leaves its pooled key unchanged (up to
    # the order of the fp32 sums)
    r1 = rng.standard_normal((1, d)).astype(np.float32)
    ta = oracle.build_tree(K, V, r1, b, 1, bf16=False)
    perm = np.concatenate([np.random.default_rng(1).permutation(b) + i * b for i in range(L // b)])
    tb = oracle.build_tree(K[perm], V[perm], r1, b, 1, bf16=False)
    assert np.abs(ta.lk[0] - tb.lk[0]).max() < 1e-5
    assert np.abs(ta.lv[0] - tb.lv[0]).max() < 1e-5

    # dominant reference: r = lam * k_c* with k_c* the child of largest norm ->
    # the pooled key is k_c* (softmax saturates)
    Kd = K.copy()
    Kd[3] *= 6.0                                   # child 3 of node 0 dominates
    rd = (60.0 * Kd[3] / np.linalg.norm(Kd[3]) ** 2 * np.sqrt(d)).astype(np.float32)[None]
    td = oracle.build_tree(Kd, V, rd, b, 1, bf16=False)
    assert np.abs(td.lk[0][0, 0] - Kd[3]).max() < 1e-4 * np.abs(Kd[3]).max()


@pytest.mark.parametrize("d", [16, 36, 128])
def test_pooler_temperature_closed_form(d):
    """P3: the pooler's weights are softmax(r . k / sqrt(d)) over a node's
    children.  Four children along orthogonal axes: child c = a_c e_c, and
    the reference r = sum_c (lambda_c sqrt(d) / a_c) e_c, so that
    r . k_c / sqrt(d) = lambda_c with lambda = (ln 3, 0, 0, ln 2).  The
    weights are then 3/7, 1/7, 1/7, 2/7 and the pooled key is
    (3 a_0 / 7, a_1 / 7, a_2 / 7, 2 a_3 / 7, 0, ...).  The three head sizes
    tell the 1/sqrt(d) temperature from a missing, halved, doubled or
    1/d one.  A second node repeats this with the children in another order,
    and the level above pools the two (its logits are again checked against
    the closed form)."""
    b = 4
    lam = np.array([np.log(3.0), 0.0, 0.0, np.log(2.0)])
    amp = np.array([2.0, -1.5, 0.75, 3.0])
    r = np.zeros(d)
    for c in range(b):
        r[c] = lam[c] * np.sqrt(d) / amp[c]
    K = np.zeros((2 * b, d))
    for c in range(b):
        K[c, c] = amp[c]
    order = [2, 0, 3, 1]                       # node 1: the same children permuted
    K[b:] = K[order]
    K32 = K.astype(np.float32)
    V = np.zeros((2 * b, d), np.float32)
    tr = oracle.build_tree(K32, V, r.astype(np.float32)[None], b, 1, bf16=False)
    want = np.zeros(d)
    wts = np.array([3.0, 1.0, 1.0, 2.0]) / 7.0
    for c in range(b):
        want[c] = wts[c] * amp[c]
    for node in range(2):
        got = tr.lk[0][node, 0].astype(np.float64)
        assert np.abs(got - want).max() < 2e-6, (d, node, got[:4], want[:4])
    # level 2 over two children given directly: logits ln 3 and 0 -> 3/4, 1/4
    u0 = np.zeros(d)
    u0[0] = 1.0
    u1 = np.zeros(d)
    u1[1] = 1.0
    r2 = np.zeros(d)
    r2[0] = np.log(3.0) * np.sqrt(d)
    t2 = oracle.build_tree(np.stack([u0, u1]).astype(np.float32), np.zeros((2, d), np.float32),
                           r2.astype(np.float32)[None], 2, 1, bf16=False)
    assert abs(float(t2.lk[0][0, 0, 0]) - 0.75) < 1e-6 and abs(float(t2.lk[0][0, 0, 1]) - 0.25) < 1e-6


@pytest.mark.parametrize("L,b,levels,R,d", [(4096 + 300, 4, 5, 3, 32), (2 * 32 ** 2 + 77, 32, 2, 4, 64),
                                            (1000, 3, 6, 2, 16)])
def test_pooler_per_reference_chains(L, b, levels, R, d):
    """P3b: with R distinct reference queries every reference pools its own
    chain -- level 1 from the tokens, level l >= 2 from its own level-(l-1)
    keys -- against the float64 whole-level pooler, level by level; values
    are the plain subtree means.  (A tree that pooled every chain with the
    first reference, or fed level l a chain of another reference, differs
    from it by far more than the fp32 rounding of its sums.)"""
    K, V, rng = rand_kv(L, d, seed=L + R)
    refs = (rng.standard_normal((R, d)) * (1.5 / np.sqrt(d))).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, levels, bf16=False)
    ref = pool_tree_f64(K, V, refs, b, levels)
    for l in range(levels):
        rk, rv = ref[l]
        scale = max(1.0, float(np.abs(rk).max()))
        assert np.abs(tr.lk[l] - rk).max() < 1e-5 * scale * (l + 1), (l + 1, float(np.abs(tr.lk[l] - rk).max()))
        assert np.abs(tr.lv[l] - rv).max() < 1e-5 * (l + 1)
        # the chains really differ between references
        if R > 1:
            assert np.abs(rk[:, 0] - rk[:, 1]).max() > 1e-2
    # bf16 storage: each level pools the stored (rounded) children; the
    # float64 pooler fed the same rounded children one level at a time
    tb = oracle.build_tree(bf16r(K), bf16r(V), refs, b, levels, bf16=True)
    for l in range(levels):
        if l == 0:
            child = np.repeat(bf16r(K)[:, None, :], R, axis=1)
        else:
            child = tb.lk[l - 1]
        n = child.shape[0] // b
        for j in range(R):
            one = pool_tree_f64(child[: n * b, j], np.zeros((n * b, d)), refs[j:j + 1], b, 1)[0][0][:, 0]
            err = np.abs(tb.lk[l][:, j] - one)
            # one bf16 rounding (half an ulp: 2^-9 relative) of an fp32 sum
            assert (err <= 2.0 ** -8 * np.abs(one) + 1e-6).all(), (l + 1, j, float(err.max()))


def _tied_setup(L, b, levels, R, d, seed):
    """A tree with R distinct references, and a group of two query heads
    q and -q: every per-head logit of head 1 is the exact negative of head
    0's (rotation commutes with negation), so every group score is exactly 0
    and every level ties throughout, across nodes and across references."""
    K, V, rng = rand_kv(L, d, seed=seed)
    refs = (rng.standard_normal((R, d)) / np.sqrt(d)).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, levels, bf16=False)
    q0 = rng.standard_normal(d).astype(np.float32)
    q = np.stack([q0, -q0])
    return tr, K, V, q


def _expected_tied_selection(L, b, levels, count):
    """Selections under exact ties with the lower-index rule: at each level the
    `count(m)` lowest node ids among the candidates."""
    sel = [set() for _ in range(levels + 1)]
    n = level_counts(L, b, levels)
    cand = list(range(n[levels]))
    for l in range(levels, 0, -1):
        keep = sorted(cand)[: count(len(cand))]
        sel[l] = set(keep)
        orph = list(range(b * n[l], n[l - 1]))
        cand = [c * b + i for c in sorted(keep) for i in range(b)] + orph
    return sel


@pytest.mark.parametrize("R", [1, 2, 3])
def test_exact_ties_topk(R):
    """P12: all group scores exactly equal; top-k keeps the k lowest node ids
    at every level (reading: ties go to the lower index), and the output is
    the float64 shared softmax in which every node takes its first
    reference's key (reading: ties across references go to the lower j)."""
    L, b, levels, d, k = 4 ** 5 + 37, 4, 5, 16, 3
    tr, K, V, q = _tied_setup(L, b, levels, R, d, seed=70 + R)
    r = oracle.query(tr, K, V, q, k=k, entries=True)
    want = _expected_tied_selection(L, b, levels, lambda m: min(k, m))
    assert sel_sets(r, levels)[1:] == want[1:]
    # output under that selection, with key j* = 0 for every summary entry
    cands = candidates_by_predicate(L, b, levels, want)
    zs, vals = [], []
    for l in range(levels, 0, -1):
        C = cands[l]
        uns = [i for i, x in enumerate(C) if x not in want[l]]
        keys0 = tr.lk[l - 1][C][:, 0]                       # the first reference's key
        kr = rope_c(keys0, np.arange(len(C)))
        zz = rope_c(q, len(C)) @ kr.T / np.sqrt(d)
        zs.append(zz[:, uns])
        vals.append(tr.lv[l - 1][[C[i] for i in uns]].astype(np.float64))
    C0 = cands[0]
    kr = rope_c(K[C0], np.arange(len(C0)))
    qp = sum(1 for x in C0 if x < L - 1)
    zs.append(rope_c(q, qp) @ kr.T / np.sqrt(d))
    vals.append(V[C0].astype(np.float64))
    out, lse = softmax_over_entries(np.concatenate(zs, axis=1), np.concatenate(vals))
    assert np.abs(r["out"] - out).max() < 2e-5
    assert np.abs(r["lse"] - lse).max() < 2e-5
    # every scored level's gap at the boundary is exactly zero (the acceptance
    # rule exempts such levels); a level taken whole has none
    fin = np.isfinite(r["gap"])
    assert fin.sum() >= levels - 1 and (r["gap"][fin] == 0).all()


@pytest.mark.parametrize("p,cap", [(0.3, 16), (0.5, 2), (0.9, 16)])
def test_exact_ties_topp(p, cap):
    """P12 for top-p: with every score equal, each candidate has softmax mass
    1/m, so the kept count is the smallest n with n/m >= p (clamped to
    [1, cap]) and the kept nodes are the n lowest ids."""
    L, b, levels, d = 4 ** 4 + 9, 4, 4, 16
    tr, K, V, q = _tied_setup(L, b, levels, 2, d, seed=91)

    def count(m):
        if m <= 1:
            return m
        n = next(i for i in range(1, m + 1) if i / m >= np.float32(p))
        if m & (m - 1) and n - 1 < cap:
            # 1/m is inexact in fp32: no running sum may sit near p (unless
            # the cap decides the count either way)
            assert min(abs(i / m - p) for i in range(1, m + 1)) > 1e-4
        # (m a power of two: 1/m and its running sums are exact in fp32)
        return max(1, min(cap, n))

    r = oracle.query(tr, K, V, q, mode="topp", p=p, cap=cap)
    want = _expected_tied_selection(L, b, levels, count)
    assert sel_sets(r, levels)[1:] == want[1:]


def test_bf16_node_rounding_is_rne():
    """b = 2 mean (a + b) / 2 in fp32 then rounded: equals torch's RNE bf16 cast."""
    rng = np.random.default_rng(11)
    L, d = 4096, 64
    V = bf16r(rng.standard_normal((L, d)))
    K = bf16r(rng.standard_normal((L, d)))
    tr = oracle.build_tree(K, V, np.zeros((1, d), np.float32), 2, 1, bf16=True)
    v32 = (torch.from_numpy(V[0::2]) + torch.from_numpy(V[1::2])) / 2.0
    expect = v32.to(torch.bfloat16).float().numpy()
    assert np.array_equal(tr.lv[0], expect)


# --------------------------------------------------------------------------- P4
def _check_certificate(s, selected_pos, mode, k, p, cap, tol=2e-5):
    m = len(s)
    S = sorted(selected_pos)
    rest = [i for i in range(m) if i not in set(S)]
    if mode == "topk":
        assert len(S) == min(k, m)
    else:
        assert 1 <= len(S) <= min(cap, m)
    if rest and S:
        assert min(s[i] for i in S) >= max(s[i] for i in rest) - tol
    if mode == "topk" and m <= 10 and len(S) < m:
        # brute force: no subset of the same size has a larger total score
        best = max(sum(s[i] for i in c) for c in itertools.combinations(range(m), len(S)))
        assert sum(s[i] for i in S) >= best - tol * len(S)
    if mode == "topp" and len(S) < min(cap, m):
        pi = np.exp(s - s.max())
        pi /= pi.sum()
        mass = pi[S].sum()
        assert mass >= p - 1e-5
        assert mass - pi[S].min() < p + 1e-5


# --------------------------------------------------------------------------- P6
@pytest.mark.parametrize("b,k,max_levels", [(2, 1, 20), (4, 2, 10), (16, 4, 5)])
def test_entries_read_grow_linearly_in_log_L(b, k, max_levels):
    """L = b^levels (one top node, no orphans): keys and values read follow the
    closed form and grow by a constant per level, i.e. O(log L)."""
    d = 8
    prev = None
    incs = []
    for lv in range(2, max_levels + 1):
        L = b ** lv
        if L > 1 << 20:
            break
        K, V, rng = rand_kv(L, d, seed=lv)
        refs = (rng.standard_normal((1, d)) / 3).astype(np.float32)
        tr = oracle.build_tree(K, V, refs, b, lv, bf16=False)
        q = rng.standard_normal((1, d)).astype(np.float32)
        r = oracle.query(tr, K, V, q, k=k)
        keys = b + (lv - 2) * k * b + k * b
        vals = (b - k) + (lv - 2) * (k * b - k) + k * b
        assert tuple(r["counts"]) == (keys, vals), (lv, r["counts"], keys, vals)
        tot = keys + vals
        if prev is not None:
            incs.append(tot - prev)
        prev = tot
    assert len(set(incs)) == 1 and incs[0] == 2 * k * b - k


# --------------------------------------------------------------------------- P7
def _sweep_cases():
    """Every (L <= 64, b, levels) geometry, four cases each, rotating the
    selection rule, R, G, the prefill block length and the seed through
    decorrelated counters so every value of every knob is hit many times."""
    cases = []
    sel_variants = {}
    for b in (2, 4, 8, 16, 32, 64):
        v = [("topk", k, 1.0, 0) for k in sorted({1, 2, b - 1, b, b + 1} - {0})]
        v += [("topp", 0, p, cap) for p in (0.1, 0.5, 0.9, 1.0) for cap in sorted({1, 2, b})]
        sel_variants[b] = v
    i = 0
    for L in range(1, 65):
        for b in (2, 4, 8, 16, 32, 64):
            maxlv = 0
            while b ** (maxlv + 1) <= 64:
                maxlv += 1
            for lv in range(0, maxlv + 2):
                variants = sel_variants[b]
                for j in range(4):
                    sv = variants[(i * 5 + j) % len(variants)]
                    R = 1 + (i // 3 + j) % 2
                    G = 1 + (i // 7 + j // 2) % 2
                    T = (0, 1, 3, 8)[(i // 11 + j) % 4]        # 0 = decode
                    cases.append((L, b, lv, sv, R, G, T, i))
                    i += 1
    return cases


_CASES = _sweep_cases()


def _check_small_case(L, b, lv, mode, k, p, cap, R, G, T, seed, fan=None):
    """P4 + P5 + P6 + P7 on one small tree (b tokens per level-1 node, fan
    nodes per node above; None: fan = b), decode (T = 0) or every row of a
    T-token prefill block."""
    d = 8
    K, V, rng = rand_kv(L + T, d, seed=seed)
    refs = (rng.standard_normal((R, d)) / np.sqrt(d)).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, lv, bf16=False, L=L, fan=fan)
    q = rng.standard_normal((G, d)).astype(np.float32)
    kmax = k if mode == "topk" else cap
    for t in (range(T) if T else [-1]):
        blk = dict(t=t, blk_k=K[L:], blk_v=V[L:]) if T else {}
        r = oracle.query(tr, K[:L], V[:L], q, mode=mode, k=k, p=p, cap=cap, kmax=kmax,
                         entries=True, **blk)
        sel = sel_sets(r, lv)
        cands = candidates_by_predicate(L, b, lv, sel, fan)
        # P7: entry list equals the node-predicate formulation
        ent = entries_from_candidates(cands, sel, lv)
        nblk = t + 1 if T else 0
        ent += [(0, L + j, len(cands[0]) + j) for j in range(nblk)]
        got = list(zip(*[x.tolist() for x in r["entries"]]))
        assert got == ent, (L, b, fan, lv, mode, k, p, cap, T, t)
        # P5: entries partition the visible tokens [0, L + nblk)
        cover = np.zeros(L + nblk, np.int64)
        for (l, x, _) in ent:
            for tkn in covered_tokens(l, x, b, fan):
                cover[tkn] += 1
        assert (cover == 1).all()
        # P4: per-level certificate on float64 scores
        thr = k if mode == "topk" else 1
        nkeys = 0
        for l in range(lv, 0, -1):
            C = cands[l]
            if len(C) <= thr:
                assert sel[l] == set(C)
                continue
            nkeys += len(C) * R
            s_, _ = group_scores_f64(q, tr.lk[l - 1][C], len(C), 10000.0)
            pos = [i for i, x in enumerate(C) if x in sel[l]]
            _check_certificate(s_, pos, mode, k, p, cap)
        # P6: counters
        nvals = sum(len(cands[l]) - len(sel[l] & set(cands[l])) for l in range(1, lv + 1))
        n0 = len(cands[0]) + nblk
        assert tuple(r["counts"]) == (nkeys + n0, nvals + n0)
        # P7: output equals a float64 softmax over E
        kw = dict(t=t, blk_k=K[L:].astype(np.float64), blk_v=V[L:].astype(np.float64)) if T else {}
        out, lse = eval_f64(tr, K, V, q, sel, **kw)
        assert np.abs(r["out"] - out).max() < 2e-5
        assert np.abs(r["lse"] - lse).max() < 2e-5


@pytest.mark.parametrize("chunk", range(8))
def test_exhaustive_64_token_trees(chunk):
    """P4 + P5 + P6 + P7 over every 64-token-or-smaller tree geometry, decode
    and prefill (blocks of 1, 3 and 8 tokens after the 64-token prefix)."""
    for (L, b, lv, (mode, k, p, cap), R, G, T, seed) in _CASES[chunk::8]:
        _check_small_case(L, b, lv, mode, k, p, cap, R, G, T, seed)


def _fan_cases():
    """Trees whose fan above level 1 differs from the chunk size of level 1
    (ZHA Figure 4 and Table II name them apart, C and F): every L <= 64 for
    each (C, F) pair, at every depth that leaves a node, selection rule, R, G
    and block length rotated as in the sweep above."""
    cases = []
    i = 0
    for (b, fan) in ((2, 3), (3, 2), (4, 2), (2, 4), (8, 2), (2, 8), (5, 3), (3, 5)):
        variants = [("topk", k, 1.0, 0) for k in (1, 2, 3)] + \
                   [("topp", 0, p, cap) for p in (0.5, 0.9) for cap in (1, 3)]
        for L in range(1, 65):
            maxlv = 0
            n = L // b
            while n >= 1:
                maxlv += 1
                n //= fan
            for lv in range(0, maxlv + 2):
                sv = variants[i % len(variants)]
                R = 1 + (i // 3) % 2
                G = 1 + (i // 5) % 2
                T = (0, 1, 3)[(i // 7) % 3]
                cases.append((L, b, fan, lv, sv, R, G, T, 5000 + i))
                i += 1
    return cases


_FAN_CASES = _fan_cases()


def check_fanout_cases(pred):
    """The fan-out sweep restricted to the (C, F) pairs pred accepts."""
    for (L, b, fan, lv, (mode, k, p, cap), R, G, T, seed) in _FAN_CASES:
        if pred(b, fan):
            _check_small_case(L, b, lv, mode, k, p, cap, R, G, T, seed, fan=fan)


@pytest.mark.parametrize("chunk", range(4))
def test_exhaustive_fanout_trees(chunk):
    """The same checks over trees with a fan F above level 1 other than the
    chunk size C of level 1: the entries still equal the node predicate
    (parents are x // F above level 1, x // C at it), partition the tokens,
    satisfy the per-level certificates and give the float64 softmax."""
    for (L, b, fan, lv, (mode, k, p, cap), R, G, T, seed) in _FAN_CASES[chunk::4]:
        _check_small_case(L, b, lv, mode, k, p, cap, R, G, T, seed, fan=fan)


@pytest.mark.parametrize("L,b,fan,levels,R,d", [(3000, 8, 3, 4, 2, 32), (5000, 3, 16, 2, 2, 16),
                                                (2 * 32 * 4 * 4 + 33, 32, 4, 3, 4, 64)])
def test_pooler_fanout_chains(L, b, fan, levels, R, d):
    """With a fan F above level 1 other than the chunk size C: level 1 pools
    C tokens, every level above pools F nodes of the level below, per
    reference chain -- against the float64 whole-level pooler with the same
    geometry, level by level (a tree that pooled C children at every level
    would not even have the same node counts)."""
    K, V, rng = rand_kv(L, d, seed=L + fan)
    refs = (rng.standard_normal((R, d)) * (1.5 / np.sqrt(d))).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, levels, bf16=False, fan=fan)
    ref = pool_tree_f64(K, V, refs, b, levels, fan=fan)
    n = L // b
    for l in range(levels):
        rk, rv = ref[l]
        assert tr.lk[l].shape[0] == rk.shape[0] == n, (l + 1, tr.lk[l].shape, rk.shape, n)
        scale = max(1.0, float(np.abs(rk).max()))
        assert np.abs(tr.lk[l] - rk).max() < 1e-5 * scale * (l + 1), (l + 1, float(np.abs(tr.lk[l] - rk).max()))
        assert np.abs(tr.lv[l] - rv).max() < 1e-5 * (l + 1)
        n //= fan


# --------------------------------------------------------------------------- P9
@pytest.mark.parametrize("P0,b,levels", [(300, 4, 3), (1000, 8, 2), (76, 2, 5)])
def test_prefill_T1_equals_decode(P0, b, levels):
    assert (P0 + 1) % b != 0
    d, G = 16, 2
    K, V, rng = rand_kv(P0 + 1, d, seed=P0)
    refs = (rng.standard_normal((1, d)) / 4).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    tdec = oracle.build_tree(K, V, refs, b, levels, bf16=False, L=P0 + 1)
    tpre = oracle.build_tree(K, V, refs, b, levels, bf16=False, L=P0)
    for k in (1, 3):
        rd = oracle.query(tdec, K, V, q, k=k)
        rp = oracle.query(tpre, K, V, q, k=k, t=0, blk_k=K[P0:P0 + 1], blk_v=V[P0:P0 + 1])
        assert np.array_equal(rd["sel"], rp["sel"])
        assert np.abs(rd["out"] - rp["out"]).max() < 1e-6


def test_prefill_empty_prefix_is_causal_attention():
    d, G, T = 32, 4, 40
    rng = np.random.default_rng(9)
    bk = rng.standard_normal((T, d)).astype(np.float32)
    bv = rng.standard_normal((T, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    empty = np.zeros((0, d), np.float32)
    tr = oracle.build_tree(empty, empty, np.zeros((1, d), np.float32), 4, 2, bf16=False)
    for t in (0, 5, T - 1):
        r = oracle.query(tr, empty, empty, q, k=2, t=t, blk_k=bk, blk_v=bv)
        ref = dense_causal(q, bk, bv, t)
        assert np.abs(r["out"] - ref).max() < 1e-5


def test_prefill_matches_f64_entry_softmax():
    """Prefill over a real prefix: output equals the float64 softmax over E."""
    P0, T, d, G, b, lv = 2000, 24, 16, 4, 8, 3
    K, V, rng = rand_kv(P0 + T, d, seed=21)
    refs = (rng.standard_normal((2, d)) / 4).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, lv, bf16=False, L=P0)
    q = rng.standard_normal((G, d)).astype(np.float32)
    for t in (0, 11, T - 1):
        r = oracle.query(tr, K, V, q, k=2, t=t, blk_k=K[P0:], blk_v=V[P0:])
        out, lse = eval_f64(tr, K, V, q, sel_sets(r, lv), t=t,
                            blk_k=K[P0:].astype(np.float64), blk_v=V[P0:].astype(np.float64))
        assert np.abs(r["out"] - out).max() < 2e-5


# --------------------------------------------------------------------------- leaf-only dispatch
@pytest.mark.parametrize("mode", ["topk", "topp"])
def test_leaf_only_is_softmax_over_reached_tokens(mode):
    """Leaf-only dispatch (ZHA Figure 3 caption: the union of the reached
    leaves is what the main attention sees): the selection is the one of the
    shared-softmax variant, and the output is the float64 softmax over the
    reached tokens alone (decode and prefill)."""
    L, d, G, b, lv = 3000, 32, 4, 8, 3
    K, V, rng = rand_kv(L + 30, d, seed=31)
    refs = (rng.standard_normal((2, d)) / np.sqrt(d)).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, lv, bf16=False, L=L)
    q = rng.standard_normal((G, d)).astype(np.float32)
    kw = dict(k=3) if mode == "topk" else dict(mode="topp", p=0.7, cap=6)
    ra = oracle.query(tr, K, V, q, **kw)
    rl = oracle.query(tr, K, V, q, leaf_only=True, **kw)
    assert np.array_equal(ra["sel"], rl["sel"])
    out, lse = eval_f64(tr, K, V, q, sel_sets(rl, lv), leaf_only=True)
    assert np.abs(rl["out"] - out).max() < 2e-5 and np.abs(rl["lse"] - lse).max() < 2e-5
    assert not np.allclose(rl["out"], ra["out"], atol=1e-3)     # the summaries did matter
    for t in (0, 17):
        rl = oracle.query(tr, K, V, q, leaf_only=True, t=t, blk_k=K[L:], blk_v=V[L:], **kw)
        out, _ = eval_f64(tr, K, V, q, sel_sets(rl, lv), t=t, leaf_only=True,
                          blk_k=K[L:].astype(np.float64), blk_v=V[L:].astype(np.float64))
        assert np.abs(rl["out"] - out).max() < 2e-5


def test_leaf_only_full_keep_is_dense():
    """Keeping every candidate reaches every token, and with the summaries out
    of the softmax the result is textbook causal attention (P1 for the
    leaf-only variant)."""
    L, d, G, b, lv = 700, 16, 2, 4, 3
    K, V, rng = rand_kv(L, d, seed=5)
    refs = (rng.standard_normal((1, d)) / 4).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, lv, bf16=False)
    q = rng.standard_normal((G, d)).astype(np.float32)
    r = oracle.query(tr, K, V, q, k=256, kmax=256, leaf_only=True)
    assert np.abs(r["out"] - dense_causal(q, K, V, L - 1)).max() < 1e-5


# --------------------------------------------------------------------------- P11 router keys
def _e4m3_torch(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _dequant_torch(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    return v * scales[..., None]


def test_router_fp8_matches_torch_cast():
    """The oracle's E4M3 encoder (nearest of all codes, ties to the even one)
    agrees with torch's float8_e4m3fn conversion of the scaled rows, over rows
    of every magnitude, with subnormal and zero elements; the scale is
    2^(e - 8) for amax = f * 2^e, f in [0.5, 1)."""
    rng = np.random.default_rng(41)
    rows = [rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 6) for _ in range(300)]
    x = rng.standard_normal(64)
    x[::3] *= 1e-4       # elements far below the row maximum: subnormal codes and zeros
    rows.append(x)
    rows.append(np.zeros(128))
    z = np.zeros(128)
    z[5] = -0.0
    z[7] = 3.0
    rows.append(z)
    for r in rows:
        r = r.astype(np.float32)
        codes, sc = oracle.router_fp8(r)
        sc = float(sc)
        amax = float(np.abs(r).max())
        if amax == 0.0:
            assert sc == 1.0
        else:
            m, e = np.frexp(amax)
            assert sc == 2.0 ** (int(e) - 8) and 128.0 <= amax / sc < 256.0
        assert np.array_equal(codes, _e4m3_torch(r / np.float32(sc)))


def test_router_fp8_codes_by_hand():
    """Codes worked out from the E4M3 definition (bias 7, 3 mantissa bits,
    subnormals m/8 * 2^-6): with the row maximum 200 the scale is 1, and
    1.0625 (halfway 1 | 1.125) -> 1.0 = 0x38, 1.1875 (1.125 | 1.25) -> 1.25 =
    0x3A, 2^-9 -> 0x01, 2^-10 (0 | 2^-9) -> 0x00, 3 * 2^-10 (2^-9 | 2^-8) ->
    0x02, -0.0 -> 0x80, 240 -> 0x77, 248 (240 | 256) -> 256 = 0x78, and 200
    (halfway 192 | 208) -> 192 = 0x74 (exponent field 14, mantissa 4), with
    the sign bit 0xF4 for -200."""
    vals = [200.0, 1.0625, 1.1875, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, -0.0, 240.0, 248.0, -200.0]
    want = [0x74, 0x38, 0x3A, 0x01, 0x00, 0x02, 0x80, 0x77, 0x78, 0xF4]
    codes, sc = oracle.router_fp8(np.array(vals, np.float32))
    assert float(sc) == 1.0
    assert [int(c) for c in codes] == want


@pytest.mark.parametrize("R,mode", [(1, "topk"), (2, "topp")])
def test_router_fp8_is_scoring_on_dequantised_keys(R, mode):
    """Routing through the E4M3 copy is the plain method on a tree whose
    summary keys are the dequantised rows (dequantised by torch): identical
    selections and outputs, bit for bit; tokens and values are untouched.
    The float64 shared softmax over that tree agrees, and the copy does
    change the result (the keys are not exactly representable)."""
    L, d, G, b, lv = 2500, 32, 4, 8, 3
    K, V, rng = rand_kv(L + 20, d, seed=43, bf16=True)
    refs = (rng.standard_normal((R, d)) / np.sqrt(d)).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, lv, bf16=True, L=L)
    tq = oracle.build_tree(K, V, refs, b, lv, bf16=True, L=L)
    for l in range(lv):
        codes, sc = oracle.router_fp8(tr.lk[l])
        tq.lk[l][...] = _dequant_torch(codes, sc)
    q = rng.standard_normal((G, d)).astype(np.float32)
    kw = dict(k=3) if mode == "topk" else dict(mode="topp", p=0.8, cap=8)
    for t in (-1, 0, 11):
        pf = dict(t=t, blk_k=K[L:], blk_v=V[L:]) if t >= 0 else {}
        r8 = oracle.query(tr, K, V, q, router_fp8=True, **kw, **pf)
        rq = oracle.query(tq, K, V, q, **kw, **pf)
        assert np.array_equal(r8["sel"], rq["sel"])
        assert np.array_equal(r8["out"], rq["out"]) and np.array_equal(r8["lse"], rq["lse"])
        f64 = dict(t=t, blk_k=K[L:].astype(np.float64), blk_v=V[L:].astype(np.float64)) if t >= 0 else {}
        out, _ = eval_f64(tq, K, V, q, sel_sets(r8, lv), **f64)
        assert np.abs(r8["out"] - out).max() < 2e-5
        r0 = oracle.query(tr, K, V, q, **kw, **pf)
        assert not np.array_equal(r0["out"], r8["out"])


# --------------------------------------------------------------------------- P10
def test_special_cases():
    L, d, b, lv, G = 3000, 32, 8, 3, 2
    K, V, rng = rand_kv(L, d, seed=4)
    r1 = (rng.standard_normal((1, d)) / 4).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    ta = oracle.build_tree(K, V, r1, b, lv, bf16=False)
    tb = oracle.build_tree(K, V, np.repeat(r1, 3, axis=0), b, lv, bf16=False)
    ra = oracle.query(ta, K, V, q, k=3)
    rb = oracle.query(tb, K, V, q, k=3)
    assert np.array_equal(ra["out"], rb["out"]) and np.array_equal(ra["sel"], rb["sel"])
    # top-p with cap 1 is top-1
    rp = oracle.query(ta, K, V, q, mode="topp", p=0.5, cap=1, kmax=1)
    rk = oracle.query(ta, K, V, q, k=1, kmax=1)
    assert np.array_equal(rp["out"], rk["out"]) and np.array_equal(rp["sel"], rk["sel"])


def test_replay():
    """Replaying the oracle's own selection reproduces it; replaying another
    selection equals the float64 evaluation under that selection."""
    L, d, b, lv, G = 5000, 16, 8, 3, 2
    K, V, rng = rand_kv(L, d, seed=8)
    refs = (rng.standard_normal((1, d)) / 4).astype(np.float32)
    tr = oracle.build_tree(K, V, refs, b, lv, bf16=False)
    q = rng.standard_normal((G, d)).astype(np.float32)
    r = oracle.query(tr, K, V, q, k=2)
    rr = oracle.query(tr, K, V, q, k=2, replay=r["sel"])
    assert np.array_equal(r["out"], rr["out"])
    # swap the top-level choice for another node
    alt = r["sel"].copy()
    ntop = L // b ** lv
    other = [x for x in range(ntop) if x not in set(alt[lv - 1])][0]
    alt[lv - 1] = sorted([alt[lv - 1][0], other])
    cand = sorted(alt[lv - 1])
    # descend under the new top choice: pick the first two children each level
    nxt = [c * b for c in cand]
    alt[lv - 2] = sorted(nxt[:2])
    alt[lv - 3] = sorted([alt[lv - 2][0] * b, alt[lv - 2][1] * b])
    ra = oracle.query(tr, K, V, q, k=2, replay=alt)
    out, _ = eval_f64(tr, K, V, q, sel_sets({"sel": alt}, lv))
    assert np.abs(ra["out"] - out).max() < 2e-5
    with pytest.raises(ValueError):
        bad = alt.copy()
        bad[0] = [L // b + 5, -1]          # not a candidate
        oracle.query(tr, K, V, q, k=2, replay=bad)
