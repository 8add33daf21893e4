"""Shared machinery of the GPU parity tests: set up a tree set on the device
through the C ABI, run the oracle on the same inputs, and apply the
acceptance rule.

Acceptance (per query, KV group): walking the levels from the top, while the
GPU and the oracle kept the same node sets so far, the kept set at the next
level must be identical unless the oracle's fp32 score gap at the selection
boundary is <= 1e-3 (top-p additionally: the running sum is within 1e-4 of
p).  At the first such exempt level the comparison of sets stops (the
candidate lists below differ) and the oracle is replayed on the GPU's
selections.  Outputs must then agree within max-abs 1e-5 (fp32 inputs) or
2e-2 (bf16 inputs); lse within the same bound.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import hierarchical_tree_indexed_amd as hti
import oracle

GAP = 1e-3
PMARGIN = 1e-4
TOL = {"f32": 1e-5, "bf16": 2e-2}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_treeset(w, Lcap, K=None, V=None, refs=None, T=0, rope_npos=None, router_fp8=False):
    """TreeSet on cuda:0 for workload w (B, Hq, Hkv, d, b, fan, levels, R, dtype)."""
    sel = select_of(w)
    cfg = hti.make_cfg(w.B, w.Hq, w.Hkv, w.d, w.b, w.levels, w.R, w.dtype, Lcap, w.rope_base, 1,
                       router_fp8=router_fp8, fan=w.fan)
    need = hti.plan(cfg, sel, T).rope_npos_needed
    cfg.rope_npos = max(need, rope_npos or 0)
    ts = hti.TreeSet(cfg, device="cuda", k_cache=K, v_cache=V)
    if refs is not None:
        ts.ref_q.copy_(refs)
    ts.rope_init()
    return ts


def select_of(w, **kw):
    return hti.make_select(w.mode, k=w.k, p=w.p, cap=w.cap, **kw)


def kmax_of(w):
    return w.k if w.mode == "topk" else w.cap


def oracle_tree(w, K_bh, V_bh, refs_h, L):
    return oracle.build_tree(K_bh[:L], V_bh[:L], refs_h, w.b, w.levels, bf16=(w.dtype == "bf16"), L=L, fan=w.F)


def oracle_tree_from_device(ts, w, bi, g, L):
    """The oracle's tree of (sequence bi, KV head g) holding the device's
    stored levels: for checks of the routing on the keys the device holds
    (the build itself is checked against the oracle's own build)."""
    tr = oracle.Tree(L, w.d, w.b, w.levels, w.R, w.dtype == "bf16", fan=w.F)
    for l in range(w.levels):
        n = tr.lk[l].shape[0]
        tr.lk[l][...] = ts.lvl_k[l][bi, g, :n].float().cpu().numpy()
        tr.lv[l][...] = ts.lvl_v[l][bi, g, :n].float().cpu().numpy()
    return tr


def router_copy_matches(ts, w, bi, g, L):
    """The device's 8-bit router copy of (bi, g) equals the oracle's encoding
    of the device's stored keys; returns the number of rows compared."""
    rows = 0
    for l in range(w.levels):
        n = w.level_counts(L)[l + 1]
        codes, sc = oracle.router_fp8(ts.lvl_k[l][bi, g, :n].float().cpu().numpy())
        assert np.array_equal(ts.lvl_kq[l][bi, g, :n].cpu().numpy(), codes), f"level {l + 1} codes"
        assert np.array_equal(ts.lvl_ks[l][bi, g, :n].cpu().numpy(), sc), f"level {l + 1} scales"
        rows += n * w.R
    return rows


def accept(w, tree, K_bh, V_bh, q_g, gout, glse, gsel, *, t=-1, blk_k=None, blk_v=None, leaf_only=False,
           router_fp8=False):
    """Apply the acceptance rule to one (query, group). Returns (exempt, maxerr)."""
    kw = dict(mode=w.mode, k=w.k, p=w.p, cap=w.cap, rope_base=w.rope_base, kmax=kmax_of(w),
              leaf_only=leaf_only, router_fp8=router_fp8)
    if t >= 0:
        kw.update(t=t, blk_k=blk_k, blk_v=blk_v)
    r = oracle.query(tree, K_bh, V_bh, q_g, **kw)
    exempt = False
    for row in range(w.levels - 1, -1, -1):
        gs = sorted(int(x) for x in gsel[row] if x >= 0)
        os_ = sorted(int(x) for x in r["sel"][row] if x >= 0)
        if gs != os_:
            amb = r["gap"][row] <= GAP or r["pmargin"][row] <= PMARGIN
            assert amb, (f"level {row + 1}: gpu kept {gs}, oracle kept {os_}, "
                         f"gap {r['gap'][row]:.3e}, pmargin {r['pmargin'][row]:.3e}")
            exempt = True
            break
    if exempt:
        r = oracle.query(tree, K_bh, V_bh, q_g, replay=np.asarray(gsel), **kw)
    err = float(np.abs(gout - r["out"]).max())
    tol = TOL[w.dtype]
    assert err <= tol, f"output max-abs error {err:.3e} > {tol}"
    lerr = float(np.abs(glse - r["lse"]).max())
    assert lerr <= tol, f"lse max-abs error {lerr:.3e} > {tol}"
    return exempt, err


def tree_close(w, gk, gv, tk, tv, level=1):
    """GPU level arrays vs oracle level arrays (one (seq, head), one level).

    fp32: within 1e-5 relative to the level's largest magnitude.
    bf16: storage rounding of two fp32 values that differ only in summation
    order may land one unit in the last place apart (level 1, whose inputs are
    exact tokens).  A child that differs by one unit moves its parent by at
    most that amount times its weight, so above level 1 the bound grows by one
    child-sized unit per level (absolute, on the level's RMS scale).
    Returns the fraction of bit-identical elements.
    """
    gk, gv = gk.float().cpu().numpy(), gv.float().cpu().numpy()
    if w.dtype == "f32":
        assert np.abs(gk - tk).max() <= 1e-5 * max(1.0, np.abs(tk).max())
        assert np.abs(gv - tv).max() <= 1e-5 * max(1.0, np.abs(tv).max())
        return 1.0
    for g_, t_ in ((gk, tk), (gv, tv)):
        rms = float(np.sqrt(np.mean(t_.astype(np.float64) ** 2))) if t_.size else 0.0
        bound = 2.0 ** -7 * np.abs(t_) + (level - 1) * 2.0 ** -7 * rms + 1e-7
        bad = np.abs(g_ - t_) > bound
        assert not bad.any(), (f"level {level}: {int(bad.sum())} elements beyond the bound, worst "
                               f"{float(np.abs(g_ - t_).max()):.3e} (rms {rms:.3e})")
    return float(np.mean(gk == tk))
