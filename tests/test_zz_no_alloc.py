"""hti_sparse_decode_static (the decode whose split workspace is the
library's static device array) against hti_sparse_decode with a caller
workspace, both called through the C ABI: the same kernels on the same
inputs, so outputs, log-sum-exps and selections must agree bit for bit.
Three calls in a row -- a larger shape, a smaller one (which must not see the
larger call's leftovers in the shared array), then the larger one again."""
import ctypes as C

import numpy as np
import pytest
import torch

import hierarchical_tree_indexed_amd as hti
import hti_workloads as W
from gpu_helpers import accept, kmax_of, log, make_treeset, oracle_tree, select_of

pytestmark = pytest.mark.gpu

DEV = "cuda"

BIG = W.DEC128K.replace(name="static_big", B=2, L=32 * 32 * 3 + 77, levels=2, needles=0, Nq=2)
SMALL = W.ZHA2M.replace(name="static_small", B=1, L=16 ** 2 * 5 + 9, levels=2, Nq=1)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _setup(w):
    K, V = W.gen_kv(w, Lcap=w.L)
    refs = W.gen_refs(w)
    ts = make_treeset(w, w.L, K.to(DEV), V.to(DEV), refs.to(DEV))
    ts.tree_build([w.L] * w.B)
    q = W.gen_queries(w).to(DEV).contiguous()
    return ts, K, V, refs, q


def _bufs(w):
    out = torch.full((w.B, w.Nq, w.Hq, w.d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((w.B, w.Nq, w.Hq), float("nan"), dtype=torch.float32, device=DEV)
    so = torch.full((w.B, w.Nq, w.Hkv, w.levels, kmax_of(w)), -7, dtype=torch.int32, device=DEV)
    return out, lse, so


def _both(ts, w, q):
    """(static result, workspace result) as numpy triples."""
    lib = hti.lib()
    sel = select_of(w)
    a, b = _bufs(w), _bufs(w)
    st = lib.hti_sparse_decode_static(C.byref(ts.c), C.byref(sel), _ptr(q), None, w.Nq, _ptr(a[0]),
                                      _ptr(a[1]), _ptr(a[2]), a[2].shape[-1], None)
    assert st == 0, lib.hti_last_error()
    ws = ts.decode_workspace(sel, w.Nq)
    ws.zero_()
    st = lib.hti_sparse_decode(C.byref(ts.c), C.byref(sel), _ptr(q), None, w.Nq, _ptr(b[0]), _ptr(b[1]),
                               _ptr(b[2]), b[2].shape[-1], _ptr(ws), ws.numel(), None)
    assert st == 0, lib.hti_last_error()
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in a], [x.cpu().numpy() for x in b]


def _same(w, got, ref):
    for name, x, y in zip(("out", "lse", "sel"), got, ref):
        assert x.shape == y.shape
        if x.dtype == np.float32:
            assert not np.isnan(y).any(), f"{w.name}: {name} of the workspace call has NaN"
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"{w.name}: {name} differs"
        else:
            assert np.array_equal(x, y), f"{w.name}: {name} differs"


def test_static_decode_matches_workspace_decode():
    big = _setup(BIG)
    small = _setup(SMALL)
    for i, (w, (ts, K, V, refs, q)) in enumerate([(BIG, big), (SMALL, small), (BIG, big)]):
        log(f"static decode call {i}: {w.name} B={w.B} Nq={w.Nq} Hkv={w.Hkv} L={w.L}")
        got, ref = _both(ts, w, q)
        _same(w, got, ref)
        if i == 1:
            # the smaller call also meets the oracle (bar of the decode tests)
            out, lse, so = got
            qh = q.cpu()
            for g in range(w.Hkv):
                tree = oracle_tree(w, K[0, g], V[0, g], refs[g], w.L)
                hs = slice(g * w.G, (g + 1) * w.G)
                accept(w, tree, K[0, g], V[0, g], qh[0, 0, hs], out[0, 0, hs], lse[0, 0, hs], so[0, 0, g])


def test_static_decode_rejects_bad_arguments():
    """Argument errors come back before anything runs (no launch)."""
    lib = hti.lib()
    assert lib.hti_sparse_decode_static(None, None, None, None, 1, None, None, None, 0, None) == -1
