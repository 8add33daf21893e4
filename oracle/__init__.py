"""CPU oracle of tree-indexed recursive sparse attention -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The product library never imports it, and this package never
imports the product library: the two share no code.

The arithmetic lives in ``hti_oracle.c`` (plain C, fp32, sequential sums,
compiled by gcc without contraction or fast-math).  This module compiles it
on demand and marshals numpy arrays.  See the C file's header for the page
passages each step follows and the readings taken where the pages are silent.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hti_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "libhti_oracle.so")
MAXLVL = 32


def compile_oracle(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    os.makedirs(_OUT_DIR, exist_ok=True)
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-Wall", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _QArgs(C.Structure):
    _fields_ = [("d", C.c_int), ("b", C.c_int), ("fan", C.c_int), ("levels", C.c_int), ("R", C.c_int),
                ("G", C.c_int), ("mode", C.c_int), ("k", C.c_int), ("cap", C.c_int),
                ("p", C.c_float), ("rope_base", C.c_double), ("Ltree", C.c_long),
                ("qpos", C.c_long), ("t", C.c_long),
                ("K", C.c_void_p), ("V", C.c_void_p),
                ("lvl_k", C.c_void_p), ("lvl_v", C.c_void_p),
                ("blk_k", C.c_void_p), ("blk_v", C.c_void_p),
                ("q", C.c_void_p), ("replay", C.c_void_p), ("kmax", C.c_int), ("leaf_only", C.c_int),
                ("router_fp8", C.c_int)]


class _QOut(C.Structure):
    _fields_ = [("out", C.c_void_p), ("lse", C.c_void_p), ("sel", C.c_void_p),
                ("gap", C.c_void_p), ("pmargin", C.c_void_p), ("counts", C.c_void_p),
                ("ent_level", C.c_void_p), ("ent_node", C.c_void_p), ("ent_pos", C.c_void_p),
                ("ent_cap", C.c_long), ("n_ent", C.c_long)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        _lib = _open(compile_oracle(force=False))
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Route every call through another build of the oracle source for the
    duration of the block (the mutation tests compile altered copies of
    hti_oracle.c to show that a planted mistake turns a pin red)."""
    global _lib
    saved = _lib
    _lib = _open(path)
    try:
        yield
    finally:
        _lib = saved


def _open(path: str):
    lib = C.CDLL(path)
    lib.orc_build.restype = C.c_int
    lib.orc_build.argtypes = [C.c_long, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                              C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.orc_query.restype = C.c_int
    lib.orc_query.argtypes = [C.POINTER(_QArgs), C.POINTER(_QOut)]
    lib.orc_router_fp8.restype = None
    lib.orc_router_fp8.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]
    return lib


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().float().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _ptr_array(arrs):
    n = max(len(arrs), 1)
    pa = (C.c_void_p * n)()
    for i, a in enumerate(arrs):
        pa[i] = a.ctypes.data
    return pa


class Tree:
    """Levels 1..levels of one (sequence, KV head): keys [n_l, R, d], values [n_l, d].
    b tokens per level-1 node (the chunk size C), fan nodes per node above
    (the fan F; None: fan = b)."""

    def __init__(self, L, d, b, levels, R, bf16, fan=None):
        fan = b if fan is None else fan
        self.L, self.d, self.b, self.fan, self.levels, self.R, self.bf16 = L, d, b, fan, levels, R, bf16
        self.lk, self.lv = [], []
        n = L
        for lvl in range(1, levels + 1):
            n //= b if lvl == 1 else fan
            self.lk.append(np.zeros((n, R, d), np.float32))
            self.lv.append(np.zeros((n, d), np.float32))


def build_tree(K, V, refs, b: int, levels: int, bf16: bool, L: int | None = None, fan: int | None = None) -> Tree:
    """Tree over the first L tokens of K, V ([*, d]); refs [R, d]; b tokens
    per level-1 node, fan nodes per node above (None: fan = b)."""
    K, V, refs = _f32(K), _f32(V), _f32(refs)
    L = K.shape[0] if L is None else L
    d = K.shape[1]
    R = refs.shape[0]
    fan = b if fan is None else fan
    assert levels <= MAXLVL and b >= 2 and fan >= 2
    tr = Tree(L, d, b, levels, R, bf16, fan)
    lk, lv = _ptr_array(tr.lk), _ptr_array(tr.lv)
    tr._keep = (K, V)
    _load().orc_build(L, d, b, fan, levels, R, int(bf16), _ptr(K), _ptr(V), _ptr(refs), lk, lv)
    return tr


def router_fp8(rows):
    """E4M3 router copy of key rows [..., d]: (codes uint8 [..., d], scales fp32 [...])."""
    rows = _f32(rows)
    d = rows.shape[-1]
    flat = rows.reshape(-1, d)
    codes = np.zeros(flat.shape, np.uint8)
    scales = np.zeros(flat.shape[0], np.float32)
    lib = _load()
    for i in range(flat.shape[0]):
        lib.orc_router_fp8(_ptr(flat[i]), d, codes[i].ctypes.data, scales[i:].ctypes.data)
    return codes.reshape(rows.shape), scales.reshape(rows.shape[:-1])


def query(tree: Tree, K, V, q, *, mode="topk", k=8, p=1.0, cap=16, rope_base=10000.0,
          qpos: int | None = None, t: int = -1, blk_k=None, blk_v=None, replay=None,
          kmax: int | None = None, entries: bool = False, leaf_only: bool = False,
          router_fp8: bool = False):
    """One query token (G heads of one KV group) over one tree.

    Decode: t = -1, query at qpos (default tree.L - 1).
    Prefill: t >= 0 is the query's index in the block blk_k/blk_v ([T, d]).
    replay: [levels, kmax] int array of selected node ids per level (row l-1 =
    level l), ascending, -1 padded.
    Returns a dict with out [G, d], lse [G], sel [levels, kmax], gap [levels],
    pmargin [levels], counts (keys, values) and optionally the entry list.
    """
    K, V, q = _f32(K), _f32(V), _f32(q)
    G, d = q.shape
    if kmax is None:
        kmax = k if mode == "topk" else cap
    a = _QArgs()
    a.d, a.b, a.fan, a.levels, a.R, a.G = d, tree.b, tree.fan, tree.levels, tree.R, G
    a.mode = 0 if mode == "topk" else 1
    a.k, a.cap, a.p, a.rope_base = k, cap, p, rope_base
    a.Ltree = tree.L
    a.qpos = (tree.L - 1) if (qpos is None and t < 0) else (-1 if qpos is None else qpos)
    a.t = t
    a.K, a.V = _ptr(K), _ptr(V)
    lk = _ptr_array([x.reshape(-1) for x in tree.lk])
    lv = _ptr_array([x.reshape(-1) for x in tree.lv])
    a.lvl_k = C.cast(lk, C.c_void_p)
    a.lvl_v = C.cast(lv, C.c_void_p)
    bk = _f32(blk_k) if blk_k is not None else None
    bv = _f32(blk_v) if blk_v is not None else None
    a.blk_k, a.blk_v = _ptr(bk), _ptr(bv)
    a.q = _ptr(q)
    rp = None
    if replay is not None:
        rp = np.ascontiguousarray(replay, dtype=np.int32).reshape(tree.levels, kmax)
    a.replay = _ptr(rp)
    a.kmax = kmax
    a.leaf_only = 1 if leaf_only else 0
    a.router_fp8 = 1 if router_fp8 else 0

    L = tree.levels
    res = dict(out=np.zeros((G, d), np.float32), lse=np.zeros(G, np.float32),
               sel=np.full((max(L, 1), kmax), -1, np.int32), gap=np.zeros(max(L, 1), np.float32),
               pmargin=np.zeros(max(L, 1), np.float32), counts=np.zeros(2, np.int64))
    o = _QOut()
    o.out, o.lse, o.sel = _ptr(res["out"]), _ptr(res["lse"]), _ptr(res["sel"])
    o.gap, o.pmargin, o.counts = _ptr(res["gap"]), _ptr(res["pmargin"]), _ptr(res["counts"])
    if entries:
        cap_e = tree.L + (0 if blk_k is None else len(blk_k)) + 16
        el, en, ep = np.zeros(cap_e, np.int32), np.zeros(cap_e, np.int64), np.zeros(cap_e, np.int64)
        o.ent_level, o.ent_node, o.ent_pos, o.ent_cap = _ptr(el), _ptr(en), _ptr(ep), cap_e
    st = _load().orc_query(C.byref(a), C.byref(o))
    if st != 0:
        raise ValueError("oracle: malformed replay selection")
    if entries:
        n = o.n_ent
        assert n <= cap_e
        res["entries"] = (el[:n].copy(), en[:n].copy(), ep[:n].copy())
    res["sel"] = res["sel"][:L]
    res["gap"] = res["gap"][:L]
    res["pmargin"] = res["pmargin"][:L]
    return res
