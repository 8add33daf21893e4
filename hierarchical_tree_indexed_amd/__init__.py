"""Tree-indexed recursive sparse attention on MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/hti.h`` (libhti.so built from
``csrc/``).  This module only marshals arguments: torch tensors provide device
memory and the current HIP stream, every step of the method runs in the
library's kernels.  There is no fallback: if the library is missing, importing
the binding's entry points raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhti.so")

MAX_LEVELS = 12
MAX_SELECT = 32
MAX_CAND = 1024
MAX_R = 8
F32, BF16 = 0, 1
TOPK, TOPP = 0, 1

STATUS = {0: "HTI_OK", -1: "HTI_ERR_INVALID_ARG", -2: "HTI_ERR_UNSUPPORTED",
          -3: "HTI_ERR_CAPACITY", -4: "HTI_ERR_WORKSPACE", -5: "HTI_ERR_LAUNCH", -6: "HTI_ERR_TIMEOUT"}

EXPORTS = ["hti_plan", "hti_rope_init", "hti_tree_build", "hti_tree_append", "hti_tree_extend",
           "hti_decode_workspace_bytes", "hti_sparse_decode", "hti_sparse_decode_static",
           "hti_decode_status", "hti_decode_step",
           "hti_prefill_workspace_bytes", "hti_sparse_prefill", "hti_last_error"]


class TreeCfg(C.Structure):
    _fields_ = [("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("d", C.c_int32),
                ("b", C.c_int32), ("levels", C.c_int32), ("R", C.c_int32), ("dtype", C.c_int32),
                ("Lcap", C.c_int64), ("rope_base", C.c_float), ("rope_npos", C.c_int32),
                ("router_fp8", C.c_int32), ("fan", C.c_int32)]


class Tree(C.Structure):
    _fields_ = [("cfg", TreeCfg), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p),
                ("lvl_k", C.c_void_p * MAX_LEVELS), ("lvl_v", C.c_void_p * MAX_LEVELS),
                ("ref_q", C.c_void_p), ("len", C.c_void_p), ("rope", C.c_void_p),
                ("lvl_kq", C.c_void_p * MAX_LEVELS), ("lvl_ks", C.c_void_p * MAX_LEVELS)]


class Select(C.Structure):
    _fields_ = [("mode", C.c_int32), ("k", C.c_int32), ("p", C.c_float), ("cap", C.c_int32),
                ("per_head", C.c_int32), ("leaf_only", C.c_int32), ("token_nodes", C.c_int32)]


class PlanOut(C.Structure):
    _fields_ = [("ncap", C.c_int64 * (MAX_LEVELS + 1)), ("cache_bytes", C.c_size_t),
                ("lvl_k_bytes", C.c_size_t * MAX_LEVELS), ("lvl_v_bytes", C.c_size_t * MAX_LEVELS),
                ("rope_bytes", C.c_size_t), ("rope_npos_needed", C.c_int32),
                ("lvl_kq_bytes", C.c_size_t * MAX_LEVELS), ("lvl_ks_bytes", C.c_size_t * MAX_LEVELS)]


class HTIError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python hierarchical_tree_indexed_amd/build.py`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        sig = {
            "hti_plan": (C.c_int, [vp, vp, i32, vp]),
            "hti_rope_init": (C.c_int, [vp, vp]),
            "hti_tree_build": (C.c_int, [vp, vp, vp]),
            "hti_tree_append": (C.c_int, [vp, vp, vp, vp]),
            "hti_tree_extend": (C.c_int, [vp, vp, vp, i32, vp]),
            "hti_decode_workspace_bytes": (C.c_size_t, [vp, vp, i32]),
            "hti_sparse_decode": (C.c_int, [vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, C.c_size_t, vp]),
            "hti_sparse_decode_static": (C.c_int, [vp, vp, vp, vp, i32, vp, vp, vp, i32, vp]),
            "hti_decode_status": (C.c_int, [vp, C.c_size_t, vp]),
            "hti_decode_step": (C.c_int, [vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, C.c_size_t, vp]),
            "hti_prefill_workspace_bytes": (C.c_size_t, [vp, vp, i32]),
            "hti_sparse_prefill": (C.c_int, [vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp,
                                             C.c_size_t, vp]),
            "hti_last_error": (C.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().hti_last_error().decode()


def _check(st: int):
    if st != 0:
        raise HTIError(st, last_error())


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_select(mode: str = "topk", k: int = 8, p: float = 1.0, cap: int = 16,
                per_head: bool = False, leaf_only: bool = False, token_nodes: bool = False) -> Select:
    """Selection rule; per_head: every query head routes on its own instead of
    its KV group sharing one selection; leaf_only: only the reached tokens are
    attended (the summaries route but do not join the softmax); token_nodes
    (prefill): the prefix token level runs node-inverted (queries grouped by
    kept level-1 node) instead of every query gathering its own token rows."""
    return Select(TOPK if mode == "topk" else TOPP, k, p, cap, 1 if per_head else 0,
                  1 if leaf_only else 0, 1 if token_nodes else 0)


def make_cfg(B, Hq, Hkv, d, b, levels, R, dtype, Lcap, rope_base=10000.0, rope_npos=1,
             router_fp8=False, fan=0) -> TreeCfg:
    """b: tokens per level-1 node (chunk size); fan: children per node above
    level 1 (0: b)."""
    return TreeCfg(B, Hq, Hkv, d, b, levels, R, F32 if dtype in ("f32", F32) else BF16,
                   Lcap, rope_base, rope_npos, int(router_fp8), int(fan))


def plan(cfg: TreeCfg, sel: Select | None = None, T: int = 0) -> PlanOut:
    out = PlanOut()
    _check(lib().hti_plan(C.byref(cfg), None if sel is None else C.byref(sel), T, C.byref(out)))
    return out


class TreeSet:
    """Device buffers of one layer's trees (B sequences x Hkv heads).

    Allocation goes through torch; the layout and sizes come from hti_plan.
    """

    def __init__(self, cfg: TreeCfg, device="cuda", k_cache=None, v_cache=None):
        self.cfg = cfg
        p = plan(cfg)
        self.plan = p
        tdt = torch.float32 if cfg.dtype == F32 else torch.bfloat16
        shape = (cfg.B, cfg.Hkv, cfg.Lcap, cfg.d)
        self.k_cache = k_cache if k_cache is not None else torch.zeros(shape, dtype=tdt, device=device)
        self.v_cache = v_cache if v_cache is not None else torch.zeros(shape, dtype=tdt, device=device)
        assert tuple(self.k_cache.shape) == shape and self.k_cache.dtype == tdt
        assert self.k_cache.is_contiguous() and self.v_cache.is_contiguous()
        self.lvl_k, self.lvl_v = [], []
        for l in range(1, cfg.levels + 1):
            n = p.ncap[l]
            self.lvl_k.append(torch.zeros((cfg.B, cfg.Hkv, n, cfg.R, cfg.d), dtype=tdt, device=device))
            self.lvl_v.append(torch.zeros((cfg.B, cfg.Hkv, n, cfg.d), dtype=tdt, device=device))
        # 8-bit router copies of the summary keys (E4M3 codes and row scales)
        self.lvl_kq, self.lvl_ks = [], []
        if cfg.router_fp8:
            for l in range(1, cfg.levels + 1):
                n = p.ncap[l]
                self.lvl_kq.append(torch.zeros((cfg.B, cfg.Hkv, n, cfg.R, cfg.d), dtype=torch.uint8, device=device))
                self.lvl_ks.append(torch.zeros((cfg.B, cfg.Hkv, n, cfg.R), dtype=torch.float32, device=device))
        self.ref_q = torch.zeros((cfg.Hkv, cfg.R, cfg.d), dtype=torch.float32, device=device)
        self.len = torch.zeros(cfg.B, dtype=torch.int64, device=device)
        self.rope = torch.zeros((cfg.rope_npos, cfg.d // 2, 2), dtype=torch.float32, device=device)
        self._dec_ws = {}
        self._refresh()

    def _refresh(self):
        t = Tree()
        t.cfg = self.cfg
        t.k_cache, t.v_cache = _ptr(self.k_cache), _ptr(self.v_cache)
        for i, (k, v) in enumerate(zip(self.lvl_k, self.lvl_v)):
            t.lvl_k[i], t.lvl_v[i] = _ptr(k), _ptr(v)
        for i, (kq, ks) in enumerate(zip(self.lvl_kq, self.lvl_ks)):
            t.lvl_kq[i], t.lvl_ks[i] = _ptr(kq), _ptr(ks)
        t.ref_q, t.len, t.rope = _ptr(self.ref_q), _ptr(self.len), _ptr(self.rope)
        self.c = t

    # ---- entry points (same names as the C ABI) ----
    def rope_init(self, stream=None):
        _check(lib().hti_rope_init(C.byref(self.c), _stream(stream)))

    def tree_build(self, L, stream=None):
        Ls = (C.c_int64 * self.cfg.B)(*([L] * self.cfg.B if isinstance(L, int) else list(L)))
        _check(lib().hti_tree_build(C.byref(self.c), Ls, _stream(stream)))

    def tree_append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        _check(lib().hti_tree_append(C.byref(self.c), _ptr(k_new), _ptr(v_new), _stream(stream)))

    def tree_extend(self, k_blk: torch.Tensor, v_blk: torch.Tensor, stream=None):
        """Append a block [B, T, Hkv, d] to every sequence and build the nodes it completes."""
        assert k_blk.shape == v_blk.shape and k_blk.dim() == 4 and k_blk.is_contiguous() and v_blk.is_contiguous()
        _check(lib().hti_tree_extend(C.byref(self.c), _ptr(k_blk), _ptr(v_blk), int(k_blk.shape[1]),
                                     _stream(stream)))

    def decode_workspace(self, sel: Select, Nq: int) -> torch.Tensor:
        """Zero-filled decode workspace for Nq queries per sequence (kept and
        reused by every decode call of that shape and routing)."""
        key = (Nq, int(sel.per_head))
        ws = self._dec_ws.get(key)
        if ws is None:
            n = lib().hti_decode_workspace_bytes(C.byref(self.cfg), C.byref(sel), Nq)
            ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=self.k_cache.device)
            self._dec_ws[key] = ws
        return ws

    def sparse_decode(self, sel: Select, q: torch.Tensor, out: torch.Tensor, lse=None,
                      sel_out=None, stream=None, split: bool = True, q_pos: torch.Tensor | None = None):
        """q_pos: [B, Nq] int64 query positions (None: every query at len - 1)."""
        B, Nq, Hq, d = q.shape
        assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        if q_pos is not None:
            assert q_pos.dtype == torch.int64 and q_pos.is_contiguous() and tuple(q_pos.shape) == (B, Nq)
        stride = 0 if sel_out is None else sel_out.shape[-1]
        ws = self.decode_workspace(sel, Nq) if split else None
        nbytes = 0 if ws is None else ws.numel()
        _check(lib().hti_sparse_decode(C.byref(self.c), C.byref(sel), _ptr(q), _ptr(q_pos), Nq, _ptr(out),
                                       _ptr(lse), _ptr(sel_out), stride, _ptr(ws), nbytes,
                                       _stream(stream)))

    def sparse_decode_static(self, sel: Select, q: torch.Tensor, out: torch.Tensor, lse=None,
                             sel_out=None, stream=None, q_pos: torch.Tensor | None = None):
        """sparse_decode whose split workspace is the library's static device
        array (no allocation); calls on one GPU must not overlap."""
        B, Nq, Hq, d = q.shape
        assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        if q_pos is not None:
            assert q_pos.dtype == torch.int64 and q_pos.is_contiguous() and tuple(q_pos.shape) == (B, Nq)
        stride = 0 if sel_out is None else sel_out.shape[-1]
        _check(lib().hti_sparse_decode_static(C.byref(self.c), C.byref(sel), _ptr(q), _ptr(q_pos), Nq,
                                              _ptr(out), _ptr(lse), _ptr(sel_out), stride, _stream(stream)))

    def decode_status(self, sel: Select, Nq: int, stream=None):
        """Raise HTIError(HTI_ERR_TIMEOUT) if a split decode with this shape's
        workspace ran out of a wait (synchronises the stream)."""
        ws = self.decode_workspace(sel, Nq)
        _check(lib().hti_decode_status(_ptr(ws), ws.numel(), _stream(stream)))

    def decode_step(self, sel: Select, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                    out: torch.Tensor, lse=None, sel_out=None, stream=None, split: bool = True):
        """tree_append(k_new, v_new) followed by sparse_decode(q), in one launch
        where the split kernel applies."""
        B, Nq, Hq, d = q.shape
        assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        assert k_new.is_contiguous() and v_new.is_contiguous()
        stride = 0 if sel_out is None else sel_out.shape[-1]
        ws = self.decode_workspace(sel, Nq) if split else None
        nbytes = 0 if ws is None else ws.numel()
        _check(lib().hti_decode_step(C.byref(self.c), C.byref(sel), _ptr(k_new), _ptr(v_new), _ptr(q), Nq,
                                     _ptr(out), _ptr(lse), _ptr(sel_out), stride, _ptr(ws), nbytes,
                                     _stream(stream)))

    def prefill_workspace_bytes(self, sel: Select, T: int) -> int:
        return lib().hti_prefill_workspace_bytes(C.byref(self.cfg), C.byref(sel), T)

    def sparse_prefill(self, sel: Select, q, k, v, out, ws, lse=None, sel_out=None, stream=None):
        B, T, Hq, d = q.shape
        for x in (q, k, v, out, ws):
            assert x.is_contiguous()
        stride = 0 if sel_out is None else sel_out.shape[-1]
        _check(lib().hti_sparse_prefill(C.byref(self.c), C.byref(sel), _ptr(q), _ptr(k), _ptr(v),
                                        T, _ptr(out), _ptr(lse), _ptr(sel_out), stride, _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))
