"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/hti.h declares, plans buffers, and rejects bad arguments with the
documented status before touching the device."""
import ctypes as C
import os
import re

import pytest

import hierarchical_tree_indexed_amd as hti

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "hti.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hti_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert set(names) == set(hti.EXPORTS)
    L = hti.lib()
    for n in names:
        assert hasattr(L, n), n


def cfg(**kw):
    base = dict(B=2, Hq=32, Hkv=8, d=128, b=32, levels=3, R=1, dtype="bf16", Lcap=1 << 17,
                rope_base=10000.0, rope_npos=1024)
    base.update(kw)
    return hti.make_cfg(**base)


def test_plan_sizes():
    c = cfg()
    p = hti.plan(c, hti.make_select("topk", k=8))
    assert list(p.ncap[:4]) == [1 << 17, 4096, 128, 4]
    assert p.cache_bytes == 2 * 8 * (1 << 17) * 128 * 2
    assert p.lvl_k_bytes[0] == 2 * 8 * 4096 * 128 * 2
    assert p.lvl_v_bytes[2] == 2 * 8 * 4 * 128 * 2
    # summary level bound 8*32 + 31 = 287 candidates -> query row 287
    assert p.rope_npos_needed == 288
    p2 = hti.plan(cfg(levels=5, b=16, Lcap=1 << 21, R=4, Hq=8, Hkv=2),
                  hti.make_select("topp", p=0.9, cap=16))
    assert p2.rope_npos_needed == 16 * 16 + 15 + 1
    p3 = hti.plan(c, hti.make_select("topk", k=8), T=8192)
    assert p3.rope_npos_needed == 287 + 8192


def test_plan_sizes_with_fan():
    """A fan above level 1 apart from the chunk size: level 1 holds
    floor(Lcap / b) nodes, every level above floor(n / fan); the candidate
    bound of a summary level is k * fan + fan - 1, of the token level
    k * b + b - 1; fan 0 is the chunk size."""
    c = cfg(b=32, levels=4, Lcap=1 << 20)
    c.fan = 8
    p = hti.plan(c, hti.make_select("topk", k=8))
    assert list(p.ncap[:5]) == [1 << 20, 1 << 15, 1 << 12, 1 << 9, 1 << 6]
    assert p.lvl_v_bytes[3] == 2 * 8 * 64 * 128 * 2
    # summary levels: at most 8 * 8 + 7 = 71 candidates (row 71); token level
    # 8 * 32 + 31 = 287 (row 287)
    assert p.rope_npos_needed == 288
    c.fan = 0
    p0 = hti.plan(c, hti.make_select("topk", k=8))
    assert list(p0.ncap[:5]) == [1 << 20, 1 << 15, 1 << 10, 1 << 5, 1]
    c.b, c.fan = 4, 48
    p1 = hti.plan(c, hti.make_select("topk", k=8))
    assert list(p1.ncap[:4]) == [1 << 20, 1 << 18, (1 << 18) // 48, (1 << 18) // 48 // 48]
    # summary bound 8 * 48 + 47 = 431 (row 431)
    assert p1.rope_npos_needed == 432


@pytest.mark.parametrize("fan", [1, 65, -3])
def test_plan_rejects_bad_fan(fan):
    c = cfg()
    c.fan = fan
    out = hti.PlanOut()
    st = hti.lib().hti_plan(C.byref(c), None, 0, C.byref(out))
    assert st == -2, hti.last_error()
    assert "fan" in hti.last_error()


@pytest.mark.parametrize("bad,status", [
    (dict(Hq=30), -1), (dict(Hq=48, Hkv=8), -2), (dict(d=96), -2), (dict(b=1), -2),
    (dict(levels=13), -1), (dict(R=9), -2), (dict(dtype=7), -1), (dict(Lcap=-1), -2),
    (dict(rope_npos=0), -1), (dict(rope_base=0.0), -1),
])
def test_plan_rejects_bad_cfg(bad, status):
    c = cfg(**{k: v for k, v in bad.items() if k != "dtype"})
    if "dtype" in bad:
        c.dtype = bad["dtype"]
    out = hti.PlanOut()
    st = hti.lib().hti_plan(C.byref(c), None, 0, C.byref(out))
    assert st == status, hti.last_error()
    assert hti.last_error()


def _tree_struct(c, fake=0x1000):
    t = hti.Tree()
    t.cfg = c
    t.k_cache = t.v_cache = fake
    for i in range(c.levels):
        t.lvl_k[i] = t.lvl_v[i] = fake
    t.ref_q = t.len = t.rope = fake
    return t


def test_decode_validation_before_launch():
    """Every error path returns before any HIP call (no GPU in this process)."""
    L = hti.lib()
    c = cfg(rope_npos=288)
    t = _tree_struct(c)
    s = hti.make_select("topk", k=8)
    out = C.c_void_p(0x2000)
    # NULL q
    assert L.hti_sparse_decode(C.byref(t), C.byref(s), None, None, 1, out, None, None, 0, None, 0, None) == -1
    # k out of range
    s_bad = hti.make_select("topk", k=33)
    assert L.hti_sparse_decode(C.byref(t), C.byref(s_bad), 0x3000, None, 1, out, None, None, 0, None, 0, None) == -2
    # top-p with p outside (0, 1]
    s_p = hti.make_select("topp", p=1.5, cap=16)
    assert L.hti_sparse_decode(C.byref(t), C.byref(s_p), 0x3000, None, 1, out, None, None, 0, None, 0, None) == -1
    # routing flag other than 0 / 1
    s_r = hti.make_select("topk", k=8)
    s_r.per_head = 2
    assert L.hti_sparse_decode(C.byref(t), C.byref(s_r), 0x3000, None, 1, out, None, None, 0, None, 0, None) == -1
    # per-head routing: the workspace grows with the units (query heads, not KV groups)
    s_h = hti.make_select("topk", k=8, per_head=True)
    assert L.hti_decode_workspace_bytes(C.byref(c), C.byref(s_h), 1) > \
        L.hti_decode_workspace_bytes(C.byref(c), C.byref(s), 1)
    assert L.hti_prefill_workspace_bytes(C.byref(c), C.byref(s_h), 64) >= \
        L.hti_prefill_workspace_bytes(C.byref(c), C.byref(s), 64)
    # RoPE table too short for the reachable positions
    t2 = _tree_struct(cfg(rope_npos=100))
    assert L.hti_sparse_decode(C.byref(t2), C.byref(s), 0x3000, None, 1, out, None, None, 0, None, 0, None) == -3
    # sel_out with too small a stride
    assert L.hti_sparse_decode(C.byref(t), C.byref(s), 0x3000, None, 1, out, None, 0x4000, 4, None, 0, None) == -1
    # a level with more candidates than the kernel's LDS holds
    t3 = _tree_struct(cfg(levels=1, b=32, rope_npos=1 << 16))      # top level 4096 nodes
    assert L.hti_sparse_decode(C.byref(t3), C.byref(s), 0x3000, None, 1, out, None, None, 0, None, 0, None) == -2
    # missing level buffer
    t4 = _tree_struct(c)
    t4.lvl_v[2] = None
    assert L.hti_sparse_decode(C.byref(t4), C.byref(s), 0x3000, None, 1, out, None, None, 0, None, 0, None) == -1
    # workspace given but too small
    assert L.hti_sparse_decode(C.byref(t), C.byref(s), 0x3000, None, 1, out, None, None, 0, 0x5000, 16,
                               None) == -4
    assert L.hti_decode_workspace_bytes(C.byref(c), C.byref(s), 1) > 16
    # Nq < 1
    assert L.hti_sparse_decode(C.byref(t), C.byref(s), 0x3000, None, 0, out, None, None, 0, None, 0, None) == -1
    # status query without a workspace
    assert L.hti_decode_status(None, 0, None) == -1
    assert L.hti_decode_status(0x5000, 2, None) == -1


def test_build_append_prefill_validation():
    L = hti.lib()
    c = cfg(rope_npos=288 + 64)
    t = _tree_struct(c)
    Ls = (C.c_int64 * 2)(10, (1 << 17) + 1)
    assert L.hti_tree_build(C.byref(t), Ls, None) == -3
    assert L.hti_tree_build(C.byref(t), None, None) == -1
    t_noref = _tree_struct(c)
    t_noref.ref_q = None
    Ls_ok = (C.c_int64 * 2)(10, 10)
    assert L.hti_tree_build(C.byref(t_noref), Ls_ok, None) == -1
    assert L.hti_tree_append(C.byref(t), None, 0x10, None) == -1
    assert L.hti_tree_extend(C.byref(t), None, 0x10, 8, None) == -1
    assert L.hti_tree_extend(C.byref(t), 0x10, 0x10, -1, None) == -1
    assert L.hti_tree_extend(C.byref(t_noref), 0x10, 0x10, 8, None) == -1
    s = hti.make_select("topk", k=8)
    need = L.hti_prefill_workspace_bytes(C.byref(c), C.byref(s), 64)
    assert need > 0
    # workspace too small
    assert L.hti_sparse_prefill(C.byref(t), C.byref(s), 0x10, 0x10, 0x10, 64, 0x10, None, None, 0,
                                0x10, need - 1, None) == -4
    # T beyond the RoPE table
    assert L.hti_sparse_prefill(C.byref(t), C.byref(s), 0x10, 0x10, 0x10, 1000, 0x10, None, None, 0,
                                0x10, 1 << 40, None) == -3
    # fp32 prefill is not offered (bf16 matrix cores)
    t32 = _tree_struct(cfg(dtype="f32", rope_npos=288 + 64))
    assert L.hti_sparse_prefill(C.byref(t32), C.byref(s), 0x10, 0x10, 0x10, 64, 0x10, None, None, 0,
                                0x10, 1 << 40, None) == -2
    assert L.hti_sparse_prefill(C.byref(t), C.byref(s), 0x10, 0x10, 0x10, 0, 0x10, None, None, 0,
                                0x10, 1 << 40, None) == -1


def test_router_fp8_cfg_and_buffers():
    """8-bit router keys: planned sizes, bf16 caches only, 0/1 flag, and the
    copies' buffers required before anything is enqueued."""
    L = hti.lib()
    c = cfg(rope_npos=288)
    c.router_fp8 = 1
    p = hti.plan(c, hti.make_select("topk", k=8))
    assert p.lvl_kq_bytes[0] == 2 * 8 * 4096 * 128 and p.lvl_ks_bytes[0] == 2 * 8 * 4096 * 4
    assert hti.plan(cfg(), None).lvl_kq_bytes[0] == 0
    out = hti.PlanOut()
    c_f32 = cfg(rope_npos=288)
    c_f32.router_fp8 = 1
    c_f32.dtype = hti.F32
    assert L.hti_plan(C.byref(c_f32), None, 0, C.byref(out)) == -2
    c_bad = cfg(rope_npos=288)
    c_bad.router_fp8 = 2
    assert L.hti_plan(C.byref(c_bad), None, 0, C.byref(out)) == -1
    # the copies' buffers: missing ones are rejected by every call that needs the tree
    t = _tree_struct(c)
    s = hti.make_select("topk", k=8)
    assert L.hti_sparse_decode(C.byref(t), C.byref(s), 0x3000, None, 1, 0x2000, None, None, 0, None, 0, None) == -1
    Ls = (C.c_int64 * 2)(10, 10)
    assert L.hti_tree_build(C.byref(t), Ls, None) == -1
    assert L.hti_tree_append(C.byref(t), 0x3000, 0x3000, None) == -1
    assert "router" in hti.last_error()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says
    why, before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()
