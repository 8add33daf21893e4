"""GPU parity of the 8-bit router keys (ZHA Figure 16: router operands,
reference-key cache and scoring in low precision, KV cache and attention in
bf16): the E4M3 copy every pooling call writes, bit for bit against the
oracle's encoder, and decode (split and unsplit) and prefill routing through
it against the oracle's routing on the same stored keys."""
import numpy as np
import pytest
import torch

import hti_workloads as W
import oracle
from gpu_helpers import accept, kmax_of, log, make_treeset, oracle_tree_from_device, select_of

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    W.DEC128K.replace(name="r8_b32_g4", L=40000 + 17, B=2, Hq=8, Hkv=2, needles=0, Nq=2),
    W.ZHA2M.replace(name="r8_topp_r4_b16", L=70000 + 5, levels=4, Nq=2),
    W.DEC128K.replace(name="r8_d64_b3_g1", d=64, b=3, levels=6, L=3000, Hq=4, Hkv=4, k=4, needles=0, Nq=2),
    # chunk 16 at level 1, fan 4 above
    W.DEC128K.replace(name="r8_c16_f4", b=16, fan=4, levels=3, L=16 * 4 * 4 * 6 + 21, B=2, Hq=8, Hkv=2,
                      needles=0, Nq=2),
]


def _setup(w, Lcap=None, Ls=None):
    Lcap = Lcap or w.L
    K, V = W.gen_kv(w, Lcap=Lcap)
    refs = W.gen_refs(w)
    ts = make_treeset(w, Lcap, K.to(DEV), V.to(DEV), refs.to(DEV), router_fp8=True)
    Ls = Ls or [w.L] * w.B
    ts.tree_build(Ls)
    torch.cuda.synchronize()
    return ts, K, V, refs, Ls


def _check_copy(ts, w, Ls):
    """lvl_kq / lvl_ks of every full node equal the oracle's encoding of the
    stored (bf16) key rows."""
    nodes = 0
    for l in range(w.levels):
        kq = ts.lvl_kq[l].cpu().numpy()
        ks = ts.lvl_ks[l].cpu().numpy()
        lk = ts.lvl_k[l].float().cpu().numpy()
        for bi in range(w.B):
            n = w.level_counts(Ls[bi])[l + 1]
            if n == 0:
                continue
            codes, sc = oracle.router_fp8(lk[bi, :, :n])
            assert np.array_equal(kq[bi, :, :n], codes), f"level {l + 1}: codes differ"
            assert np.array_equal(ks[bi, :, :n], sc), f"level {l + 1}: scales differ"
            nodes += n * w.Hkv
    return nodes


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_router_copy_matches_oracle(w):
    log(f"router copy {w.name}: build, append, extend")
    Lcap = w.L + 3 * w.b ** 2 + 40
    Ls = [w.L - 7 * bi for bi in range(w.B)]
    ts, K, V, refs, Ls = _setup(w, Lcap=Lcap, Ls=Ls)
    nodes = _check_copy(ts, w, Ls)
    # appends that complete nodes, then a block that completes more
    for i in range(w.b + 1):
        kn, vn = W.gen_append(w, i)
        ts.tree_append(kn.to(DEV).contiguous(), vn.to(DEV).contiguous())
    T = 2 * w.b ** 2 + 5
    blk = torch.randn((w.B, T, w.Hkv, w.d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    ts.tree_extend(blk.to(DEV).contiguous(), blk.flip(1).to(DEV).contiguous())
    torch.cuda.synchronize()
    L1 = ts.len.cpu().tolist()
    assert L1 == [min(x + w.b + 1 + T, Lcap) for x in Ls]
    nodes1 = _check_copy(ts, w, L1)
    log(f"  {nodes} nodes after the build, {nodes1} after append + extend: identical")


def _decode(ts, w, q, split):
    out = torch.empty((w.B, q.shape[1], w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, q.shape[1], w.Hq), dtype=torch.float32, device=DEV)
    sel = torch.empty((w.B, q.shape[1], w.Hkv, max(w.levels, 1), kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_decode(select_of(w), q.to(DEV).contiguous(), out, lse, sel, split=split)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_decode_router_fp8(w, split):
    ts, K, V, refs, Ls = _setup(w)
    q = W.gen_queries(w)
    out, lse, sel = _decode(ts, w, q, split)
    nex, emax, e0 = 0, 0.0, 0.0
    for bi in range(w.B):
        for g in range(w.Hkv):
            tr = oracle_tree_from_device(ts, w, bi, g, Ls[bi])
            for qi in range(q.shape[1]):
                hs = slice(g * w.G, (g + 1) * w.G)
                Kb, Vb = K[bi, g, : Ls[bi]], V[bi, g, : Ls[bi]]
                ex, err = accept(w, tr, Kb, Vb, q[bi, qi, hs], out[bi, qi, hs], lse[bi, qi, hs],
                                 sel[bi, qi, g], router_fp8=True)
                nex += ex
                emax = max(emax, err)
                r0 = oracle.query(tr, Kb, Vb, q[bi, qi, hs], mode=w.mode, k=w.k, p=w.p, cap=w.cap,
                                  kmax=kmax_of(w))
                e0 = max(e0, float(np.abs(r0["out"] - out[bi, qi, hs]).max()))
    log(f"  {w.name} split={split}: exempt={nex} max_err={emax:.2e} (vs routing on the bf16 keys {e0:.2e})")
    assert emax < e0     # the 8-bit keys were used


@pytest.mark.parametrize("Hq,Hkv,R,k,levels,P0,T,d", [(32, 8, 1, 8, 2, 32 * 32 * 12 + 70, 70, 128),
                                                      (16, 8, 2, 8, 2, 32 * 32 * 5 + 31, 40, 128),
                                                      (32, 8, 1, 8, 3, 32 * 32 * 3 + 9, 33, 128),
                                                      (8, 2, 2, 4, 2, 32 * 32 * 9 + 17, 50, 64)])
def test_prefill_router_fp8(Hq, Hkv, R, k, levels, P0, T, d):
    """Summary levels scored through the 8-bit copy in the prefill walk and in
    the matrix-core scoring of the top level (d = 128 and 64)."""
    w = W.PREFILL.replace(name="r8_pf", Hq=Hq, Hkv=Hkv, R=R, k=k, levels=levels, L=P0, T=T, d=d)
    K, V = W.gen_kv(w, Lcap=P0)
    refs = W.gen_refs(w)
    ts = make_treeset(w, P0, K.to(DEV), V.to(DEV), refs.to(DEV), T=T, router_fp8=True)
    ts.tree_build([P0] * w.B)
    qb, kb, vb = W.gen_block(w)
    sel = select_of(w)
    ws = torch.empty(ts.prefill_workspace_bytes(sel, T), dtype=torch.uint8, device=DEV)
    out = torch.empty((w.B, T, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, T, w.Hq), dtype=torch.float32, device=DEV)
    so = torch.empty((w.B, T, w.Hkv, max(w.levels, 1), kmax_of(w)), dtype=torch.int32, device=DEV)
    ts.sparse_prefill(sel, qb.to(DEV).contiguous(), kb.to(DEV).contiguous(), vb.to(DEV).contiguous(),
                      out, ws, lse, so)
    torch.cuda.synchronize()
    out, lse, so = out.cpu().numpy(), lse.cpu().numpy(), so.cpu().numpy()
    nex, emax = 0, 0.0
    for bi in range(w.B):
        for g in range(w.Hkv):
            tr = oracle_tree_from_device(ts, w, bi, g, P0)
            bk = kb[bi, :, g].float().numpy()
            bv = vb[bi, :, g].float().numpy()
            for t in range(0, T, 3):
                hs = slice(g * w.G, (g + 1) * w.G)
                ex, err = accept(w, tr, K[bi, g, :P0], V[bi, g, :P0], qb[bi, t, hs], out[bi, t, hs],
                                 lse[bi, t, hs], so[bi, t, g], t=t, blk_k=bk, blk_v=bv, router_fp8=True)
                nex += ex
                emax = max(emax, err)
    log(f"  prefill router_fp8 P0={P0} T={T} R={R}: exempt={nex} max_err={emax:.2e}")
