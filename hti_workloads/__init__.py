"""Workload definitions and seeded synthetic input generators.

This module holds no arithmetic of the method: it only names the five
workloads (sizes, branching, selection rule) and draws seeded N(0,1) inputs
for them.  Both the CPU oracle's tests and the HIP path's tests and benchmark
take their inputs from here, so the two sides always see the same tensors.

Recipe (every tensor has its own derived random stream, so changing one
workload knob never shifts another tensor's values):
  * K, V caches: i.i.d. N(0,1) drawn in fp32, rounded round-to-nearest-even to
    the workload's dtype, layout [B, Hkv, Lcap, d], keys stored un-rotated;
  * reference queries r: N(0,1)/sqrt(d), fp32, layout [Hkv, R, d];
  * decode queries: i.i.d. N(0,1) in the workload dtype, layout [B, Nq, Hq, d];
  * needles: at `needles` positions drawn uniformly without replacement from
    [0, L), the key of KV head g is replaced by 4 * u_g, u_g the unit vector of
    the mean of the group's query vectors (a diagnostic of retrieval only);
  * appended tokens (decode loop): N(0,1) k, v per step, [B, Hkv, d];
  * prefill block: q [B, T, Hq, d], k/v [B, T, Hkv, d], N(0,1).
"""
from __future__ import annotations

import dataclasses
import math

import torch

F32 = "f32"
BF16 = "bf16"

TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}

# random-stream ids
_S_K, _S_V, _S_REF, _S_Q, _S_NEEDLE, _S_APPEND, _S_BQ, _S_BK, _S_BV = range(1, 10)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str
    L: int                 # cached tokens (decode) or prefix length (prefill)
    b: int                 # branching factor
    levels: int            # tree levels above the tokens
    mode: str = "topk"     # "topk" | "topp"
    k: int = 8
    p: float = 1.0
    cap: int = 16
    R: int = 1             # reference queries per KV head
    Nq: int = 1            # decode queries per sequence
    T: int = 0             # prefill block length (0 = decode workload)
    needles: int = 0
    steps: int = 0         # decode loop: appended tokens per sequence
    rope_base: float = 10000.0
    seed: int = 0
    fan: int = 0           # children per node above level 1 (0: b, the chunk size of level 1)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def ref_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def F(self) -> int:
        """Children per node above level 1."""
        return self.fan or self.b

    def level_counts(self, L: int | None = None) -> list[int]:
        """Full-node counts n_0 = L, n_1 = floor(L / b), n_l = floor(n_{l-1} / F)."""
        n = [self.L if L is None else L]
        for lvl in range(1, self.levels + 1):
            n.append(n[-1] // (self.b if lvl == 1 else self.F))
        return n

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, with the sizes the method is measured at.
TINY = Workload("tiny_decode_4k", B=1, Hq=1, Hkv=1, d=64, dtype=F32, L=4096, b=16,
                levels=2, k=4, Nq=16)
DEC128K = Workload("decode_128k", B=1, Hq=32, Hkv=8, d=128, dtype=BF16, L=131072, b=32,
                   levels=3, k=8, Nq=1, needles=8)
DEC1M = Workload("decode_1m_b4", B=4, Hq=32, Hkv=8, d=128, dtype=BF16, L=1048576, b=32,
                 levels=4, k=8, Nq=1, needles=16, steps=256)
PREFILL = Workload("prefill_524k_t8192", B=1, Hq=32, Hkv=8, d=128, dtype=BF16, L=524288,
                   b=32, levels=3, k=8, T=8192)
ZHA2M = Workload("zha_topp_2m_r4", B=1, Hq=8, Hkv=2, d=128, dtype=BF16, L=2097152, b=16,
                 levels=5, mode="topp", p=0.9, cap=16, R=4, Nq=1)

WORKLOADS = {w.name: w for w in (TINY, DEC128K, DEC1M, PREFILL, ZHA2M)}


def _gen(seed: int, stream: int, sub: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1_000_003 + stream) * 1_000_003 + sub) & ((1 << 62) - 1))
    return g


def _randn(shape, gen, device, dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def gen_kv(w: Workload, Lcap: int | None = None, device="cpu"):
    """K, V caches [B, Hkv, Lcap, d]; rows >= L are zero (free capacity)."""
    Lcap = w.L + w.steps if Lcap is None else Lcap
    assert Lcap >= w.L
    dt = TORCH_DTYPE[w.dtype]
    K = torch.zeros((w.B, w.Hkv, Lcap, w.d), dtype=dt, device=device)
    V = torch.zeros_like(K)
    for bi in range(w.B):
        for h in range(w.Hkv):
            sub = bi * 4096 + h
            K[bi, h, : w.L] = _randn((w.L, w.d), _gen(w.seed, _S_K, sub, device), device, dt)
            V[bi, h, : w.L] = _randn((w.L, w.d), _gen(w.seed, _S_V, sub, device), device, dt)
    return K, V


def gen_refs(w: Workload, device="cpu") -> torch.Tensor:
    """Reference queries [Hkv, R, d], fp32, N(0,1)/sqrt(d)."""
    r = torch.randn((w.Hkv, w.R, w.d), generator=_gen(w.seed, _S_REF), dtype=torch.float32)
    return (r * w.ref_scale).to(device)


def gen_queries(w: Workload, step: int = 0, device="cpu") -> torch.Tensor:
    """Decode queries [B, Nq, Hq, d] in the workload dtype."""
    return _randn((w.B, w.Nq, w.Hq, w.d), _gen(w.seed, _S_Q, step), "cpu",
                  TORCH_DTYPE[w.dtype]).to(device)


def needle_positions(w: Workload) -> torch.Tensor:
    """[B, needles] int64 positions, uniform without replacement in [0, L)."""
    out = torch.empty((w.B, w.needles), dtype=torch.int64)
    for bi in range(w.B):
        g = _gen(w.seed, _S_NEEDLE, bi)
        if w.L <= 1 << 24:
            out[bi] = torch.randperm(w.L, generator=g)[: w.needles]
        else:  # pragma: no cover - larger than every workload
            raise ValueError("context too long for needle sampling")
    return out


def plant_needles(w: Workload, K: torch.Tensor, q: torch.Tensor) -> torch.Tensor:
    """Overwrite needle keys in K (in place) with 4 * unit(mean of the group's queries).

    q: [B, Nq, Hq, d] (the first query of each sequence defines the direction).
    Returns the needle positions [B, needles].
    """
    pos = needle_positions(w)
    if w.needles == 0:
        return pos
    for bi in range(w.B):
        qb = q[bi, 0].float().cpu().view(w.Hkv, w.G, w.d).mean(dim=1)       # [Hkv, d]
        u = qb / qb.norm(dim=-1, keepdim=True)
        key = (4.0 * u).to(K.dtype).to(K.device)                             # [Hkv, d]
        idx = pos[bi].to(K.device)
        for h in range(w.Hkv):
            K[bi, h, idx] = key[h]
    return pos


def gen_append(w: Workload, step: int, device="cpu"):
    """One appended token per sequence: k, v [B, Hkv, d]."""
    dt = TORCH_DTYPE[w.dtype]
    k = _randn((w.B, w.Hkv, w.d), _gen(w.seed, _S_APPEND, 2 * step), "cpu", dt)
    v = _randn((w.B, w.Hkv, w.d), _gen(w.seed, _S_APPEND, 2 * step + 1), "cpu", dt)
    return k.to(device), v.to(device)


def gen_block(w: Workload, device="cpu"):
    """Prefill block q [B, T, Hq, d], k, v [B, T, Hkv, d]."""
    dt = TORCH_DTYPE[w.dtype]
    q = _randn((w.B, w.T, w.Hq, w.d), _gen(w.seed, _S_BQ), "cpu", dt)
    k = _randn((w.B, w.T, w.Hkv, w.d), _gen(w.seed, _S_BK), "cpu", dt)
    v = _randn((w.B, w.T, w.Hkv, w.d), _gen(w.seed, _S_BV), "cpu", dt)
    return q.to(device), k.to(device), v.to(device)
