"""Seeded random geometries against the oracle: decode (split over
workgroups and one workgroup per unit) and prefill (walked and node-inverted
token level), drawn over branching factors (and, in a second set, fans above
level 1 apart from the chunk size), depths, head groups, head dims,
reference counts, cache dtypes, both selection rules and ragged lengths --
combinations the hand-picked cases do not pair up.  The draws are fixed by
their seeds, so a failure names a reproducible geometry."""
import numpy as np
import pytest

import hti_workloads as W
from test_gpu_parity import _check_decode, _check_prefill, _setup

pytestmark = pytest.mark.gpu


def _draw(rng, i, prefill):
    d = int(rng.choice([64, 128]))
    dtype = "f32" if (not prefill and rng.random() < 0.3) else "bf16"
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3]))
    b = int(rng.integers(2, 33))
    levels = int(rng.integers(1, 4))
    while b ** levels > 40000:
        levels -= 1
    R = int(rng.choice([1, 2, 4]))
    mode = "topk" if rng.random() < 0.6 else "topp"
    k = int(rng.integers(1, 9))
    p = float(rng.choice([0.5, 0.8, 0.95, 1.0]))
    cap = int(rng.integers(1, 17))
    span = b ** levels
    L = int(rng.integers(1, 5)) * span + int(rng.integers(0, span))
    return W.DEC128K.replace(name=f"rnd_{'pf' if prefill else 'dec'}{i}", B=int(rng.integers(1, 3)),
                             Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, L=L, b=b, levels=levels, mode=mode, k=k,
                             p=p, cap=cap, R=R, needles=0, seed=1000 + i)


DECODE_RANDOM = [_draw(np.random.default_rng(7000 + i), i, False) for i in range(32)]
PREFILL_RANDOM = [_draw(np.random.default_rng(9000 + i), i, True) for i in range(16)]


def _draw_fan(rng, i, prefill):
    """A geometry whose fan above level 1 is drawn apart from the chunk size."""
    w = _draw(rng, i, prefill)
    fan = int(rng.integers(2, 33))
    levels = max(2, w.levels)
    while w.b * fan ** (levels - 1) > 40000 and levels > 2:
        levels -= 1
    span = w.b * fan ** (levels - 1)
    L = int(rng.integers(1, 4)) * span + int(rng.integers(0, span))
    return w.replace(name=w.name.replace("rnd_", "rndfan_"), fan=fan, levels=levels, L=L, seed=3000 + i)


DECODE_FAN_RANDOM = [_draw_fan(np.random.default_rng(7500 + i), i, False) for i in range(12)]
PREFILL_FAN_RANDOM = [_draw_fan(np.random.default_rng(9500 + i), i, True) for i in range(6)]


def _desc(w):
    return (f"{w.name}: B={w.B} G={w.Hq // w.Hkv} Hkv={w.Hkv} d={w.d} {w.dtype} b={w.b} fan={w.F} levels={w.levels} "
            f"R={w.R} {w.mode} k={w.k} p={w.p} cap={w.cap} L={w.L}")


@pytest.mark.parametrize("w", DECODE_RANDOM + DECODE_FAN_RANDOM, ids=lambda w: w.name)
def test_decode_random_geometry(w):
    print(_desc(w), flush=True)
    Ls = [w.L] + [max(1, w.L - 1 - 311 * i) for i in range(1, w.B)]
    ts, K, V, refs, _ = _setup(w, Lcap=w.L, Ls=Ls)
    q = W.gen_queries(w)
    trees, _, _, _ = _check_decode(ts, w, K, V, refs, Ls, q)
    _check_decode(ts, w, K, V, refs, Ls, q, trees=trees, split=False)


@pytest.mark.parametrize("token_nodes", [False, True])
@pytest.mark.parametrize("w", PREFILL_RANDOM + PREFILL_FAN_RANDOM, ids=lambda w: w.name)
def test_prefill_random_geometry(w, token_nodes):
    T = int(np.random.default_rng(w.seed).integers(1, 160))
    print(_desc(w), f"T={T} token_nodes={token_nodes}", flush=True)
    _check_prefill(w, w.L, T, token_nodes=token_nodes)
