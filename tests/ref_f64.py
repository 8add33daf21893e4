"""Independent float64 formulations used to pin the oracle (tests only).

Nothing here shares code with the oracle or with the GPU library.  Each helper
is a *different* formulation of something the method reduces to:

* RoPE as multiplication of the complex numbers x_j + i x_{j+d/2} by
  e^{i pos theta_j} (the rotate-half form written as complex arithmetic);
* dense causal attention (the textbook routine the method must reduce to when
  every node is selected);
* the entry set E written as a predicate over *all* nodes ("a node is a
  candidate iff it is a top node, an orphan, or a child of a selected
  candidate"), not as the oracle's level-by-level candidate lists;
* the shared softmax evaluated in float64 over that entry set;
* the tree's pooled keys and mean values as whole-level float64 array
  operations (log-sum-exp weights), one chain of keys per reference query.
"""
from __future__ import annotations

import numpy as np


def thetas(d: int, base: float) -> np.ndarray:
    return base ** (-2.0 * np.arange(d // 2) / d)


def rope_c(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """RoPE via complex multiplication; x [..., d], pos broadcastable to x[..., 0]."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    ang = np.asarray(pos, np.float64)[..., None] * thetas(d, base)
    z = z * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def dense_causal(q: np.ndarray, K: np.ndarray, V: np.ndarray, qpos: int, base=10000.0):
    """Textbook attention of q [G, d] at absolute position qpos over tokens 0..qpos."""
    n = qpos + 1
    qr = rope_c(q, qpos, base)
    kr = rope_c(K[:n], np.arange(n), base)
    z = qr @ kr.T / np.sqrt(q.shape[-1])
    w = np.exp(z - z.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return w @ np.asarray(V[:n], np.float64)


def fan_in(level: int, b: int, fan: int | None) -> int:
    """Children per node of `level` (>= 1): b tokens at level 1, fan nodes above."""
    return b if level == 1 or fan is None else fan


def level_counts(L: int, b: int, levels: int, fan: int | None = None) -> list[int]:
    n = [L]
    for lvl in range(1, levels + 1):
        n.append(n[-1] // fan_in(lvl, b, fan))
    return n


def candidates_by_predicate(L: int, b: int, levels: int, sel: list[set], fan: int | None = None):
    """Candidate sets per level from the node predicate.

    sel[l] = set of selected node ids at level l (l = 1..levels; sel[0] unused).
    A level-l node x is a candidate iff l is the top level, or x has no full
    parent (x >= f * n_{l+1}, f the fan-in of level l + 1), or its parent
    x // f is a candidate and selected.
    Returns {l: sorted list of candidate ids}.
    """
    n = level_counts(L, b, levels, fan)
    memo = {}

    def is_cand(l: int, x: int) -> bool:
        key = (l, x)
        if key in memo:
            return memo[key]
        f = fan_in(l + 1, b, fan) if l < levels else 0
        if l == levels or x >= f * n[l + 1]:
            r = True
        else:
            par = x // f
            r = is_cand(l + 1, par) and par in sel[l + 1]
        memo[key] = r
        return r

    return {l: [x for x in range(n[l]) if is_cand(l, x)] for l in range(levels + 1)}


def entries_from_candidates(cands: dict, sel: list[set], levels: int):
    """Entry list (level, node, position) implied by the candidate sets."""
    ent = []
    for l in range(levels, 0, -1):
        for pos, x in enumerate(cands[l]):
            if x not in sel[l]:
                ent.append((l, x, pos))
    for pos, x in enumerate(cands[0]):
        ent.append((0, x, pos))
    return ent


def covered_tokens(level: int, node: int, b: int, fan: int | None = None) -> range:
    span = 1
    for lvl in range(1, level + 1):
        span *= fan_in(lvl, b, fan)
    return range(node * span, (node + 1) * span)


def group_scores_f64(q: np.ndarray, keys: np.ndarray, qpos: int, base: float):
    """Per-head logits [G, m, R] and group scores (max over R of the head mean).

    keys [m, R, d] un-rotated; candidate i at position i, query at qpos.
    """
    d = q.shape[-1]
    qr = rope_c(q, qpos, base)                                         # [G, d]
    m = keys.shape[0]
    kr = rope_c(keys, np.arange(m)[:, None], base)                     # [m, R, d]
    z = np.einsum("gd,mrd->gmr", qr, kr) / np.sqrt(d)
    gm = z.mean(axis=0)                                                # [m, R]
    jstar = gm.argmax(axis=1)
    s = gm[np.arange(m), jstar]
    zsel = z[:, np.arange(m), jstar]                                   # [G, m]
    return s, zsel


def softmax_over_entries(zs: np.ndarray, vals: np.ndarray):
    """zs [G, E] logits, vals [E, d] -> out [G, d], lse [G] in float64."""
    M = zs.max(axis=1, keepdims=True)
    w = np.exp(zs - M)
    den = w.sum(axis=1, keepdims=True)
    return (w @ vals) / den, (M + np.log(den))[:, 0]


def pool_tree_f64(K: np.ndarray, V: np.ndarray, refs: np.ndarray, b: int, levels: int, L: int | None = None,
                  fan: int | None = None):
    """The tree's levels in float64, written as whole-level array operations.

    Each reference query r_j pools its own chain of keys: level 1 pools the
    token keys, level l >= 2 pools the level-(l-1) keys of that same
    reference.  A node's weights are the softmax over its children (b tokens
    at level 1, fan nodes above; fan None means b) of
    r_j . k_child / sqrt(d) (taken in the log domain: log-sum-exp with the
    children's maximum), its key the weighted sum of the children's keys and
    its value the plain mean of the children's values.  Only full nodes.
    Returns [(keys [n_l, R, d], values [n_l, d]) for l = 1..levels].
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    refs = np.asarray(refs, np.float64)
    L = K.shape[0] if L is None else L
    R, d = refs.shape
    keys = np.repeat(K[:L, None, :], R, axis=1)            # [n, R, d]: level 0, one chain per reference
    vals = V[:L]
    out = []
    for lvl in range(1, levels + 1):
        f = fan_in(lvl, b, fan)
        n = keys.shape[0] // f
        ch = keys[: n * f].reshape(n, f, R, d)               # [node, child, ref, d]
        logit = np.einsum("ncrd,rd->ncr", ch, refs) / np.sqrt(d)
        lse = logit.max(axis=1, keepdims=True)
        lse = lse + np.log(np.exp(logit - lse).sum(axis=1, keepdims=True))
        w = np.exp(logit - lse)                              # [node, child, ref]
        keys = np.einsum("ncr,ncrd->nrd", w, ch)
        vals = vals[: n * f].reshape(n, f, d).mean(axis=1)
        out.append((keys, vals))
    return out
