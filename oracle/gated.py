"""TALON confidence-gated budget tree (oracle; test infrastructure only).

Follows the TALON page, key designs 1 and 2, for one round:

* Root Top-K initialisation: P_1 = the top K_root tokens of the first position
  (the children of the root), kept whatever their probability.
* For d = 1, 2, ...: the pool S_d = {(v, w) : v in P_d, w in V} over the whole
  vocabulary, each with path probability p(v, w) = p(v) * P(w | x_{<=v}); the
  anchor m_d = max over S_d; keep P_{d+1} = {u in S_d : p(u) >= mu * m_d}.
* Global budget: if the kept set is larger than N - |T|, keep only its
  N - |T| highest path scores and stop growing.

Readings: the per-position logits stand for P(w | x_{<=v}) (one distribution
per depth, parent independent); |T| counts every non-root node added so far,
including the root layer; growth also stops at depth L or when |T| = N.
The gate is taken in log space: log p(u) = Z(u) - Lsum_d with
Z(u) = sum of the path's logits, so p(u) >= mu * m_d is exactly
Z(u) - Z_max >= ln(mu), evaluated in float64. Within a depth the order is
larger Z, then the parent's position in P_d, then the token's rank at its
position (logit descending, id ascending).
"""
from __future__ import annotations

import math

import numpy as np

from .rowsweep import logsumexp_row, rank_order
from .treeout import Tree


def build_gated(z_rows: np.ndarray, K_root: int, mu: float, N: int, full_pool: bool = True) -> Tree:
    """One round. z_rows float64 [L, V]. With full_pool the candidate pool is the literal
    P_d x V; otherwise it is P_d x (top N-|T| tokens), which the dominance argument shows
    to be the same set of survivors (tested on small inputs)."""
    L, V = z_rows.shape
    if not (1 <= K_root <= V and K_root <= N and 0.0 < mu <= 1.0 and L >= 1):
        raise ValueError("bad arguments")
    ln_mu = math.log(float(mu))
    lse = [logsumexp_row(z_rows[d]) for d in range(L)]
    Lsum = [0.0]
    for v in lse:
        Lsum.append(Lsum[-1] + v)
    ranks = [rank_order(z_rows[d]) for d in range(L)]
    rank_of = [np.empty(V, dtype=np.int64) for _ in range(L)]
    for d in range(L):
        rank_of[d][ranks[d]] = np.arange(V)

    t = Tree()
    # root layer: top K_root tokens of position 1
    layer = []  # (Z, index in t) in this depth's order
    for k in range(K_root):
        v = int(ranks[0][k])
        Z = float(z_rows[0, v])
        i = t.add(0, v, 1, Z - Lsum[1])
        layer.append((Z, i))
    d = 1
    while d < L and t.n < N:
        room = N - t.n
        zrow = z_rows[d]
        parZ = np.array([Z for Z, _ in layer])
        if full_pool:
            cand_tok = np.arange(V)
        else:
            cand_tok = ranks[d][:min(room, V)]
        Zpool = parZ[:, None] + zrow[cand_tok][None, :]         # [n_par, n_cand]
        Zmax = float(np.max(Zpool))
        keep = (Zpool - Zmax) >= ln_mu
        pi, ci = np.nonzero(keep)
        Zk = Zpool[pi, ci]
        toks = cand_tok[ci]
        rk = rank_of[d][toks]
        order = np.lexsort((rk, pi, -Zk))
        truncated = order.shape[0] > room
        order = order[:room]
        new_layer = []
        for o in order:
            Z = float(Zk[o])
            s = Z - Lsum[d + 1]
            s = min(s, t.score[layer[pi[o]][1]])
            i = t.add(layer[pi[o]][1], int(toks[o]), d + 1, s)
            new_layer.append((Z, i))
        layer = new_layer
        d += 1
        if truncated:
            break
    return t
