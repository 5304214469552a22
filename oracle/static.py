"""Static D x K grid expansion, the fixed-shape tree builder TALON compares against
(oracle; test infrastructure only).

Follows the TALON page, research background: the static expansion of Eagle-3 grows the
tree to a preset depth D with a preset width K; at every depth each of the K kept nodes
is expanded by its top K tokens (K x K leaves) and the best K of those become the kept
nodes of the next depth.

Readings (the page gives the shape, not the details):

* The per-position logits stand for the children's distribution at that depth, the same
  for every parent (as for the other builders here), and a path's score is the sum of its
  log-probabilities, i.e. Z(u) - Lsum_d with Z(u) the sum of the path's logits.
* Depth 1 holds the top K tokens of position 1; depth d + 1 the best K of the pool
  P_d x V, ranked by larger Z, then the parent's position in P_d, then the token's rank
  at its position (logit descending, id ascending). The tree is the union of the kept
  nodes, K per depth, K * D in all; no final re-ranking is applied.
* A node's stored score is min(own, parent's), as for the gated tree, so rounding never
  lets a child outscore its parent.

The pool is written over the whole vocabulary, P_d x V; only each parent's top K tokens
can reach the best K, which is what the K x K grid restricts it to.
"""
from __future__ import annotations

import numpy as np

from .rowsweep import logsumexp_row, rank_order
from .treeout import Tree


def build_static(z_rows: np.ndarray, K: int, D: int) -> Tree:
    """One round. z_rows float64 [L, V]; 1 <= K <= V, 1 <= D <= L."""
    L, V = z_rows.shape
    if not (1 <= K <= V and 1 <= D <= L):
        raise ValueError("bad arguments")
    Lsum = [0.0]
    for d in range(L):
        Lsum.append(Lsum[-1] + logsumexp_row(z_rows[d]))
    ranks = [rank_order(z_rows[d]) for d in range(D)]
    rank_of = []
    for d in range(D):
        ro = np.empty(V, dtype=np.int64)
        ro[ranks[d]] = np.arange(V)
        rank_of.append(ro)

    t = Tree()
    layer = []  # (Z, node index) in this depth's order
    for k in range(K):
        v = int(ranks[0][k])
        Z = float(z_rows[0, v])
        layer.append((Z, t.add(0, v, 1, Z - Lsum[1])))
    for d in range(1, D):
        parZ = np.array([Z for Z, _ in layer])
        Zpool = parZ[:, None] + z_rows[d][None, :]  # [K, V], the whole pool
        pi, ci = np.nonzero(np.ones_like(Zpool, dtype=bool))
        Zk = Zpool[pi, ci]
        order = np.lexsort((rank_of[d][ci], pi, -Zk))[:K]
        new_layer = []
        for o in order:
            Z = float(Zk[o])
            par = layer[pi[o]][1]
            s = min(Z - Lsum[d + 1], t.score[par])
            new_layer.append((Z, t.add(par, int(ci[o]), d + 1, s)))
        layer = new_layer
    return t
