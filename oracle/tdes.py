"""GRAFT: target-distilled edge scores (TDES) with a best-first builder, and the state-aware
budget (SABA) (oracle; test infrastructure only).

Follows the GRAFT page:

* Edge score, method "target-distilled edge scoring": an MLP maps the parent's and the
  child's projected token embeddings and a depth embedding to a scalar,
  f(p, c, d) = w . ReLU(W [g_p(e_p); g_c(e_c); e_d] + b) + b0. The projections depend only
  on the token id, so they enter here as precomputed tables Gp[v] = g_p(e_v) and
  Gc[v] = g_c(e_v); Ed[d - 1] = e_d.
* Inference: a prefix's score is the sum of its edges' scores, and the builder keeps
  adding the highest-scoring prefix from a max-heap until the budget is reached.
* Budget, "state-aware budget allocation": B_t maximises G(B) / C(B) with
  G(B) = a_t B^beta and C(B) = B c_verify + c_fixed.

Readings (the page refers to an equation it does not print, and says nothing of weights):

* An edge v = (p, c, d) scores S(v) = log q_d(c) + s * f(p, c, d): the draft's log-prob
  (DDTree's edge score, the page's background) plus the learned correction scaled by the
  positive scale s the page lists among the parameters; the parameters are random, seeded
  (no trained weights).
* The candidate children at depth d are the top K tokens of position d (DDTree's
  restriction); the root's token is the last verified token (an input).
* Heap order: larger score first; equal scores by the parent's node index, then by the
  child's position in its parent's children sorted by (edge score descending, token rank
  ascending). Nodes are returned in the order they are taken (parent before child).
  Because f can be positive, a child can outscore its parent, so this tree is in general
  not the Top-B of the prefix scores.
* The budget maximiser is taken over integers 1..B_max, the smallest on ties.
"""
from __future__ import annotations

import heapq
import math

import numpy as np

from .rowsweep import logsumexp_row, rank_order
from .treeout import Tree


def mlp_edge(p_tok: int, c_tok: int, d: int, prm: dict) -> float:
    """f(p, c, d) for one edge; prm holds Gp [V, hp], Gc [V, hc], Ed [L, hd], W [H, hp+hc+hd],
    b [H], w [H], b0 (float64 arrays)."""
    x = np.concatenate([prm["Gp"][p_tok], prm["Gc"][c_tok], prm["Ed"][d - 1]])
    hidden = np.maximum(prm["W"] @ x + prm["b"], 0.0)
    return float(prm["w"] @ hidden + prm["b0"])


def candidates(z_rows: np.ndarray, K: int):
    """Per depth d = 1..L: the top K tokens of position d (rank order) and their log-probs."""
    L = z_rows.shape[0]
    toks, lps = [], []
    for d in range(L):
        lse = logsumexp_row(z_rows[d])
        ids = rank_order(z_rows[d])[:K]
        toks.append([int(v) for v in ids])
        lps.append([float(z_rows[d, v]) - lse for v in ids])
    return toks, lps


def edge_rows(z_rows: np.ndarray, root_tok: int, prm: dict, K: int, s: float):
    """For each depth d and parent token index pi (the root at d = 1, else the parent's index
    in C_{d-1}): the K children's edge scores S = log q_d(c) + s f(p, c, d), and the
    children's positions sorted by (S descending, rank ascending)."""
    L = z_rows.shape[0]
    toks, lps = candidates(z_rows, K)
    rows = {}
    for d in range(1, L + 1):
        parents = [root_tok] if d == 1 else toks[d - 2]
        for pi, p_tok in enumerate(parents):
            S = [lps[d - 1][ci] + s * mlp_edge(p_tok, toks[d - 1][ci], d, prm) for ci in range(K)]
            order = sorted(range(K), key=lambda ci: (-S[ci], ci))
            rows[(d, pi)] = (S, order)
    return toks, rows


def build_tdes(z_rows: np.ndarray, root_tok: int, prm: dict, K: int, B: int, s: float):
    """One round's best-first tree over S_TDES. Returns (tree, gap): gap is the smallest
    margin between the taken prefix and the best other one on the heap over all steps
    (inf when no step had a rival)."""
    L, V = z_rows.shape
    if not (1 <= K <= V and B >= 0):
        raise ValueError("bad arguments")
    toks, rows = edge_rows(z_rows, root_tok, prm, K, s)
    t = Tree()
    pidx = [0]  # per node: index of its token in C_depth (the root: 0)
    heap = []

    def push_children(n):
        d = t.depth[n] + 1
        if d > L:
            return
        S, order = rows[(d, pidx[n])]
        for j, ci in enumerate(order):
            heapq.heappush(heap, (-(t.score[n] + S[ci]), n, j, ci))

    push_children(0)
    gap = math.inf
    while t.n < B and heap:
        negS, n, j, ci = heapq.heappop(heap)
        if heap:
            gap = min(gap, heap[0][0] - negS)
        d = t.depth[n] + 1
        m = t.add(n, toks[d - 1][ci], d, -negS)
        pidx.append(ci)
        push_children(m)
    return t, gap


def saba_budget(a: float, beta: float, c_verify: float, c_fixed: float, B_max: int) -> int:
    """argmax over B = 1..B_max of a B^beta / (B c_verify + c_fixed), smallest B on ties."""
    if not (a > 0 and 0 < beta < 1 and c_verify > 0 and c_fixed >= 0 and B_max >= 1):
        raise ValueError("bad arguments")
    best, arg = -math.inf, 1
    for Bc in range(1, B_max + 1):
        u = a * Bc ** beta / (Bc * c_verify + c_fixed)
        if u > best:
            best, arg = u, Bc
    return arg
