"""Marginal (parent-independent) draft tree: the B best prefixes (oracle; test infrastructure only).

What it computes (DARTree summary, background "tree verification and DDTree";
DDTree blog sections 2.1-2.3): among all prefixes u = (u_1..u_d), d <= L, of
the per-position drafts, take the B with the largest
    s_beta(u) = sum_{i<=d} log q_i(u_i) + beta*d          (DARTree, eq. for s_beta)
under the factorised block distribution. Ancestors carry at least their
descendants' score (DDTree blog 2.2, DARTree Lemma 1 proof), so the B best form
a prefix-closed tree, and by the S_K restriction (DDTree blog 2.3) it suffices
to look at each position's top K = min(B, V) tokens.

Two independent computations are given:
* ``heap_topb``: DDTree's best-first enumeration over rank descriptors (blog
  section 3.1) with a max-heap, popping B prefixes. Successors of a popped
  descriptor rho: its first child (rho, top-1) whenever d < L, and its next
  sibling when the last rank can still grow. The blog's text pushes the first
  child only when the last rank is the top one; that rule never reaches the
  children of lower-ranked prefixes and contradicts the blog's own
  predecessor-chain argument, so the rule that matches the argument is used.
* ``sort_topb``: plain enumeration of every prefix over the given candidate
  lists, then one sort (used over S_K on tiny inputs, and over the full
  vocabulary as brute force).

Exact ties. log q_i(v) = z_i(v) - LSE_i, so for prefixes of equal depth the
score differs only through Z(u) = sum_i z_i(u_i); with bf16 logits many such
sums are exactly equal. Scores are therefore formed as
    Z(child) = Z(parent) + z                  (float64, in depth order)
    s(child) = min((Z - Lsum_d) + beta*d, s(parent)),   Lsum_d = sum_{i<=d} LSE_i
so that equal-Z prefixes of one depth get bit-identical scores, and the clamp
keeps the child <= parent invariant of Lemma 1 exact under rounding.

Total order (ties broken as Lemma 1 asks, ancestor first): larger s first; then
smaller depth; then larger Z; then the parent's position within its own depth's
order; then the token's rank at its position. The B selected prefixes are
returned depth by depth, each depth in this order.
"""
from __future__ import annotations

import heapq

import numpy as np

from .rowsweep import logsumexp_row, rank_order
from .treeout import Tree


def lse_prefix_sums(lse: np.ndarray) -> list:
    """Lsum[d] = LSE_1 + ... + LSE_d (float64, left to right); Lsum[0] = 0."""
    out = [0.0]
    for v in lse:
        out.append(out[-1] + float(v))
    return out


def child_score(z_par: float, s_par: float, z: float, d: int, Lsum: list, beta: float):
    """(Z, s) of a depth-d child whose parent has (z_par, s_par)."""
    Z = z_par + z
    s = (Z - Lsum[d]) + beta * d
    return Z, min(s, s_par)


def heap_topb(zk: np.ndarray, lse: np.ndarray, B: int, beta: float):
    """DDTree best-first over rank descriptors. zk: [L, K] logits of each position's
    candidates in rank order. Returns the popped nodes, in pop order, as dicts."""
    L, K = zk.shape
    if beta > 0:
        raise ValueError("Lemma 1 needs beta <= 0")
    Lsum = lse_prefix_sums(lse)
    popped_at = [0] * (L + 1)
    out = []
    heap = []

    def push(desc, z_par, s_par, ppos, parent_idx):
        d = len(desc)
        Z, s = child_score(z_par, s_par, float(zk[d - 1, desc[-1]]), d, Lsum, beta)
        key = (-s, d, -Z, ppos, desc[-1])
        heapq.heappush(heap, (key, desc, Z, s, ppos, parent_idx, z_par, s_par))

    if L >= 1 and K >= 1 and B >= 1:
        push((0,), 0.0, 0.0, 0, -1)
    while heap and len(out) < B:
        key, desc, Z, s, ppos, parent_idx, z_par, s_par = heapq.heappop(heap)
        d = len(desc)
        pos = popped_at[d]
        popped_at[d] += 1
        idx = len(out)
        out.append(dict(desc=desc, depth=d, Z=Z, s=s, ppos=ppos, pos=pos, rank=desc[-1], parent=parent_idx))
        if d < L:
            push(desc + (0,), Z, s, pos, idx)
        if desc[-1] + 1 < K:
            push(desc[:-1] + (desc[-1] + 1,), z_par, s_par, ppos, parent_idx)
    return out


def sort_topb(zk: np.ndarray, lse: np.ndarray, B: int, beta: float):
    """Enumerate every prefix over the candidate lists zk [L, K] and sort (plain definition).

    Returns the B first nodes in the total order as dicts (same fields as heap_topb,
    with 'parent' an index into the returned list). Memory grows as K**L."""
    L, K = zk.shape
    Lsum = lse_prefix_sums(lse)
    levels = []  # per depth: dict of arrays in that depth's order
    prevZ = np.zeros(1)
    prevS = np.zeros(1)
    prevPos = np.zeros(1, dtype=np.int64)
    prevDesc = [()]
    for d in range(1, L + 1):
        n_par = prevZ.shape[0]
        Z = (prevZ[:, None] + zk[d - 1][None, :]).reshape(-1)
        s_raw = (Z - Lsum[d]) + beta * d
        s = np.minimum(s_raw, np.repeat(prevS, K))
        ppos = np.repeat(prevPos, K)
        rank = np.tile(np.arange(K), n_par)
        par_local = np.repeat(np.arange(n_par), K)
        order = np.lexsort((rank, ppos, -Z, -s))
        lev = dict(Z=Z[order], s=s[order], ppos=ppos[order], rank=rank[order], par_local=par_local[order])
        levels.append(lev)
        # positions of this depth in its own order: index after sorting
        prevZ, prevS = lev["Z"], lev["s"]
        prevPos = np.arange(Z.shape[0], dtype=np.int64)
    # global order over all depths
    allS = np.concatenate([lv["s"] for lv in levels])
    allD = np.concatenate([np.full(lv["s"].shape[0], d + 1) for d, lv in enumerate(levels)])
    allZ = np.concatenate([lv["Z"] for lv in levels])
    allP = np.concatenate([lv["ppos"] for lv in levels])
    allR = np.concatenate([lv["rank"] for lv in levels])
    allPos = np.concatenate([np.arange(lv["s"].shape[0]) for lv in levels])
    order = np.lexsort((allR, allP, -allZ, allD, -allS))[:B]
    out = []
    for g in order:
        out.append(dict(depth=int(allD[g]), Z=float(allZ[g]), s=float(allS[g]), ppos=int(allP[g]),
                        pos=int(allPos[g]), rank=int(allR[g])))
    return out


def nodes_to_tree(nodes, tokens_by_rank: np.ndarray) -> Tree:
    """Canonical tree from selected nodes (each with depth, pos, ppos, rank, s).

    Nodes are laid out depth by depth, each depth in its order; a node's parent is
    the depth-(d-1) node whose position is its ppos. tokens_by_rank[d-1, k] is the
    token id of rank k at position d."""
    t = Tree()
    by_depth = {}
    for nd in nodes:
        by_depth.setdefault(nd["depth"], []).append(nd)
    index_of = {(0, 0): 0}
    for d in sorted(by_depth):
        for nd in sorted(by_depth[d], key=lambda x: x["pos"]):
            p = index_of[(d - 1, nd["ppos"])]
            i = t.add(p, int(tokens_by_rank[d - 1, nd["rank"]]), d, nd["s"])
            index_of[(d, nd["pos"])] = i
    return t


def build_marginal(z_rows: np.ndarray, K: int, B: int, beta: float) -> Tree:
    """One round: z_rows float64 [L, V]. K = 0 means min(B, V). Heap best-first over S_K,
    asserted equal (node for node, in pop order) to a sort when S_K is small."""
    L, V = z_rows.shape
    K = min(B, V) if K == 0 else K
    if not (1 <= K <= V and B >= 1 and L >= 1):
        raise ValueError("bad sizes")
    lse = np.array([logsumexp_row(z_rows[d]) for d in range(L)])
    ranks = np.stack([rank_order(z_rows[d])[:K] for d in range(L)])
    zk = np.take_along_axis(z_rows, ranks, axis=1)
    nodes = heap_topb(zk, lse, B, float(beta))
    if K ** L <= 2_000_000:
        ref = sort_topb(zk, lse, B, float(beta))
        a = [(n["depth"], n["pos"], n["ppos"], n["rank"], n["s"]) for n in nodes]
        b = [(n["depth"], n["pos"], n["ppos"], n["rank"], n["s"]) for n in ref]
        assert a == b, "Lemma 1: best-first pops differ from the global Top-B"
    return nodes_to_tree(nodes, ranks)


def brute_force(z_rows: np.ndarray, B: int, beta: float) -> Tree:
    """Every prefix over the full vocabulary (depth <= L), sorted; for tiny V**L only."""
    L, V = z_rows.shape
    lse = np.array([logsumexp_row(z_rows[d]) for d in range(L)])
    ranks = np.stack([rank_order(z_rows[d]) for d in range(L)])
    zk = np.take_along_axis(z_rows, ranks, axis=1)
    nodes = sort_topb(zk, lse, B, float(beta))
    return nodes_to_tree(nodes, ranks)
