"""DARTree depth-wise super-tree with a causal correction head, then deferred Top-B (oracle).

Follows Algorithm 1 of the DARTree summary ("DARTree construction") step by
step, for one round:

  S_0 = {root}, state r(root) = r_0, s(root) = 0
  for d = 1..gamma:
      C_d = TopK(L_d^base, K)                                  (step 4)
      correct C_d for every branch of S_{d-1} at once           (steps 5-6)
      child score s(u_{1:d}) = s(u_{<d}) + log q~_d(u_d | u_{<d}) + beta   (step 8)
      S_d = the global top-W children                           (step 9)
      carry the new state from (r, u_d)                          (step 10)
  T = TopB over S = union of S_d of s                          (step 12)

The correction head g is the synthetic Markov head of the workload: the state of
a branch is its last token (the root's is root_tok), and
    h_b = bf16(E[tok_b] @ U_d)              (rank-64 state, rounded to bf16)
    z_b = base_d + h_b @ P                  (corrected logits over the full V)
    log q~_d(c | b) = z_b[c] - logsumexp(z_b)
so q~ is normalised over the whole vocabulary and evaluated at the candidates
C_d, which come from the base logits and are shared by all branches. Markov
correction (one-step transition from the previous token) is the DARTree
summary's background "parallel drafting and causal correction".

Ties: a depth keeps its children in order of larger s, then the parent's
position in S_{d-1}, then the candidate's rank. The final Top-B uses larger s,
then smaller depth (ancestor first, Lemma 1), then the position within S_d.
A child's score is clamped to its parent's so Lemma 1's monotonicity holds
exactly; it is checked by running the deferred selection both as one sort
and as a best-first heap over the super-tree and asserting the same result.
"""
from __future__ import annotations

import heapq

import numpy as np

from .rowsweep import logsumexp_row, rank_order
from .treeout import Tree


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (8 significant bits, ties to even),
    returned as float64. Rounds directly from float64 on each value's binade grid
    (no intermediate float32 rounding)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    m, e = np.frexp(x[nz])          # x = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: m * 2**8 rounded to an integer, ties to even
    q = np.round(m * 256.0)         # numpy rounds half to even
    out[nz] = np.ldexp(q / 256.0, e)
    return out


def build_depthwise(base_rows: np.ndarray, E: np.ndarray, U: np.ndarray, P: np.ndarray,
                    root_tok: int, K: int, W: int, B: int, beta: float, with_super: bool = False):
    """One round. base_rows float64 [L, V]; E float64-convertible [V, dm] (rows gathered);
    U [L, dm, rank]; P [rank, V]. Returns the canonical Tree; with_super also returns the
    super-tree levels and the selection gaps (per depth at the width cut, then at the B cut)."""
    L, V = base_rows.shape
    if beta > 0:
        raise ValueError("Lemma 1 needs beta <= 0")
    if not (1 <= K <= V and W >= 1 and B >= 1):
        raise ValueError("bad sizes")
    P64 = np.asarray(P, dtype=np.float64)
    levels = []
    gaps = []   # per depth: score of the W-th kept child minus the first dropped one
    # S_{d-1} as parallel lists; depth 0 is the root alone
    prev_tok = [int(root_tok)]
    prev_s = [0.0]
    for d in range(1, L + 1):
        base = base_rows[d - 1]
        cand = rank_order(base)[:K]
        Ud = np.asarray(U[d - 1], dtype=np.float64)
        Erows = np.asarray(E[np.array(prev_tok)], dtype=np.float64)
        H = bf16_round(Erows @ Ud)                         # [n_b, rank]
        Z = base[None, :] + H @ P64                         # [n_b, V]
        children = []
        for b in range(len(prev_tok)):
            lse_b = logsumexp_row(Z[b])
            for k, c in enumerate(cand):
                s = prev_s[b] + (Z[b, c] - lse_b) + beta
                s = min(s, prev_s[b])
                children.append((-s, b, k, int(c), s))
        children.sort()
        kept = children[:W]
        gaps.append(kept[-1][4] - children[W][4] if len(children) > W else np.inf)
        levels.append([dict(s=s, ppos=b, rank=k, token=c) for (_, b, k, c, s) in kept])
        prev_tok = [c for (_, _, _, c, _) in kept]
        prev_s = [s for (_, _, _, _, s) in kept]
    tree = deferred_topb(levels, B)
    if with_super:
        flat = sorted(-nd["s"] for lev in levels for nd in lev)
        gaps.append(flat[B] - flat[B - 1] if len(flat) > B else np.inf)
        return tree, levels, gaps
    return tree


def deferred_topb(levels, B: int) -> Tree:
    """T = TopB over the super-tree by (s desc, depth asc, position in S_d asc); built by
    sort and by a best-first heap (Lemma 1), asserted equal, laid out depth by depth."""
    flat = []
    for d, lev in enumerate(levels, start=1):
        for pos, nd in enumerate(lev):
            flat.append((-nd["s"], d, pos))
    by_sort = sorted(flat)[:B]
    # heap: start from the depth-1 layer, pop, push the popped node's children in S
    kids = {}
    for d, lev in enumerate(levels, start=1):
        for pos, nd in enumerate(lev):
            kids.setdefault((d - 1, nd["ppos"]), []).append((-nd["s"], d, pos))
    heap = list(kids.get((0, 0), []))
    heapq.heapify(heap)
    by_heap = []
    while heap and len(by_heap) < B:
        item = heapq.heappop(heap)
        by_heap.append(item)
        for ch in kids.get((item[1], item[2]), []):
            heapq.heappush(heap, ch)
    assert by_heap == by_sort, "Lemma 1: best-first differs from Top-B over the super-tree"
    chosen = sorted((d, pos) for (_, d, pos) in by_sort)
    t = Tree()
    index_of = {(0, 0): 0}
    for d, pos in chosen:
        nd = levels[d - 1][pos]
        p = index_of[(d - 1, nd["ppos"])]
        index_of[(d, pos)] = t.add(p, nd["token"], d, nd["s"])
    return t


def build_sequential(base_rows: np.ndarray, E: np.ndarray, U: np.ndarray, P: np.ndarray,
                     root_tok: int, K: int, B: int, beta: float, with_gaps: bool = False):
    """The exact path-dependent best-first tree the DARTree summary sets against its own
    method ("decoupling causal correction from best-first search"; the tree-construction
    ablation's "sequential correction with heap"): a max-heap of candidate prefixes; each
    step pops the best one, runs the correction head once for that node alone (its own
    token history; with the Markov head, its last token), scores its children over C_{d+1}
    and pushes them, before the next pop. B nodes are popped (or the heap runs dry).

    Same correction and child score as build_depthwise, the clamp to the parent included.
    Heap order: larger s, then smaller depth (ancestor first), then the parent's pop order,
    then the candidate's rank. The tree is laid out depth by depth, each depth in pop order
    (which within a depth is the depth-wise builder's S_d order). with_gaps also returns,
    per pop, the popped score minus the best one left in the heap when the two are at the
    same depth or the pop is the last (inf otherwise)."""
    L, V = base_rows.shape
    if beta > 0:
        raise ValueError("Lemma 1 needs beta <= 0")
    if not (1 <= K <= V and B >= 1):
        raise ValueError("bad sizes")
    P64 = np.asarray(P, dtype=np.float64)
    cands = [rank_order(base_rows[d])[:K] for d in range(L)]

    def expand(pop_index, depth, tok, s, heap):
        """One correction call for one node: push its children at depth + 1."""
        if depth >= L:
            return
        erow = np.asarray(E[np.array([tok])], dtype=np.float64)[0]  # rows by index array, as above
        h = bf16_round(erow @ np.asarray(U[depth], dtype=np.float64))
        z = base_rows[depth] + h @ P64
        lse = logsumexp_row(z)
        for k, c in enumerate(cands[depth]):
            cs = min(s + (z[c] - lse) + beta, s)
            heapq.heappush(heap, (-cs, depth + 1, pop_index, k, int(c)))

    popped = []  # (s, depth, parent pop index, token), pop index = position + 1 (root = 0)
    gaps = []
    heap = []
    expand(0, 0, int(root_tok), 0.0, heap)
    while heap and len(popped) < B:
        ns, d, par, _k, c = heapq.heappop(heap)
        if with_gaps:
            last = len(popped) + 1 == B
            gaps.append(-ns - (-heap[0][0]) if heap and (heap[0][1] == d or last) else np.inf)
        popped.append((-ns, d, par, c))
        if len(popped) < B:  # the last node's children could never be popped
            expand(len(popped), d, c, -ns, heap)
    # canonical layout: depth by depth, pop order within a depth
    order = sorted(range(len(popped)), key=lambda i: (popped[i][1], i))
    index_of = {0: 0}
    t = Tree()
    for i in order:
        s, d, par, c = popped[i]
        index_of[i + 1] = t.add(index_of[par], c, d, s)
    return (t, gaps) if with_gaps else t
