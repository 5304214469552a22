"""Flattened tree outputs: parent array, tokens, depths, scores, ancestor mask (oracle).

The DARTree summary (background, "tree verification") flattens the draft tree
and builds a tree-attention mask under which every node sees only the verified
context and its own root-to-node path; the DDTree blog (section 4.2) keys the
mask on each token's parent position and its checklist asks for a hand-drawn
mask of a depth-3 tree. Row i of the mask has bit j set iff node j is node i
or one of its ancestors; word j >> 5, bit j & 31, least significant bit first.
Node 0 is the root (the verified context); B and N count non-root nodes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Tree:
    """One round's tree in canonical order: the root is node 0, then depth by depth,
    each depth in its selection order, so parent[i] < i."""
    parent: list = field(default_factory=lambda: [-1])
    token: list = field(default_factory=lambda: [-1])
    depth: list = field(default_factory=lambda: [0])
    score: list = field(default_factory=lambda: [0.0])

    @property
    def n(self) -> int:
        """Number of non-root nodes."""
        return len(self.parent) - 1

    def add(self, parent: int, token: int, depth: int, score: float) -> int:
        self.parent.append(int(parent))
        self.token.append(int(token))
        self.depth.append(int(depth))
        self.score.append(float(score))
        return len(self.parent) - 1

    def arrays(self, cap: int):
        """Padded arrays of length cap+1: unused slots hold -1 (ints) and -inf (scores)."""
        par = np.full(cap + 1, -1, dtype=np.int32)
        tok = np.full(cap + 1, -1, dtype=np.int32)
        dep = np.full(cap + 1, -1, dtype=np.int32)
        sc = np.full(cap + 1, -np.inf, dtype=np.float64)
        m = len(self.parent)
        par[:m] = self.parent
        tok[:m] = self.token
        dep[:m] = self.depth
        sc[:m] = self.score
        return par, tok, dep, sc

    def paths(self) -> list:
        """Root-to-node token paths, one tuple per node (the root's is ())."""
        out = [()]
        for i in range(1, len(self.parent)):
            out.append(out[self.parent[i]] + (self.token[i],))
        return out


def mask_words(cap: int) -> int:
    return (cap + 1 + 31) // 32


def ancestor_mask(parent, cap: int) -> np.ndarray:
    """uint32 [cap+1, words]: row i = bits of i and of every ancestor of i (walked up the parent chain)."""
    W = mask_words(cap)
    m = np.zeros((cap + 1, W), dtype=np.uint32)
    for i in range(len(parent)):
        j = i
        while j >= 0:
            m[i, j >> 5] |= np.uint32(1) << np.uint32(j & 31)
            j = parent[j]
    return m


def check_invariants(t: Tree, B: int, L: int) -> None:
    """Prefix closure and score monotonicity (DARTree Lemma 1 proof: a child never outscores its parent)."""
    assert t.parent[0] == -1 and t.depth[0] == 0 and t.token[0] == -1
    assert t.n <= B
    seen = set()
    for i in range(1, len(t.parent)):
        p = t.parent[i]
        assert 0 <= p < i, (i, p)
        assert t.depth[i] == t.depth[p] + 1
        assert 1 <= t.depth[i] <= L
        assert t.score[i] <= t.score[p]
        assert t.depth[i] >= t.depth[i - 1], "canonical order is depth-major"
        key = (p, t.token[i])
        assert key not in seen, "two children of one node carry the same token"
        seen.add(key)
