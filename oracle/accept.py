"""Tree verification walks (oracle; test infrastructure only).

Greedy (T = 0), DARTree summary background "speculative sampling": accept the
draft tokens that match the target's greedy prediction; at the first mismatch
emit the target's prediction and end the round. On a tree: at node j take
t* = argmax of the target row j (the smallest id among equal maxima, the course
notes' greedy tie-break); descend to the child carrying t* if there is one,
otherwise stop and emit t* as the round's extra token.

Residual sampling (T > 0), DARTree summary (same section) and the course notes'
three-token worked example: a draft token x proposed from q is accepted with
probability min(1, p(x)/q(x)); after a rejection the next draw uses the
normalised positive residual (p - q)_+ / sum (p - q)_+. When that sum is zero,
p = q and the rejection had probability zero, so nothing is renormalised (the
notes' degenerate case). At a node the children are tried in canonical order,
each against the current residual with q fixed; when every child is rejected,
or at a leaf, one token is drawn from the current residual -- the bonus token
after a fully accepted path, the correction token otherwise.

Exact target-sample matching (DARTree summary, same section: DFlash checks
drafts by matching exact samples of the target): at node j draw x from
p = softmax(target[j] / T) by inverse CDF with the walk's next uniform; descend to
the child carrying x (the first in canonical order) or, with none, stop and emit
x. Every committed token is then a sample of the target's own distribution, for
any tree. At T = 0 the draw is the argmax and the rule is the greedy walk.

p = softmax(target[j] / T) for node j; q = softmax(draft[depth(j)] / T), the
position its children were drafted from. Acceptance is tested without a
division as u * q(c) < p'(c); sampling is by inverse CDF in id order: the
smallest v with sum_{w <= v} p'(w) > u * sum p'.
"""
from __future__ import annotations

import numpy as np

from .philox import uniform


def softmax_row(z: np.ndarray, T: float) -> np.ndarray:
    x = np.asarray(z, dtype=np.float64) / T
    m = np.max(x)
    e = np.exp(x - m)
    return e / np.sum(e)


def children_lists(parent) -> list:
    kids = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        kids[parent[i]].append(i)
    return kids


def walk_greedy(parent, token, depth, target_rows: np.ndarray):
    """T = 0 walk for one round. target_rows float64 [n+1, V]. Returns (accept_len, accept_node, next_token)."""
    kids = children_lists(parent)
    j = 0
    while True:
        t_star = int(np.argmax(target_rows[j]))
        nxt = -1
        for c in kids[j]:
            if token[c] == t_star:
                nxt = c
                break
        if nxt < 0:
            return depth[j], j, t_star
        j = nxt


class ResidualTables:
    """Per node: the children's (q(c), p'(c)) at the moment each is tried, and the
    residual left when all of them are rejected (the distribution of the extra token)."""

    def __init__(self, parent, token, depth, target_rows: np.ndarray, draft_rows: np.ndarray, T: float):
        self.kids = children_lists(parent)
        n1 = len(parent)
        self.qc = [[] for _ in range(n1)]
        self.pc = [[] for _ in range(n1)]
        self.final = [None] * n1
        L = draft_rows.shape[0]
        for j in range(n1):
            p_res = softmax_row(target_rows[j], T)
            if self.kids[j]:
                q = softmax_row(draft_rows[min(depth[j], L - 1)], T)
                for c in self.kids[j]:
                    x = token[c]
                    self.qc[j].append(float(q[x]))
                    self.pc[j].append(float(p_res[x]))
                    diff = np.maximum(p_res - q, 0.0)
                    tot = float(np.sum(diff))
                    if tot > 0.0:
                        p_res = diff / tot
            self.final[j] = p_res


def sample_inverse_cdf(p: np.ndarray, u: float) -> int:
    cdf = np.cumsum(p)
    v = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
    if v >= p.shape[0]:
        v = int(np.nonzero(p > 0)[0][-1])
    return v


def walk_sampled(tab: ResidualTables, depth, seed: int, trial: int, rnd: int):
    """T > 0 walk for one (trial, round) with the Philox stream. Returns (accept_len, accept_node, next_token)."""
    j = 0
    step = 0
    while True:
        nxt = -1
        for i, c in enumerate(tab.kids[j]):
            u = uniform(seed, trial, rnd, step)
            step += 1
            if u * tab.qc[j][i] < tab.pc[j][i]:
                nxt = c
                break
        if nxt < 0:
            u = uniform(seed, trial, rnd, step)
            return depth[j], j, sample_inverse_cdf(tab.final[j], u)
        j = nxt


def inverse_cdf_margin(p: np.ndarray, u: float, v: int) -> float:
    """How far the draw's target mass u * sum(p) lies from the CDF boundaries of the token v
    it selected, as a fraction of sum(p): min(cdf[v] - target, target - cdf[v - 1])."""
    cdf = np.cumsum(p)
    tot = cdf[-1]
    tgt = u * tot
    hi = cdf[v] - tgt
    lo = tgt - (cdf[v - 1] if v > 0 else 0.0)
    return float(min(abs(hi), abs(lo)) / tot)


def walk_sampled_margin(tab: ResidualTables, depth, seed: int, trial: int, rnd: int):
    """walk_sampled plus the smallest decision margin of the walk: |u q(c) - p'(c)| over the
    acceptance tests it made and the draw's distance to its CDF boundaries. A device walk
    whose probabilities differ from these by float rounding can only decide differently
    where this margin is of the order of that rounding. Returns ((accept_len,
    accept_node, next_token), margin)."""
    j = 0
    step = 0
    margin = np.inf
    while True:
        nxt = -1
        for i, c in enumerate(tab.kids[j]):
            u = uniform(seed, trial, rnd, step)
            step += 1
            margin = min(margin, abs(u * tab.qc[j][i] - tab.pc[j][i]))
            if u * tab.qc[j][i] < tab.pc[j][i]:
                nxt = c
                break
        if nxt < 0:
            u = uniform(seed, trial, rnd, step)
            v = sample_inverse_cdf(tab.final[j], u)
            margin = min(margin, inverse_cdf_margin(tab.final[j], u, v))
            return (depth[j], j, v), float(margin)
        j = nxt


def exact_outcomes(tab: ResidualTables):
    """Exact law of the walk: stop[j] = P(the walk ends at node j); the extra token then
    follows tab.final[j]. Also returns reach[j] = P(the walk visits j)."""
    n1 = len(tab.kids)
    reach = np.zeros(n1)
    stop = np.zeros(n1)
    reach[0] = 1.0
    for j in range(n1):
        r = reach[j]
        for i, c in enumerate(tab.kids[j]):
            q, p = tab.qc[j][i], tab.pc[j][i]
            a = min(1.0, p / q) if q > 0.0 else 1.0
            reach[c] = r * a
            r = r * (1.0 - a)
        stop[j] = r
    return stop, reach


def walk_match(parent, token, depth, target_rows: np.ndarray, T: float, seed: int, trial: int, rnd: int):
    """Target-sample matching for one (trial, round): one Philox uniform per visited node
    (step 0, 1, ...). Returns (accept_len, accept_node, next_token)."""
    kids = children_lists(parent)
    j = 0
    step = 0
    while True:
        u = uniform(seed, trial, rnd, step)
        step += 1
        x = sample_inverse_cdf(softmax_row(target_rows[j], T), u)
        nxt = -1
        for c in kids[j]:
            if token[c] == x:
                nxt = c
                break
        if nxt < 0:
            return depth[j], j, x
        j = nxt


def walk_match_margin(parent, token, depth, target_rows: np.ndarray, T: float, seed: int, trial: int, rnd: int):
    """walk_match plus the smallest distance of its draws' target masses to their CDF
    boundaries (as a fraction of the row's mass). Returns ((accept_len, accept_node,
    next_token), margin)."""
    kids = children_lists(parent)
    j = 0
    step = 0
    margin = np.inf
    while True:
        u = uniform(seed, trial, rnd, step)
        step += 1
        p = softmax_row(target_rows[j], T)
        x = sample_inverse_cdf(p, u)
        margin = min(margin, inverse_cdf_margin(p, u, x))
        nxt = -1
        for c in kids[j]:
            if token[c] == x:
                nxt = c
                break
        if nxt < 0:
            return (depth[j], j, x), float(margin)
        j = nxt


def match_outcomes(parent, token, target_rows: np.ndarray, T: float):
    """Exact law of target-sample matching: reach[c] = reach[j] p_j(token c) for the first
    child of j carrying that token; stop[j] = reach[j] times the p_j-mass of the tokens no
    child of j carries, and the emitted token then follows p_j restricted to those tokens.
    Returns (stop, reach, emit) with emit[j] that restricted, renormalised law (None when
    the restricted mass is 0)."""
    kids = children_lists(parent)
    n1 = len(parent)
    reach = np.zeros(n1)
    stop = np.zeros(n1)
    emit = [None] * n1
    reach[0] = 1.0
    for j in range(n1):
        p = softmax_row(target_rows[j], T)
        free = p.copy()
        for c in kids[j]:
            x = token[c]
            if free[x] > 0.0:  # the first child carrying x takes the draws of x
                reach[c] = reach[j] * p[x]
                free[x] = 0.0
        m = float(np.sum(free))
        stop[j] = reach[j] * m
        emit[j] = free / m if m > 0.0 else None
    return stop, reach, emit
