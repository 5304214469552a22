"""Round-parallel runs of the oracle for the full-size parity tests (test infrastructure).

Rounds are independent, so the oracle's per-round functions are mapped over a pool of
worker processes. The workers are spawned and import numpy and ``oracle`` only (never
torch or the HIP library), so they never touch the GPU. Each task carries one round's
stored inputs (bf16 bits or float32), widened inside the worker exactly as the tests
widen them. Workers: min(16, cpu count).
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

from oracle import accept, depthwise, gated, marginal, rowsweep, static

_pool = None


def n_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    """fn over items in worker processes, results in order."""
    global _pool
    items = list(items)
    if len(items) <= 1:
        return [fn(x) for x in items]
    if _pool is None:
        _pool = cf.ProcessPoolExecutor(max_workers=n_workers(), mp_context=mp.get_context("spawn"))
    return list(_pool.map(fn, items, chunksize=1))


# ---------------------------------------------------------------- per-round tasks
def marginal_task(args):
    """(logits [L, V], dtype, K, B, beta) -> (Tree, gap). gap = score of the B-th minus the
    (B+1)-th prefix when they lie at different depths (inf otherwise): within one depth both
    sides order by exact logit sums, so only a cut between depths compares scores that carry
    each side's own LSE rounding."""
    x, dtype, K, B, beta = args
    z = rowsweep.as_f64(x, dtype)
    t = marginal.build_marginal(z, K, B, beta)
    L, V = z.shape
    Ke = min(B, V) if K == 0 else K
    lse = np.array([rowsweep.logsumexp_row(z[d]) for d in range(L)])
    ranks = np.stack([rowsweep.rank_order(z[d])[:Ke] for d in range(L)])
    zk = np.take_along_axis(z, ranks, axis=1)
    pops = marginal.heap_topb(zk, lse, B + 1, float(beta))
    if len(pops) <= B or pops[B - 1]["depth"] == pops[B]["depth"]:
        return t, np.inf
    return t, pops[B - 1]["s"] - pops[B]["s"]


def gated_task(args):
    """(logits [L, V] bf16 bits, K_root, mu, N) -> Tree (top-K restricted pool)."""
    x, K_root, mu, N = args
    return gated.build_gated(rowsweep.as_f64(x, "bf16"), K_root, mu, N, full_pool=False)


def static_task(args):
    """(logits [L, V] bf16 bits, K, D) -> Tree."""
    x, K, D = args
    return static.build_static(rowsweep.as_f64(x, "bf16"), K, D)


class GatheredRows:
    """Rows of E for the tokens a round can ask for (its root token and every position's
    top-K candidates), indexed like the full table; any other token raises."""

    def __init__(self, tokens, rows_bf16):
        self.rows = {int(t): i for i, t in enumerate(tokens)}
        self.data = (np.asarray(rows_bf16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)

    def __getitem__(self, idx):
        idx = np.atleast_1d(np.asarray(idx))
        return self.data[[self.rows[int(t)] for t in idx]].astype(np.float64)


def gather_head_rows(E_bits, base_bits, root_tok: int, K: int):
    """The tokens a depth-wise round can use as states and their E rows (bf16 bits)."""
    z = rowsweep.as_f64(base_bits, "bf16")
    toks = {int(root_tok)}
    for d in range(z.shape[0]):
        toks.update(int(t) for t in rowsweep.rank_order(z[d])[:K])
    toks = sorted(toks)
    return toks, np.asarray(E_bits[toks])


def depthwise_task(args):
    """(base [L, V] bf16 bits, (tokens, E rows), U bits, P bits, root, K, W, B, beta)
    -> (Tree, gaps)."""
    base, (toks, erows), U_bits, P_bits, root, K, W, B, beta = args
    widen = lambda b: (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    tree, _, gaps = depthwise.build_depthwise(rowsweep.as_f64(base, "bf16"), GatheredRows(toks, erows), widen(U_bits),
                                              widen(P_bits), int(root), K, W, B, beta, with_super=True)
    return tree, gaps


def sequential_task(args):
    """(base [L, V] bf16 bits, (tokens, E rows), U bits, P bits, root, K, B, beta) -> (Tree, gaps)."""
    base, (toks, erows), U_bits, P_bits, root, K, B, beta = args
    widen = lambda b: (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return depthwise.build_sequential(rowsweep.as_f64(base, "bf16"), GatheredRows(toks, erows), widen(U_bits),
                                      widen(P_bits), int(root), K, B, beta, with_gaps=True)


def greedy_task(args):
    """(parent, token, depth, target rows [n+1, V] bf16 bits) -> (accept_len, node, token)."""
    par, tok, dep, tgt = args
    return accept.walk_greedy(par, tok, dep, rowsweep.as_f64(tgt, "bf16"))


def sampled_task(args):
    """(parent, token, depth, target rows [n+1, V], draft rows [L, V] (bf16 bits), T, seed,
    trials, round) -> ([((accept_len, node, token), margin) per trial], stop law)."""
    par, tok, dep, tgt, dr, T, seed, trials, rnd = args
    tab = accept.ResidualTables(par, tok, dep, rowsweep.as_f64(tgt, "bf16"), rowsweep.as_f64(dr, "bf16"), T)
    outs = [accept.walk_sampled_margin(tab, dep, seed, t, rnd) for t in trials]
    stop, _ = accept.exact_outcomes(tab)
    return outs, stop


def match_task(args):
    """(parent, token, depth, target rows [n+1, V] bf16 bits, T, seed, trials, round)
    -> [((accept_len, node, token), margin) per trial]."""
    par, tok, dep, tgt, T, seed, trials, rnd = args
    rows = rowsweep.as_f64(tgt, "bf16")
    return [accept.walk_match_margin(par, tok, dep, rows, T, seed, t, rnd) for t in trials]


class TokenRows:
    """Rows of a [V, h] table for the tokens a round can ask for, indexed like the table."""

    def __init__(self, tokens, rows):
        self.at = {int(t): i for i, t in enumerate(tokens)}
        self.rows = np.asarray(rows, dtype=np.float64)

    def __getitem__(self, tok):
        return self.rows[self.at[int(tok)]]


def gather_tdes_params(prm, base_bits, dtype, root_tok: int, K: int):
    """The edge MLP's parameters for one round, float64, with Gp and Gc cut down to the
    tokens the round can use (its root token and every position's top-K candidates)."""
    z = rowsweep.as_f64(base_bits, dtype)
    toks = {int(root_tok)}
    for d in range(z.shape[0]):
        toks.update(int(t) for t in rowsweep.rank_order(z[d])[:K])
    toks = sorted(toks)
    out = {k: np.asarray(prm[k], dtype=np.float32).astype(np.float64) for k in ("Ed", "W", "b", "w")}
    out["Gp"] = TokenRows(toks, np.asarray(prm["Gp"], dtype=np.float32)[toks])
    out["Gc"] = TokenRows(toks, np.asarray(prm["Gc"], dtype=np.float32)[toks])
    out["b0"] = float(np.float32(prm["b0"]))
    return out


def tdes_task(args):
    """(logits [L, V], dtype, root token, float64 params, K, budget, s) -> (Tree, gap)."""
    from oracle import tdes
    x, dtype, root, prm, K, B, s = args
    return tdes.build_tdes(rowsweep.as_f64(x, dtype), int(root), prm, K, B, s)
