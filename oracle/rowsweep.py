"""Row log-softmax and top-K (oracle; test infrastructure only).

Follows the DDTree blog, section 3.3 ("probability computation and caching"):
scores are compared as log-probabilities, log q, so that products do not
underflow, and each position needs its top-K tokens with their log-probs. The
DARTree summary's Algorithm 1 selects C_d = TopK(L_d^base, K) from the base
logits of each depth. Ties between equal logits go to the smaller vocabulary
index, the greedy tie-break the course notes give for equal maximum logits.
"""
from __future__ import annotations

import numpy as np


def as_f64(logits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored logits to float64 exactly. dtype is 'bf16' (uint16 bits) or 'f32'."""
    if dtype == "bf16":
        return (np.asarray(logits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(logits, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def logsumexp_row(z: np.ndarray) -> float:
    """ln sum_v exp(z_v), written as max plus the log of a shifted sum."""
    z = np.asarray(z, dtype=np.float64)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logits")
    m = float(np.max(z))
    return m + float(np.log(np.sum(np.exp(z - m))))


def rank_order(z: np.ndarray) -> np.ndarray:
    """Token ids of one row sorted by (logit descending, id ascending).

    A stable sort of -z keeps equal logits in ascending id order; -0.0 and +0.0
    compare equal, so they are ordered by id as well.
    """
    return np.argsort(-np.asarray(z, dtype=np.float64), kind="stable")


def topk_logsoftmax(z_rows: np.ndarray, K: int):
    """For each row: lse, the top-K ids (rank order), their logits and log-probs lp = z - lse.

    z_rows: float64 [rows, V]. Returns (lse [rows], ids [rows, K] int64,
    zk [rows, K] float64, lp [rows, K] float64).
    """
    z_rows = np.asarray(z_rows, dtype=np.float64)
    rows, V = z_rows.shape
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    lse = np.empty(rows)
    ids = np.empty((rows, K), dtype=np.int64)
    zk = np.empty((rows, K))
    for i in range(rows):
        lse[i] = logsumexp_row(z_rows[i])
        order = rank_order(z_rows[i])[:K]
        ids[i] = order
        zk[i] = z_rows[i, order]
    lp = zk - lse[:, None]
    return lse, ids, zk, lp
