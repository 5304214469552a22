"""Seeded synthetic inputs for the draft-tree hot path.

This module only draws random numbers and stores them; it holds none of the
method's arithmetic (no softmax, no selection, no scoring). Both the CPU
oracle and the HIP path consume exactly the bytes produced here.

Stand-in for the pages' workloads: the pages measure on GSM8K, MATH-500,
HumanEval, MT-Bench and others with Qwen3 drafters and targets. None of that is
used. The logits take the pages' shapes instead: Qwen3's vocabulary width
V = 151,936, a DFlash block of L = 16 positions, budgets B = 64..128, and one
planted boosted token per position standing in for the peaked distributions of
a real drafter.

Recipes (all tensors row-major, numpy PCG64 via ``default_rng(seed)``, drawn in
the order listed; fp32 -> bf16 is round-to-nearest-even, stored as uint16):

* tiny marginal (seed 1): z = 2*N(0,1) fp32 [R=4, L=4, V=32].
* DDTree shape (seed 2): z = 3*N(0,1) fp32 [R, L, V]; tok = integers(0, V, [R, L]);
  boost = uniform(2, 12, [R, L]); z[r, l, tok[r, l]] += boost -> bf16.
* DARTree correction head (seed 3): E = 0.02*N [V, d_model], U = 0.02*N
  [L, d_model, rank], P = 0.02*N [rank, V] -> bf16; root_tok = integers(0, V, [R]).
  Its base logits are the DDTree-shape tensor.
* TALON (seed 4): z = 3*N(0,1) [R, L, V]; tok = integers(0, V, [R, L]);
  b = uniform(0, 12, [R]); z[r, l, tok[r, l]] += b[r] -> bf16.
* Verification (seed 5): noise = N(0,1) [R, n+1, V];
  target[r, j] = bf16(float(draft[r, min(depth[r, j], L-1)]) + noise[r, j]).
"""
from __future__ import annotations

import numpy as np

V_QWEN3 = 151936
PHILOX_SEED = 0x5EED5EED


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (uint16), round to nearest, ties to even. Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_from_bf16(b: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> fp32, exact widening."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def tiny_marginal(seed: int = 1, R: int = 4, L: int = 4, V: int = 32) -> np.ndarray:
    """fp32 logits [R, L, V] ~ 2*N(0,1)."""
    rng = np.random.default_rng(seed)
    return (np.float32(2.0) * rng.standard_normal((R, L, V), dtype=np.float32)).astype(np.float32)


def ddtree_logits(seed: int = 2, R: int = 64, L: int = 16, V: int = V_QWEN3,
                  boost_lo: float = 2.0, boost_hi: float = 12.0) -> np.ndarray:
    """bf16 bits [R, L, V]: 3*N(0,1) plus one planted token per position boosted by U(lo, hi)."""
    rng = np.random.default_rng(seed)
    out = np.empty((R, L, V), dtype=np.uint16)
    # Draw the normals round by round (same stream as one big draw) to bound memory.
    zs = []
    for r in range(R):
        zs.append(np.float32(3.0) * rng.standard_normal((L, V), dtype=np.float32))
    tok = rng.integers(0, V, (R, L))
    boost = rng.uniform(boost_lo, boost_hi, (R, L))
    for r in range(R):
        z = zs[r]
        z[np.arange(L), tok[r]] += boost[r].astype(np.float32)
        out[r] = bf16_from_f32(z)
        zs[r] = None
    return out


def talon_logits(seed: int = 4, R: int = 64, L: int = 16, V: int = V_QWEN3) -> np.ndarray:
    """bf16 bits [R, L, V]: 3*N(0,1) plus one planted token per position, boost b_r ~ U(0, 12) per round."""
    rng = np.random.default_rng(seed)
    zs = [np.float32(3.0) * rng.standard_normal((L, V), dtype=np.float32) for _ in range(R)]
    tok = rng.integers(0, V, (R, L))
    b = rng.uniform(0.0, 12.0, (R,))
    out = np.empty((R, L, V), dtype=np.uint16)
    for r in range(R):
        z = zs[r]
        z[np.arange(L), tok[r]] += np.float32(b[r])
        out[r] = bf16_from_f32(z)
        zs[r] = None
    return out


def correction_head(seed: int = 3, R: int = 64, L: int = 16, V: int = V_QWEN3,
                    d_model: int = 1024, rank: int = 64):
    """Synthetic Markov correction head: E [V, d_model], U [L, d_model, rank], P [rank, V] (bf16 bits), root_tok [R]."""
    rng = np.random.default_rng(seed)
    E = np.empty((V, d_model), dtype=np.uint16)
    step = 8192
    for v0 in range(0, V, step):
        v1 = min(V, v0 + step)
        E[v0:v1] = bf16_from_f32(np.float32(0.02) * rng.standard_normal((v1 - v0, d_model), dtype=np.float32))
    U = bf16_from_f32(np.float32(0.02) * rng.standard_normal((L, d_model, rank), dtype=np.float32))
    P = bf16_from_f32(np.float32(0.02) * rng.standard_normal((rank, V), dtype=np.float32))
    root_tok = rng.integers(0, V, (R,)).astype(np.int32)
    return E, U, P, root_tok


def verification_target(draft_bf16: np.ndarray, depth: np.ndarray, seed: int = 5,
                        rows: int | None = None) -> np.ndarray:
    """Target logits [R, rows, V] bf16 bits, draft-correlated: bf16(float(draft[r, min(depth, L-1)]) + N(0,1)).

    ``depth[r, j]`` is the depth of tree node j in round r (0 for the root); slots
    beyond a round's tree may hold any value >= 0 (their rows are still drawn so
    the stream does not depend on tree sizes). ``rows`` defaults to depth.shape[1].
    """
    R, L, V = draft_bf16.shape
    rows = depth.shape[1] if rows is None else rows
    rng = np.random.default_rng(seed)
    out = np.empty((R, rows, V), dtype=np.uint16)
    draft = f32_from_bf16(draft_bf16)
    for r in range(R):
        noise = rng.standard_normal((rows, V), dtype=np.float32)
        pos = np.minimum(np.maximum(depth[r], 0), L - 1)
        out[r] = bf16_from_f32(draft[r, pos] + noise)
    return out


def edge_mlp(seed: int = 6, R: int = 64, L: int = 16, V: int = V_QWEN3, hp: int = 64, hc: int = 64,
             hd: int = 16, H: int = 128):
    """Random-init edge MLP (no trained weights), float32: projected token tables Gp [V, hp] and
    Gc [V, hc] ~ N(0, 1), depth embeddings Ed [L, hd] ~ N(0, 1), W [H, hp+hc+hd] ~ N(0, 1/fan_in),
    b [H] ~ N(0, 0.1^2), w [H] ~ N(0, 2/H), b0 = 0, scale s = 1; root_tok [R] uniform."""
    rng = np.random.default_rng(seed)
    n = hp + hc + hd
    prm = dict(Gp=rng.standard_normal((V, hp), dtype=np.float32), Gc=rng.standard_normal((V, hc), dtype=np.float32),
               Ed=rng.standard_normal((L, hd), dtype=np.float32),
               W=(rng.standard_normal((H, n), dtype=np.float32) / np.float32(np.sqrt(n))).astype(np.float32),
               b=(np.float32(0.1) * rng.standard_normal(H, dtype=np.float32)).astype(np.float32),
               w=(rng.standard_normal(H, dtype=np.float32) * np.float32(np.sqrt(2.0 / H))).astype(np.float32),
               b0=0.0, s=1.0)
    root_tok = rng.integers(0, V, (R,)).astype(np.int32)
    return prm, root_tok


def tie_rows(V: int, rows: int, seed: int = 11) -> np.ndarray:
    """bf16 rows with many exact ties: values drawn from a small grid, so the top-K and argmax tie-breaks matter."""
    rng = np.random.default_rng(seed)
    grid = np.array([-3.0, -1.0, 0.0, 0.5, 1.0, 2.0, 2.5, 3.0], dtype=np.float32)
    z = grid[rng.integers(0, len(grid), (rows, V))]
    return bf16_from_f32(z)
