"""GPU parity: the sequential correction-with-heap builder (exact path-dependent best-first,
one correction per popped node) against the oracle, and against the depth-wise builder at
W = B, which gives the same tree."""
import numpy as np
import pytest
import torch

import draft_tree_construction_amd as dt
import synth
from oracle import depthwise, rowsweep
import oracle_pool as op
from parity_util import TOL, assert_tree_equal, dev_bf16, dev_f32, tree_to_host

pytestmark = pytest.mark.gpu


def head_on_device(E, U, P, root):
    Ed, Ud, Pd = dev_bf16(E), dev_bf16(U), dev_bf16(P)
    return Ed, dt.prepare_depthwise_head(Ud, Pd), torch.from_numpy(root.astype(np.int32)).cuda()


def check(base_host, dtype, E, U, P, root, K, B, beta, dm):
    """All rounds on the GPU against the oracle; a round with a pop decided within TOL (same
    depth, or the last pop) is checked for validity and shared scores only."""
    R = base_host.shape[0]
    bd = dev_bf16(base_host) if dtype == "bf16" else dev_f32(base_host)
    Ed, head, rd = head_on_device(E, U, P, root)
    h = tree_to_host(dt.build_tree_sequential(bd, Ed, head, dm, 64, rd, K, B, beta))
    E64, U64, P64 = (synth.f32_from_bf16(x).astype(np.float64) for x in (E, U, P))
    exact = near = 0
    for r in range(R):
        ref, gaps = depthwise.build_sequential(rowsweep.as_f64(base_host[r], dtype), E64, U64, P64, int(root[r]),
                                               K, B, beta, with_gaps=True)
        tie = min(gaps, default=np.inf) <= TOL
        near += tie
        exact += assert_tree_equal(h, r, ref, B, near_tie=tie)
    assert exact == R - near and exact >= 1, (exact, near, R)   # every round without a near tie is identical
    return exact, R


@pytest.mark.parametrize("R,L,V,dm,K,B,beta,seed", [
    (4, 6, 600, 256, 8, 40, -0.5, 1),
    (3, 16, 2000, 512, 8, 128, -0.2, 2),
    (3, 5, 1001, 256, 4, 30, 0.0, 3),     # odd V: ragged 32-token block, element loads
    (40, 4, 500, 256, 16, 60, -0.1, 4),   # two 32-round column tiles
    (130, 3, 400, 256, 4, 12, -0.1, 7),   # five column tiles: one wave per tile
    (2, 7, 300, 256, 1, 20, 0.0, 5),      # K = 1: a chain of L nodes, then the heap runs dry
    (3, 3, 64, 256, 3, 128, -0.3, 6),     # budget above the 39 prefixes: all of them
    (2, 1, 64, 256, 8, 1, 0.0, 8),        # L = 1, B = 1: the best root child
    (2, 3, 8, 256, 8, 30, -0.2, 9),       # K = V = 8: one 32-token block, most chunks empty
    (2, 4, 600, 256, 64, 128, -0.1, 10),  # K = 64, B = 128: pools of up to 8192 entries
    (2, 64, 300, 256, 4, 128, -0.2, 11),  # L = DTREE_MAX_L: chains down to depth 64
])
def test_sequential_small(R, L, V, dm, K, B, beta, seed):
    base = synth.ddtree_logits(seed=seed, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=200 + seed, R=R, L=L, V=V, d_model=dm, rank=64)
    check(base, "bf16", E, U, P, root, K, B, beta, dm)


def test_sequential_float32_base():
    R, L, V, dm = 3, 5, 700, 256
    rng = np.random.default_rng(18)
    base = (2.0 * rng.standard_normal((R, L, V))).astype(np.float32)
    E, U, P, root = synth.correction_head(seed=19, R=R, L=L, V=V, d_model=dm, rank=64)
    check(base, "f32", E, U, P, root, 8, 40, -0.3, dm)


def test_sequential_equals_depthwise_width_b():
    """Same inputs, same tree as the depth-wise builder at W = B (both on the GPU)."""
    R, L, V, dm, K, B = 6, 8, 3000, 256, 8, 64
    base = synth.ddtree_logits(seed=21, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=22, R=R, L=L, V=V, d_model=dm, rank=64)
    bd = dev_bf16(base)
    Ed, head, rd = head_on_device(E, U, P, root)
    hs = tree_to_host(dt.build_tree_sequential(bd, Ed, head, dm, 64, rd, K, B, -0.2))
    hw = tree_to_host(dt.build_tree_depthwise_prepared(bd, Ed, head, dm, 64, rd, K, B, B, -0.2))
    same = 0
    for r in range(R):
        if all(np.array_equal(hs[k][r], hw[k][r]) for k in ("parent", "token", "depth", "mask", "n")):
            np.testing.assert_allclose(hs["score"][r], hw["score"][r], rtol=0, atol=TOL)
            same += 1
    assert same >= R - 1, same


def test_sequential_full_config_sampled_rounds():
    """Exact best-first at the depth-wise workload's full size (R=64, L=16, V=151936,
    d_model=1024, K=8, B=128, beta=0) in one call; eight rounds checked against the oracle."""
    base = synth.ddtree_logits(seed=2)
    E, U, P, root = synth.correction_head(seed=3)
    bd = dev_bf16(base)
    Ed, head, rd = head_on_device(E, U, P, root)
    h = tree_to_host(dt.build_tree_sequential(bd, Ed, head, 1024, 64, rd, 8, 128, 0.0))
    rounds = list(range(0, 64, 8))
    tasks = [(base[r], op.gather_head_rows(E, base[r], int(root[r]), 8), U, P, int(root[r]), 8, 128, 0.0)
             for r in rounds]
    ref = op.pmap(op.sequential_task, tasks)
    exact = sum(assert_tree_equal(h, r, t, 128, near_tie=min(g) <= TOL) for r, (t, g) in zip(rounds, ref))
    assert exact >= 6, exact
