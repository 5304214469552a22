"""GPU parity: DARTree depth-wise super-tree + deferred Top-B (a3 + a4 + a6) against the oracle."""
import numpy as np
import pytest
import torch

import draft_tree_construction_amd as dt
import synth
from oracle import depthwise, marginal, rowsweep
import oracle_pool as op
from parity_util import TOL, assert_tree_equal, assert_tree_valid, dev_bf16, dev_f32, tree_to_host

pytestmark = pytest.mark.gpu


def head_to_device(E, U, P, root):
    return dev_bf16(E), dev_bf16(U), dev_bf16(P), torch.from_numpy(root.astype(np.int32)).cuda()


def check(base_host, dtype, E, U, P, root, K, W, B, beta, rounds=None):
    """Run all rounds on the GPU; compare the given rounds with the oracle. A round whose
    oracle selection gap (width cut of any depth, or the B cut) is <= 1e-5 is checked for
    validity and shared-prefix scores only. Returns (exact rounds, compared rounds)."""
    R = base_host.shape[0]
    bd = dev_bf16(base_host) if dtype == "bf16" else dev_f32(base_host)
    Ed, Ud, Pd, rd = head_to_device(E, U, P, root)
    tr = dt.build_tree_depthwise(bd, Ed, Ud, Pd, rd, K, W, B, beta)
    h = tree_to_host(tr)
    E64, U64, P64 = (synth.f32_from_bf16(x).astype(np.float64) for x in (E, U, P))
    rounds = range(R) if rounds is None else rounds
    exact = near = 0
    for r in rounds:
        z = rowsweep.as_f64(base_host[r], dtype)
        ref, _, gaps = depthwise.build_depthwise(z, E64, U64, P64, int(root[r]), K, W, B, beta, with_super=True)
        tie = min(gaps) <= TOL
        near += tie
        exact += assert_tree_equal(h, r, ref, B, near_tie=tie)
    n = len(list(rounds))
    assert exact == n - near, (exact, near, n)  # every round without a near tie is identical
    return exact, n


@pytest.mark.parametrize("R,L,V,dm,K,W,B,beta,seed", [
    (4, 6, 600, 64, 8, 32, 40, -0.5, 1),
    (3, 16, 2000, 128, 8, 32, 128, -0.5, 2),
    (3, 5, 1001, 64, 4, 16, 30, -0.2, 3),     # odd V: ragged 32-token block
    (2, 4, 500, 64, 16, 64, 100, 0.0, 4),     # two 32-branch tiles per round
    (3, 7, 300, 64, 5, 1, 7, -0.1, 5),        # width 1: one corrected chain
    (3, 5, 900, 64, 32, 32, 90, -0.3, 6),     # L K^2 > 4096: log q~ rows staged depth by depth
    (2, 3, 700, 64, 64, 16, 40, 0.0, 7),      # K = 64: sixteen sorted lists per depth
    (2, 4, 800, 64, 10, 100, 128, -0.2, 8),   # W = 100 (two keys per lane), ragged last list
    (12, 16, 2500, 64, 8, 32, 128, -0.5, 9),  # three tile groups: 88 V chunks, partials one by one
    (8, 16, 2500, 64, 8, 32, 128, -0.5, 10),  # two tile groups: 128 V chunks
    (2, 64, 600, 64, 4, 8, 128, -0.3, 11),    # L = DTREE_MAX_L: 64 depths, 512 super-tree nodes
])
def test_depthwise_small(R, L, V, dm, K, W, B, beta, seed):
    base = synth.ddtree_logits(seed=seed, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=100 + seed, R=R, L=L, V=V, d_model=dm, rank=64)
    exact, n = check(base, "bf16", E, U, P, root, K, W, B, beta)
    assert exact >= (n + 1) // 2, (exact, n)


def test_depthwise_float32_base():
    R, L, V, dm = 3, 5, 700, 64
    rng = np.random.default_rng(8)
    base = (2.0 * rng.standard_normal((R, L, V))).astype(np.float32)
    E, U, P, root = synth.correction_head(seed=9, R=R, L=L, V=V, d_model=dm, rank=64)
    exact, n = check(base, "f32", E, U, P, root, 8, 16, 40, -0.3)
    assert exact >= n - 1


def test_depthwise_loose_bound_uses_running_max():
    """A head large enough that the max-logit bound exceeds 10 nats switches tiles to the
    running-max path; results must still match."""
    R, L, V, dm = 2, 4, 800, 64
    base = synth.ddtree_logits(seed=6, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=7, R=R, L=L, V=V, d_model=dm, rank=64)
    U = synth.bf16_from_f32(synth.f32_from_bf16(U) * np.float32(40.0))
    P = synth.bf16_from_f32(synth.f32_from_bf16(P) * np.float32(40.0))
    exact, n = check(base, "bf16", E, U, P, root, 8, 32, 60, -0.5)
    assert exact >= n - 1


def test_depthwise_zero_correction_is_marginal_tree():
    """U = 0 makes every branch's correction vanish; with W >= B and K >= B the depth-wise
    tree is the marginal Top-B tree (fp32 logits: no exact ties)."""
    R, L, V, B = 3, 6, 500, 32
    rng = np.random.default_rng(10)
    base = (2.0 * rng.standard_normal((R, L, V))).astype(np.float32)
    E, U, P, root = synth.correction_head(seed=11, R=R, L=L, V=V, d_model=64, rank=64)
    U[:] = 0
    Ed, Ud, Pd, rd = head_to_device(E, U, P, root)
    tr = dt.build_tree_depthwise(dev_f32(base), Ed, Ud, Pd, rd, B, B, B, -0.25)
    h = tree_to_host(tr)
    for r in range(R):
        ref = marginal.build_marginal(rowsweep.as_f64(base[r], "f32"), B, B, -0.25)
        assert_tree_equal(h, r, ref, B)


_HEAD = {}


def full_head():
    if "h" not in _HEAD:
        _HEAD["h"] = (synth.ddtree_logits(seed=2), synth.correction_head(seed=3))
    return _HEAD["h"]


def check_full(K, W, B, beta, rounds):
    """The DARTree config at full size in one launch: the given rounds against the oracle
    (run round-parallel on E rows gathered per round), and every round of the batch for the
    super-tree invariants: a valid monotone prefix-closed tree of B nodes, at most W nodes
    per depth, each depth-d token among the top K of base position d."""
    base, (E, U, P, root) = full_head()
    Ed, Ud, Pd, rd = head_to_device(E, U, P, root)
    h = tree_to_host(dt.build_tree_depthwise(dev_bf16(base), Ed, Ud, Pd, rd, K, W, B, beta))
    for r in range(base.shape[0]):
        n, par, tok, dep, sc = assert_tree_valid(h, r, B)
        assert n == B
        z = rowsweep.as_f64(base[r], "bf16")
        for d in range(1, base.shape[1] + 1):
            at = [i for i in range(1, n + 1) if dep[i] == d]
            assert len(at) <= W
            if at:
                kth = np.partition(z[d - 1], -K)[-K]
                assert all(z[d - 1, tok[i]] >= kth for i in at)
    tasks = [(base[r], op.gather_head_rows(E, base[r], int(root[r]), K), U, P, int(root[r]), K, W, B, beta)
             for r in rounds]
    ref = op.pmap(op.depthwise_task, tasks)
    exact = sum(assert_tree_equal(h, r, t, B, near_tie=min(g) <= TOL) for r, (t, g) in zip(rounds, ref))
    near = sum(min(g) <= TOL for _, g in ref)
    assert exact == len(rounds) - near   # every round without a near tie is identical
    return exact, near


def test_depthwise_full_dartree_config():
    """DARTree config at full size: R=64, L=16, V=151936, E 151936x1024, U 16x1024x64,
    P 64x151936, W=32, K=8, B=128, beta=-0.5; 32 rounds against the oracle (rounds where a
    width or budget cut falls within 1e-5 are checked for validity and shared scores, and
    counted), invariants on all 64."""
    exact, near = check_full(8, 32, 128, -0.5, list(range(0, 64, 2)))
    assert exact >= 16 and near <= 8, (exact, near)


def test_depthwise_one_round_over_two_tiles():
    """K = 40 pads a round to 64 state slots: each tile holds 32 states of one round."""
    R, L, V, dm = 2, 5, 900, 64
    base = synth.ddtree_logits(seed=13, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=113, R=R, L=L, V=V, d_model=dm, rank=64)
    exact, n = check(base, "bf16", E, U, P, root, 40, 16, 60, -0.3)
    assert exact >= n - 1



def test_depthwise_width_b_exact_best_first():
    """W = B = 128 (K = 8, W*K = 1024 children per depth): the exact corrected best-first tree."""
    R, L, V, dm = 3, 6, 900, 64
    base = synth.ddtree_logits(seed=16, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=116, R=R, L=L, V=V, d_model=dm, rank=64)
    exact, n = check(base, "bf16", E, U, P, root, 8, 128, 128, 0.0)
    assert exact >= n - 1


def test_depthwise_fixed_width_keeps_every_branch():
    """DARTree (fixed): W = B / L, B = L * W, no depth bonus."""
    R, L, V, dm = 3, 16, 1200, 64
    base = synth.ddtree_logits(seed=17, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=117, R=R, L=L, V=V, d_model=dm, rank=64)
    exact, n = check(base, "bf16", E, U, P, root, 8, 8, 128, 0.0)
    assert exact >= n - 1


def test_depthwise_full_config_exact_best_first():
    """Full DARTree shapes with W = B = 128 (exact best-first, beta = 0): 8 rounds against the
    oracle, invariants on all 64."""
    exact, near = check_full(8, 128, 128, 0.0, list(range(3, 64, 8)))
    assert exact >= 6, (exact, near)


@pytest.mark.parametrize("R,L,V,dm,K,W,B,beta,seed", [
    (3, 6, 1001, 64, 8, 32, 60, -0.5, 21),            # ragged V
    (64, 16, 151936, 1024, 8, 32, 128, -0.5, 3),      # the DARTree config
])
def test_depthwise_prepared_head_gives_the_same_tree(R, L, V, dm, K, W, B, beta, seed):
    """The head prepared once (P^T, U^T, column bounds) and reused over two calls gives the
    builder's tree exactly, on a small ragged shape and the full DARTree config."""
    if V == 151936:
        base, (E, U, P, root) = full_head()
    else:
        base = synth.ddtree_logits(seed=seed, R=R, L=L, V=V)
        E, U, P, root = synth.correction_head(seed=100 + seed, R=R, L=L, V=V, d_model=dm, rank=64)
    bd = dev_bf16(base)
    Ed, Ud, Pd, rd = head_to_device(E, U, P, root)
    want = tree_to_host(dt.build_tree_depthwise(bd, Ed, Ud, Pd, rd, K, W, B, beta))
    head = dt.prepare_depthwise_head(Ud, Pd)
    for _ in range(2):
        got = tree_to_host(dt.build_tree_depthwise_prepared(bd, Ed, head, dm, 64, rd, K, W, B, beta))
        for k in ("parent", "token", "depth", "mask", "n", "score"):
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)
