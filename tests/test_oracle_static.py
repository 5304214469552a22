"""Pins for the oracle's static D x K grid expansion (CPU only)."""
import itertools

import numpy as np
import pytest
from scipy.special import log_softmax

from oracle import static


@pytest.mark.parametrize("seed", range(6))
def test_each_depth_is_the_exact_top_k_paths_of_that_length(seed):
    """With one child distribution per position, the best K of the K x K grid at depth d
    are the K best of all V^d paths of length d (brute force over a tiny vocabulary):
    the prefix of a top-K path is itself top-K, and its last token is among its
    position's top K. Continuous logits, so no ties."""
    rng = np.random.default_rng(seed)
    L, V = 4, 5
    K = int(rng.integers(1, V + 1))
    D = int(rng.integers(1, L + 1))
    z = rng.standard_normal((L, V)) * 2.0
    t = static.build_static(z, K, D)
    paths = t.paths()
    lp = log_softmax(z, axis=1)
    for d in range(1, D + 1):
        allp = sorted(itertools.product(range(V), repeat=d), key=lambda p: -sum(lp[i, p[i]] for i in range(d)))
        got = [paths[i] for i in range(1, t.n + 1) if t.depth[i] == d]
        assert got == allp[:K]  # same set, and within a depth in score order
        for i in range(1, t.n + 1):
            if t.depth[i] == d:
                exact = sum(lp[j, paths[i][j]] for j in range(d))
                assert abs(t.score[i] - exact) < 1e-12


def test_width_one_is_the_greedy_chain():
    rng = np.random.default_rng(3)
    L, V = 6, 40
    z = rng.standard_normal((L, V)) * 3.0
    t = static.build_static(z, 1, L)
    assert t.n == L
    assert t.token[1:] == [int(np.argmax(z[d])) for d in range(L)]
    assert t.parent[1:] == list(range(L))


def test_shape_k_per_depth_and_parents_in_previous_depth():
    rng = np.random.default_rng(4)
    L, V, K, D = 8, 300, 10, 6
    z = rng.standard_normal((L, V)) * 2.5
    t = static.build_static(z, K, D)
    assert t.n == K * D
    for d in range(1, D + 1):
        idx = [i for i in range(1, t.n + 1) if t.depth[i] == d]
        assert idx == list(range(1 + (d - 1) * K, 1 + d * K))
        for i in idx:
            assert t.parent[i] < i and t.depth[t.parent[i]] == d - 1
            assert t.score[i] <= t.score[t.parent[i]]
    # every (parent, token) pair appears once
    assert len(set(zip(t.parent[1:], t.token[1:]))) == t.n


def test_equal_logits_follow_parent_position_then_token_rank():
    """All paths of a depth tie: the reading orders them by the parent's position, then
    by the token's rank (equal logits: ascending id), so depth 2 holds the first kept
    node's K smallest ids."""
    z = np.zeros((3, 7))
    t = static.build_static(z, 3, 3)
    assert t.token[1:4] == [0, 1, 2]
    assert t.parent[4:7] == [1, 1, 1] and t.token[4:7] == [0, 1, 2]
    assert t.parent[7:10] == [4, 4, 4]
    assert abs(t.score[9] - 3 * np.log(1 / 7)) < 1e-12


def test_bad_arguments_raise():
    z = np.zeros((2, 4))
    for K, D in [(0, 1), (5, 1), (2, 0), (2, 3)]:
        with pytest.raises(ValueError):
            static.build_static(z, K, D)
