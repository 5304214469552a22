"""GPU parity: one row sweep shared by several builders (dtree_topk_lists and the *_lists
builders). The lists against the oracle's top-K; the builders from lists against the
oracle and, bit for bit, against the same builders sweeping the logits themselves."""
import numpy as np
import pytest
import torch

import draft_tree_construction_amd as dt
import synth
from oracle import rowsweep
from parity_util import TOL, assert_tree_equal, dev_bf16, dev_f32, tree_to_host
from test_gpu_builders import oracle_marginal

pytestmark = pytest.mark.gpu


def assert_same_tree(a: dt.Tree, b: dt.Tree):
    ha, hb = tree_to_host(a), tree_to_host(b)
    for k in ha:
        np.testing.assert_array_equal(ha[k], hb[k], err_msg=k)


@pytest.mark.parametrize("rows,V,K,dtype,seed", [
    (7, 100003, 64, "bf16", 2),   # odd V: unaligned rows, split rows, ragged tail
    (16, 32, 8, "f32", 1),
    (9, 40000, 128, "bf16", 8),
    (3, 64, 64, "f32", 4),        # K = V
])
def test_topk_lists_against_oracle(rows, V, K, dtype, seed):
    rng = np.random.default_rng(seed)
    x = (3.0 * rng.standard_normal((rows, V))).astype(np.float32)
    host = synth.bf16_from_f32(x) if dtype == "bf16" else x
    z = rowsweep.as_f64(host, dtype)
    d = dev_bf16(host) if dtype == "bf16" else dev_f32(host)
    li = dt.topk_lists(d, K)
    torch.cuda.synchronize()
    zk, ids, lse = li.zk.cpu().numpy(), li.ids.cpu().numpy(), li.lse.cpu().numpy()
    r_lse, r_ids, _, _ = rowsweep.topk_logsoftmax(z, K)
    np.testing.assert_array_equal(ids, r_ids)
    np.testing.assert_array_equal(zk.astype(np.float64), np.take_along_axis(z, r_ids.astype(np.int64), axis=1))
    np.testing.assert_allclose(lse, r_lse, rtol=0, atol=TOL)


@pytest.mark.parametrize("R,L,V,K,B,beta", [
    (6, 16, 20000, 64, 64, 0.0),
    (4, 7, 500, 16, 100, -0.3),
    (3, 1, 1000, 10, 10, 0.0),
])
def test_marginal_lists_against_oracle(R, L, V, K, B, beta):
    host = synth.ddtree_logits(seed=20 + V, R=R, L=L, V=V)
    d = dev_bf16(host)
    tr = dt.build_tree_marginal_lists(dt.topk_lists(d, K), R, L, B, beta)
    h = tree_to_host(tr)
    for r in range(R):
        ref, gap = oracle_marginal(rowsweep.as_f64(host[r], "bf16"), K, B, beta)
        assert_tree_equal(h, r, ref, B, near_tie=gap <= TOL)
    assert_same_tree(tr, dt.build_tree_marginal(d, K, B, beta))


def test_marginal_lists_full_config_equals_marginal():
    """The DDTree-shape config (R = 64, L = 16, V = 151,936, K = B = 64): the tree from
    shared lists is the standalone builder's, bit for bit, on every round."""
    d = dev_bf16(synth.ddtree_logits(seed=2))
    assert_same_tree(dt.build_tree_marginal_lists(dt.topk_lists(d, 64), 64, 16, 64, 0.0),
                     dt.build_tree_marginal(d, 64, 64, 0.0))


@pytest.mark.parametrize("R,L,V,dm,K,ks,W,B,beta,seed", [
    (4, 6, 600, 64, 8, 64, 32, 40, -0.5, 1),     # lists of 64 feed K = 8
    (3, 5, 1001, 64, 4, 4, 16, 30, -0.2, 3),     # ks = K; odd V
    (2, 4, 500, 64, 16, 128, 64, 100, 0.0, 4),   # the widest lists
])
def test_depthwise_lists_equals_prepared(R, L, V, dm, K, ks, W, B, beta, seed):
    base = synth.ddtree_logits(seed=seed, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=seed + 100, R=R, L=L, V=V, d_model=dm)
    bd, Ed, Ud, Pd = dev_bf16(base), dev_bf16(E), dev_bf16(U), dev_bf16(P)
    rd = torch.from_numpy(root.astype(np.int32)).cuda()
    head = dt.prepare_depthwise_head(Ud, Pd)
    a = dt.build_tree_depthwise_lists(bd, dt.topk_lists(bd, ks), Ed, head, dm, 64, rd, K, W, B, beta)
    b = dt.build_tree_depthwise_prepared(bd, Ed, head, dm, 64, rd, K, W, B, beta)
    assert_same_tree(a, b)


def test_depthwise_lists_full_config_equals_prepared():
    """The DARTree config (K = 8, W = 32, B = 128) from the marginal builder's lists of 64:
    every round's tree equals the standalone builder's, bit for bit."""
    base = synth.ddtree_logits(seed=2)
    E, U, P, root = synth.correction_head(seed=3)
    bd, Ed, Ud, Pd = dev_bf16(base), dev_bf16(E), dev_bf16(U), dev_bf16(P)
    rd = torch.from_numpy(root.astype(np.int32)).cuda()
    head = dt.prepare_depthwise_head(Ud, Pd)
    li = dt.topk_lists(bd, 64)
    a = dt.build_tree_depthwise_lists(bd, li, Ed, head, 1024, 64, rd, 8, 32, 128, -0.5)
    b = dt.build_tree_depthwise_prepared(bd, Ed, head, 1024, 64, rd, 8, 32, 128, -0.5)
    assert_same_tree(a, b)
    assert_same_tree(dt.build_tree_marginal_lists(li, 64, 16, 64, 0.0), dt.build_tree_marginal(bd, 64, 64, 0.0))
