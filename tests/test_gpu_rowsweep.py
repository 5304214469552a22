"""GPU parity: fused row log-softmax + top-K (a1) against the oracle, via the C ABI."""
import numpy as np
import pytest
import torch

import draft_tree_construction_amd as dt
import synth
from oracle import rowsweep
from parity_util import TOL, dev_bf16, dev_f32

pytestmark = pytest.mark.gpu


def run_and_compare(host, dtype, K):
    z = rowsweep.as_f64(host, dtype)
    d = dev_bf16(host) if dtype == "bf16" else dev_f32(host)
    lse, ids, lp = dt.topk_logsoftmax(d, K)
    torch.cuda.synchronize()
    lse, ids, lp = lse.cpu().numpy(), ids.cpu().numpy(), lp.cpu().numpy()
    r_lse, r_ids, _, r_lp = rowsweep.topk_logsoftmax(z, K)
    np.testing.assert_array_equal(ids, r_ids)
    assert_lse_close(lse, r_lse)
    np.testing.assert_allclose(lp, r_lp, rtol=0, atol=TOL)


def assert_lse_close(got, want):
    """lse is returned as float32: within 1e-5, or within float32's half-ulp for |lse| >= 64."""
    np.testing.assert_allclose(got, want, rtol=2.0 ** -24, atol=TOL)


@pytest.mark.parametrize("rows,V,K,dtype,seed", [
    (16, 32, 8, "f32", 1),        # tiny config rows
    (7, 100003, 64, "bf16", 2),   # odd V: unaligned rows, split rows, ragged tail
    (5, 8191, 17, "bf16", 3),
    (3, 64, 64, "f32", 4),        # K = V
    (2, 1, 1, "bf16", 5),         # V = 1
    (33, 2049, 8, "f32", 6),
    (9, 40000, 64, "bf16", 7),
    (9, 40000, 128, "bf16", 8),   # the marginal envelope's widest list
    (4, 151936, 128, "bf16", 9),
    (3, 262144, 128, "bf16", 10),  # a wider vocabulary than Qwen3's, split rows, K = 128
])
def test_rowsweep_random(rows, V, K, dtype, seed):
    rng = np.random.default_rng(seed)
    x = (3.0 * rng.standard_normal((rows, V))).astype(np.float32)
    host = synth.bf16_from_f32(x) if dtype == "bf16" else x
    run_and_compare(host, dtype, K)


@pytest.mark.parametrize("V,K", [(4096, 64), (151936, 64), (3000, 8), (151936, 128)])
def test_rowsweep_planted_ties(V, K):
    """Rows drawn from an 8-value grid: thousands of exact ties at the K-th value."""
    run_and_compare(synth.tie_rows(V, 6, seed=V), "bf16", K)


def test_rowsweep_constant_and_sorted_rows():
    V = 20000
    rows = np.stack([np.zeros(V), np.arange(V), -np.arange(V), np.full(V, -7.5)]).astype(np.float32)
    run_and_compare(synth.bf16_from_f32(rows), "bf16", 64)
    run_and_compare(rows, "f32", 64)
    # large magnitudes: the exponent's fp32 rounding of log2 e must only ever scale x - max(x)
    big = np.stack([np.arange(V) * 0.5 + 1.0e5, 1.0e5 - np.arange(V) * 0.5, np.arange(V) * 0.5 - 1.0e5]).astype(np.float32)
    run_and_compare(big, "f32", 64)
    run_and_compare(synth.bf16_from_f32(rows), "bf16", 128)


def test_rowsweep_full_ddtree_shape_sampled():
    """All 1024 rows of the DDTree-shape workload in one launch (the benchmarked
    configuration); 64 rows spread over the batch are checked against the oracle."""
    host = synth.ddtree_logits(seed=2)                   # [64, 16, 151936]
    flat = host.reshape(-1, host.shape[-1])
    d = dev_bf16(flat)
    lse, ids, lp = dt.topk_logsoftmax(d, 64)
    torch.cuda.synchronize()
    lse, ids, lp = lse.cpu().numpy(), ids.cpu().numpy(), lp.cpu().numpy()
    pick = np.linspace(0, flat.shape[0] - 1, 64).astype(int)
    r_lse, r_ids, _, r_lp = rowsweep.topk_logsoftmax(rowsweep.as_f64(flat[pick], "bf16"), 64)
    np.testing.assert_array_equal(ids[pick], r_ids)
    assert_lse_close(lse[pick], r_lse)
    np.testing.assert_allclose(lp[pick], r_lp, rtol=0, atol=TOL)
    # every row: ids distinct, lp non-increasing and <= 0
    assert np.all(np.diff(lp, axis=1) <= 0) and np.all(lp <= 0)


@pytest.mark.parametrize("rows", [3, 40])
def test_rowsweep_top_values_in_one_lane(rows):
    """The row's largest values all in the 16-element spans of one thread of every 4096-element
    chunk (a stride the sweep's layout maps to one lane): the lanes' own maxima then certify a
    low bound, far more spans reach it than a wave lists, and the sweep must still return the
    exact top-K. Also a second pattern with the large values on a 64-element stride. Few rows
    split each row over several workgroups; 40 rows give one workgroup per row."""
    V = 151936
    rng = np.random.default_rng(31 + rows)
    x = rng.standard_normal((rows, V)).astype(np.float32)
    v = np.arange(V)
    one_lane = ((v % 4096) // 16) == 5
    x[0, one_lane] += (8.0 + rng.uniform(0.0, 2.0, one_lane.sum())).astype(np.float32)
    strided = (v % 64) == 3
    x[1, strided] += (6.0 + rng.uniform(0.0, 1.0, strided.sum())).astype(np.float32)
    x[2, ::4096] += 12.0
    host = synth.bf16_from_f32(x)
    for K in (8, 64, 128):
        run_and_compare(host, "bf16", K)
