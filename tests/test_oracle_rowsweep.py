"""Pins for the oracle's row log-softmax and top-K (CPU only)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import rowsweep


def test_lse_matches_torch_logsumexp():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((6, 5000)) * 3.0
    lse, _, _, lp = rowsweep.topk_logsoftmax(z, 4)
    ref = torch.logsumexp(torch.from_numpy(z), dim=1).numpy()
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)
    ref_lp = torch.log_softmax(torch.from_numpy(z), dim=1).numpy()
    _, ids, _, _ = rowsweep.topk_logsoftmax(z, 4)
    np.testing.assert_allclose(lp, np.take_along_axis(ref_lp, ids, 1), atol=1e-12)


def test_closed_forms():
    # a constant row: every log-prob is -ln V
    z = np.full((1, 1000), 7.25)
    lse, ids, _, lp = rowsweep.topk_logsoftmax(z, 5)
    assert abs(lse[0] - (7.25 + math.log(1000))) < 1e-12
    np.testing.assert_allclose(lp, -math.log(1000), atol=1e-12)
    assert list(ids[0]) == [0, 1, 2, 3, 4]  # ties go to the smaller id
    # two values a > b, n_a copies of a: lse = a + ln(n_a + (V - n_a) e^{b-a})
    z = np.zeros((1, 10))
    z[0, [3, 7]] = 2.0
    lse, ids, _, _ = rowsweep.topk_logsoftmax(z, 3)
    assert abs(lse[0] - (2.0 + math.log(2 + 8 * math.exp(-2.0)))) < 1e-12
    assert list(ids[0]) == [3, 7, 0]


def test_topk_order_with_planted_ties():
    b = synth.tie_rows(4096, 5)
    z = rowsweep.as_f64(b, "bf16")
    K = 64
    _, ids, zk, _ = rowsweep.topk_logsoftmax(z, K)
    for r in range(z.shape[0]):
        # the K selected are the K largest under (value desc, id asc)
        kth_val, kth_id = zk[r, -1], ids[r, -1]
        rest = np.setdiff1d(np.arange(z.shape[1]), ids[r])
        assert np.all((z[r, rest] < kth_val) | ((z[r, rest] == kth_val) & (rest > kth_id)))
        for i in range(K - 1):
            assert zk[r, i] > zk[r, i + 1] or (zk[r, i] == zk[r, i + 1] and ids[r, i] < ids[r, i + 1])


def test_signed_zero_is_a_tie():
    z = np.array([[-0.0, 0.0, -1.0, -0.0]])
    _, ids, _, _ = rowsweep.topk_logsoftmax(z, 3)
    assert list(ids[0]) == [0, 1, 3]


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        rowsweep.topk_logsoftmax(np.array([[0.0, np.inf]]), 1)


def test_bf16_widening_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0], dtype=np.float32)
    b = synth.bf16_from_f32(x)
    back = synth.f32_from_bf16(b)
    # bf16 keeps 8 significant bits: 1e-3 rounds; the others are exact
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 3.140625
    assert abs(back[3] - 1e-3) <= 2 ** -8 * 1e-3
    np.testing.assert_array_equal(rowsweep.as_f64(b, "bf16"), back.astype(np.float64))
