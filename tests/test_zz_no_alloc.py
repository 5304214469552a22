"""GPU: build_tree_marginal_noalloc (the library's own scratch, no workspace) gives exactly
build_tree_marginal's tree, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents, which the second must not depend on)."""
import ctypes

import numpy as np
import pytest
import torch

import draft_tree_construction_amd as dt
import synth
from parity_util import dev_bf16, tree_to_host

pytestmark = pytest.mark.gpu


def noalloc_call(x, K, B, beta, out):
    R, L, V = x.shape
    st = out.c_struct()
    rc = dt.lib().build_tree_marginal_noalloc(ctypes.c_void_p(x.data_ptr()), dt.DTREE_BF16, R, L, V, K, B,
                                              float(beta), ctypes.byref(st),
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, dt.lib().dtree_last_error()
    return out


@pytest.mark.parametrize("first,second", [((64, 16, 151936, 64, 64, 0.0), (3, 5, 20001, 16, 40, -0.3)),
                                          ((8, 16, 151936, 0, 64, -0.1), (2, 16, 151936, 64, 128, 0.0))])
def test_noalloc_matches_workspace_builder(first, second):
    for i, (R, L, V, K, B, beta) in enumerate((first, second)):
        x = dev_bf16(synth.ddtree_logits(seed=70 + i, R=R, L=L, V=V))
        want = tree_to_host(dt.build_tree_marginal(x, K, B, beta))
        got = tree_to_host(noalloc_call(x, K, B, beta, dt.Tree.empty(R, B, x.device)))
        for k in ("parent", "token", "depth", "mask", "n"):
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)
        np.testing.assert_array_equal(got["score"], want["score"])
