"""Helpers shared by the GPU parity tests: moving seeded inputs to the device, and
comparing a device tree with the oracle's under the tolerance rules.

Rules (scores and log-probs: |diff| <= 1e-5; topology, tokens and accepted lengths
bit-exact wherever the oracle's selection boundary has a score gap above 1e-5).
"""
from __future__ import annotations

import numpy as np
import torch

import draft_tree_construction_amd as dt
from oracle import treeout

TOL = 1e-5


def dev_bf16(bits: np.ndarray, device="cuda:0") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def dev_f32(x: np.ndarray, device="cuda:0") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def tree_to_host(tr: dt.Tree):
    torch.cuda.synchronize()
    return dict(parent=tr.parent.cpu().numpy(), token=tr.token.cpu().numpy(), depth=tr.depth.cpu().numpy(),
                score=tr.score.cpu().numpy(), mask=tr.mask.cpu().numpy().view(np.uint32),
                n=tr.n_nodes.cpu().numpy())


def oracle_to_device(trees, cap: int, device="cuda:0") -> dt.Tree:
    """Oracle Trees (one per round) -> a device Tree struct."""
    R = len(trees)
    out = dt.Tree.empty(R, cap, device)
    par = np.stack([t.arrays(cap)[0] for t in trees])
    tok = np.stack([t.arrays(cap)[1] for t in trees])
    dep = np.stack([t.arrays(cap)[2] for t in trees])
    sc = np.stack([t.arrays(cap)[3] for t in trees]).astype(np.float32)
    mk = np.stack([treeout.ancestor_mask(t.parent, cap) for t in trees])
    out.parent.copy_(torch.from_numpy(par))
    out.token.copy_(torch.from_numpy(tok))
    out.depth.copy_(torch.from_numpy(dep))
    out.score.copy_(torch.from_numpy(sc))
    out.mask.copy_(torch.from_numpy(mk.view(np.int32)))
    out.n_nodes.copy_(torch.from_numpy(np.array([t.n for t in trees], dtype=np.int32)))
    return out


def device_round(h, r: int):
    n = int(h["n"][r])
    par = [int(x) for x in h["parent"][r, :n + 1]]
    tok = [int(x) for x in h["token"][r, :n + 1]]
    dep = [int(x) for x in h["depth"][r, :n + 1]]
    sc = [float(x) for x in h["score"][r, :n + 1]]
    return n, par, tok, dep, sc


def paths_of(par, tok):
    out = [()]
    for i in range(1, len(par)):
        out.append(out[par[i]] + (tok[i],))
    return out


def assert_tree_valid(h, r: int, cap: int, monotone: bool = True):
    """Device round r is a well-formed tree: root slot, parents before children, depth =
    parent's + 1, scores never above the parent's (monotone), distinct (parent, token)
    pairs, the ancestor mask, and -1 padding past n_nodes."""
    n, par, tok, dep, sc = device_round(h, r)
    assert 0 <= n <= cap
    assert par[0] == -1 and dep[0] == 0 and tok[0] == -1
    for i in range(1, n + 1):
        assert 0 <= par[i] < i and dep[i] == dep[par[i]] + 1
        assert not monotone or sc[i] <= sc[par[i]]
    assert len(set(zip(par[1:], tok[1:]))) == n
    np.testing.assert_array_equal(h["mask"][r], treeout.ancestor_mask(par, cap))
    assert np.all(h["parent"][r, n + 1:] == -1) and np.all(h["token"][r, n + 1:] == -1)
    return n, par, tok, dep, sc


def assert_tree_equal(h, r: int, ref, cap: int, near_tie: bool = False):
    """Device round r must equal the oracle tree `ref` exactly (topology, tokens, depths,
    padding, mask) with scores within TOL. With near_tie (the oracle saw a selection gap
    <= TOL) only validity and the scores of shared prefixes are checked. Returns True if
    the exact comparison was made."""
    n, par, tok, dep, sc = assert_tree_valid(h, r, cap)
    if near_tie:
        got = dict(zip(paths_of(par, tok), sc))
        want = dict(zip(ref.paths(), ref.score))
        for p in set(got) & set(want):
            assert abs(got[p] - want[p]) <= TOL
        return False
    assert n == ref.n, (n, ref.n)
    assert par == ref.parent and tok == ref.token and dep == ref.depth
    np.testing.assert_allclose(sc, ref.score, rtol=0, atol=TOL)
    return True


_CACHE = {}


def full_verification_case():
    """The verification workload at full size, built once per test session: DDTree-shape
    draft logits [64, 16, 151936] (seed 2), the oracle's marginal trees (K = B = 64) and
    draft-correlated target logits [64, 65, 151936] (seed 5) on those trees' depths."""
    if "verify" not in _CACHE:
        import synth
        import oracle_pool as op
        draft = synth.ddtree_logits(seed=2)
        trees = [t for t, _ in op.pmap(op.marginal_task, [(draft[r], "bf16", 64, 64, 0.0) for r in range(64)])]
        depth = np.stack([t.arrays(64)[2] for t in trees])
        target = synth.verification_target(draft, depth, seed=5)
        _CACHE["verify"] = (draft, trees, target)
    return _CACHE["verify"]


def compare_with_margins(got, want_with_margins, tol=1e-6):
    """Trial-by-trial comparison of device walks with the oracle's, where the oracle also
    gives each walk's smallest decision margin. A mismatch is allowed only where that
    margin is <= tol (a decision within float rounding of its threshold); returns
    (mismatches, comparisons)."""
    bad = n = 0
    for g, (w, m) in zip(got, want_with_margins):
        n += 1
        if tuple(int(x) for x in g) != tuple(int(x) for x in w):
            assert m <= tol, (g, w, m)
            bad += 1
    return bad, n
