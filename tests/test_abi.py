"""The C-ABI library loads, exports every declared symbol, sizes workspaces, and rejects bad
arguments on the host before any launch (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import draft_tree_construction_amd as dt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "dtree.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol():
    L = dt.lib()
    decl = declared_symbols()
    assert set(decl) == set(dt.SYMBOLS)
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings():
    L = dt.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.dtree_status_string(code)
    assert L.dtree_status_string(7) == b"unknown status"


def test_workspace_sizes():
    ws = dt.workspace_size
    assert ws(dt.OP_MARGINAL, 64, 16, 151936, 64, 64) > 64 * 16 * 64 * 8
    assert ws(dt.OP_GATED, 64, 16, 151936, 0, 60) > 0
    assert ws(dt.OP_ACCEPT, 64, 16, 151936, 0, 64) > 64 * 65 * 2374 * 8
    assert ws(dt.OP_DEPTHWISE, 64, 16, 151936, 8, 128, 32, 64, 1024) > 0
    assert ws(dt.OP_DEPTHWISE, 64, 16, 151936, 8, 128, 32, 64, 0) == 0   # needs d_model
    assert ws(dt.OP_TOPK, 1024, 1, 151936, 64) == 0          # no split needed
    assert ws(dt.OP_TOPK, 2, 1, 151936, 64) > 0              # split rows need partials
    assert ws(99, 1, 1, 1) == 0
    assert ws(dt.OP_MARGINAL, -1, 16, 100, 8, 8) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def tree(cap):
    return dt.CTree(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, cap)


def marg(**kw):
    a = dict(logits=FAKE, dtype=0, R=4, L=4, V=32, K=8, B=8, beta=0.0, t=tree(8), ws=FAKE, nbytes=0)
    a.update(kw)
    t = a["t"]
    return dt.lib().build_tree_marginal(a["logits"], a["dtype"], a["R"], a["L"], a["V"], a["K"], a["B"],
                                        a["beta"], ctypes.byref(t) if t is not None else None, a["ws"],
                                        a["nbytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(beta=0.5), -2),
    (dict(beta=float("nan")), -1),
    (dict(dtype=3), -1),
    (dict(K=33), -1),
    (dict(K=129, V=1000), -4),
    (dict(K=65, V=1000), -3),          # K up to 128 is in the envelope: next check is the workspace
    (dict(B=129, t=tree(129)), -4),
    (dict(L=65), -4),
    (dict(t=tree(7)), -1),
    (dict(t=None), -1),
    (dict(logits=None), -1),
    (dict(ws=None), -3),
    (dict(nbytes=10), -3),
    (dict(ws=ctypes.c_void_p(0x1010), nbytes=1 << 40), -1),   # ws must be 256-byte aligned
])
def test_marginal_validation(kw, code):
    assert marg(**kw) == code
    assert dt.lib().dtree_last_error()


def test_zero_rounds_is_a_no_op():
    assert marg(R=0, ws=None, logits=None) == 0


def test_gated_validation():
    L = dt.lib()
    t = tree(60)
    def call(K_root=10, mu=0.03, N=60, V=151936, cap_t=t):
        return L.build_tree_gated(FAKE, 0, 4, 16, V, K_root, mu, N, ctypes.byref(cap_t), FAKE, 0, None)
    assert call(mu=0.0) == -1
    assert call(mu=1.5) == -1
    assert call(K_root=61) == -1
    assert call(K_root=0) == -1
    assert call(N=200, cap_t=tree(200)) == -4
    assert call(K_root=65, N=100, cap_t=tree(100)) == -4
    assert call() == -3


def test_static_validation():
    L = dt.lib()
    def call(K=10, D=6, Lp=16, V=151936, cap_t=None):
        ct = tree(K * D) if cap_t is None else cap_t
        return L.build_tree_static(FAKE, 0, 4, Lp, V, K, D, ctypes.byref(ct), FAKE, 0, None)
    assert call(K=0) == -1
    assert call(D=0) == -1
    assert call(D=17) == -1
    assert call(K=20, V=10) == -1
    assert call(K=65, D=1) == -4
    assert call(K=16, D=9) == -4
    assert call(cap_t=tree(59)) == -1
    assert call() == -3
    assert dt.workspace_size(dt.OP_STATIC, 4, 16, 151936, 10) >= dt.workspace_size(dt.OP_TOPK, 64, 1, 151936, 10)
    assert dt.workspace_size(dt.OP_STATIC, 4, 16, 151936, 0) == 0
    assert L.build_tree_static(None, 0, 0, 16, 100, 10, 6, ctypes.byref(tree(60)), None, 0, None) == 0


def test_tdes_validation():
    L = dt.lib()
    def call(K=32, B=128, hp=64, hc=64, hd=16, H=128, s=1.0, b0=0.0, cap=None, Gp=FAKE, V=151936, nbytes=0):
        ct = tree(B if cap is None else cap)
        return L.build_tree_tdes(FAKE, 0, 4, 16, V, FAKE, Gp, FAKE, FAKE, FAKE, FAKE, FAKE, b0, s, hp, hc, hd, H, K, B,
                                 None, ctypes.byref(ct), FAKE, nbytes, None)
    assert call(K=0) == -1
    assert call(K=40, V=30) == -1
    assert call(s=0.0) == -1
    assert call(s=-1.0) == -1
    assert call(b0=float("nan")) == -1
    assert call(cap=64) == -1
    assert call(K=65) == -4
    assert call(B=129, cap=129) == -4
    assert call(hp=66) == -4
    assert call(hd=6) == -4
    assert call(H=129) == -4
    assert call(Gp=0x1004) == -1
    assert call() == -3
    need = dt.workspace_size(dt.OP_TDES, 4, 16, 151936, 32)
    assert need >= 4 * 16 * 32 * 32 * 5


@pytest.mark.parametrize("cv,cf,beta,bmax", [(1.0, 10.0, 0.5, 128), (0.37, 20.0, 0.5, 128), (0.05, 7.9, 0.3, 64),
                                             (1.0, 0.0, 0.5, 128), (0.01, 500.0, 0.5, 128), (0.2, 3.0, 0.8, 16)])
def test_saba_budget_matches_oracle(cv, cf, beta, bmax):
    """The library's closed form against the oracle's exhaustive argmax."""
    from oracle import tdes
    for a in (1.0, 3.5):
        assert dt.saba_budget(a, beta, cv, cf, bmax) == tdes.saba_budget(a, beta, cv, cf, bmax)


def test_saba_budget_rejects_bad_arguments():
    for args in [(0.0, 0.5, 1.0, 1.0, 8), (1.0, 1.0, 1.0, 1.0, 8), (1.0, 0.5, 0.0, 1.0, 8), (1.0, 0.5, 1.0, -1.0, 8),
                 (1.0, 0.5, 1.0, 1.0, 0), (1.0, 0.5, 1.0, float("nan"), 8)]:
        with pytest.raises(dt.DTreeError):
            dt.saba_budget(*args)


def test_depthwise_validation():
    L = dt.lib()
    def call(rank=64, dm=1024, K=8, W=32, B=128, beta=-0.5, cap=128, E=FAKE):
        t = tree(cap)
        return L.build_tree_depthwise(FAKE, 0, 4, 16, 151936, E, FAKE, FAKE, dm, rank, FAKE, K, W, B, beta,
                                      ctypes.byref(t), FAKE, 0, None)
    assert call(beta=0.1) == -2
    assert call(E=ctypes.c_void_p(0x1002)) == -1   # E, U, P are read with 16-byte loads
    assert call(rank=32) == -4
    assert call(dm=1000) == -4
    assert call(W=129, K=4) == -4
    assert call(K=9, W=64*2) == -4
    assert call() == -3


def test_accept_validation():
    L = dt.lib()
    t = tree(64)
    def call(T=1.0, n=1, draft=FAKE, V=151936):
        o = FAKE
        return L.accept_tree(ctypes.byref(t), FAKE, draft, 0, 4, 16, V, T, 1, 0, n, o, o, o, FAKE, 0, None)
    assert call(T=-1.0) == -1
    assert call(T=float("inf")) == -1
    assert call(n=0) == -1
    assert call(draft=None) == -1
    assert call(V=300000) == -4
    assert call() == -3
    assert L.accept_tree(ctypes.byref(t), FAKE, FAKE, 0, 4, 16, 151936, 1.0, 1, 0, 1, FAKE, FAKE, FAKE,
                         ctypes.c_void_p(0x1008), 1 << 40, None) == -1   # misaligned workspace
    assert L.accept_tree(None, FAKE, FAKE, 0, 4, 16, 100, 1.0, 1, 0, 1, FAKE, FAKE, FAKE, FAKE, 0, None) == -1


def test_accept_match_validation():
    L = dt.lib()
    t = tree(64)
    def call(T=1.0, n=1, V=151936, ws=FAKE, nbytes=0):
        o = FAKE
        return L.accept_tree_match(ctypes.byref(t), FAKE, 0, 4, V, T, 1, 0, n, o, o, o, ws, nbytes, None)
    assert call(T=-1.0) == -1
    assert call(T=float("nan")) == -1
    assert call(n=0) == -1
    assert call(V=300000) == -4
    assert call() == -3
    assert call(ws=ctypes.c_void_p(0x1008), nbytes=1 << 40) == -1   # misaligned workspace
    assert L.accept_tree_match(None, FAKE, 0, 4, 100, 1.0, 1, 0, 1, FAKE, FAKE, FAKE, FAKE, 0, None) == -1


def test_topk_validation():
    L = dt.lib()
    def call(K=8, V=32, rows=4, dtype=0):
        return L.dtree_topk_logsoftmax(FAKE, dtype, rows, V, K, FAKE, FAKE, FAKE, None, 0, None)
    assert call(K=0) == -1
    assert call(K=33) == -1
    assert call(K=129, V=200) == -4
    assert call(K=100, V=50) == -1    # K > V (the envelope allows up to 128)
    assert call(dtype=5) == -1
    assert call(rows=2, V=151936, K=8) == -3   # split rows need a workspace
    assert call(rows=0) == 0


def test_marginal_noalloc_validation():
    """The no-workspace variant checks like build_tree_marginal and rejects a scratch need
    beyond DTREE_NOALLOC_SCRATCH_BYTES (4 MiB) before touching the device."""
    L = dt.lib()
    def call(R=4, V=32, K=8, B=8, beta=0.0, t=None):
        t = tree(B) if t is None else t
        return L.build_tree_marginal_noalloc(FAKE, 0, R, 4 if V == 32 else 16, V, K, B, beta, ctypes.byref(t), None)
    assert call(beta=0.5) == -2
    assert call(K=33) == -1
    assert call(B=129, t=tree(129)) == -4
    assert call(R=4096, V=151936, K=64, B=64) == -4
    assert b"DTREE_NOALLOC_SCRATCH_BYTES" in L.dtree_last_error()
    assert call(R=0) == 0


def test_depthwise_head_validation():
    L = dt.lib()
    ws = dt.workspace_size
    assert ws(dt.OP_DEPTHWISE_HEAD, 0, 16, 151936, 0, 0, 0, 64, 1024) >= 151936 * 128
    full = ws(dt.OP_DEPTHWISE, 64, 16, 151936, 8, 128, 32, 64, 1024)
    prep = ws(dt.OP_DEPTHWISE_PREPARED, 64, 16, 151936, 8, 128, 32, 64, 1024)
    head = ws(dt.OP_DEPTHWISE_HEAD, 0, 16, 151936, 0, 0, 0, 64, 1024)
    assert prep > 0 and prep + head == full
    def prep_call(rank=64, dm=1024, nbytes=1 << 40, head=FAKE2):
        return L.dtree_prepare_depthwise_head(FAKE2, FAKE2, 16, 151936, dm, rank, head, nbytes, None)
    assert prep_call(rank=32) == -4
    assert prep_call(dm=100) == -4
    assert prep_call(nbytes=10) == -3
    assert prep_call(head=None) == -3
    assert prep_call(head=ctypes.c_void_p(0x1010)) == -1
    t = tree(128)
    def build(head=FAKE2, beta=-0.5, nbytes=0):
        return L.build_tree_depthwise_prepared(FAKE2, 0, 4, 16, 1000, FAKE2, head, 1024, 64, FAKE2, 8, 32, 128, beta,
                                               ctypes.byref(t), FAKE2, nbytes, None)
    assert build(head=None) == -1
    assert build(beta=0.5) == -2
    assert build() == -3


FAKE2 = ctypes.c_void_p(0x100000)  # 256-byte aligned, never dereferenced


def test_sequential_validation():
    """build_tree_sequential rejects bad arguments on the host before any launch."""
    L = dt.lib()
    assert dt.workspace_size(dt.OP_SEQUENTIAL, 64, 16, 151936, 8, 128, 0, 64, 1024) > 0
    assert dt.workspace_size(dt.OP_SEQUENTIAL, 64, 16, 151936, 0, 128, 0, 64, 1024) == 0
    def call(K=8, B=128, beta=0.0, dm=1024, rank=64, head=FAKE2, E=FAKE2, cap=None, R=4):
        t = tree(B if cap is None else cap)
        return L.build_tree_sequential(FAKE2, 0, R, 16, 1000, E, head, dm, rank, FAKE2, K, B, beta,
                                       ctypes.byref(t), FAKE2, 0, None)
    assert call(beta=0.1) == -2
    assert call(K=65) == -4
    assert call(B=129, cap=129) == -4
    assert call(rank=32) == -4
    assert call(dm=1088) == -4         # d_model % 256 != 0
    assert call(cap=64) == -1          # the tree's cap must equal B
    assert call(head=None) == -1
    assert call(head=ctypes.c_void_p(0x100010)) == -1   # head must be 256-byte aligned
    assert call(E=ctypes.c_void_p(0x100002)) == -1      # E is read with 16-byte loads
    assert call() == -3
    assert call(R=0) == 0


def test_lists_entry_points_validation():
    """dtree_topk_lists and the builders that take its lists reject bad arguments on the host."""
    L = dt.lib()
    def lists(K=64, V=1000, zk=FAKE2, rows=64, nbytes=0, ws=FAKE2):
        return L.dtree_topk_lists(FAKE2, 0, rows, V, K, zk, FAKE2, FAKE2, ws, nbytes, None)
    assert lists(K=0) == -1
    assert lists(K=65, V=64) == -1
    assert lists(K=129, V=1000) == -4
    assert lists(zk=None) == -1
    assert lists(rows=0, zk=None) == 0
    assert lists(rows=2, V=1 << 20, ws=None) == -3   # two long rows are split: partials need a workspace
    t = tree(64)
    def marg(K=64, B=64, beta=0.0, Lp=16, cap=None, zk=FAKE2, R=4):
        ct = t if cap is None else tree(cap)
        return L.build_tree_marginal_lists(zk, FAKE2, FAKE2, R, Lp, K, B, beta, ctypes.byref(ct), None)
    assert marg(beta=0.5) == -2
    assert marg(beta=float("nan")) == -1
    assert marg(K=0) == -1                     # the lists' K, never the automatic 0
    assert marg(K=129) == -4
    assert marg(Lp=65) == -4
    assert marg(B=129, cap=129) == -4
    assert marg(cap=63) == -1
    assert marg(zk=None) == -1
    assert marg(R=0, zk=None) == 0
    ws = dt.workspace_size
    prep = ws(dt.OP_DEPTHWISE_PREPARED, 64, 16, 151936, 8, 128, 32, 64, 1024)
    dl = ws(dt.OP_DEPTHWISE_LISTS, 64, 16, 151936, 8, 128, 32, 64, 1024)
    assert 0 < dl < prep                       # no candidate lists or sweep partials of its own
    t2 = tree(128)
    def dw(K=8, ks=64, head=FAKE2, beta=-0.5, nbytes=0, zk=FAKE2):
        return L.build_tree_depthwise_lists(FAKE2, 0, zk, FAKE2, ks, 4, 16, 1000, FAKE2, head, 1024, 64, FAKE2, K, 32,
                                            128, beta, ctypes.byref(t2), FAKE2, nbytes, None)
    assert dw(K=9, ks=8) == -1
    assert dw(ks=129) == -4
    assert dw(K=65, ks=128) == -4
    assert dw(beta=0.5) == -2
    assert dw(head=None) == -1
    assert dw(head=ctypes.c_void_p(0x100010)) == -1
    assert dw(zk=None) == -1
    assert dw() == -3
