"""Python binding of libdtree.so, the gfx950 draft-tree construction library.

Argument marshalling only: every step of the hot path runs in the HIP kernels behind
the C ABI declared in include/dtree.h. PyTorch provides device memory and the
current stream. There is no CPU fallback: if libdtree.so is missing or fails to
load, every call raises.

Entry points (same names as the C ABI):
    topk_logsoftmax(logits, K)                          -> (lse, ids, lp)
    build_tree_marginal(logits, K, B, beta)             -> Tree
    build_tree_marginal_noalloc(logits, K, B, beta, out) -> Tree (no workspace, no allocation)
    build_tree_depthwise(logits, E, U, P, root_tok, K, W, B, beta) -> Tree
    prepare_depthwise_head(U, P) -> head;  build_tree_depthwise_prepared(logits, E, head, d_model, rank,
        root_tok, K, W, B, beta) -> Tree  (the head's transposes done once)
    build_tree_sequential(logits, E, head, d_model, rank, root_tok, K, B, beta) -> Tree
        (exact best-first, one correction per popped node)
    build_tree_gated(logits, K_root, mu, N)             -> Tree
    build_tree_static(logits, K, D)                     -> Tree  (K*D nodes)
    build_tree_tdes(logits, root_tok, mlp, K, B, budget=None) -> Tree
    saba_budget(a, beta, c_verify, c_fixed, B_max)      -> int   (host only)
    accept_tree(tree, target, draft, temperature, seed, trial0, n_trials)
        -> (accept_len, accept_node, next_token), each [n_trials, R]
    accept_tree_narrow(tree, target, draft, temperature, seed, trial0, n_trials)
        (accept_tree with one workgroup per round; same outputs)
    accept_tree_match(tree, target, temperature, seed, trial0, n_trials)   (same outputs)
Logits are torch.bfloat16 or torch.float32 device tensors ([R, L, V] for the builders).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdtree.so")

DTREE_BF16, DTREE_F32 = 0, 1
OP_TOPK, OP_MARGINAL, OP_DEPTHWISE, OP_GATED, OP_ACCEPT, OP_STATIC, OP_TDES, OP_DEPTHWISE_HEAD, \
    OP_DEPTHWISE_PREPARED, OP_SEQUENTIAL, OP_DEPTHWISE_LISTS = range(11)
STATUS = {0: "DTREE_OK", -1: "DTREE_E_INVAL", -2: "DTREE_E_BETA", -3: "DTREE_E_WORKSPACE",
          -4: "DTREE_E_UNSUPPORTED", -5: "DTREE_E_HIP"}

# every symbol include/dtree.h declares
SYMBOLS = ("dtree_workspace_size", "dtree_topk_logsoftmax", "dtree_topk_lists", "build_tree_marginal",
           "build_tree_marginal_lists", "build_tree_marginal_noalloc",
           "build_tree_depthwise", "dtree_prepare_depthwise_head", "build_tree_depthwise_prepared",
           "build_tree_depthwise_lists",
           "build_tree_sequential",
           "build_tree_gated", "build_tree_static", "build_tree_tdes", "dtree_saba_budget", "accept_tree", "accept_tree_narrow", "accept_tree_match", "dtree_status_string", "dtree_last_error")


class DTreeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class CTree(ctypes.Structure):
    _fields_ = [("parent", ctypes.c_void_p), ("token", ctypes.c_void_p), ("depth", ctypes.c_void_p),
                ("score", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("n_nodes", ctypes.c_void_p),
                ("cap", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdtree.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m draft_tree_construction_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    u64 = ctypes.c_uint64
    L.dtree_workspace_size.restype = sz
    L.dtree_workspace_size.argtypes = [i32] * 9
    L.dtree_topk_logsoftmax.restype = i32
    L.dtree_topk_logsoftmax.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.dtree_topk_lists.restype = i32
    L.dtree_topk_lists.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.build_tree_marginal_lists.restype = i32
    L.build_tree_marginal_lists.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, ctypes.POINTER(CTree), vp]
    L.build_tree_depthwise_lists.restype = i32
    L.build_tree_depthwise_lists.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, vp, i32, i32,
                                             i32, f32, ctypes.POINTER(CTree), vp, sz, vp]
    L.build_tree_marginal.restype = i32
    L.build_tree_marginal.argtypes = [vp, i32, i32, i32, i32, i32, i32, f32, ctypes.POINTER(CTree), vp, sz, vp]
    L.build_tree_marginal_noalloc.restype = i32
    L.build_tree_marginal_noalloc.argtypes = [vp, i32, i32, i32, i32, i32, i32, f32, ctypes.POINTER(CTree), vp]
    L.build_tree_depthwise.restype = i32
    L.build_tree_depthwise.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, i32, vp, i32, i32, i32, f32,
                                       ctypes.POINTER(CTree), vp, sz, vp]
    L.dtree_prepare_depthwise_head.restype = i32
    L.dtree_prepare_depthwise_head.argtypes = [vp, vp, i32, i32, i32, i32, vp, sz, vp]
    L.build_tree_depthwise_prepared.restype = i32
    L.build_tree_depthwise_prepared.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, i32, vp, i32, i32, i32, f32,
                                                ctypes.POINTER(CTree), vp, sz, vp]
    L.build_tree_sequential.restype = i32
    L.build_tree_sequential.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, i32, vp, i32, i32, f32,
                                        ctypes.POINTER(CTree), vp, sz, vp]
    L.build_tree_gated.restype = i32
    L.build_tree_gated.argtypes = [vp, i32, i32, i32, i32, i32, f32, i32, ctypes.POINTER(CTree), vp, sz, vp]
    L.build_tree_static.restype = i32
    L.build_tree_static.argtypes = [vp, i32, i32, i32, i32, i32, i32, ctypes.POINTER(CTree), vp, sz, vp]
    L.build_tree_tdes.restype = i32
    L.build_tree_tdes.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, f32, f32, i32, i32, i32, i32,
                                  i32, i32, vp, ctypes.POINTER(CTree), vp, sz, vp]
    L.dtree_saba_budget.restype = i32
    L.dtree_saba_budget.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double, i32]
    L.accept_tree.restype = i32
    L.accept_tree.argtypes = [ctypes.POINTER(CTree), vp, vp, i32, i32, i32, i32, f32, u64, u64, i32, vp, vp, vp,
                              vp, sz, vp]
    L.accept_tree_narrow.restype = i32
    L.accept_tree_narrow.argtypes = L.accept_tree.argtypes
    L.accept_tree_match.restype = i32
    L.accept_tree_match.argtypes = [ctypes.POINTER(CTree), vp, i32, i32, i32, f32, u64, u64, i32, vp, vp, vp, vp, sz,
                                    vp]
    L.dtree_status_string.restype = ctypes.c_char_p
    L.dtree_status_string.argtypes = [i32]
    L.dtree_last_error.restype = ctypes.c_char_p
    L.dtree_last_error.argtypes = []
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        raise DTreeError(rc, lib().dtree_last_error().decode())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTREE_BF16
    if t.dtype == torch.float32:
        return DTREE_F32
    raise TypeError("logits must be torch.bfloat16 or torch.float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _require_device(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("inputs must be contiguous device tensors")


def workspace_size(op: int, R: int, L: int, V: int, K: int = 0, B_or_N: int = 0, W: int = 0, rank: int = 0,
                   d_model: int = 0) -> int:
    return int(lib().dtree_workspace_size(op, R, L, V, K, B_or_N, W, rank, d_model))


def _workspace(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


@dataclass
class Tree:
    """Device outputs of a builder: per round [cap+1] slots (slot 0 = root)."""
    parent: torch.Tensor
    token: torch.Tensor
    depth: torch.Tensor
    score: torch.Tensor
    mask: torch.Tensor
    n_nodes: torch.Tensor
    cap: int

    @staticmethod
    def empty(R: int, cap: int, dev) -> "Tree":
        words = (cap + 1 + 31) // 32
        i32 = dict(dtype=torch.int32, device=dev)
        return Tree(torch.empty(R, cap + 1, **i32), torch.empty(R, cap + 1, **i32), torch.empty(R, cap + 1, **i32),
                    torch.empty(R, cap + 1, dtype=torch.float32, device=dev),
                    torch.empty(R, cap + 1, words, dtype=torch.int32, device=dev),
                    torch.empty(R, **i32), cap)

    def c_struct(self) -> CTree:
        return CTree(self.parent.data_ptr(), self.token.data_ptr(), self.depth.data_ptr(), self.score.data_ptr(),
                     self.mask.data_ptr(), self.n_nodes.data_ptr(), self.cap)


def topk_logsoftmax(logits: torch.Tensor, K: int, ws: torch.Tensor | None = None):
    """logits [rows, V] -> lse [rows] f32, ids [rows, K] i32, lp [rows, K] f32."""
    _require_device(logits)
    rows, V = logits.shape
    dev = logits.device
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    ids = torch.empty(rows, K, dtype=torch.int32, device=dev)
    lp = torch.empty(rows, K, dtype=torch.float32, device=dev)
    need = workspace_size(OP_TOPK, rows, 1, V, K)
    ws = _workspace(need, dev) if ws is None else ws
    _check(lib().dtree_topk_logsoftmax(_ptr(logits), _dtype(logits), rows, V, K, _ptr(lse), _ptr(ids), _ptr(lp),
                                       _ptr(ws), ws.numel(), _stream(dev)))
    return lse, ids, lp


@dataclass
class Lists:
    """dtree_topk_lists' result for [R*L] rows: zk, ids [rows, K] and lse [rows] (float64)."""
    zk: torch.Tensor
    ids: torch.Tensor
    lse: torch.Tensor

    @property
    def K(self) -> int:
        return self.ids.shape[1]

    @staticmethod
    def empty(rows: int, K: int, dev) -> "Lists":
        return Lists(torch.empty(rows, K, dtype=torch.float32, device=dev),
                     torch.empty(rows, K, dtype=torch.int32, device=dev),
                     torch.empty(rows, dtype=torch.float64, device=dev))


def topk_lists(logits: torch.Tensor, K: int, ws: torch.Tensor | None = None, out: Lists | None = None) -> Lists:
    """logits [R, L, V] or [rows, V] -> the candidate lists the *_lists builders take."""
    _require_device(logits)
    V = logits.shape[-1]
    rows = logits.numel() // V
    dev = logits.device
    out = Lists.empty(rows, K, dev) if out is None else out
    need = workspace_size(OP_TOPK, rows, 1, V, K)
    ws = _workspace(need, dev) if ws is None else ws
    _check(lib().dtree_topk_lists(_ptr(logits), _dtype(logits), rows, V, K, _ptr(out.zk), _ptr(out.ids),
                                  _ptr(out.lse), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def build_tree_marginal_lists(lists: Lists, R: int, L: int, B: int, beta: float, out: Tree | None = None) -> Tree:
    """build_tree_marginal from topk_lists over the same logits (K = the lists' K)."""
    _require_device(lists.zk, lists.ids, lists.lse)
    dev = lists.zk.device
    out = Tree.empty(R, B, dev) if out is None else out
    st = out.c_struct()
    _check(lib().build_tree_marginal_lists(_ptr(lists.zk), _ptr(lists.ids), _ptr(lists.lse), R, L, lists.K, B,
                                           float(beta), ctypes.byref(st), _stream(dev)))
    return out


def build_tree_marginal(logits: torch.Tensor, K: int, B: int, beta: float, ws: torch.Tensor | None = None,
                        out: Tree | None = None) -> Tree:
    _require_device(logits)
    R, L, V = logits.shape
    dev = logits.device
    out = Tree.empty(R, B, dev) if out is None else out
    ws = _workspace(workspace_size(OP_MARGINAL, R, L, V, K, B), dev) if ws is None else ws
    st = out.c_struct()
    _check(lib().build_tree_marginal(_ptr(logits), _dtype(logits), R, L, V, K, B, float(beta), ctypes.byref(st),
                                     _ptr(ws), ws.numel(), _stream(dev)))
    return out


def build_tree_marginal_noalloc(logits: torch.Tensor, K: int, B: int, beta: float, out: Tree) -> Tree:
    """build_tree_marginal with the library's own per-device scratch (no workspace); `out`
    must be given, so the call allocates nothing."""
    _require_device(logits)
    R, L, V = logits.shape
    st = out.c_struct()
    _check(lib().build_tree_marginal_noalloc(_ptr(logits), _dtype(logits), R, L, V, K, B, float(beta),
                                             ctypes.byref(st), _stream(logits.device)))
    return out


def build_tree_depthwise(logits: torch.Tensor, E: torch.Tensor, U: torch.Tensor, P: torch.Tensor,
                         root_tok: torch.Tensor, K: int, W: int, B: int, beta: float,
                         ws: torch.Tensor | None = None, out: Tree | None = None) -> Tree:
    """E [V, d_model], U [L, d_model, rank], P [rank, V] bf16; root_tok [R] int32."""
    _require_device(logits, E, U, P, root_tok)
    for t in (E, U, P):
        if t.dtype != torch.bfloat16:
            raise TypeError("E, U, P must be torch.bfloat16")
    if root_tok.dtype != torch.int32:
        raise TypeError("root_tok must be int32")
    R, L, V = logits.shape
    d_model, rank = U.shape[1], U.shape[2]
    dev = logits.device
    out = Tree.empty(R, B, dev) if out is None else out
    ws = _workspace(workspace_size(OP_DEPTHWISE, R, L, V, K, B, W, rank, d_model), dev) if ws is None else ws
    st = out.c_struct()
    _check(lib().build_tree_depthwise(_ptr(logits), _dtype(logits), R, L, V, _ptr(E), _ptr(U), _ptr(P), d_model, rank,
                                      _ptr(root_tok), K, W, B, float(beta), ctypes.byref(st), _ptr(ws), ws.numel(),
                                      _stream(dev)))
    return out


def prepare_depthwise_head(U: torch.Tensor, P: torch.Tensor, V: int | None = None,
                           head: torch.Tensor | None = None) -> torch.Tensor:
    """U [L, d_model, rank], P [rank, V] bf16 -> the prepared head (a uint8 device buffer)."""
    _require_device(U, P)
    L, d_model, rank = U.shape
    V = P.shape[1] if V is None else V
    dev = U.device
    need = workspace_size(OP_DEPTHWISE_HEAD, 0, L, V, 0, 0, 0, rank, d_model)
    head = _workspace(need, dev) if head is None else head
    _check(lib().dtree_prepare_depthwise_head(_ptr(U), _ptr(P), L, V, d_model, rank, _ptr(head), head.numel(),
                                              _stream(dev)))
    return head


def build_tree_depthwise_prepared(logits: torch.Tensor, E: torch.Tensor, head: torch.Tensor, d_model: int, rank: int,
                                  root_tok: torch.Tensor, K: int, W: int, B: int, beta: float,
                                  ws: torch.Tensor | None = None, out: Tree | None = None) -> Tree:
    """build_tree_depthwise with a head from prepare_depthwise_head."""
    _require_device(logits, E, head, root_tok)
    if E.dtype != torch.bfloat16 or root_tok.dtype != torch.int32:
        raise TypeError("E must be torch.bfloat16 and root_tok int32")
    R, L, V = logits.shape
    dev = logits.device
    out = Tree.empty(R, B, dev) if out is None else out
    ws = _workspace(workspace_size(OP_DEPTHWISE_PREPARED, R, L, V, K, B, W, rank, d_model), dev) if ws is None else ws
    st = out.c_struct()
    _check(lib().build_tree_depthwise_prepared(_ptr(logits), _dtype(logits), R, L, V, _ptr(E), _ptr(head), d_model,
                                               rank, _ptr(root_tok), K, W, B, float(beta), ctypes.byref(st), _ptr(ws),
                                               ws.numel(), _stream(dev)))
    return out


def build_tree_depthwise_lists(logits: torch.Tensor, lists: Lists, E: torch.Tensor, head: torch.Tensor, d_model: int,
                               rank: int, root_tok: torch.Tensor, K: int, W: int, B: int, beta: float,
                               ws: torch.Tensor | None = None, out: Tree | None = None) -> Tree:
    """build_tree_depthwise_prepared with C_d from topk_lists over the same logits (K <= the
    lists' K)."""
    _require_device(logits, lists.zk, lists.ids, E, head, root_tok)
    if E.dtype != torch.bfloat16 or root_tok.dtype != torch.int32:
        raise TypeError("E must be torch.bfloat16 and root_tok int32")
    R, L, V = logits.shape
    dev = logits.device
    out = Tree.empty(R, B, dev) if out is None else out
    ws = _workspace(workspace_size(OP_DEPTHWISE_LISTS, R, L, V, K, B, W, rank, d_model), dev) if ws is None else ws
    st = out.c_struct()
    _check(lib().build_tree_depthwise_lists(_ptr(logits), _dtype(logits), _ptr(lists.zk), _ptr(lists.ids), lists.K, R,
                                            L, V, _ptr(E), _ptr(head), d_model, rank, _ptr(root_tok), K, W, B,
                                            float(beta), ctypes.byref(st), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def build_tree_sequential(logits: torch.Tensor, E: torch.Tensor, head: torch.Tensor, d_model: int, rank: int,
                          root_tok: torch.Tensor, K: int, B: int, beta: float, ws: torch.Tensor | None = None,
                          out: Tree | None = None) -> Tree:
    """Exact path-dependent best-first tree, one correction per popped node, with a head from
    prepare_depthwise_head."""
    _require_device(logits, E, head, root_tok)
    if E.dtype != torch.bfloat16 or root_tok.dtype != torch.int32:
        raise TypeError("E must be torch.bfloat16 and root_tok int32")
    R, L, V = logits.shape
    dev = logits.device
    out = Tree.empty(R, B, dev) if out is None else out
    ws = _workspace(workspace_size(OP_SEQUENTIAL, R, L, V, K, B, 0, rank, d_model), dev) if ws is None else ws
    st = out.c_struct()
    _check(lib().build_tree_sequential(_ptr(logits), _dtype(logits), R, L, V, _ptr(E), _ptr(head), d_model, rank,
                                       _ptr(root_tok), K, B, float(beta), ctypes.byref(st), _ptr(ws), ws.numel(),
                                       _stream(dev)))
    return out


def build_tree_gated(logits: torch.Tensor, K_root: int, mu: float, N: int, ws: torch.Tensor | None = None,
                     out: Tree | None = None) -> Tree:
    _require_device(logits)
    R, L, V = logits.shape
    dev = logits.device
    out = Tree.empty(R, N, dev) if out is None else out
    ws = _workspace(workspace_size(OP_GATED, R, L, V, 0, N), dev) if ws is None else ws
    st = out.c_struct()
    _check(lib().build_tree_gated(_ptr(logits), _dtype(logits), R, L, V, K_root, float(mu), N, ctypes.byref(st),
                                  _ptr(ws), ws.numel(), _stream(dev)))
    return out


def build_tree_static(logits: torch.Tensor, K: int, D: int, ws: torch.Tensor | None = None,
                      out: Tree | None = None) -> Tree:
    """Static D x K grid: K nodes per depth to depth D (cap = K*D)."""
    _require_device(logits)
    R, L, V = logits.shape
    dev = logits.device
    out = Tree.empty(R, K * D, dev) if out is None else out
    ws = _workspace(workspace_size(OP_STATIC, R, L, V, K), dev) if ws is None else ws
    st = out.c_struct()
    _check(lib().build_tree_static(_ptr(logits), _dtype(logits), R, L, V, K, D, ctypes.byref(st), _ptr(ws),
                                   ws.numel(), _stream(dev)))
    return out


def build_tree_tdes(logits: torch.Tensor, root_tok: torch.Tensor, mlp: dict, K: int, B: int,
                    budget: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                    out: Tree | None = None) -> Tree:
    """GRAFT edge-scored best-first tree. mlp: float32 device tensors Gp [V, hp], Gc [V, hc],
    Ed [L, hd], W [H, hp+hc+hd], b [H], w [H] and floats b0, s. budget: int32 [R] or None."""
    names = ("Gp", "Gc", "Ed", "W", "b", "w")
    _require_device(logits, root_tok, *(mlp[k] for k in names))
    for k in names:
        if mlp[k].dtype != torch.float32 or not mlp[k].is_contiguous():
            raise TypeError(f"{k} must be a contiguous float32 tensor")
    if root_tok.dtype != torch.int32 or (budget is not None and budget.dtype != torch.int32):
        raise TypeError("root_tok and budget must be int32")
    R, L, V = logits.shape
    hp, hc, hd = mlp["Gp"].shape[1], mlp["Gc"].shape[1], mlp["Ed"].shape[1]
    H = mlp["W"].shape[0]
    dev = logits.device
    out = Tree.empty(R, B, dev) if out is None else out
    ws = _workspace(workspace_size(OP_TDES, R, L, V, K), dev) if ws is None else ws
    st = out.c_struct()
    _check(lib().build_tree_tdes(_ptr(logits), _dtype(logits), R, L, V, _ptr(root_tok), *(_ptr(mlp[k]) for k in names),
                                 float(mlp["b0"]), float(mlp["s"]), hp, hc, hd, H, K, B,
                                 None if budget is None else _ptr(budget), ctypes.byref(st), _ptr(ws), ws.numel(),
                                 _stream(dev)))
    return out


def saba_budget(a: float, beta: float, c_verify: float, c_fixed: float, B_max: int) -> int:
    """GRAFT's budget: argmax over B in [1, B_max] of a B^beta / (B c_verify + c_fixed) (host)."""
    rc = lib().dtree_saba_budget(float(a), float(beta), float(c_verify), float(c_fixed), int(B_max))
    _check(rc if rc < 0 else 0)
    return rc


def _accept(fn: str, tree: Tree, target: torch.Tensor, draft: torch.Tensor | None, temperature: float, seed: int,
            trial0: int, n_trials: int, ws: torch.Tensor | None, outs):
    _require_device(target, draft)
    R, rows, V = target.shape
    if rows != tree.cap + 1:
        raise ValueError("target must have cap+1 rows per round")
    L = draft.shape[1] if draft is not None else 1
    dev = target.device
    if outs is None:
        outs = tuple(torch.empty(n_trials, R, dtype=torch.int32, device=dev) for _ in range(3))
    ws = _workspace(workspace_size(OP_ACCEPT, R, L, V, 0, tree.cap), dev) if ws is None else ws
    st = tree.c_struct()
    _check(getattr(lib(), fn)(ctypes.byref(st), _ptr(target), _ptr(draft), _dtype(target), R, L, V, float(temperature),
                              int(seed), int(trial0), int(n_trials), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
                              _ptr(ws), ws.numel(), _stream(dev)))
    return outs


def accept_tree(tree: Tree, target: torch.Tensor, draft: torch.Tensor | None, temperature: float, seed: int,
                trial0: int = 0, n_trials: int = 1, ws: torch.Tensor | None = None, outs=None):
    """target [R, cap+1, V]; draft [R, L, V] (None allowed at temperature 0)."""
    return _accept("accept_tree", tree, target, draft, temperature, seed, trial0, n_trials, ws, outs)


def accept_tree_narrow(tree: Tree, target: torch.Tensor, draft: torch.Tensor | None, temperature: float, seed: int,
                       trial0: int = 0, n_trials: int = 1, ws: torch.Tensor | None = None, outs=None):
    """accept_tree with one workgroup per round (for a walk that runs beside other work)."""
    return _accept("accept_tree_narrow", tree, target, draft, temperature, seed, trial0, n_trials, ws, outs)


def accept_tree_match(tree: Tree, target: torch.Tensor, temperature: float, seed: int, trial0: int = 0,
                      n_trials: int = 1, ws: torch.Tensor | None = None, outs=None):
    """Exact target-sample matching; target [R, cap+1, V]."""
    _require_device(target)
    R, rows, V = target.shape
    if rows != tree.cap + 1:
        raise ValueError("target must have cap+1 rows per round")
    dev = target.device
    if outs is None:
        outs = tuple(torch.empty(n_trials, R, dtype=torch.int32, device=dev) for _ in range(3))
    ws = _workspace(workspace_size(OP_ACCEPT, R, 1, V, 0, tree.cap), dev) if ws is None else ws
    st = tree.c_struct()
    _check(lib().accept_tree_match(ctypes.byref(st), _ptr(target), _dtype(target), R, V, float(temperature), int(seed),
                                   int(trial0), int(n_trials), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(ws),
                                   ws.numel(), _stream(dev)))
    return outs
