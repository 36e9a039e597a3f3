"""ctypes binding of libtreedraft.so (the C ABI in include/treedraft.h).

Argument marshalling only: every function checks the torch tensors it is
given (device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream, and raises TreedraftError on a non-OK status.  All
computation happens in the library's HIP kernels.  If the library is missing
this module raises at import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TREEDRAFT_LIB selects another build of the library (e.g. for A/B timing).
LIB_PATH = os.environ.get("TREEDRAFT_LIB") or os.path.join(_HERE, "libtreedraft.so")

TD_OK, TD_EINVAL, TD_ECAPACITY, TD_EUNSUPPORTED, TD_EHIP, TD_ESYNC = range(6)
TD_F32, TD_BF16 = 0, 1
TD_STEP_DRAFT, TD_STEP_VERIFY = 1, 2
STATUS_NAMES = {0: "TD_OK", 1: "TD_EINVAL", 2: "TD_ECAPACITY", 3: "TD_EUNSUPPORTED", 4: "TD_EHIP",
                5: "TD_ESYNC"}

# every symbol declared in include/treedraft.h
EXPORTED = ["td_abi_version", "td_last_error", "td_draft_topk_workspace", "td_draft_topk",
            "td_build_tree", "td_tree_mask", "td_tree_verify_attn_workspace",
            "td_tree_verify_attn", "td_accept", "td_step_args_bytes", "td_verify_step_workspace",
            "td_verify_step", "td_workspace_status", "td_verify_step_noalloc",
            "td_verify_step_events", "td_kv_commit", "td_flex_budget",
            "td_verify_layer_workspace", "td_tree_qkv", "td_lm_head_argmax", "td_fit_cost",
            "td_verify_step_kernels", "td_verify_step_kernel_events"]


class StepArgs(ctypes.Structure):
    """td_step_args, field for field."""
    _fields_ = [
        ("logits", c_void_p), ("logits_dtype", c_int), ("batch", c_int32), ("block", c_int32),
        ("vocab", c_int32), ("pos_stride", c_int64), ("topk", c_int32),
        ("n_max", c_int32), ("use_stop", c_int32), ("cost_a", c_double), ("cost_b", c_double),
        ("cost_c", c_double), ("cost_knee", c_int32), ("l_ar", c_double), ("ahat0", c_double),
        ("root_token", c_void_p), ("branch", c_int32), ("min_logrho", c_double),
        ("q", c_void_p), ("k_ctx", c_void_p), ("v_ctx", c_void_p), ("ctx_offsets", c_void_p),
        ("ctx_lengths", c_void_p), ("total_ctx", c_int64), ("max_ctx", c_int64), ("k_tree", c_void_p), ("v_tree", c_void_p),
        ("hq", c_int32), ("hkv", c_int32), ("head_dim", c_int32), ("scale", c_float),
        ("attn_dtype", c_int),
        ("target_token", c_void_p),
        ("commit", c_int32), ("next_root", c_void_p),
        ("topk_id", c_void_p), ("topk_logq", c_void_p), ("lse", c_void_p),
        ("n_nodes", c_void_p), ("node_token", c_void_p), ("node_parent", c_void_p),
        ("node_depth", c_void_p), ("node_logrho", c_void_p), ("ahat", c_void_p),
        ("speedup", c_void_p), ("mask", c_void_p), ("out", c_void_p),
        ("accept_len", c_void_p), ("accept_path", c_void_p), ("bonus_token", c_void_p),
        ("stages", c_int32),
    ]


class TreedraftError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tree_draft_build_amd.build`"
                          " (the HIP library is required; there is no CPU path)")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    lib.td_abi_version.restype = c_int
    lib.td_last_error.restype = ctypes.c_char_p
    lib.td_draft_topk_workspace.argtypes = [c_int32] * 4
    lib.td_draft_topk_workspace.restype = c_size_t
    lib.td_draft_topk.argtypes = [P, c_int, c_int32, c_int32, c_int32, c_int64, c_int32, P, P, P, P,
                                  c_size_t, P]
    lib.td_build_tree.argtypes = [P, P, c_int32, c_int32, c_int32, c_int32, c_int32, c_double,
                                  c_double, c_double, c_int32, c_double, c_double, c_int32,
                                  c_double, P, P, P, P, P, P, P, P, P]
    lib.td_flex_budget.argtypes = [c_int32] * 5 + [P, P]
    lib.td_flex_budget.restype = None
    lib.td_fit_cost.argtypes = [P, P, c_int32, c_int32, c_int32, P, P, P, P, P]
    lib.td_fit_cost.restype = c_int
    lib.td_verify_layer_workspace.argtypes = [c_int32] * 6
    lib.td_verify_layer_workspace.restype = c_size_t
    lib.td_tree_qkv.argtypes = [P, P, P, P, P, P, P, c_int32, c_int32, c_int32, c_int32, c_int32,
                                c_int32, c_double, P, P, P, P, c_size_t, P]
    lib.td_lm_head_argmax.argtypes = [P, P, P, c_int32, c_int32, c_int32, c_int32, c_int32, P, P,
                                      c_size_t, P]
    lib.td_tree_mask.argtypes = [P, P, c_int32, c_int32, P, P]
    lib.td_tree_verify_attn_workspace.argtypes = [c_int32] * 5 + [c_int64, c_int64]
    lib.td_tree_verify_attn_workspace.restype = c_size_t
    lib.td_tree_verify_attn.argtypes = [P, P, P, P, P, c_int64, c_int64, P, P, P, P, c_int32, c_int32,
                                        c_int32, c_int32, c_int32, c_float, c_int, P, P, c_size_t, P]
    lib.td_kv_commit.argtypes = [P, P, P, P, P, c_int32, c_int32, c_int32, c_int32, c_int32, c_int,
                                 P, P, P, P, P, P]
    lib.td_accept.argtypes = [P, P, P, P, c_int32, c_int32, c_int32, P, P, P, P]
    lib.td_step_args_bytes.restype = c_size_t
    lib.td_verify_step_workspace.argtypes = [ctypes.POINTER(StepArgs)]
    lib.td_verify_step_workspace.restype = c_size_t
    lib.td_verify_step.argtypes = [ctypes.POINTER(StepArgs), P, c_size_t, P]
    lib.td_workspace_status.argtypes = [P, c_size_t, P]
    lib.td_verify_step_noalloc.argtypes = [ctypes.POINTER(StepArgs), P]
    lib.td_verify_step_events.argtypes = [ctypes.POINTER(StepArgs), P, c_size_t, P, P, P]
    lib.td_verify_step_kernels.argtypes = [ctypes.POINTER(StepArgs)]
    lib.td_verify_step_kernels.restype = c_int32
    lib.td_verify_step_kernel_events.argtypes = [ctypes.POINTER(StepArgs), P, c_size_t, P, c_int32,
                                                 c_int32, P, P]
    for name in ("td_draft_topk", "td_build_tree", "td_tree_mask", "td_tree_verify_attn",
                 "td_accept", "td_verify_step", "td_workspace_status", "td_verify_step_noalloc",
                 "td_verify_step_events", "td_kv_commit", "td_tree_qkv",
                 "td_lm_head_argmax", "td_verify_step_kernel_events"):
        getattr(lib, name).restype = c_int
    if lib.td_step_args_bytes() != ctypes.sizeof(StepArgs):
        raise ImportError("td_step_args layout differs between the library and this binding")
    return lib


lib = _load()


def last_error() -> str:
    return lib.td_last_error().decode()


def _check(st):
    if st != TD_OK:
        raise TreedraftError(st, last_error())


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _dt(t):
    if t.dtype == torch.bfloat16:
        return TD_BF16
    if t.dtype == torch.float32:
        return TD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------------

def draft_topk_workspace(batch, block, vocab, K) -> int:
    return int(lib.td_draft_topk_workspace(batch, block, vocab, K))


def draft_topk_alloc_workspace(batch, block, vocab, K, device):
    """Zero-filled workspace.  It holds per-workgroup epoch words, so one
    buffer serves any number of calls of the same shape; zero it again
    before a call with a different batch, block, vocab or K."""
    return torch.zeros(max(16, draft_topk_workspace(batch, block, vocab, K)), dtype=torch.uint8,
                       device=device)


def draft_topk(logits, K, out=None, workspace=None, stream=None):
    """logits [batch][block][vocab] (bf16 or f32, device).  Returns
    (topk_id int32[b][B][K], topk_logq f64[b][B][K], lse f64[b][B])."""
    _dev(logits, "logits")
    b, B, V = logits.shape
    dev = logits.device
    if out is None:
        out = (torch.empty((b, B, K), dtype=torch.int32, device=dev),
               torch.empty((b, B, K), dtype=torch.float64, device=dev),
               torch.empty((b, B), dtype=torch.float64, device=dev))
    ids, lq, lse = out
    if workspace is None:
        workspace = draft_topk_alloc_workspace(b, B, V, K, dev)
    _check(lib.td_draft_topk(_ptr(logits), _dt(logits), b, B, V, V, K, _ptr(ids), _ptr(lq),
                             _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return ids, lq, lse


def workspace_status(workspace, stream=None):
    """Wait for the stream, then read and clear the status word of a top-K or
    verify-step workspace.  Returns TD_OK, or TD_ESYNC when a cross-workgroup
    hand-off gave up since the last check (last_error() says which)."""
    _dev(workspace, "workspace")
    st = lib.td_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    if st not in (TD_OK, TD_ESYNC):
        _check(st)
    return st


def alloc_tree(batch, n_max, device):
    W = n_max + 1
    return dict(n_nodes=torch.empty(batch, dtype=torch.int32, device=device),
                node_token=torch.empty((batch, W), dtype=torch.int32, device=device),
                node_parent=torch.empty((batch, W), dtype=torch.int32, device=device),
                node_depth=torch.empty((batch, W), dtype=torch.int32, device=device),
                node_logrho=torch.empty((batch, W), dtype=torch.float64, device=device),
                ahat=torch.empty(batch, dtype=torch.float64, device=device),
                speedup=torch.empty(batch, dtype=torch.float64, device=device))


def build_tree(topk_id, topk_logq, n_max, use_stop, cost=(1.0, 0.0, 0.0, 0), l_ar=1.0, ahat0=1.0,
               root_token=None, out=None, stream=None, branch=0, min_logrho=float("-inf")):
    """branch: children per node (0: K); min_logrho: selective verification
    threshold on log rho (-inf: off)."""
    _dev(topk_id, "topk_id", torch.int32)
    b, B, K = topk_id.shape
    _dev(topk_logq, "topk_logq", torch.float64, (b, B, K))
    if root_token is not None:
        _dev(root_token, "root_token", torch.int32, (b,))
    t = alloc_tree(b, n_max, topk_id.device) if out is None else out
    ca, cb, cc, knee = cost
    _check(lib.td_build_tree(_ptr(topk_id), _ptr(topk_logq), b, B, K, n_max, int(bool(use_stop)),
                             float(ca), float(cb), float(cc), int(knee), float(l_ar), float(ahat0),
                             int(branch), float(min_logrho), _ptr(root_token), _ptr(t["n_nodes"]), _ptr(t["node_token"]),
                             _ptr(t["node_parent"]), _ptr(t["node_depth"]), _ptr(t["node_logrho"]),
                             _ptr(t["ahat"]), _ptr(t["speedup"]), _stream(stream)))
    return t


def flex_budget(batch, switch_batch, K, n_max, block):
    """(branch, n_max) for a step of `batch` sequences under the batch-size
    switch (td_flex_budget)."""
    br, nm = ctypes.c_int32(0), ctypes.c_int32(0)
    lib.td_flex_budget(int(batch), int(switch_batch), int(K), int(n_max), int(block),
                       ctypes.byref(br), ctypes.byref(nm))
    return br.value, nm.value


def fit_cost(n, t, knee_min, knee_max):
    """Least-squares fit of C(N) = a + b N + c max(0, N - knee) to measured
    (n, t) pairs (host arrays).  Returns (a, b, c, knee, rss)."""
    import numpy as np
    n = np.ascontiguousarray(n, dtype=np.float64)
    t = np.ascontiguousarray(t, dtype=np.float64)
    if n.shape != t.shape:
        raise ValueError("n and t differ in length")
    a, b, c, r = c_double(), c_double(), c_double(), c_double()
    k = c_int32()
    _check(lib.td_fit_cost(n.ctypes.data_as(c_void_p), t.ctypes.data_as(c_void_p), len(n),
                           int(knee_min), int(knee_max), ctypes.byref(a), ctypes.byref(b),
                           ctypes.byref(c), ctypes.byref(k), ctypes.byref(r)))
    return a.value, b.value, c.value, k.value, r.value


def tree_mask(node_parent, n_nodes, out=None, stream=None):
    _dev(node_parent, "node_parent", torch.int32)
    b, nq = node_parent.shape
    _dev(n_nodes, "n_nodes", torch.int32, (b,))
    words = (nq + 63) // 64
    mask = torch.empty((b, nq, words), dtype=torch.int64, device=node_parent.device) \
        if out is None else out
    _check(lib.td_tree_mask(_ptr(node_parent), _ptr(n_nodes), b, nq, _ptr(mask), _stream(stream)))
    return mask


def tree_verify_attn_workspace(batch, nq_max, hq, hkv, head_dim, total_ctx, max_ctx) -> int:
    return int(lib.td_tree_verify_attn_workspace(batch, nq_max, hq, hkv, head_dim, total_ctx,
                                                 max_ctx))


def tree_verify_attn_alloc_workspace(batch, nq_max, hq, hkv, head_dim, total_ctx, max_ctx, device):
    """Workspace for the per-chunk partials (no state is kept between calls;
    zero-filled only for tidiness)."""
    return torch.zeros(max(16, tree_verify_attn_workspace(batch, nq_max, hq, hkv, head_dim,
                                                          total_ctx, max_ctx)),
                       dtype=torch.uint8, device=device)


def tree_verify_attn(q, k_ctx, v_ctx, ctx_offsets, total_ctx, max_ctx, k_tree, v_tree, mask,
                     n_nodes, scale, out=None, workspace=None, stream=None, ctx_lengths=None):
    """q [b][nq][hq][d]; k_ctx/v_ctx [total][hkv][d]; k_tree/v_tree [b][nq][hkv][d];
    ctx_lengths int64 [b] or None (the context is the first ctx_lengths[b]
    rows of sequence b's region; None: the whole region)."""
    _dev(q, "q")
    b, nq, hq, d = q.shape
    hkv = k_tree.shape[2]
    for name, t, shp in (("k_tree", k_tree, (b, nq, hkv, d)), ("v_tree", v_tree, (b, nq, hkv, d)),
                         ("k_ctx", k_ctx, (total_ctx, hkv, d)), ("v_ctx", v_ctx, (total_ctx, hkv, d))):
        _dev(t, name, q.dtype, shp)
    _dev(ctx_offsets, "ctx_offsets", torch.int64, (b + 1,))
    if ctx_lengths is not None:
        _dev(ctx_lengths, "ctx_lengths", torch.int64, (b,))
    _dev(mask, "mask", torch.int64, (b, nq, (nq + 63) // 64))
    _dev(n_nodes, "n_nodes", torch.int32, (b,))
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = tree_verify_attn_alloc_workspace(b, nq, hq, hkv, d, total_ctx, max_ctx,
                                                     q.device)
    _check(lib.td_tree_verify_attn(_ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_offsets),
                                   _ptr(ctx_lengths), total_ctx,
                                   max_ctx, _ptr(k_tree), _ptr(v_tree), _ptr(mask), _ptr(n_nodes), b,
                                   nq, hq, hkv, d, float(scale), _dt(q), _ptr(out), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))
    return out


def accept(node_token, node_parent, n_nodes, target_token, block, out=None, stream=None):
    _dev(node_token, "node_token", torch.int32)
    b, W = node_token.shape
    _dev(node_parent, "node_parent", torch.int32, (b, W))
    _dev(n_nodes, "n_nodes", torch.int32, (b,))
    _dev(target_token, "target_token", torch.int32, (b, W))
    dev = node_token.device
    if out is None:
        out = (torch.empty(b, dtype=torch.int32, device=dev),
               torch.empty((b, block + 1), dtype=torch.int32, device=dev),
               torch.empty(b, dtype=torch.int32, device=dev))
    alen, path, bonus = out
    _check(lib.td_accept(_ptr(node_token), _ptr(node_parent), _ptr(n_nodes), _ptr(target_token), b,
                         W - 1, block, _ptr(alen), _ptr(path), _ptr(bonus), _stream(stream)))
    return alen, path, bonus


def kv_commit(k_tree, v_tree, accept_len, accept_path, bonus_token, k_cache, v_cache, ctx_offsets,
              ctx_lengths, next_root=None, stream=None):
    """Append each sequence's accepted path (root first) from the tree K/V to
    its context region of k_cache / v_cache; ctx_lengths advances in place.
    next_root (int32 [b], optional) receives the bonus tokens."""
    _dev(k_tree, "k_tree")
    b, nq, hkv, d = k_tree.shape
    _dev(v_tree, "v_tree", k_tree.dtype, k_tree.shape)
    _dev(accept_len, "accept_len", torch.int32, (b,))
    _dev(accept_path, "accept_path", torch.int32)
    block = accept_path.shape[1] - 1
    _dev(bonus_token, "bonus_token", torch.int32, (b,))
    _dev(k_cache, "k_cache", k_tree.dtype)
    _dev(v_cache, "v_cache", k_tree.dtype, k_cache.shape)
    _dev(ctx_offsets, "ctx_offsets", torch.int64, (b + 1,))
    _dev(ctx_lengths, "ctx_lengths", torch.int64, (b,))
    if next_root is not None:
        _dev(next_root, "next_root", torch.int32, (b,))
    _check(lib.td_kv_commit(_ptr(k_tree), _ptr(v_tree), _ptr(accept_len), _ptr(accept_path),
                            _ptr(bonus_token), b, nq, block, hkv, d, _dt(k_tree), _ptr(k_cache),
                            _ptr(v_cache), _ptr(ctx_offsets), _ptr(ctx_lengths), _ptr(next_root),
                            _stream(stream)))


def verify_layer_workspace(batch, nq_max, hq, hkv, head_dim, vocab, device):
    n = int(lib.td_verify_layer_workspace(batch, nq_max, hq, hkv, head_dim, vocab))
    if n == 0:
        raise TreedraftError(TD_EINVAL, "invalid verify-layer shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def tree_qkv(embed, w_qkv, node_token, node_depth, n_nodes, ctx_offsets, hq, hkv, head_dim,
             rope_base, ctx_lengths=None, out=None, workspace=None, stream=None):
    """Q / K / V of the tree tokens with rotary positions (bf16).  Returns
    (q [b][nq][hq][d], k_tree [b][nq][hkv][d], v_tree)."""
    _dev(embed, "embed", torch.bfloat16)
    vocab, hidden = embed.shape
    _dev(w_qkv, "w_qkv", torch.bfloat16, ((hq + 2 * hkv) * head_dim, hidden))
    _dev(node_token, "node_token", torch.int32)
    b, nq = node_token.shape
    _dev(node_depth, "node_depth", torch.int32, (b, nq))
    _dev(n_nodes, "n_nodes", torch.int32, (b,))
    _dev(ctx_offsets, "ctx_offsets", torch.int64, (b + 1,))
    if ctx_lengths is not None:
        _dev(ctx_lengths, "ctx_lengths", torch.int64, (b,))
    dev = embed.device
    if out is None:
        out = (torch.empty((b, nq, hq, head_dim), dtype=torch.bfloat16, device=dev),
               torch.empty((b, nq, hkv, head_dim), dtype=torch.bfloat16, device=dev),
               torch.empty((b, nq, hkv, head_dim), dtype=torch.bfloat16, device=dev))
    q, k, v = out
    if workspace is None:
        workspace = verify_layer_workspace(b, nq, hq, hkv, head_dim, vocab, dev)
    _check(lib.td_tree_qkv(_ptr(embed), _ptr(w_qkv), _ptr(node_token), _ptr(node_depth),
                           _ptr(n_nodes), _ptr(ctx_offsets), _ptr(ctx_lengths), b, nq, vocab, hq,
                           hkv, head_dim, float(rope_base), _ptr(q), _ptr(k), _ptr(v),
                           _ptr(workspace), workspace.numel(), _stream(stream)))
    return q, k, v


def lm_head_argmax(hidden_rows, w_lm, n_nodes, out=None, workspace=None, stream=None):
    """Greedy target token of every tree row: argmax over the vocabulary of
    hidden_rows [b][nq][hq][d] (or [b][nq][hidden]) times w_lm [vocab][hidden]."""
    _dev(hidden_rows, "hidden_rows", torch.bfloat16)
    b, nq = hidden_rows.shape[:2]
    hidden = hidden_rows[0, 0].numel()
    _dev(w_lm, "w_lm", torch.bfloat16)
    vocab = w_lm.shape[0]
    if w_lm.shape[1] != hidden:
        raise ValueError("w_lm must have shape [vocab][hidden]")
    _dev(n_nodes, "n_nodes", torch.int32, (b,))
    head_dim = 128 if hidden % 128 == 0 else 64
    hq = hidden // head_dim
    if out is None:
        out = torch.empty((b, nq), dtype=torch.int32, device=w_lm.device)
    if workspace is None:
        workspace = verify_layer_workspace(b, nq, hq, hq, head_dim, vocab, w_lm.device)
    _check(lib.td_lm_head_argmax(_ptr(hidden_rows), _ptr(w_lm), _ptr(n_nodes), b, nq, hq, head_dim,
                                 vocab, _ptr(out), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# the fused verify step

class VerifyStep:
    """Argument block and buffers of td_verify_step for one fixed problem.

    All tensors are device tensors; outputs and the (zero-filled) workspace
    are allocated once, so repeated calls allocate nothing and can be
    captured in a HIP graph."""

    def __init__(self, *, batch, block, vocab, topk, n_max, use_stop, cost, l_ar, ahat0, hq, hkv,
                 head_dim, scale, logits_dtype, attn_dtype, total_ctx, max_ctx, device, branch=0,
                 min_logrho=float("-inf")):
        dev = device
        W = n_max + 1
        self.topk_id = torch.empty((batch, block, topk), dtype=torch.int32, device=dev)
        self.topk_logq = torch.empty((batch, block, topk), dtype=torch.float64, device=dev)
        self.lse = torch.empty((batch, block), dtype=torch.float64, device=dev)
        self.tree = alloc_tree(batch, n_max, dev)
        self.mask = torch.empty((batch, W, (W + 63) // 64), dtype=torch.int64, device=dev)
        adt = torch.bfloat16 if attn_dtype == TD_BF16 else torch.float32
        self.out = torch.empty((batch, W, hq, head_dim), dtype=adt, device=dev)
        self.accept_len = torch.empty(batch, dtype=torch.int32, device=dev)
        self.accept_path = torch.empty((batch, block + 1), dtype=torch.int32, device=dev)
        self.bonus_token = torch.empty(batch, dtype=torch.int32, device=dev)
        a = StepArgs()
        a.logits_dtype, a.batch, a.block, a.vocab, a.pos_stride, a.topk = (
            logits_dtype, batch, block, vocab, vocab, topk)
        a.n_max, a.use_stop = n_max, int(bool(use_stop))
        a.cost_a, a.cost_b, a.cost_c, a.cost_knee = float(cost[0]), float(cost[1]), float(cost[2]), int(cost[3])
        a.l_ar, a.ahat0 = float(l_ar), float(ahat0)
        a.branch, a.min_logrho = int(branch), float(min_logrho)
        a.total_ctx, a.max_ctx = int(total_ctx), int(max_ctx)
        a.hq, a.hkv, a.head_dim, a.scale, a.attn_dtype = hq, hkv, head_dim, float(scale), attn_dtype
        t = self.tree
        for name, ten in (("topk_id", self.topk_id), ("topk_logq", self.topk_logq),
                          ("lse", self.lse), ("n_nodes", t["n_nodes"]),
                          ("node_token", t["node_token"]), ("node_parent", t["node_parent"]),
                          ("node_depth", t["node_depth"]), ("node_logrho", t["node_logrho"]),
                          ("ahat", t["ahat"]), ("speedup", t["speedup"]), ("mask", self.mask),
                          ("out", self.out), ("accept_len", self.accept_len),
                          ("accept_path", self.accept_path), ("bonus_token", self.bonus_token)):
            setattr(a, name, ten.data_ptr())
        self.args = a
        self.workspace = torch.zeros(max(16, int(lib.td_verify_step_workspace(ctypes.byref(a)))),
                                     dtype=torch.uint8, device=dev)

    def set_inputs(self, logits, q, k_ctx, v_ctx, ctx_offsets, k_tree, v_tree, target_token,
                   root_token=None, ctx_lengths=None, commit=False, next_root=None):
        """commit: after acceptance, append the accepted path's K/V to the
        contexts (k_ctx / v_ctx rows after ctx_lengths[b], which advances);
        next_root receives the bonus tokens."""
        if commit and ctx_lengths is None:
            raise ValueError("commit needs ctx_lengths")
        a = self.args
        a.logits = logits.data_ptr()
        a.q, a.k_ctx, a.v_ctx = q.data_ptr(), k_ctx.data_ptr(), v_ctx.data_ptr()
        a.ctx_offsets = ctx_offsets.data_ptr()
        a.ctx_lengths = None if ctx_lengths is None else ctx_lengths.data_ptr()
        a.commit = int(bool(commit))
        a.next_root = None if next_root is None else next_root.data_ptr()
        a.k_tree, a.v_tree = k_tree.data_ptr(), v_tree.data_ptr()
        a.target_token = target_token.data_ptr()
        a.root_token = None if root_token is None else root_token.data_ptr()
        self._keep = (logits, q, k_ctx, v_ctx, ctx_offsets, k_tree, v_tree, target_token, root_token,
                      ctx_lengths, next_root)

    def status(self, stream=None):
        """TD_OK, or TD_ESYNC if a hand-off of an earlier call gave up
        (waits for the stream; clears the status word)."""
        return workspace_status(self.workspace, stream)

    def run_timed(self, start, stop, stream=None, stages=0):
        """Enqueue the step with torch timing events attached to its kernels:
        start.elapsed_time(stop) is then the execution time of the selected
        stages' kernels, first start to last end (both events must have been
        recorded once before, so that their HIP events exist)."""
        self.args.stages = stages
        _check(lib.td_verify_step_events(ctypes.byref(self.args), _ptr(self.workspace),
                                         self.workspace.numel(), _stream(stream),
                                         c_void_p(start.cuda_event), c_void_p(stop.cuda_event)))

    def kernels(self, stages=0):
        """How many kernels the step enqueues for these arguments (both
        stages: 2 when the context split runs inside the first kernel, else 3)."""
        self.args.stages = stages
        return int(lib.td_verify_step_kernels(ctypes.byref(self.args)))

    def run_kernels_timed(self, first, last, start, stop, stream=None, stages=0):
        """Enqueue the whole step with torch timing events on its kernels
        first .. last (0-based, launch order): start.elapsed_time(stop) is
        their execution time, first start to last end (both events must have
        been recorded once before, so that their HIP events exist)."""
        self.args.stages = stages
        _check(lib.td_verify_step_kernel_events(ctypes.byref(self.args), _ptr(self.workspace),
                                                self.workspace.numel(), _stream(stream), first, last,
                                                c_void_p(start.cuda_event), c_void_p(stop.cuda_event)))

    def run(self, stream=None, stages=0):
        """Enqueue the step (stages: TD_STEP_DRAFT | TD_STEP_VERIFY, 0 = both)."""
        self.args.stages = stages
        _check(lib.td_verify_step(ctypes.byref(self.args), _ptr(self.workspace),
                                  self.workspace.numel(), _stream(stream)))
