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
LIB_PATH = os.path.join(_HERE, "libtreedraft.so")

TD_OK, TD_EINVAL, TD_ECAPACITY, TD_EUNSUPPORTED, TD_EHIP = range(5)
TD_F32, TD_BF16 = 0, 1
STATUS_NAMES = {0: "TD_OK", 1: "TD_EINVAL", 2: "TD_ECAPACITY", 3: "TD_EUNSUPPORTED", 4: "TD_EHIP"}

# every symbol declared in include/treedraft.h
EXPORTED = ["td_abi_version", "td_last_error", "td_draft_topk_workspace", "td_draft_topk",
            "td_build_tree", "td_tree_mask", "td_tree_verify_attn_workspace",
            "td_tree_verify_attn", "td_accept"]


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
                                  c_double, c_double, c_int32, c_double, c_double, P, P, P, P, P, P,
                                  P, P, P]
    lib.td_tree_mask.argtypes = [P, P, c_int32, c_int32, P, P]
    lib.td_tree_verify_attn_workspace.argtypes = [c_int32] * 5 + [c_int64, c_int64]
    lib.td_tree_verify_attn_workspace.restype = c_size_t
    lib.td_tree_verify_attn.argtypes = [P, P, P, P, c_int64, c_int64, P, P, P, P, c_int32, c_int32,
                                        c_int32, c_int32, c_int32, c_float, c_int, P, P, c_size_t, P]
    lib.td_accept.argtypes = [P, P, P, P, c_int32, c_int32, c_int32, P, P, P, P]
    for name in ("td_draft_topk", "td_build_tree", "td_tree_mask", "td_tree_verify_attn",
                 "td_accept"):
        getattr(lib, name).restype = c_int
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
    """Zero-filled workspace (its arrival counters must start at zero; each
    call leaves them zero, so the buffer can be reused)."""
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
               root_token=None, out=None, stream=None):
    _dev(topk_id, "topk_id", torch.int32)
    b, B, K = topk_id.shape
    _dev(topk_logq, "topk_logq", torch.float64, (b, B, K))
    if root_token is not None:
        _dev(root_token, "root_token", torch.int32, (b,))
    t = alloc_tree(b, n_max, topk_id.device) if out is None else out
    ca, cb, cc, knee = cost
    _check(lib.td_build_tree(_ptr(topk_id), _ptr(topk_logq), b, B, K, n_max, int(bool(use_stop)),
                             float(ca), float(cb), float(cc), int(knee), float(l_ar), float(ahat0),
                             _ptr(root_token), _ptr(t["n_nodes"]), _ptr(t["node_token"]),
                             _ptr(t["node_parent"]), _ptr(t["node_depth"]), _ptr(t["node_logrho"]),
                             _ptr(t["ahat"]), _ptr(t["speedup"]), _stream(stream)))
    return t


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
    """Zero-filled workspace (arrival counters start at zero and every call
    leaves them zero, so the buffer can be reused)."""
    return torch.zeros(max(16, tree_verify_attn_workspace(batch, nq_max, hq, hkv, head_dim,
                                                          total_ctx, max_ctx)),
                       dtype=torch.uint8, device=device)


def tree_verify_attn(q, k_ctx, v_ctx, ctx_offsets, total_ctx, max_ctx, k_tree, v_tree, mask,
                     n_nodes, scale, out=None, workspace=None, stream=None):
    """q [b][nq][hq][d]; k_ctx/v_ctx [total][hkv][d]; k_tree/v_tree [b][nq][hkv][d]."""
    _dev(q, "q")
    b, nq, hq, d = q.shape
    hkv = k_tree.shape[2]
    for name, t, shp in (("k_tree", k_tree, (b, nq, hkv, d)), ("v_tree", v_tree, (b, nq, hkv, d)),
                         ("k_ctx", k_ctx, (total_ctx, hkv, d)), ("v_ctx", v_ctx, (total_ctx, hkv, d))):
        _dev(t, name, q.dtype, shp)
    _dev(ctx_offsets, "ctx_offsets", torch.int64, (b + 1,))
    _dev(mask, "mask", torch.int64, (b, nq, (nq + 63) // 64))
    _dev(n_nodes, "n_nodes", torch.int32, (b,))
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = tree_verify_attn_alloc_workspace(b, nq, hq, hkv, d, total_ctx, max_ctx,
                                                     q.device)
    _check(lib.td_tree_verify_attn(_ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_offsets), total_ctx,
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
