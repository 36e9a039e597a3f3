"""CPU oracle of the verify-side path (TEST INFRASTRUCTURE ONLY).

Thin ctypes wrapper over ``oracle/liboracle.so`` (built from ``oracle.c`` by
``oracle/build.py``).  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use this package; the HIP library never does.

Each function follows one stage of budget-aware tree speculative decoding
(BASTION technical summary, "Methodik" §1-§3; greedy acceptance from
"Experimentelle Ergebnisse"); see the comments in ``oracle.c``.

Parity unpinned: none of these functions; every one has a pin in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_double, c_int, c_int32, c_int64, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load(path=None):
    global _lib
    if _lib is None or path is not None:
        if path is None and not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        # TD_ORACLE_LIB: another build of the same source (the sanitizer check)
        lib = ctypes.CDLL(path or os.environ.get("TD_ORACLE_LIB") or LIB_PATH)
        P = c_void_p
        lib.or_draft_topk.argtypes = [P, c_int, c_int, c_int, c_int, c_int64, c_int, P, P, P]
        lib.or_build_tree.argtypes = [P, P, c_int, c_int, c_int, c_int, c_int, c_double, c_double,
                                      c_double, c_int, c_double, c_double, P, P, P, P, P, P, P, P, P,
                                      c_int, c_double]
        lib.or_flex_budget.argtypes = [c_int, c_int, c_int, c_int, c_int, P, P]
        lib.or_flex_budget.restype = None
        lib.or_tree_qkv.argtypes = [P, P, P, P, P, P, P, c_int, c_int, c_int, c_int, c_int, c_int,
                                    c_int, c_double, P, P, P]
        lib.or_lm_head_argmax.argtypes = [P, P, P, c_int, c_int, c_int, c_int, P, P, P]
        lib.or_tree_qkv.restype = c_int
        lib.or_lm_head_argmax.restype = c_int
        lib.or_tree_mask.argtypes = [P, P, c_int, c_int, P]
        lib.or_tree_attn.argtypes = [P, P, P, P, P, P, P, P, P, c_int, c_int, c_int, c_int, c_int,
                                     c_double, c_int, P, c_int32, c_int32, c_int32]
        lib.or_kv_commit.argtypes = [P, P, P, P, P, c_int, c_int, c_int, c_int, c_int, c_int, P, P,
                                     P, P, P]
        lib.or_accept.argtypes = [P, P, P, P, c_int, c_int, c_int, P, P, P]
        lib.or_set_threads.argtypes = [c_int]
        lib.or_set_threads.restype = c_int
        for f in (lib.or_draft_topk, lib.or_build_tree, lib.or_tree_mask, lib.or_tree_attn,
                  lib.or_accept, lib.or_kv_commit):
            f.restype = c_int
        _lib = lib
    return _lib


def use_library(path=None):
    """Point the wrapper at another build of oracle.c (the mutation tests load
    copies with planted mistakes); None restores the default library."""
    global _lib
    _lib = None
    if path is not None:
        _load(path)


def set_threads(n: int = 0) -> int:
    """Threads the oracle spreads independent outputs over (n <= 0: keep the
    current setting); returns the count in effect.  Results do not depend on
    it: every output is computed by one thread in the same order."""
    return int(_load().or_set_threads(int(n)))


def _p(a):
    return None if a is None else a.ctypes.data_as(c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def _dtype_code(arr) -> int:
    if arr.dtype == np.float32:
        return 0
    if arr.dtype == np.uint16:
        return 1
    raise TypeError("logits/attention inputs must be float32 or bf16 bits (uint16)")


def draft_topk(logits: np.ndarray, K: int):
    """logits [batch][block][vocab] float32 or bf16 bits.
    Returns (topk_id int32[b][B][K], topk_logq f64[b][B][K], lse f64[b][B])."""
    logits = np.ascontiguousarray(logits)
    b, B, V = logits.shape
    ids = np.empty((b, B, K), np.int32)
    lq = np.empty((b, B, K), np.float64)
    lse = np.empty((b, B), np.float64)
    _check(_load().or_draft_topk(_p(logits), _dtype_code(logits), b, B, V, V, K, _p(ids), _p(lq),
                                 _p(lse)), "or_draft_topk")
    return ids, lq, lse


def build_tree(topk_id, topk_logq, n_max, use_stop, cost=(1.0, 0.0, 0.0, 0), l_ar=1.0,
               ahat0=1.0, root_token=None, want_curve=False, branch=0, min_logrho=-math.inf):
    """Best-first tree.  Returns dict of node arrays [b][n_max+1] (index 0 = root),
    n_nodes[b] (draft nodes), ahat[b], speedup[b] and optionally s_curve.
    branch: children per node (0: K); min_logrho: no node below this log rho."""
    topk_id = _c(topk_id, np.int32)
    topk_logq = _c(topk_logq, np.float64)
    b, B, K = topk_id.shape
    W = n_max + 1
    out = dict(n_nodes=np.empty(b, np.int32), node_token=np.empty((b, W), np.int32),
               node_parent=np.empty((b, W), np.int32), node_depth=np.empty((b, W), np.int32),
               node_logrho=np.empty((b, W), np.float64), ahat=np.empty(b, np.float64),
               speedup=np.empty(b, np.float64))
    curve = np.empty((b, W), np.float64) if want_curve else None
    rt = None if root_token is None else _c(root_token, np.int32)
    ca, cb, cc, knee = cost
    _check(_load().or_build_tree(_p(topk_id), _p(topk_logq), b, B, K, n_max, int(bool(use_stop)),
                                 ca, cb, cc, int(knee), l_ar, ahat0, _p(rt), _p(out["n_nodes"]),
                                 _p(out["node_token"]), _p(out["node_parent"]),
                                 _p(out["node_depth"]), _p(out["node_logrho"]), _p(out["ahat"]),
                                 _p(out["speedup"]), _p(curve), int(branch), float(min_logrho)),
           "or_build_tree")
    if want_curve:
        out["s_curve"] = curve
    return out


def flex_budget(batch, switch_batch, K, n_max, block):
    """(branch, n_max) of a step of `batch` sequences under the batch-size
    switch (single branch at or above switch_batch)."""
    br, nm = ctypes.c_int(0), ctypes.c_int(0)
    _load().or_flex_budget(int(batch), int(switch_batch), int(K), int(n_max), int(block),
                           ctypes.byref(br), ctypes.byref(nm))
    return br.value, nm.value


def tree_mask(node_parent, n_nodes, nq_max=None):
    node_parent = _c(node_parent, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    b, W = node_parent.shape
    nq_max = W if nq_max is None else nq_max
    assert nq_max == W
    words = (nq_max + 63) // 64
    mask = np.empty((b, nq_max, words), np.uint64)
    _check(_load().or_tree_mask(_p(node_parent), _p(n_nodes), b, nq_max, _p(mask)), "or_tree_mask")
    return mask


def tree_attn(q, k_ctx, v_ctx, ctx_offsets, k_tree, v_tree, mask, n_nodes, hq, hkv, d, scale,
              seqs=None, row_limit=-1, ctx_lengths=None):
    """float64 output [len(seqs)][nq_max][hq][d]; seqs = contiguous range (b0, b1).
    ctx_lengths [batch] (optional): sequence b's context is the first
    ctx_lengths[b] rows of its region (None: the whole region)."""
    arrs = [np.ascontiguousarray(x) for x in (q, k_ctx, v_ctx, k_tree, v_tree)]
    q, k_ctx, v_ctx, k_tree, v_tree = arrs
    dt = _dtype_code(q)
    for x in arrs:
        assert x.dtype == q.dtype
    ctx_offsets = _c(ctx_offsets, np.int64)
    mask = _c(mask, np.uint64)
    n_nodes = _c(n_nodes, np.int32)
    batch, nq_max = q.shape[0], q.shape[1]
    b0, b1 = (0, batch) if seqs is None else seqs
    out = np.empty((b1 - b0, nq_max, hq, d), np.float64)
    lens = None if ctx_lengths is None else _c(ctx_lengths, np.int64)
    _check(_load().or_tree_attn(_p(q), _p(k_ctx), _p(v_ctx), _p(ctx_offsets), _p(lens), _p(k_tree),
                                _p(v_tree), _p(mask), _p(n_nodes), batch, nq_max, hq, hkv, d,
                                float(scale), dt, _p(out), b0, b1, int(row_limit)), "or_tree_attn")
    return out


def accept(node_token, node_parent, n_nodes, target_token, block):
    node_token = _c(node_token, np.int32)
    node_parent = _c(node_parent, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    target_token = _c(target_token, np.int32)
    b, W = node_token.shape
    alen = np.empty(b, np.int32)
    path = np.empty((b, block + 1), np.int32)
    bonus = np.empty(b, np.int32)
    _check(_load().or_accept(_p(node_token), _p(node_parent), _p(n_nodes), _p(target_token), b,
                             W - 1, block, _p(alen), _p(path), _p(bonus)), "or_accept")
    return alen, path, bonus


def kv_commit(k_tree, v_tree, accept_len, accept_path, bonus_token, k_cache, v_cache, ctx_offsets,
              ctx_lengths, hkv, d):
    """Append each sequence's accepted path (root first) from the tree K/V to
    its context region.  k_cache / v_cache [total][hkv][d] and ctx_lengths
    [batch] are updated IN PLACE; returns next_root [batch] (the bonus)."""
    k_tree = np.ascontiguousarray(k_tree)
    v_tree = np.ascontiguousarray(v_tree)
    dt = _dtype_code(k_tree)
    for x in (v_tree, k_cache, v_cache):
        assert x.dtype == k_tree.dtype and x.flags.c_contiguous
    assert ctx_lengths.dtype == np.int64 and ctx_lengths.flags.c_contiguous
    accept_len = _c(accept_len, np.int32)
    accept_path = _c(accept_path, np.int32)
    bonus = _c(bonus_token, np.int32)
    ctx_offsets = _c(ctx_offsets, np.int64)
    batch, nq_max = k_tree.shape[0], k_tree.shape[1]
    block = accept_path.shape[1] - 1
    nxt = np.empty(batch, np.int32)
    _check(_load().or_kv_commit(_p(k_tree), _p(v_tree), _p(accept_len), _p(accept_path), _p(bonus),
                                batch, nq_max, block, hkv, d, dt, _p(k_cache), _p(v_cache),
                                _p(ctx_offsets), _p(ctx_lengths), _p(nxt)), "or_kv_commit")
    return nxt


def tree_qkv(embed, w_qkv, node_token, node_depth, n_nodes, ctx_offsets, hq, hkv, d, rope_base,
             ctx_lengths=None):
    """Projection of the tree tokens' embeddings with rotary positions.
    embed [vocab][hidden], w_qkv [(hq + 2 hkv) d][hidden] bf16 bits (uint16).
    Returns float64 q [b][nq][hq][d], k, v [b][nq][hkv][d] (zero beyond the tree)."""
    embed = np.ascontiguousarray(embed, dtype=np.uint16)
    w_qkv = np.ascontiguousarray(w_qkv, dtype=np.uint16)
    node_token = _c(node_token, np.int32)
    node_depth = _c(node_depth, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    ctx_offsets = _c(ctx_offsets, np.int64)
    lens = None if ctx_lengths is None else _c(ctx_lengths, np.int64)
    b, nq = node_token.shape
    vocab, hidden = embed.shape
    assert w_qkv.shape == ((hq + 2 * hkv) * d, hidden)
    q = np.empty((b, nq, hq, d))
    k = np.empty((b, nq, hkv, d))
    v = np.empty((b, nq, hkv, d))
    _check(_load().or_tree_qkv(_p(embed), _p(w_qkv), _p(node_token), _p(node_depth), _p(n_nodes),
                               _p(ctx_offsets), _p(lens), b, nq, hidden, vocab, hq, hkv, d,
                               float(rope_base), _p(q), _p(k), _p(v)), "or_tree_qkv")
    return q, k, v


def lm_head_argmax(rows, w_lm, n_nodes):
    """Greedy token of every tree row: argmax over the vocabulary of
    rows [b][nq][hidden] (bf16 bits) times w_lm [vocab][hidden] (bf16 bits),
    ties to the smaller id; -1 beyond the tree.  Returns (target, best,
    second): the two largest float64 logits of each row."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    w_lm = np.ascontiguousarray(w_lm, dtype=np.uint16)
    n_nodes = _c(n_nodes, np.int32)
    b, nq, hidden = rows.shape
    vocab = w_lm.shape[0]
    assert w_lm.shape[1] == hidden
    tgt = np.empty((b, nq), np.int32)
    best = np.empty((b, nq))
    second = np.empty((b, nq))
    _check(_load().or_lm_head_argmax(_p(rows), _p(w_lm), _p(n_nodes), b, nq, hidden, vocab,
                                     _p(tgt), _p(best), _p(second)), "or_lm_head_argmax")
    return tgt, best, second
