"""The tachometer: the verification latency of a tree of N draft nodes,
measured on this GPU, and the fit of the budget controller's cost model to it
(BASTION, "Methodik" §3, latency modelling: a roofline model of the
verification latency, calibrated on observed runtimes so that kernel fusion
and scheduling overheads are accounted for; the explanatory part's
"tachometer" measures how long verifying a tree of a given size takes on the
device).

The verification measured here is this library's own one-layer pass over a
tree of N nodes: the tree tokens' Q/K/V projection with rotary positions
(td_tree_qkv), tree attention against the context (td_tree_verify_attn) and
the LM-head argmax that yields the target tokens (td_lm_head_argmax), on
N + 1 query rows.  Times are HIP-event averages of back-to-back calls on the
launch stream.  td_fit_cost then fits C(N) = a + b N + c max(0, N - knee);
divided by a, the fit is in units of one single-token verification (the
autoregressive step: L_AR = 1), the form td_build_tree's stop takes.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as td

DEFAULT_SIZES = (0, 1, 2, 4, 8, 12, 16, 24, 32, 40, 48, 64, 80, 96, 128, 160, 192, 224, 255)


class VerifyPass:
    """Buffers of the one-layer verification for one tree capacity."""

    def __init__(self, *, batch, nq_max, hq, hkv, head_dim, vocab, weights, k_ctx, v_ctx,
                 ctx_offsets, ctx_lengths=None, scale, rope_base, device):
        self.batch, self.nq_max = batch, nq_max
        self.hq, self.hkv, self.head_dim, self.vocab = hq, hkv, head_dim, vocab
        self.w = weights
        self.k_ctx, self.v_ctx, self.off, self.lens = k_ctx, v_ctx, ctx_offsets, ctx_lengths
        self.total_ctx = int(k_ctx.shape[0])
        self.scale, self.rope_base = scale, rope_base
        bf = torch.bfloat16
        self.q = torch.empty((batch, nq_max, hq, head_dim), dtype=bf, device=device)
        self.kt = torch.empty((batch, nq_max, hkv, head_dim), dtype=bf, device=device)
        self.vt = torch.empty_like(self.kt)
        self.out = torch.empty_like(self.q)
        self.mask = torch.empty((batch, nq_max, (nq_max + 63) // 64), dtype=torch.int64,
                                device=device)
        self.target = torch.empty((batch, nq_max), dtype=torch.int32, device=device)
        self.ws_layer = td.verify_layer_workspace(batch, nq_max, hq, hkv, head_dim, vocab, device)
        self.ws_attn = td.tree_verify_attn_alloc_workspace(batch, nq_max, hq, hkv, head_dim,
                                                           self.total_ctx, self.total_ctx, device)

    def run(self, tree):
        """tree: device arrays node_token, node_parent, node_depth [b][nq_max],
        n_nodes [b] (from td.build_tree); leaves the target tokens in .target."""
        td.tree_qkv(self.w["embed"], self.w["w_qkv"], tree["node_token"], tree["node_depth"],
                    tree["n_nodes"], self.off, self.hq, self.hkv, self.head_dim, self.rope_base,
                    ctx_lengths=self.lens, out=(self.q, self.kt, self.vt),
                    workspace=self.ws_layer)
        td.tree_mask(tree["node_parent"], tree["n_nodes"], out=self.mask)
        td.tree_verify_attn(self.q, self.k_ctx, self.v_ctx, self.off, self.total_ctx,
                            self.total_ctx, self.kt, self.vt, self.mask, tree["n_nodes"],
                            self.scale, out=self.out, workspace=self.ws_attn,
                            ctx_lengths=self.lens)
        td.lm_head_argmax(self.out, self.w["w_lm"], tree["n_nodes"], out=self.target,
                          workspace=self.ws_layer)


def measure(topk_id, topk_logq, sizes=DEFAULT_SIZES, reps=20, warmup=3, **pass_kw):
    """Verification time (microseconds per call) of trees of each size N in
    `sizes`, built best-first with a fixed budget N from the given top-K
    tables.  Returns a list of (N, n_nodes realised, microseconds)."""
    stream = torch.cuda.current_stream()
    points = []
    for n in sizes:
        tree = td.build_tree(topk_id, topk_logq, int(n), False)
        vp = VerifyPass(nq_max=int(n) + 1, **pass_kw)
        for _ in range(warmup):
            vp.run(tree)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            vp.run(tree)
        t1.record(stream)
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / reps
        points.append((int(n), int(tree["n_nodes"].max()), us))
        del vp
    return points


def fit(points, knee_min=0, knee_max=None):
    """Fit of C(N) to measured points; returns absolute (microseconds) and
    normalised (a = 1, L_AR = 1) coefficients."""
    n = np.array([p[1] for p in points], dtype=np.float64)
    t = np.array([p[2] for p in points], dtype=np.float64)
    kmax = int(n.max()) if knee_max is None else knee_max
    a, b, c, knee, rss = td.fit_cost(n, t, knee_min, kmax)
    tss = float(((t - t.mean()) ** 2).sum())
    return {"a_us": a, "b_us": b, "c_us": c, "knee": knee, "rss": rss,
            "r2": 1.0 - rss / tss if tss > 0 else 1.0,
            "cost": (1.0, b / a, c / a, knee), "l_ar": 1.0}
