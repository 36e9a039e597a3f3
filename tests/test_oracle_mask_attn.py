"""Pins of the oracle's stage (b') ancestor mask and stage (c) tree attention.

The pages have the target score the whole tree in one parallel pass; a tree
row can only depend on its own root path (prefix tree, BASTION "Methodik" §1).
Pins:
  * mask: ancestor sets by walking parent pointers; popcount = depth + 1;
  * attention: torch's scaled_dot_product_attention in float64 on the CPU
    with an explicit boolean mask (library special case); a chain tree is
    causal attention; a root-only tree is plain decode attention; a star tree
    admits only context, root and self; one wrong mask bit is visible.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tree_draft_build_amd import workload as wl


def random_tree(rng, n, nq_max):
    par = np.full(nq_max, -1, np.int32)
    for i in range(1, n + 1):
        par[i] = rng.integers(0, i)
    return par


def anc_sets(par, n):
    out = []
    for i in range(n + 1):
        s, u = {i}, i
        while u > 0:
            u = int(par[u])
            s.add(u)
        out.append(s)
    return out


@pytest.mark.parametrize("nq_max", [1, 2, 17, 64, 65, 129, 200])
def test_mask_is_ancestor_or_self(nq_max):
    rng = np.random.default_rng(nq_max)
    b = 3
    n_nodes = np.array([nq_max - 1, rng.integers(0, nq_max), 0], np.int32)
    par = np.stack([random_tree(rng, int(n), nq_max) for n in n_nodes])
    mask = oracle.tree_mask(par, n_nodes)
    W = (nq_max + 63) // 64
    assert mask.shape == (b, nq_max, W)
    for bi in range(b):
        n = int(n_nodes[bi])
        sets = anc_sets(par[bi], n)
        depth = [len(s) - 1 for s in sets]
        for i in range(nq_max):
            bits = {w * 64 + t for w in range(W) for t in range(64)
                    if (int(mask[bi, i, w]) >> t) & 1}
            if i <= n:
                assert bits == sets[i]
                assert len(bits) == depth[i] + 1
            else:
                assert bits == set()


def _sdpa_reference(inp, par, n_nodes, hq, hkv, d, scale, dtype):
    """Row-by-row float64 SDPA with a boolean mask built from parent walks."""
    q = wl.logits_as_f64(inp["q"], dtype)
    kc, vc = wl.logits_as_f64(inp["k_ctx"], dtype), wl.logits_as_f64(inp["v_ctx"], dtype)
    kt, vt = wl.logits_as_f64(inp["k_tree"], dtype), wl.logits_as_f64(inp["v_tree"], dtype)
    off = inp["ctx_offsets"]
    batch, nq = q.shape[:2]
    out = np.zeros((batch, nq, hq, d))
    rep = hq // hkv
    for b in range(batch):
        n = int(n_nodes[b])
        L = int(off[b + 1] - off[b])
        keys = np.concatenate([kc[off[b]:off[b + 1]], kt[b]], 0)     # [L+nq][hkv][d]
        vals = np.concatenate([vc[off[b]:off[b + 1]], vt[b]], 0)
        allow = np.zeros((nq, L + nq), bool)
        allow[:, :L] = True
        for i, s in enumerate(anc_sets(par[b], n)):
            for j in s:
                allow[i, L + j] = True
        Q = torch.from_numpy(q[b, :n + 1]).permute(1, 0, 2)            # [hq][rows][d]
        K = torch.from_numpy(keys).permute(1, 0, 2).repeat_interleave(rep, 0)
        V = torch.from_numpy(vals).permute(1, 0, 2).repeat_interleave(rep, 0)
        M = torch.from_numpy(allow[:n + 1])
        o = F.scaled_dot_product_attention(Q, K, V, attn_mask=M, scale=scale)
        out[b, :n + 1] = o.permute(1, 0, 2).numpy()
    return out


def small_cfg(dtype, law="normal", hq=4, hkv=2, d=16, n_max=9, batch=3):
    return wl.CONFIGS["tiny"].replace(name="t", index=77, batch=batch, hq=hq, hkv=hkv, head_dim=d,
                                      n_max=n_max, attn_dtype=dtype, ctx_law="uniform",
                                      ctx_p0=1, ctx_p1=40, attn_law=law)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 4), (8, 1)])
def test_attention_matches_torch_sdpa(dtype, hq, hkv):
    cfg = small_cfg(dtype, hq=hq, hkv=hkv)
    inp = wl.make_attn_inputs(cfg)
    rng = np.random.default_rng(hq * 10 + hkv)
    n_nodes = np.array([cfg.n_max, 3, 0], np.int32)
    par = np.stack([random_tree(rng, int(n), cfg.nq_max) for n in n_nodes])
    mask = oracle.tree_mask(par, n_nodes)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    got = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"], inp["k_tree"],
                           inp["v_tree"], mask, n_nodes, hq, hkv, cfg.head_dim, scale)
    want = _sdpa_reference(inp, par, n_nodes, hq, hkv, cfg.head_dim, scale, dtype)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    for b, n in enumerate(n_nodes):                  # padding rows are zero
        assert np.all(got[b, n + 1:] == 0)


def _plain_rows(inp, b, rows_keys, hq, hkv, d, scale, dtype):
    """Attention for given explicit key lists (row -> list of (kind, idx))."""
    q = wl.logits_as_f64(inp["q"], dtype)
    kc, vc = wl.logits_as_f64(inp["k_ctx"], dtype), wl.logits_as_f64(inp["v_ctx"], dtype)
    kt, vt = wl.logits_as_f64(inp["k_tree"], dtype), wl.logits_as_f64(inp["v_tree"], dtype)
    off = inp["ctx_offsets"]
    out = {}
    for i, keys in rows_keys.items():
        for h in range(hq):
            g = h // (hq // hkv)
            K = np.stack([kc[off[b] + j, g] if kind == "c" else kt[b, j, g] for kind, j in keys])
            V = np.stack([vc[off[b] + j, g] if kind == "c" else vt[b, j, g] for kind, j in keys])
            s = K @ q[b, i, h] * scale
            p = np.exp(s - s.max())
            out[(i, h)] = (p / p.sum()) @ V
    return out


@pytest.mark.parametrize("shape", ["chain", "star", "root"])
def test_attention_special_trees(shape):
    cfg = small_cfg("f32", batch=1, n_max=6)
    inp = wl.make_attn_inputs(cfg)
    L = int(inp["ctx_len"][0])
    n = {"chain": 6, "star": 6, "root": 0}[shape]
    par = np.full(cfg.nq_max, -1, np.int32)
    for i in range(1, n + 1):
        par[i] = i - 1 if shape == "chain" else 0
    mask = oracle.tree_mask(par[None], np.array([n], np.int32))
    scale = 1.0 / math.sqrt(cfg.head_dim)
    got = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"], inp["k_tree"],
                           inp["v_tree"], mask, np.array([n], np.int32), cfg.hq, cfg.hkv,
                           cfg.head_dim, scale)
    ctx = [("c", j) for j in range(L)]
    if shape == "chain":      # causal over context + chain
        rows = {i: ctx + [("t", j) for j in range(i + 1)] for i in range(n + 1)}
    elif shape == "star":     # context + root + itself
        rows = {i: ctx + [("t", 0)] + ([("t", i)] if i else []) for i in range(n + 1)}
    else:                     # decode attention over context + the root
        rows = {0: ctx + [("t", 0)]}
    want = _plain_rows(inp, 0, rows, cfg.hq, cfg.hkv, cfg.head_dim, scale, "f32")
    for (i, h), o in want.items():
        np.testing.assert_allclose(got[0, i, h], o, rtol=0, atol=1e-12)


def test_one_wrong_mask_bit_is_visible():
    cfg = small_cfg("bf16", law="mask_sensitive", batch=1, n_max=12, d=64)
    inp = wl.make_attn_inputs(cfg)
    par = np.array([-1, 0, 1, 2, 0, 4, 1, 6, 7, 8, 3, 10, 11], np.int32)
    n_nodes = np.array([12], np.int32)
    mask = oracle.tree_mask(par[None], n_nodes)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    args = (inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"], inp["k_tree"], inp["v_tree"])
    base = oracle.tree_attn(*args, mask, n_nodes, cfg.hq, cfg.hkv, cfg.head_dim, scale)
    bad = mask.copy()
    bad[0, 9, 0] ^= np.uint64(1 << 5)            # row 9 wrongly admits node 5
    flipped = oracle.tree_attn(*args, bad, n_nodes, cfg.hq, cfg.hkv, cfg.head_dim, scale)
    diff = np.abs(flipped - base).max(axis=-1)
    assert diff[0, 9].min() > 0.1                 # far beyond the bf16 tolerance 2e-2
    assert np.all(diff[0, :9] == 0) and np.all(diff[0, 10:] == 0)


def test_thread_count_does_not_change_results():
    """The oracle's outputs are the same, bit for bit, on one thread and on
    several (each output is computed by one thread in a fixed order)."""
    import oracle as orc
    from tree_draft_build_amd import workload as wl
    cfg = wl.CONFIGS["tiny_fixed"].replace(batch=3, n_max=12)
    x = wl.make_logits(cfg)
    inp = wl.make_attn_inputs(cfg)
    res = []
    before = orc.set_threads(0)
    try:
        for n in (1, 4):
            orc.set_threads(n)
            ids, lq, lse = orc.draft_topk(x, cfg.topk)
            tr = orc.build_tree(ids, lq, cfg.n_max, False)
            m = orc.tree_mask(tr["node_parent"], tr["n_nodes"])
            o = orc.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                              inp["k_tree"], inp["v_tree"], m, tr["n_nodes"], cfg.hq, cfg.hkv,
                              cfg.head_dim, wl.attn_scale(cfg))
            res.append((ids, lq, lse, tr["node_token"], tr["node_logrho"], o))
    finally:
        orc.set_threads(before)
    for a, b in zip(*res):
        assert np.array_equal(a, b)
