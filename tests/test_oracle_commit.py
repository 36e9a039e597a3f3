"""Pins of the oracle's KV commit (the step after acceptance) and of its
context-length form of tree attention.

After the target has verified the tree in one pass, decoding continues from
the accepted prefix (BASTION page, "Problemstellung"); the keys and values the
verification computed for that prefix are kept as context (the FlexDraft page,
"Methodik" §3, decoupled execution: the verification's KV cache is reused).
Pins:
  * the committed rows are, in order, the root and the nodes whose token
    paths are the prefixes of the target's greedy chain g_1, g_2, ... (the
    chain computed here from the synthetic target directly, not from the
    oracle's acceptance walk); the bonus g_{A+1} is the next root;
  * lengths grow by A + 1; rows outside the appended range are untouched;
    a full region takes no row beyond its end;
  * decode invariance: the tree pass's attention row of the deepest accepted
    node equals plain decode attention of that node's query over the
    committed context (its key set is the same);
  * attention over the first ctx_lengths[b] rows of each region equals
    attention over a compacted copy of those rows.
"""
import numpy as np
import pytest

import oracle
from tree_draft_build_amd import workload as wl

CFG = wl.CONFIGS["tiny_fixed"].replace(name="commit", index=60, batch=3, spike_lo=14.0,
                                       spike_hi=20.0)


def paths_of(tok, par, n):
    paths = [()]
    for j in range(1, n + 1):
        paths.append(paths[int(par[j])] + (int(tok[j]),))
    return paths


def setup(cfg=CFG, room=None):
    x = wl.make_logits(cfg)
    ids, lq, _ = oracle.draft_topk(x, cfg.topk)
    tr = oracle.build_tree(ids, lq, cfg.n_max, False)
    lf = wl.logits_as_f64(x, cfg.logit_dtype)
    tg = wl.target_tokens(cfg, lf, tr["node_token"], tr["node_parent"], tr["n_nodes"])
    alen, path, bonus = oracle.accept(tr["node_token"], tr["node_parent"], tr["n_nodes"], tg,
                                      cfg.block)
    inp = wl.make_attn_inputs(cfg)
    b, nq, hkv, d = cfg.batch, cfg.nq_max, cfg.hkv, cfg.head_dim
    # tag every tree row: element 0 of every KV head carries 1000 b + node
    kt = inp["k_tree"].copy()
    kt[:, :, :, 0] = (1000 * np.arange(b)[:, None, None] + np.arange(nq)[None, :, None])
    L = inp["ctx_len"].astype(np.int64)
    room = cfg.block + 3 if room is None else room
    region = L + room
    off = np.zeros(b + 1, np.int64)
    off[1:] = np.cumsum(region)
    # rows past the last region: spare room that no correct commit writes
    pad = cfg.block + 2
    kc = np.full((off[-1] + pad, hkv, d), 7.0, np.float32)
    vc = np.full((off[-1] + pad, hkv, d), -7.0, np.float32)
    for s in range(b):
        o0 = inp["ctx_offsets"][s]
        kc[off[s]:off[s] + L[s]] = inp["k_ctx"][o0:o0 + L[s]]
        vc[off[s]:off[s] + L[s]] = inp["v_ctx"][o0:o0 + L[s]]
    return dict(x=x, lf=lf, tr=tr, tg=tg, alen=alen, path=path, bonus=bonus, inp=inp, kt=kt,
                L=L, off=off, kc=kc, vc=vc)


def test_commit_follows_greedy_chain():
    s = setup()
    tr, inp = s["tr"], s["inp"]
    kc, vc, lens = s["kc"].copy(), s["vc"].copy(), s["L"].copy()
    nxt = oracle.kv_commit(s["kt"], inp["v_tree"], s["alen"], s["path"], s["bonus"], kc, vc,
                           s["off"], lens, CFG.hkv, CFG.head_dim)
    tm = wl.TargetModel(CFG, s["lf"])
    deep = 0
    for b in range(CFG.batch):
        n = int(tr["n_nodes"][b])
        paths = paths_of(tr["node_token"][b], tr["node_parent"][b], n)
        where = {p: i for i, p in enumerate(paths)}
        chain = ()
        nodes = [0]
        while True:                                   # the target's greedy chain in the tree
            g = tm.token(b, chain)
            if chain + (g,) not in where:
                break
            chain = chain + (g,)
            nodes.append(where[chain])
        A = len(nodes) - 1
        deep = max(deep, A)
        assert lens[b] == s["L"][b] + A + 1
        assert nxt[b] == tm.token(b, chain)           # the bonus: g_{A+1}
        base = s["off"][b] + s["L"][b]
        got = kc[base:base + A + 1, :, 0].astype(np.int64)
        assert np.all(got == (1000 * b + np.array(nodes))[:, None])
        np.testing.assert_array_equal(kc[base:base + A + 1], s["kt"][b, nodes])
        np.testing.assert_array_equal(vc[base:base + A + 1], inp["v_tree"][b, nodes])
        # untouched: the old context and the room past the appended rows
        np.testing.assert_array_equal(kc[s["off"][b]:base], s["kc"][s["off"][b]:base])
        assert np.all(kc[base + A + 1:s["off"][b + 1]] == 7.0)
        assert np.all(vc[base + A + 1:s["off"][b + 1]] == -7.0)
    assert deep >= 2                                  # the case reaches deep acceptances


def test_committed_prefix_reproduces_tree_attention():
    """The deepest accepted node u sees context + its root path in the tree
    pass; after the commit, its query over the committed context (with u's
    own row as the only tree row) sees the same keys."""
    s = setup()
    tr, inp = s["tr"], s["inp"]
    cfg = CFG
    mask = oracle.tree_mask(tr["node_parent"], tr["n_nodes"])
    tree_out = oracle.tree_attn(inp["q"], s["kc"], s["vc"], s["off"], s["kt"], inp["v_tree"], mask,
                                tr["n_nodes"], cfg.hq, cfg.hkv, cfg.head_dim, wl.attn_scale(cfg),
                                ctx_lengths=s["L"])
    kc, vc, lens = s["kc"].copy(), s["vc"].copy(), s["L"].copy()
    oracle.kv_commit(s["kt"], inp["v_tree"], s["alen"], s["path"], s["bonus"], kc, vc, s["off"],
                     lens, cfg.hkv, cfg.head_dim)
    nq = cfg.nq_max
    for b in range(cfg.batch):
        A = int(s["alen"][b])
        u = int(s["path"][b, A])
        q1 = np.zeros_like(inp["q"])
        q1[b, 0] = inp["q"][b, u]
        k1 = np.zeros_like(s["kt"])
        v1 = np.zeros_like(inp["v_tree"])
        k1[b, 0] = s["kt"][b, u]
        v1[b, 0] = inp["v_tree"][b, u]
        lens1 = lens.copy()
        lens1[b] -= 1                                 # u's own row is the tree root here
        n0 = np.zeros(cfg.batch, np.int32)
        m0 = oracle.tree_mask(np.full((cfg.batch, nq), -1, np.int32), n0)
        dec = oracle.tree_attn(q1, kc, vc, s["off"], k1, v1, m0, n0, cfg.hq, cfg.hkv, cfg.head_dim,
                               wl.attn_scale(cfg), seqs=(b, b + 1), ctx_lengths=lens1)
        np.testing.assert_allclose(dec[0, 0], tree_out[b, u], rtol=0, atol=1e-12)


def test_commit_stops_at_the_region_end():
    s = setup(room=2)
    inp = s["inp"]
    kc, vc, lens = s["kc"].copy(), s["vc"].copy(), s["L"].copy()
    oracle.kv_commit(s["kt"], inp["v_tree"], s["alen"], s["path"], s["bonus"], kc, vc, s["off"],
                     lens, CFG.hkv, CFG.head_dim)
    for b in range(CFG.batch):
        A = int(s["alen"][b])
        assert lens[b] == s["L"][b] + min(A + 1, 2)
        assert lens[b] <= s["off"][b + 1] - s["off"][b]
    assert (s["alen"] + 1 > 2).any()                  # some sequence overflowed its room
    assert np.all(kc[s["off"][-1]:] == 7.0) and np.all(vc[s["off"][-1]:] == -7.0)


def test_attention_over_context_lengths_equals_compacted():
    s = setup()
    tr, inp, cfg = s["tr"], s["inp"], CFG
    rng = np.random.default_rng(3)
    lens = np.array([rng.integers(0, int(l) + 1) for l in s["L"]], np.int64)
    lens[0] = 0                                       # an empty context
    mask = oracle.tree_mask(tr["node_parent"], tr["n_nodes"])
    got = oracle.tree_attn(inp["q"], s["kc"], s["vc"], s["off"], s["kt"], inp["v_tree"], mask,
                           tr["n_nodes"], cfg.hq, cfg.hkv, cfg.head_dim, wl.attn_scale(cfg),
                           ctx_lengths=lens)
    off2 = np.zeros(cfg.batch + 1, np.int64)
    off2[1:] = np.cumsum(lens)
    kc2 = np.concatenate([s["kc"][s["off"][b]:s["off"][b] + lens[b]] for b in range(cfg.batch)])
    vc2 = np.concatenate([s["vc"][s["off"][b]:s["off"][b] + lens[b]] for b in range(cfg.batch)])
    want = oracle.tree_attn(inp["q"], kc2, vc2, off2, s["kt"], inp["v_tree"], mask, tr["n_nodes"],
                            cfg.hq, cfg.hkv, cfg.head_dim, wl.attn_scale(cfg))
    np.testing.assert_array_equal(got, want)
