"""Pins of the oracle's stage (b): best-first construction of the prefix-closed
tree and the S(N) stop (BASTION "Methodik" §2 and §3).

Pins, none of which reuses the oracle's code:
  * brute force: every prefix-closed tree of size n over tiny vocabularies;
    its best A_hat equals best-first's for every n (the pages' optimality claim);
  * closed form: the best-first order is the global sort of all candidate
    nodes under (log rho desc, depth asc, token asc, parent rank asc);
  * invariants: rho non-increasing along paths, A_hat concave in n, prefix
    closure, depth <= B, sibling tokens distinct and inside the top-K;
  * the stop: N* is the smallest argmax of S over the fixed-budget order, and
    S is unimodal for convex C;
  * special cases: K = 1 gives the top-1 chain; K = V gives A_hat = ahat0 + B
    for the full tree; the pages' worked cat/dog example.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from tree_draft_build_amd import workload as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# candidate universe written out independently of the oracle
# ---------------------------------------------------------------------------

def universe(ids, lq, B, K):
    """All candidate nodes as dicts keyed by rank path (j_1..j_d)."""
    nodes = {}
    for d in range(1, B + 1):
        for ranks in itertools.product(range(K), repeat=d):
            parent = ranks[:-1]
            plr = 0.0 if d == 1 else nodes[parent]["lr"]
            lr = plr + lq[d - 1][ranks[-1]]
            toks = tuple(int(ids[t][ranks[t]]) for t in range(d))
            nodes[ranks] = dict(lr=lr, depth=d, token=toks[-1], toks=toks, parent=parent)
    return nodes


def enum_trees(nodes, K, B, n):
    """Every prefix-closed tree (set of rank paths, root implicit) with n nodes.
    Extension-list enumeration: each rooted subtree is produced exactly once."""
    def children(p):
        return [p + (j,) for j in range(K)] if len(p) < B else []

    def rec(chosen, ext, left):
        if left == 0:
            yield chosen
            return
        for i, node in enumerate(ext):
            yield from rec(chosen + [node], ext[i + 1:] + children(node), left - 1)

    yield from rec([], children(()), n)


def oracle_paths(tree, b=0):
    """Token paths of the oracle's inserted nodes, in insertion order."""
    n = int(tree["n_nodes"][b])
    paths = [()]
    for j in range(1, n + 1):
        paths.append(paths[int(tree["node_parent"][b, j])] + (int(tree["node_token"][b, j]),))
    return paths[1:]


def tiny_tables(seed, V, B, coarse=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, B, V)) * 1.5
    if coarse:
        x = np.round(x * 2) / 2       # exact ties inside and across positions
    return x.astype(np.float32)


def degenerate_tables(V, B):
    """Exactly tied and one-hot positions: -1000 underflows to exactly zero
    mass, so q is exactly 1/2 (two tied tokens) or exactly 1 (one-hot).  Then
    nodes at different depths carry identical log rho and the depth key of
    the tie-break decides."""
    x = np.full((1, B, V), -1000.0, np.float32)
    for k in range(B):
        if k % 2 == 0:
            x[0, k, 0] = x[0, k, 1] = 0.0      # q = 1/2, 1/2
        else:
            x[0, k, (k // 2) % V] = 0.0        # q = 1
    return x


# ---------------------------------------------------------------------------

@pytest.mark.parametrize("V,K,B,nmax", [(2, 2, 3, 7), (3, 3, 2, 7), (3, 3, 3, 6), (4, 2, 3, 7),
                                         (4, 3, 2, 7), (2, 2, 4, 7)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_best_first_is_optimal_bruteforce(V, K, B, nmax, seed):
    x = tiny_tables(seed * 31 + V * 7 + B, V, B)
    ids, lq, _ = oracle.draft_topk(x, K)
    nodes = universe(ids[0], lq[0], B, K)
    n_all = len(nodes)
    tree = oracle.build_tree(ids, lq, n_all, use_stop=False, ahat0=0.0)
    lr_order = tree["node_logrho"][0, 1:]
    for n in range(1, min(nmax, n_all) + 1):
        best_val, second, best_sets = -1.0, -1.0, []
        for t in enum_trees(nodes, K, B, n):
            a = sum(math.exp(nodes[p]["lr"]) for p in t)
            if a > best_val + 1e-12:
                second, best_val, best_sets = best_val, a, [t]
            elif a > best_val - 1e-12:
                best_sets.append(t)
            elif a > second:
                second = a
        bf = float(np.sum(np.exp(lr_order[:n])))
        assert bf == pytest.approx(best_val, abs=1e-12), (n, bf, best_val)
        if len(best_sets) == 1:
            want = sorted(nodes[p]["toks"] for p in best_sets[0])
            got = sorted(oracle_paths(tree)[:n])
            assert got == want


def _global_order(nodes):
    keys = {}

    def key(p):
        if p == ():
            return ()
        if p not in keys:
            nd = nodes[p]
            keys[p] = (-nd["lr"], nd["depth"], nd["token"], key(nd["parent"]))
        return keys[p]

    return sorted(nodes, key=key)


@pytest.mark.parametrize("V,K,B", [(3, 3, 4), (5, 3, 3), (4, 4, 3), (6, 2, 5)])
@pytest.mark.parametrize("coarse", [False, True, "degenerate"])
def test_best_first_order_is_global_sort(V, K, B, coarse):
    if coarse == "degenerate":
        x = degenerate_tables(V, B)
    else:
        x = tiny_tables(V * 100 + K * 10 + B, V, B, coarse=coarse)
    ids, lq, _ = oracle.draft_topk(x, K)
    nodes = universe(ids[0], lq[0], B, K)
    tree = oracle.build_tree(ids, lq, len(nodes), use_stop=False)
    want = [nodes[p]["toks"] for p in _global_order(nodes)]
    assert oracle_paths(tree) == want
    if coarse:  # the tie keys were exercised
        lrs = [nodes[p]["lr"] for p in nodes]
        assert len(set(lrs)) < len(lrs)
    if coarse == "degenerate":  # equal log rho at different depths occurs
        by_lr = {}
        for p in nodes:
            by_lr.setdefault(nodes[p]["lr"], set()).add(nodes[p]["depth"])
        assert any(len(dset) > 1 for dset in by_lr.values())


def check_invariants(tree, ids, lq, B, K, ahat0=1.0):
    for b in range(tree["n_nodes"].shape[0]):
        n = int(tree["n_nodes"][b])
        par, tok = tree["node_parent"][b], tree["node_token"][b]
        dep, lr = tree["node_depth"][b], tree["node_logrho"][b]
        assert dep[0] == 0 and lr[0] == 0.0 and par[0] == -1
        for i in range(1, n + 1):
            p = par[i]
            assert 0 <= p < i                          # prefix closed, parent first
            assert dep[i] == dep[p] + 1 <= B
            assert lr[i] <= lr[p]                      # rho non-increasing on paths
            assert tok[i] in ids[b, dep[i] - 1]        # token from q_{d}'s top-K
            j = list(ids[b, dep[i] - 1]).index(tok[i])
            assert lr[i] == pytest.approx(lr[p] + lq[b, dep[i] - 1, j], abs=1e-12)
        assert np.all(np.diff(lr[1:n + 1]) <= 0)       # popped scores non-increasing
        # A_hat increments are the popped rho: non-increasing, so A_hat is concave
        inc = np.exp(lr[1:n + 1])
        assert np.all(np.diff(inc) <= 1e-300)
        assert tree["ahat"][b] == pytest.approx(ahat0 + inc.sum(), rel=1e-12)
        for i in range(0, n + 1):                      # siblings carry distinct tokens
            kids = [tok[c] for c in range(1, n + 1) if par[c] == i]
            assert len(kids) == len(set(kids)) <= K
        assert np.all(tok[n + 1:] == -1) and np.all(par[n + 1:] == -1)


@pytest.mark.parametrize("name", ["tiny_fixed", "tiny", "qwen3_8b", "qwen3_8b_stress"])
def test_invariants_on_configs(name):
    cfg = wl.CONFIGS[name]
    x = wl.make_logits(cfg)
    ids, lq, _ = oracle.draft_topk(x, cfg.topk)
    tree = oracle.build_tree(ids, lq, cfg.n_max, cfg.use_stop,
                             (cfg.cost_a, cfg.cost_b, cfg.cost_c, cfg.cost_knee), cfg.l_ar,
                             cfg.ahat0)
    check_invariants(tree, ids, lq, cfg.block, cfg.topk, cfg.ahat0)
    if not cfg.use_stop:
        assert np.all(tree["n_nodes"] == cfg.n_max)


def _cost(n, c):
    return c[0] + c[1] * n + c[2] * max(0, n - c[3])


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b", "qwen3_8b_stress", "llama31_8b"])
def test_stop_is_smallest_argmax_of_S(name):
    cfg = wl.CONFIGS[name]
    seqs = [0, 1] if cfg.batch > 1 else [0]
    x = wl.make_logits(cfg, seqs)
    ids, lq, _ = oracle.draft_topk(x, cfg.topk)
    cost = (cfg.cost_a, cfg.cost_b, cfg.cost_c, cfg.cost_knee)
    full = oracle.build_tree(ids, lq, cfg.n_max, False, cost, cfg.l_ar, cfg.ahat0, want_curve=True)
    stop = oracle.build_tree(ids, lq, cfg.n_max, True, cost, cfg.l_ar, cfg.ahat0, want_curve=True)
    for b in range(len(seqs)):
        # S written out from the popped scores, independently of the oracle's loop
        lr = full["node_logrho"][b]
        S = [(cfg.ahat0 + np.exp(lr[1:n + 1]).sum()) * cfg.l_ar / _cost(n, cost)
             for n in range(cfg.n_max + 1)]
        np.testing.assert_allclose(full["s_curve"][b], S, rtol=1e-12)
        nstar = int(np.argmax(np.asarray(S)))           # first maximiser
        assert int(stop["n_nodes"][b]) == nstar
        # unimodal: once S falls it keeps falling
        d = np.diff(S)
        if np.any(d <= 0):
            first = int(np.argmax(d <= 0))
            assert np.all(d[first:] <= 0)
        # the stopped tree is the prefix of the fixed-budget order
        for key in ("node_token", "node_parent", "node_depth"):
            np.testing.assert_array_equal(stop[key][b, :nstar + 1], full[key][b, :nstar + 1])
        assert stop["speedup"][b] == pytest.approx(S[nstar], rel=1e-12)


def test_k1_is_top1_chain():
    cfg = wl.CONFIGS["tiny"]
    x = wl.make_logits(cfg)
    ids, lq, lse = oracle.draft_topk(x, 1)
    xf = wl.logits_as_f64(x, "f32")[0]
    tree = oracle.build_tree(ids, lq, cfg.block + 3, use_stop=False)
    n = int(tree["n_nodes"][0])
    assert n == cfg.block                               # runs out of candidates at depth B
    for d in range(1, n + 1):
        assert tree["node_parent"][0, d] == d - 1 and tree["node_depth"][0, d] == d
        assert tree["node_token"][0, d] == int(np.argmax(xf[d - 1]))
        # rho_d = prod_k max_v q_k(v)
        want = sum(xf[k].max() - math.log(np.exp(xf[k] - xf[k].max()).sum()) - xf[k].max()
                   for k in range(d))
        assert tree["node_logrho"][0, d] == pytest.approx(want, abs=1e-10)


@pytest.mark.parametrize("V,B", [(3, 3), (4, 2), (2, 5)])
def test_full_tree_ahat_closed_form(V, B):
    # K = V: each depth level's rho sum to 1, so the whole tree has A_hat = ahat0 + B
    x = tiny_tables(V + 10 * B, V, B)
    ids, lq, _ = oracle.draft_topk(x, V)
    total = sum(V ** d for d in range(1, B + 1))
    tree = oracle.build_tree(ids, lq, total, use_stop=False, ahat0=1.0)
    assert int(tree["n_nodes"][0]) == total
    assert tree["ahat"][0] == pytest.approx(1.0 + B, abs=1e-12)


def test_worked_example_cat_dog():
    g = json.load(open(os.path.join(GOLDEN, "toy_cat_dog.json")))
    p_cat, p_dog = g["position_1"]["cat"], g["position_1"]["dog"]
    V, B, K = 8, 2, 2
    CAT, DOG = 0, 1
    # position 1: the pages' 80/20 split; the other six words carry ~e^-60
    x = np.full((1, B, V), -60.0, np.float32)
    x[0, 0, CAT], x[0, 0, DOG] = math.log(p_cat), math.log(p_dog)
    # position 2: a flat next word (1/8 each), our choice, so that both
    # depth-1 words are taken before any depth-2 word
    x[0, 1, :] = 0.0
    ids, lq, _ = oracle.draft_topk(x, K)
    assert list(ids[0, 0]) == [CAT, DOG]
    cost = (1.0, 0.02, 0.0, 0)
    tree = oracle.build_tree(ids, lq, 6, use_stop=False, cost=cost, want_curve=True)
    paths = oracle_paths(tree)
    rho = np.exp(tree["node_logrho"][0, 1:7])
    assert paths[:2] == [(CAT,), (DOG,)]                # both branches first
    # logits are float32: ln 0.8 is stored to a relative 6e-8, hence rtol 1e-7
    np.testing.assert_allclose(rho, [0.8, 0.2, 0.1, 0.1, 0.025, 0.025], rtol=1e-7, atol=0)
    assert {p[0] for p in paths if len(p) == 2} == {CAT, DOG}   # both branch again
    np.testing.assert_allclose(np.cumsum(rho) + 1.0, [1.8, 2.0, 2.1, 2.2, 2.225, 2.25], rtol=1e-7,
                               atol=0)
    # S(N) = A_hat / (1 + 0.02 N) rises to N = 4 and then falls
    stop = oracle.build_tree(ids, lq, 6, use_stop=True, cost=cost)
    assert int(stop["n_nodes"][0]) == 4
    assert stop["speedup"][0] == pytest.approx(2.2 / 1.08, rel=1e-7)


def test_root_token_and_empty_budget():
    cfg = wl.CONFIGS["tiny"]
    x = wl.make_logits(cfg)
    ids, lq, _ = oracle.draft_topk(x, cfg.topk)
    tree = oracle.build_tree(ids, lq, 0, use_stop=False, root_token=np.array([777]))
    assert int(tree["n_nodes"][0]) == 0 and tree["node_token"][0, 0] == 777
    assert tree["ahat"][0] == 1.0
