"""Pins of selective verification and the batch-size switch in the oracle's
tree construction (FlexDraft page, "Methodik" §3, Flex-Decoding).

Readings: a candidate's cumulative draft confidence is its path score rho
(the product of the drafter's marginals along its path, the same quantity
BASTION's surrogate sums); selective verification prunes branches whose
confidence falls below a threshold tau; in the sequential mode of large
batches only one branch is drafted (each position's top-1 token).
Pins (the candidate universe is written out independently of the oracle):
  * threshold: the tree is the first min(N, #{rho >= tau}) candidates of the
    global sort of all candidates (ties exactly at tau are kept);
  * branch cap b: the tree is the global sort restricted to ranks < b;
    b = 1 gives the top-1 chain with closed-form scores;
  * with the S(N) stop as well, the tree stops at the first of the three
    limits;
  * the batch switch's closed form.
"""
import math

import numpy as np
import pytest

import oracle
from test_oracle_tree import _global_order, oracle_paths, tiny_tables, universe


def global_order(nodes):
    """(rank path, node) pairs in the global order of all candidates."""
    return [(p, nodes[p]) for p in _global_order(nodes)]


def tables(seed, V=4, B=4):
    x = tiny_tables(seed, V, B)
    ids, lq, _ = oracle.draft_topk(x, V)
    return ids, lq


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("n_max", [5, 40])
def test_threshold_is_a_prefix_of_the_global_order(seed, n_max):
    ids, lq = tables(seed)
    K, B = 3, 4
    order = global_order(universe(ids[0], lq[0], B, K))
    scores = [v["lr"] for _, v in order]
    for tau in (scores[0] + 0.5, scores[2], (scores[6] + scores[7]) / 2, scores[-1] - 1.0):
        assert tau < 0
        tree = oracle.build_tree(ids[:, :, :K], lq[:, :, :K], n_max, False, min_logrho=tau)
        want_n = min(n_max, sum(1 for x in scores if x >= tau))
        assert int(tree["n_nodes"][0]) == want_n
        want_paths = [v["toks"] for _, v in order[:want_n]]
        assert oracle_paths(tree) == want_paths
        assert all(tree["node_logrho"][0, 1:want_n + 1] >= tau)


@pytest.mark.parametrize("branch", [1, 2])
def test_branch_cap_is_the_order_over_low_ranks(branch):
    ids, lq = tables(7)
    K, B = 4, 4
    sub = universe(ids[0], lq[0], B, branch)           # ranks < branch only
    order = global_order(sub)
    n = min(len(order), 9)
    tree = oracle.build_tree(ids, lq, n, False, branch=branch)
    assert oracle_paths(tree) == [v["toks"] for _, v in order[:n]]
    if branch == 1:
        # the top-1 chain: depth d holds position d's best token
        assert int(tree["n_nodes"][0]) == B
        lr = np.cumsum([lq[0, d, 0] for d in range(B)])
        np.testing.assert_allclose(tree["node_logrho"][0, 1:B + 1], lr, rtol=0, atol=1e-15)
        assert list(tree["node_token"][0, 1:B + 1]) == [int(ids[0, d, 0]) for d in range(B)]


def test_threshold_with_the_budget_stop():
    """Three limits: budget, S(N) stop, threshold; the tree ends at the first."""
    ids, lq = tables(3, V=6, B=5)
    cost = (1.0, 0.05, 0.2, 3)
    full = oracle.build_tree(ids, lq, 30, False, cost=cost, want_curve=True)
    stop = oracle.build_tree(ids, lq, 30, True, cost=cost)
    n_stop = int(stop["n_nodes"][0])
    lr = full["node_logrho"][0, 1:31]
    for cut in range(0, 12):
        tau = lr[cut] if cut < len(lr) else -math.inf
        t = oracle.build_tree(ids, lq, 30, True, cost=cost, min_logrho=tau)
        n_tau = int(np.sum(lr >= tau))
        assert int(t["n_nodes"][0]) == min(n_stop, n_tau)
        assert oracle_paths(t) == oracle_paths(full)[:min(n_stop, n_tau)]


def test_nonnegative_threshold_is_off():
    ids, lq = tables(5)
    a = oracle.build_tree(ids, lq, 12, False)
    for tau in (0.0, 3.0):
        b = oracle.build_tree(ids, lq, 12, False, min_logrho=tau)
        for k in ("n_nodes", "node_token", "node_parent"):
            np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("batch,switch,want", [(1, 8, (8, 64)), (7, 8, (8, 64)), (8, 8, (1, 16)),
                                               (64, 8, (1, 16)), (64, 0, (8, 64))])
def test_batch_switch_closed_form(batch, switch, want):
    assert oracle.flex_budget(batch, switch, 8, 64, 16) == want
    assert oracle.flex_budget(batch, switch, 8, 4, 16)[1] == (4 if want[0] == 1 else 4)
