"""Pins of the oracle's one-layer verification stand-in: the projection of
the tree tokens with rotary positions (position = context length + depth)
and the LM-head argmax that gives the target's greedy token at every node.

Pins (none retypes the oracle's formulas):
  * at position 0 the rotation is the identity, so q, k, v equal a library
    matrix product of the embedding rows with the projection;
  * rotation as complex multiplication: head pairs (x_j, x_{j+d/2}) read as
    complex numbers are multiplied by exp(i pos base^(-2j/d)) (numpy complex
    exponential), checked against the unrotated product;
  * the relative-position property: shifting every position by s leaves all
    query-key dot products unchanged, and rotation keeps every norm;
  * rows beyond the tree are zero; a node without a token reads row 0;
  * argmax: numpy's argmax of a float64 matrix product; planted duplicate
    vocabulary rows go to the smaller id; best and runner-up logits.
"""
import numpy as np
import pytest

import oracle
from tree_draft_build_amd import workload as wl

SHAPE = wl.LayerShape(vocab=97, hq=4, hkv=2, head_dim=32, rope_base=1e4)
CFG = wl.CONFIGS["tiny_fixed"].replace(name="layer", index=90, batch=2, n_max=9, vocab=97,
                                       hq=4, hkv=2, head_dim=32)


def f64(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def tree_rows(seed=0):
    rng = np.random.default_rng(seed)
    nq = CFG.nq_max
    tok = rng.integers(0, SHAPE.vocab, size=(CFG.batch, nq)).astype(np.int32)
    depth = np.minimum(np.arange(nq), 4)[None, :].repeat(CFG.batch, 0).astype(np.int32)
    n_nodes = np.array([nq - 1, 4], np.int32)
    return tok, depth, n_nodes


def run_qkv(w, tok, depth, n_nodes, lens):
    off = np.zeros(CFG.batch + 1, np.int64)
    off[1:] = np.cumsum(np.maximum(lens, 1) + 40)
    return oracle.tree_qkv(w["embed"], w["w_qkv"], tok, depth, n_nodes, off, SHAPE.hq, SHAPE.hkv,
                           SHAPE.head_dim, SHAPE.rope_base, ctx_lengths=np.asarray(lens, np.int64))


def plain_projection(w, tok):
    y = f64(w["embed"])[tok] @ f64(w["w_qkv"]).T          # [b][nq][out]
    H, D = SHAPE.hq, SHAPE.head_dim
    return (y[..., :H * D].reshape(*tok.shape, H, D),
            y[..., H * D:(H + SHAPE.hkv) * D].reshape(*tok.shape, SHAPE.hkv, D),
            y[..., (H + SHAPE.hkv) * D:].reshape(*tok.shape, SHAPE.hkv, D))


def test_position_zero_is_the_plain_projection():
    w = wl.layer_weights(CFG, SHAPE)
    tok, depth, n_nodes = tree_rows()
    depth[:] = 0
    q, k, v = run_qkv(w, tok, depth, n_nodes, [0, 0])
    pq, pk, pv = plain_projection(w, tok)
    for b in range(CFG.batch):
        r = int(n_nodes[b]) + 1
        np.testing.assert_allclose(q[b, :r], pq[b, :r], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(k[b, :r], pk[b, :r], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(v[b, :r], pv[b, :r], rtol=1e-12, atol=1e-12)
        assert not q[b, r:].any() and not k[b, r:].any() and not v[b, r:].any()


def test_rotation_is_complex_multiplication():
    w = wl.layer_weights(CFG, SHAPE)
    tok, depth, n_nodes = tree_rows(1)
    lens = [37, 1200]
    q, k, v = run_qkv(w, tok, depth, n_nodes, lens)
    pq, pk, pv = plain_projection(w, tok)
    D = SHAPE.head_dim
    inv = SHAPE.rope_base ** (-2.0 * np.arange(D // 2) / D)
    for b in range(CFG.batch):
        for i in range(int(n_nodes[b]) + 1):
            pos = lens[b] + int(depth[b, i])
            rot = np.exp(1j * pos * inv)
            for got, plain in ((q[b, i], pq[b, i]), (k[b, i], pk[b, i])):
                z = (plain[:, :D // 2] + 1j * plain[:, D // 2:]) * rot
                np.testing.assert_allclose(got[:, :D // 2], z.real, rtol=1e-10, atol=1e-10)
                np.testing.assert_allclose(got[:, D // 2:], z.imag, rtol=1e-10, atol=1e-10)
            np.testing.assert_array_equal(v[b, i], pv[b, i])     # values are not rotated


def test_relative_positions_and_norms():
    w = wl.layer_weights(CFG, SHAPE)
    tok, depth, n_nodes = tree_rows(2)
    qa, ka, _ = run_qkv(w, tok, depth, n_nodes, [10, 500])
    qb, kb, _ = run_qkv(w, tok, depth, n_nodes, [10 + 777, 500 + 3])
    q0, k0, _ = run_qkv(w, tok, np.zeros_like(depth), n_nodes, [0, 0])
    g = SHAPE.hq // SHAPE.hkv
    for b in range(CFG.batch):
        r = int(n_nodes[b]) + 1
        np.testing.assert_allclose(np.linalg.norm(qa[b, :r], axis=-1),
                                   np.linalg.norm(q0[b, :r], axis=-1), rtol=1e-10)
        kk_a = np.repeat(ka[b, :r], g, axis=1)
        kk_b = np.repeat(kb[b, :r], g, axis=1)
        dots_a = np.einsum("ihd,jhd->hij", qa[b, :r], kk_a)
        dots_b = np.einsum("ihd,jhd->hij", qb[b, :r], kk_b)
        np.testing.assert_allclose(dots_a, dots_b, rtol=1e-8, atol=1e-8)


def test_missing_token_reads_row_zero():
    w = wl.layer_weights(CFG, SHAPE)
    tok, depth, n_nodes = tree_rows(3)
    tok2 = tok.copy()
    tok2[0, 0] = -1
    tok[0, 0] = 0
    a = run_qkv(w, tok, depth, n_nodes, [5, 5])
    bq = run_qkv(w, tok2, depth, n_nodes, [5, 5])
    for x, y in zip(a, bq):
        np.testing.assert_array_equal(x, y)


def test_argmax_matches_library_product_with_ties():
    w = wl.layer_weights(CFG, SHAPE)
    rows = wl.hidden_rows(CFG, CFG.nq_max, SHAPE.hidden)
    w_lm = w["w_lm"].copy()
    n_nodes = np.array([CFG.nq_max - 1, 3], np.int32)
    logits = f64(rows) @ f64(w_lm).T
    top = logits.argmax(-1)
    # plant exact ties: copy each row's winner into a smaller and a larger id
    for b in range(CFG.batch):
        t = int(top[b, 0])
        if t > 0:
            w_lm[t - 1] = w_lm[t]
    tgt, best, second = oracle.lm_head_argmax(rows, w_lm, n_nodes)
    logits = f64(rows) @ f64(w_lm).T
    for b in range(CFG.batch):
        for i in range(CFG.nq_max):
            if i > n_nodes[b]:
                assert tgt[b, i] == -1
                continue
            lg = logits[b, i]
            assert tgt[b, i] == int(np.flatnonzero(lg == lg.max())[0])     # smallest id of the max
            srt = np.sort(lg)[::-1]
            assert best[b, i] == pytest.approx(srt[0], abs=1e-12)
            assert second[b, i] == pytest.approx(srt[1], abs=1e-12)
    assert any(tgt[b, 0] == int(top[b, 0]) - 1 for b in range(CFG.batch) if top[b, 0] > 0)
