"""Pins of the oracle's stage (a): the log-softmax normaliser lse_k and the
top-K table of each drafter position (path scores need q_k, BASTION
"Methodik" §1).  Each pin is independent of the oracle's own code: closed
forms, a library special case (torch.logsumexp in float64) and brute force
(NumPy lexsort)."""
import math

import numpy as np
import pytest
import torch

import oracle
from tree_draft_build_amd import workload as wl


def _bf16(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_lse_constant_row_closed_form():
    # lse of V equal logits c is c + ln V exactly (up to the last bit).
    for V, c in [(1, 0.0), (7, -3.25), (32000, 1.5), (151936, 10.0)]:
        x = np.full((1, 2, V), c, np.float32)
        _, lq, lse = oracle.draft_topk(x, 1)
        assert lse == pytest.approx(c + math.log(V), abs=1e-12, rel=1e-14)
        # every token then has q = 1/V
        assert lq[0, 0, 0] == pytest.approx(-math.log(V), abs=1e-12)


def test_lse_single_spike_closed_form():
    # one logit s, the other V-1 equal to c: lse = s + log1p((V-1) e^{c-s})
    V, s, c = 1000, 30.0, -2.0
    x = np.full((1, 1, V), c, np.float32)
    x[0, 0, 417] = s
    ids, lq, lse = oracle.draft_topk(x, 3)
    want = s + math.log1p((V - 1) * math.exp(c - s))
    assert lse[0, 0] == pytest.approx(want, abs=1e-12)
    assert ids[0, 0, 0] == 417
    # ties among the flat tokens go to the smaller ids
    assert list(ids[0, 0, 1:]) == [0, 1]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lse_matches_torch_logsumexp(dtype):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((2, 5, 3001)) * 3).astype(np.float32)
    x[:, :, 11] += 9.0
    stored = x if dtype == "f32" else _bf16(x)
    _, lq, lse = oracle.draft_topk(stored, 4)
    xf = wl.logits_as_f64(stored, dtype)
    ref = torch.logsumexp(torch.from_numpy(xf), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)
    # the top-K log q are the raw logits minus lse
    ids, _, _ = oracle.draft_topk(stored, 4)
    got = np.take_along_axis(xf, ids.astype(np.int64), axis=-1) - ref[..., None]
    np.testing.assert_allclose(lq, got, rtol=0, atol=1e-12)


def test_logq_full_vocab_normalises():
    # with K = V every token is listed and the probabilities sum to one
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((3, 4, 50)) * 2).astype(np.float32)
    _, lq, _ = oracle.draft_topk(x, 50)
    np.testing.assert_allclose(np.exp(lq).sum(-1), 1.0, atol=1e-13)


def _brute_topk(xf, K):
    out = np.empty(xf.shape[:-1] + (K,), np.int32)
    ids = np.arange(xf.shape[-1])
    for idx in np.ndindex(*xf.shape[:-1]):
        order = np.lexsort((ids, -xf[idx]))  # primary: value desc, then id asc
        out[idx] = order[:K]
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 4, 8, 32])
def test_topk_matches_bruteforce_with_ties(dtype, K):
    rng = np.random.default_rng(100 + K)
    # coarse values so that many ties exist, both in f32 and after bf16 rounding
    x = np.round(rng.standard_normal((2, 6, 700)) * 2, 1).astype(np.float32)
    x[0, 0, :] = 1.0            # an all-tied row
    x[1, 2, 650:] = 50.0        # ties at the top, late ids
    stored = x if dtype == "f32" else _bf16(x)
    ids, _, _ = oracle.draft_topk(stored, K)
    want = _brute_topk(wl.logits_as_f64(stored, dtype), K)
    np.testing.assert_array_equal(ids, want)


def test_topk_on_config_rows():
    cfg = wl.CONFIGS["qwen3_8b"]
    x = wl.make_logits(cfg)[:, :2]
    ids, lq, _ = oracle.draft_topk(x, cfg.topk)
    want = _brute_topk(wl.logits_as_f64(x, "bf16"), cfg.topk)
    np.testing.assert_array_equal(ids, want)
    assert np.all(np.diff(lq, axis=-1) <= 0)
