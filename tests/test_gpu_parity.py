"""GPU parity: every stage of the HIP library against the CPU oracle, through
the C ABI, on seeded synthetic inputs.

Bars: top-K ids, tree node sets/order (near-tie rule in helpers.compare_tree),
masks and acceptance bit-exact; log q, lse and log rho within 1e-5;
attention within 2e-2 (bf16) / 1e-4 (f32) absolute plus a relative
Frobenius bound per row.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from helpers import attn_close, compare_tree, cost_of, oracle_front, paths_of, targets_by_path
from tree_draft_build_amd import workload as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def td():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tree_draft_build_amd import binding
    return binding


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev_logits(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x).to(DEV)


def dev_attn(x):
    return dev_logits(np.ascontiguousarray(x))


def host_out(t, dtype):
    if dtype == "bf16":
        return wl.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def np_tree(t):
    return {k: v.cpu().numpy() for k, v in t.items()}


# ---------------------------------------------------------------------------
# stage (a)
# ---------------------------------------------------------------------------

def check_topk(ids_g, lq_g, lse_g, ids_o, lq_o, lse_o):
    np.testing.assert_array_equal(ids_g, ids_o)
    assert np.abs(lse_g - lse_o).max() < 1e-5
    assert np.abs(lq_g - lq_o).max() < 1e-5


@pytest.mark.parametrize("name,seqs", [("tiny", None), ("qwen3_8b", None), ("llama31_8b", None),
                                       ("batched", [0, 7, 15]), ("long", [0, 33, 63])])
def test_topk_configs(td, name, seqs):
    cfg = wl.CONFIGS[name]
    say("topk", name, seqs)
    x = wl.make_logits(cfg) if seqs is None or cfg.batch <= 4 else None
    if x is None:
        full = wl.make_logits(cfg)
        sub = full[seqs]
    else:
        full = sub = x
        seqs = list(range(cfg.batch))
    ids, lq, lse = td.draft_topk(dev_logits(full), cfg.topk)
    torch.cuda.synchronize()
    ids_o, lq_o, lse_o = oracle.draft_topk(sub, cfg.topk)
    check_topk(ids.cpu().numpy()[seqs], lq.cpu().numpy()[seqs], lse.cpu().numpy()[seqs], ids_o,
               lq_o, lse_o)


@pytest.mark.parametrize("V", [8, 1000, 4099, 33000])
@pytest.mark.parametrize("K", [1, 4, 8, 13, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_ragged_and_ties(td, V, K, dtype):
    if K > V:
        pytest.skip("K > V")
    say("topk ragged", V, K, dtype)
    rng = np.random.default_rng(V * 7 + K)
    x = np.round(rng.standard_normal((3, 5, V)) * 2, 1).astype(np.float32)  # many ties
    x[0, 0] = 1.5                                                           # all tied
    x[1, 1, -3:] = 40.0                                                     # tied top at the tail
    x[2, 3] = np.linspace(-3.0, 9.0, V)                                     # ascending: every element a new max
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    ids, lq, lse = td.draft_topk(dev_logits(x), K)
    torch.cuda.synchronize()
    check_topk(ids.cpu().numpy(), lq.cpu().numpy(), lse.cpu().numpy(), *oracle.draft_topk(x, K))


def test_topk_pos_stride(td):
    """Rows placed with a stride larger than the vocabulary (padded rows)."""
    say("topk pos_stride")
    rng = np.random.default_rng(3)
    V, S = 1000, 1024
    big = wl.f32_to_bf16_bits(rng.standard_normal((2, 4, S)).astype(np.float32) * 3)
    dev = dev_logits(big)
    K = 8
    ids = torch.empty((2, 4, K), dtype=torch.int32, device=DEV)
    lq = torch.empty((2, 4, K), dtype=torch.float64, device=DEV)
    lse = torch.empty((2, 4), dtype=torch.float64, device=DEV)
    ws = td.draft_topk_alloc_workspace(2, 4, V, K, DEV)
    st = td.lib.td_draft_topk(td._ptr(dev), td.TD_BF16, 2, 4, V, S, K, td._ptr(ids), td._ptr(lq),
                              td._ptr(lse), td._ptr(ws), ws.numel(), td._stream())
    assert st == 0, td.last_error()
    torch.cuda.synchronize()
    check_topk(ids.cpu().numpy(), lq.cpu().numpy(), lse.cpu().numpy(),
               *oracle.draft_topk(np.ascontiguousarray(big[:, :, :V]), K))


# ---------------------------------------------------------------------------
# stage (b), (b'), (d) with identical inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "tiny_fixed", "qwen3_8b", "qwen3_8b_stress",
                                  "llama31_8b", "batched"])
def test_build_tree_same_inputs(td, name):
    cfg = wl.CONFIGS[name]
    say("build_tree", name)
    x = wl.make_logits(cfg, list(range(min(cfg.batch, 4))))
    orc = oracle_front(cfg, x)
    ids = torch.from_numpy(orc["ids"]).to(DEV)
    lq = torch.from_numpy(orc["lq"]).to(DEV)
    root = torch.arange(x.shape[0], dtype=torch.int32, device=DEV) + 100
    t = np_tree(td.build_tree(ids, lq, cfg.n_max, cfg.use_stop, cost_of(cfg), cfg.l_ar, cfg.ahat0,
                              root_token=root))
    for b in range(x.shape[0]):
        compare_tree(b, t, orc, cfg.use_stop)
        assert t["node_token"][b, 0] == 100 + b
        n = int(t["n_nodes"][b])
        assert t["ahat"][b] == pytest.approx(cfg.ahat0 + np.exp(t["node_logrho"][b, 1:n + 1]).sum(),
                                             rel=1e-12)
    # with identical inputs and no near ties the trees are identical
    same = all(np.array_equal(t[k], orc["tree"][k]) for k in ("n_nodes", "node_token",
                                                               "node_parent", "node_depth"))
    if same:
        np.testing.assert_array_equal(t["node_logrho"], orc["tree"]["node_logrho"])


@pytest.mark.parametrize("n_max", [0, 1, 63, 64, 127, 255])
@pytest.mark.parametrize("K", [1, 3, 8, 32])
def test_build_tree_capacity_edges(td, n_max, K):
    """Fixed budgets up to the cap, K up to the cap, peaked and flat tables."""
    say("build_tree edges", n_max, K)
    rng = np.random.default_rng(n_max * 40 + K)
    B, V = 16, 64
    x = (rng.standard_normal((2, B, V)) * 1.5).astype(np.float32)
    x[1, :, 5] += 12.0       # peaked sequence: deep chains
    ids, lq, _ = oracle.draft_topk(x, K)
    cfg = wl.CONFIGS["tiny_fixed"].replace(block=B, vocab=V, topk=K, n_max=n_max)
    orc = dict(ids=ids, lq=lq,
               tree=oracle.build_tree(ids, lq, n_max, False),
               full=oracle.build_tree(ids, lq, n_max, False, want_curve=True))
    t = np_tree(td.build_tree(torch.from_numpy(ids).to(DEV), torch.from_numpy(lq).to(DEV), n_max,
                              False))
    for b in range(2):
        compare_tree(b, t, orc, False)
        avail = sum(K ** d for d in range(1, B + 1)) if K > 1 else B
        assert t["n_nodes"][b] == min(n_max, avail)


def test_tree_mask_same_inputs(td):
    say("tree_mask")
    rng = np.random.default_rng(11)
    for nq in (1, 2, 17, 64, 65, 129, 256):
        b = 5
        n_nodes = np.array([nq - 1, rng.integers(0, nq), 0, nq // 2, 1 if nq > 1 else 0], np.int32)
        par = np.full((b, nq), -1, np.int32)
        for bi in range(b):
            for i in range(1, int(n_nodes[bi]) + 1):
                par[bi, i] = rng.integers(0, i)
        m = td.tree_mask(torch.from_numpy(par).to(DEV), torch.from_numpy(n_nodes).to(DEV))
        torch.cuda.synchronize()
        want = oracle.tree_mask(par, n_nodes)
        np.testing.assert_array_equal(m.cpu().numpy().view(np.uint64), want)


def test_accept_same_inputs(td):
    say("accept")
    cfg = wl.CONFIGS["qwen3_8b_stress"].replace(batch=1)
    x = wl.make_logits(cfg)
    orc = oracle_front(cfg, x)
    tree = orc["tree"]
    lf = wl.logits_as_f64(x, "bf16")
    W = cfg.n_max + 1
    rows = []
    for seed in range(64):               # many target draws over one tree
        rows.append(wl.target_tokens(cfg, lf, tree["node_token"], tree["node_parent"],
                                     tree["n_nodes"], seed=seed)[0])
    tg = np.stack(rows)
    rep = lambda a: np.repeat(a, 64, axis=0)
    args_np = (rep(tree["node_token"]), rep(tree["node_parent"]), rep(tree["n_nodes"]), tg)
    alen, path, bonus = td.accept(*[torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
                                    for a in args_np], cfg.block)
    torch.cuda.synchronize()
    a_o, p_o, b_o = oracle.accept(*args_np, cfg.block)
    np.testing.assert_array_equal(alen.cpu().numpy(), a_o)
    np.testing.assert_array_equal(path.cpu().numpy(), p_o)
    np.testing.assert_array_equal(bonus.cpu().numpy(), b_o)
    assert a_o.max() > 1                  # some deep acceptances happened


# ---------------------------------------------------------------------------
# stage (c) with identical inputs
# ---------------------------------------------------------------------------

def run_attn(td, cfg, inp, par, n_nodes):
    mask = oracle.tree_mask(par, n_nodes)
    dq = dev_attn(inp["q"])
    kc, vc = dev_attn(inp["k_ctx"]), dev_attn(inp["v_ctx"])
    kt, vt = dev_attn(inp["k_tree"]), dev_attn(inp["v_tree"])
    off = torch.from_numpy(inp["ctx_offsets"]).to(DEV)
    total = int(inp["ctx_offsets"][-1])
    maxc = int(inp["ctx_len"].max()) if len(inp["ctx_len"]) else 0
    out = td.tree_verify_attn(dq, kc, vc, off, total, maxc, kt, vt,
                              torch.from_numpy(mask.view(np.int64)).to(DEV),
                              torch.from_numpy(n_nodes).to(DEV), wl.attn_scale(cfg))
    torch.cuda.synchronize()
    return host_out(out, cfg.attn_dtype), mask


def random_parents(rng, n_nodes, nq):
    par = np.full((len(n_nodes), nq), -1, np.int32)
    for b, n in enumerate(n_nodes):
        for i in range(1, int(n) + 1):
            par[b, i] = rng.integers(max(0, i - 4), i)     # deep-ish random trees
    return par


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (4, 1)])
def test_attention_small_ragged(td, dtype, d, hq, hkv):
    say("attn small", dtype, d, hq, hkv)
    cfg = wl.CONFIGS["qwen3_8b"].replace(name="s", index=50, batch=5, n_max=20, hq=hq, hkv=hkv,
                                         head_dim=d, attn_dtype=dtype, ctx_law="uniform",
                                         ctx_p0=0, ctx_p1=700)
    inp = wl.make_attn_inputs(cfg)
    rng = np.random.default_rng(hq + d)
    n_nodes = np.array([20, 0, 7, 1, 13], np.int32)
    par = random_parents(rng, n_nodes, cfg.nq_max)
    got, mask = run_attn(td, cfg, inp, par, n_nodes)
    want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                            inp["k_tree"], inp["v_tree"], mask, n_nodes, hq, hkv, d,
                            wl.attn_scale(cfg))
    attn_close(got, want, dtype, f"attn {dtype} d{d} {hq}/{hkv}", n_nodes)


def test_attention_empty_context(td):
    say("attn empty ctx")
    cfg = wl.CONFIGS["qwen3_8b"].replace(name="e", index=51, batch=3, n_max=5, ctx_law="fixed",
                                         ctx_p0=0)
    inp = wl.make_attn_inputs(cfg)
    n_nodes = np.array([5, 0, 2], np.int32)
    par = random_parents(np.random.default_rng(0), n_nodes, cfg.nq_max)
    got, mask = run_attn(td, cfg, inp, par, n_nodes)
    want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                            inp["k_tree"], inp["v_tree"], mask, n_nodes, cfg.hq, cfg.hkv,
                            cfg.head_dim, wl.attn_scale(cfg))
    attn_close(got, want, "bf16", "empty context", n_nodes)


@pytest.mark.parametrize("name", ["tiny_masksens", "qwen3_8b_masksens"])
def test_attention_mask_sensitive(td, name):
    """Tree keys dominate the softmax, so one wrong mask bit would move a row
    by far more than the tolerance."""
    cfg = wl.CONFIGS[name]
    say("attn mask-sensitive", name)
    x = wl.make_logits(cfg)
    orc = oracle_front(cfg, x)
    tree = orc["tree"]
    inp = wl.make_attn_inputs(cfg)
    got, mask = run_attn(td, cfg, inp, tree["node_parent"], tree["n_nodes"])
    want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                            inp["k_tree"], inp["v_tree"], mask, tree["n_nodes"], cfg.hq, cfg.hkv,
                            cfg.head_dim, wl.attn_scale(cfg))
    attn_close(got, want, cfg.attn_dtype, name, tree["n_nodes"])
    assert int(tree["n_nodes"][0]) == cfg.n_max


@pytest.mark.parametrize("law", ["normal", "mask_sensitive"])
def test_attention_row_group_paths(td, law):
    """Every tree row of sequences whose trees take each of the split kernel's
    row-group paths (8 sequences x 4096 keys x 8 KV heads: 1024-key chunks,
    320 work items, the 64-key ring), where trees of more than 4 row groups
    of 16 rows take 3 row groups per wave in row blocks of at most 12:
    17 row groups (n_nodes 64) in blocks of 9 and 8; 11, 5, 8 and 4
    (n_nodes 40, 16, 30, 12) in one block; 13 and 16 (50, 63) in two; one
    sequence has no tree beyond the root.  (Five row groups per wave are
    checked row by row by the long pipeline case.)"""
    say("attn row-group paths", law)
    cfg = wl.CONFIGS["qwen3_8b"].replace(name="rg5", index=52, batch=8, n_max=64, use_stop=False,
                                         ctx_law="fixed", ctx_p0=4096, attn_law=law)
    inp = wl.make_attn_inputs(cfg)
    n_nodes = np.array([64, 40, 16, 30, 12, 50, 63, 0], np.int32)
    par = random_parents(np.random.default_rng(52), n_nodes, cfg.nq_max)
    got, mask = run_attn(td, cfg, inp, par, n_nodes)
    for b0, b1 in ((0, 5), (5, 8)):
        want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                                inp["k_tree"], inp["v_tree"], mask, n_nodes, cfg.hq, cfg.hkv,
                                cfg.head_dim, wl.attn_scale(cfg), seqs=(b0, b1))
        attn_close(got[b0:b1], want, "bf16", f"row-group paths {law} seqs {b0}..{b1 - 1}",
                   n_nodes[b0:b1])


@pytest.mark.parametrize("law", ["normal", "mask_sensitive"])
def test_attention_five_group_path(td, law):
    """The split kernel's five-row-groups-per-wave path on every tree row:
    64 sequences x 512 keys x 8 KV heads make 96 chunks of 1024 keys, 768
    work items (more than two per compute unit), so trees of more than 4
    row groups take 5 per wave on the 64-key ring.  Trees of 17, 11, 5, 8,
    4, 13, 16 and 1 row groups (n_nodes 64, 40, 16, 30, 12, 50, 63, 0) repeat
    over the batch; sequences 0-7 and 63 are compared with the oracle."""
    say("attn five-group path", law)
    cfg = wl.CONFIGS["qwen3_8b"].replace(name="rg5b", index=53, batch=64, n_max=64, use_stop=False,
                                         ctx_law="fixed", ctx_p0=512, attn_law=law)
    inp = wl.make_attn_inputs(cfg)
    n_nodes = np.resize(np.array([64, 40, 16, 30, 12, 50, 63, 0], np.int32), cfg.batch)
    par = random_parents(np.random.default_rng(53), n_nodes, cfg.nq_max)
    got, mask = run_attn(td, cfg, inp, par, n_nodes)
    for b0, b1 in ((0, 8), (63, 64)):
        want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                                inp["k_tree"], inp["v_tree"], mask, n_nodes, cfg.hq, cfg.hkv,
                                cfg.head_dim, wl.attn_scale(cfg), seqs=(b0, b1))
        attn_close(got[b0:b1], want, "bf16", f"five-group path {law} seqs {b0}..{b1 - 1}",
                   n_nodes[b0:b1])


def attn_inputs_with_lengths(cfg, lens):
    """make_attn_inputs for explicit context lengths."""
    parts = [wl.attn_inputs_for_seq(cfg, b, int(n)) for b, n in enumerate(lens)]
    out = {k: np.concatenate([p[k] for p in parts], axis=0) if k in ("k_ctx", "v_ctx")
           else np.stack([p[k] for p in parts], axis=0) for k in parts[0]}
    lens = np.asarray(lens, np.int64)
    out["ctx_offsets"] = wl.ctx_offsets(cfg, lens)
    out["ctx_len"] = lens
    return out


@pytest.mark.parametrize("case", ["longest_first", "many_sequences"])
def test_attention_chunk_order(td, case):
    """Work items take the chunks longest first up to 64 sequences (every
    full chunk, then the last chunks by decreasing length, ties by sequence)
    and in sequence order beyond; the partial rows keep the sequence order.
    longest_first: 24 sequences, 29,941 keys x 8 KV heads (1024-key chunks,
    40 chunks, 320 work items): exact multiples of the chunk, empty and one-key contexts,
    last chunks of equal length in different sequences, and more work items
    than compute units.  many_sequences: 70 sequences (the scan over groups
    of 64; 2048-key chunks), three of them several chunks long.  Every tree row of the
    compared sequences against the oracle."""
    say("attn chunk order", case)
    if case == "longest_first":
        lens = [3000, 952, 0, 1024, 2048, 5000, 1, 1023, 1025, 476, 1500, 2047,
                904, 3000, 64, 700, 1, 1100, 2100, 952, 0, 900, 1024, 1100]
        cmp = [(0, 12), (12, 24)]
    else:
        rng = np.random.default_rng(54)
        lens = rng.integers(0, 1200, 70)
        lens[[3, 40, 66]] = [9000, 5000, 7777]
        lens[[10, 65]] = 0
        cmp = [(0, 12), (38, 42), (62, 70)]
    cfg = wl.CONFIGS["qwen3_8b"].replace(name="co", index=54, batch=len(lens), n_max=8,
                                         use_stop=False, ctx_law="fixed", ctx_p0=0)
    inp = attn_inputs_with_lengths(cfg, lens)
    n_nodes = np.resize(np.array([8, 3, 0, 5, 1, 8, 2], np.int32), cfg.batch)
    par = random_parents(np.random.default_rng(54), n_nodes, cfg.nq_max)
    got, mask = run_attn(td, cfg, inp, par, n_nodes)
    for b0, b1 in cmp:
        want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                                inp["k_tree"], inp["v_tree"], mask, n_nodes, cfg.hq, cfg.hkv,
                                cfg.head_dim, wl.attn_scale(cfg), seqs=(b0, b1))
        attn_close(got[b0:b1], want, "bf16", f"chunk order {case} seqs {b0}..{b1 - 1}",
                   n_nodes[b0:b1])


def test_attention_split_invariance(td):
    """One sequence (5000 keys, a 16-node tree) alone and as sequence 0 of a
    batch of 12: alone its context splits into 256-key chunks (20 partials
    per row), in the batch into 4096-key chunks (2 partials).  Both results
    meet the oracle bound, and they agree with each other far more tightly
    (only the summation order of the partials differs)."""
    say("attn split invariance")
    cfg = wl.CONFIGS["qwen3_8b"].replace(name="si", index=55, batch=12, n_max=16, use_stop=False,
                                         ctx_law="fixed", ctx_p0=0)
    lens = [5000] + [20000 + 997 * i for i in range(11)]
    n_nodes = np.array([16, 3, 0, 16, 5, 1, 8, 2, 16, 4, 7, 9], np.int32)
    par = random_parents(np.random.default_rng(55), n_nodes, cfg.nq_max)
    inp = attn_inputs_with_lengths(cfg, lens)
    got_b, mask_b = run_attn(td, cfg, inp, par, n_nodes)
    one = cfg.replace(batch=1)
    inp1 = attn_inputs_with_lengths(one, lens[:1])
    got_1, mask_1 = run_attn(td, one, inp1, par[:1], n_nodes[:1])
    np.testing.assert_array_equal(mask_1[0], mask_b[0])
    want = oracle.tree_attn(inp1["q"], inp1["k_ctx"], inp1["v_ctx"], inp1["ctx_offsets"],
                            inp1["k_tree"], inp1["v_tree"], mask_1, n_nodes[:1], cfg.hq, cfg.hkv,
                            cfg.head_dim, wl.attn_scale(cfg))
    attn_close(got_1, want, "bf16", "split invariance: alone", n_nodes[:1])
    attn_close(got_b[:1], want, "bf16", "split invariance: in the batch", n_nodes[:1])
    rows = int(n_nodes[0]) + 1
    diff = np.abs(got_1[0, :rows] - got_b[0, :rows]).max()
    assert diff <= 2e-3, f"alone vs in the batch: {diff:.3g}"


# ---------------------------------------------------------------------------
# end to end: the whole path on the GPU vs the whole path in the oracle
# ---------------------------------------------------------------------------

def gpu_pipeline(td, cfg, x, inp):
    ids, lq, lse = td.draft_topk(dev_logits(x), cfg.topk)
    t = td.build_tree(ids, lq, cfg.n_max, cfg.use_stop, cost_of(cfg), cfg.l_ar, cfg.ahat0)
    mask = td.tree_mask(t["node_parent"], t["n_nodes"])
    off = torch.from_numpy(inp["ctx_offsets"]).to(DEV)
    total = int(inp["ctx_offsets"][-1])
    out = td.tree_verify_attn(dev_attn(inp["q"]), dev_attn(inp["k_ctx"]), dev_attn(inp["v_ctx"]),
                              off, total, int(inp["ctx_len"].max()), dev_attn(inp["k_tree"]),
                              dev_attn(inp["v_tree"]), mask, t["n_nodes"], wl.attn_scale(cfg))
    torch.cuda.synchronize()
    return dict(ids=ids.cpu().numpy(), lq=lq.cpu().numpy(), lse=lse.cpu().numpy(), tree=np_tree(t),
                mask=mask.cpu().numpy().view(np.uint64), out=host_out(out, cfg.attn_dtype),
                t_dev=t)


@pytest.mark.parametrize("name,sample", [("tiny", None), ("tiny_fixed", None), ("qwen3_8b", None),
                                         ("qwen3_8b_stress", None), ("llama31_8b", [0, 3]),
                                         ("batched", [0, 9]), ("long", [5, 40]),
                                         ("two_seq_k4", None), ("few_slices", None)])
def test_pipeline(td, name, sample):
    cfg = wl.CONFIGS[name]
    say("pipeline", name, sample)
    x = wl.make_logits(cfg)
    inp = wl.make_attn_inputs(cfg)
    g = gpu_pipeline(td, cfg, x, inp)
    seqs = list(range(cfg.batch)) if sample is None else sample
    orc = oracle_front(cfg, x[seqs])
    check_topk(g["ids"][seqs], g["lq"][seqs], g["lse"][seqs], orc["ids"], orc["lq"], orc["lse"])
    sub_tree = {k: v[seqs] for k, v in g["tree"].items()}
    for i in range(len(seqs)):
        compare_tree(i, sub_tree, orc, cfg.use_stop)
    # mask of the GPU tree, checked against the oracle's mask of the same tree
    np.testing.assert_array_equal(g["mask"][seqs],
                                  oracle.tree_mask(sub_tree["node_parent"], sub_tree["n_nodes"]))
    # attention of the GPU tree on every row of the sampled sequences
    for b in seqs:
        want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                                inp["k_tree"], inp["v_tree"], g["mask"], g["tree"]["n_nodes"],
                                cfg.hq, cfg.hkv, cfg.head_dim, wl.attn_scale(cfg), seqs=(b, b + 1))
        attn_close(g["out"][b:b + 1], want, cfg.attn_dtype, f"{name} seq {b}",
                   g["tree"]["n_nodes"][b:b + 1])
    # acceptance on the GPU tree with the synthetic target
    lf = wl.logits_as_f64(x, cfg.logit_dtype)
    tg = targets_by_path(cfg, lf, g["tree"])
    alen, path, bonus = td.accept(g["t_dev"]["node_token"], g["t_dev"]["node_parent"],
                                  g["t_dev"]["n_nodes"], torch.from_numpy(tg).to(DEV), cfg.block)
    torch.cuda.synchronize()
    a_o, p_o, b_o = oracle.accept(g["tree"]["node_token"], g["tree"]["node_parent"],
                                  g["tree"]["n_nodes"], tg, cfg.block)
    np.testing.assert_array_equal(alen.cpu().numpy(), a_o)
    np.testing.assert_array_equal(path.cpu().numpy(), p_o)
    np.testing.assert_array_equal(bonus.cpu().numpy(), b_o)
    assert np.all(a_o <= np.maximum(0, g["tree"]["node_depth"].max(axis=1)))


@pytest.mark.parametrize("name", ["tiny_fixed", "qwen3_8b_stress", "batched", "llama31_8b"])
@pytest.mark.parametrize("branch,cut", [(0, 9), (1, None), (3, 20), (2, None)])
def test_build_tree_selective(td, name, branch, cut):
    """Selective verification (threshold on log rho between the oracle's
    cut-th and next node) and the branch cap, same inputs, GPU vs oracle."""
    cfg = wl.CONFIGS[name]
    say("build_tree selective", name, branch, cut)
    x = wl.make_logits(cfg, list(range(min(cfg.batch, 4))))
    ids, lq, _ = oracle.draft_topk(x, cfg.topk)
    tau = float("-inf")
    if cut is not None:
        ref = oracle.build_tree(ids, lq, cfg.n_max, False, branch=branch)
        lr = ref["node_logrho"][0, 1:]
        tau = float((lr[cut - 1] + lr[cut]) / 2) if cut < int(ref["n_nodes"][0]) else -1e300
    kw = dict(branch=branch, min_logrho=tau)
    orc = dict(ids=ids, lq=lq,
               tree=oracle.build_tree(ids, lq, cfg.n_max, cfg.use_stop, cost_of(cfg), cfg.l_ar,
                                      cfg.ahat0, **kw),
               full=oracle.build_tree(ids, lq, cfg.n_max, False, cost_of(cfg), cfg.l_ar, cfg.ahat0,
                                      want_curve=True, **kw))
    t = np_tree(td.build_tree(torch.from_numpy(ids).to(DEV), torch.from_numpy(lq).to(DEV),
                              cfg.n_max, cfg.use_stop, cost_of(cfg), cfg.l_ar, cfg.ahat0, **kw))
    for b in range(x.shape[0]):
        compare_tree(b, t, orc, cfg.use_stop)
        n = int(t["n_nodes"][b])
        assert np.all(t["node_logrho"][b, 1:n + 1] >= tau)
        if branch == 1:
            assert n <= cfg.block
