"""GPU: the KV commit of the accepted path (td_kv_commit and the verify
step's fused commit) and attention over context lengths, against the oracle;
and a multi-step synthetic decode loop in which every step's tree, attention,
acceptance and committed context match the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import test_oracle_commit as toc
from helpers import attn_close, compare_tree, cost_of, oracle_front, targets_by_path
from tree_draft_build_amd import workload as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def td():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tree_draft_build_amd import binding
    return binding


def dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("room", [None, 2])
def test_kv_commit_matches_oracle(td, room):
    print("[case] kv_commit", room, flush=True)
    s = toc.setup(room=room)
    inp, cfg = s["inp"], toc.CFG
    kc, vc, lens = s["kc"].copy(), s["vc"].copy(), s["L"].copy()
    nxt = oracle.kv_commit(s["kt"], inp["v_tree"], s["alen"], s["path"], s["bonus"], kc, vc,
                           s["off"], lens, cfg.hkv, cfg.head_dim)
    gk, gv, gl = dev(s["kc"]), dev(s["vc"]), dev(s["L"])
    groot = torch.full((cfg.batch,), -5, dtype=torch.int32, device=DEV)
    td.kv_commit(dev(s["kt"]), dev(inp["v_tree"]), dev(s["alen"]), dev(s["path"]), dev(s["bonus"]),
                 gk, gv, dev(s["off"]), gl, next_root=groot)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(gl), lens)
    np.testing.assert_array_equal(host(groot), nxt)
    np.testing.assert_array_equal(host(gk), kc)
    np.testing.assert_array_equal(host(gv), vc)


def test_attention_over_context_lengths(td):
    """bf16 at the Qwen3-8B head shape: each sequence's context is a prefix
    of its region (one empty, one full), the rest of the region is garbage."""
    print("[case] attn ctx lengths", flush=True)
    cfg = wl.CONFIGS["qwen3_8b"].replace(name="lens", index=61, batch=4, n_max=20,
                                         ctx_law="uniform", ctx_p0=300, ctx_p1=1200)
    inp = wl.make_attn_inputs(cfg)
    region = inp["ctx_len"].astype(np.int64)
    lens = np.array([0, region[1], region[2] // 2, 7], np.int64)
    n_nodes = np.array([20, 3, 0, 11], np.int32)
    rng = np.random.default_rng(61)
    par = np.full((cfg.batch, cfg.nq_max), -1, np.int32)
    for b, n in enumerate(n_nodes):
        for i in range(1, int(n) + 1):
            par[b, i] = rng.integers(max(0, i - 3), i)
    mask = oracle.tree_mask(par, n_nodes)
    out = td.tree_verify_attn(dev(inp["q"]), dev(inp["k_ctx"]), dev(inp["v_ctx"]),
                              dev(inp["ctx_offsets"]), int(inp["ctx_offsets"][-1]),
                              int(region.max()), dev(inp["k_tree"]), dev(inp["v_tree"]),
                              dev(mask.view(np.int64)), dev(n_nodes), wl.attn_scale(cfg),
                              ctx_lengths=dev(lens))
    torch.cuda.synchronize()
    got = wl.bf16_bits_to_f32(host(out)).astype(np.float64)
    want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"], inp["k_tree"],
                            inp["v_tree"], mask, n_nodes, cfg.hq, cfg.hkv, cfg.head_dim,
                            wl.attn_scale(cfg), ctx_lengths=lens)
    attn_close(got, want, "bf16", "context lengths", n_nodes)


@pytest.mark.parametrize("name,steps", [("qwen3_8b_stress", 4), ("tiny_masksens", 3)])
def test_multi_step_decode(td, name, steps):
    """The fused step with commit, step after step: the bonus of one step is
    the next root, the accepted path's K/V extend the contexts in place; each
    step's outputs match the oracle pipeline run on the same state."""
    base = wl.CONFIGS[name].replace(batch=2, ctx_law="uniform", ctx_p0=200, ctx_p1=700)
    print("[case] decode", name, steps, flush=True)
    cfg0 = base.replace(index=70)
    inp0 = wl.make_attn_inputs(cfg0)
    L0 = inp0["ctx_len"].astype(np.int64)
    room = steps * (base.block + 1)
    region = L0 + room
    off = np.zeros(base.batch + 1, np.int64)
    off[1:] = np.cumsum(region)
    kc = np.zeros((off[-1], base.hkv, base.head_dim), inp0["k_ctx"].dtype)
    vc = np.zeros_like(kc)
    for b in range(base.batch):
        o = inp0["ctx_offsets"][b]
        kc[off[b]:off[b] + L0[b]] = inp0["k_ctx"][o:o + L0[b]]
        vc[off[b]:off[b] + L0[b]] = inp0["v_ctx"][o:o + L0[b]]
    lens = L0.copy()
    root = np.array([11, 22], np.int32)
    gk, gv, gl, goff = dev(kc), dev(vc), dev(lens), dev(off)
    groot = dev(root)
    gnext = torch.empty(base.batch, dtype=torch.int32, device=DEV)
    vs = td.VerifyStep(batch=base.batch, block=base.block, vocab=base.vocab, topk=base.topk,
                       n_max=base.n_max, use_stop=base.use_stop, cost=cost_of(base), l_ar=base.l_ar,
                       ahat0=base.ahat0, hq=base.hq, hkv=base.hkv, head_dim=base.head_dim,
                       scale=wl.attn_scale(base),
                       logits_dtype=td.TD_BF16 if base.logit_dtype == "bf16" else td.TD_F32,
                       attn_dtype=td.TD_BF16 if base.attn_dtype == "bf16" else td.TD_F32,
                       total_ctx=int(off[-1]), max_ctx=int(region.max()), device=DEV)
    total_accepted = 0
    for step in range(steps):
        cfg = base.replace(index=80 + step)
        x = wl.make_logits(cfg)
        inp = wl.make_attn_inputs(cfg)           # this step's q and tree K/V
        gl_before = host(gl).copy()
        np.testing.assert_array_equal(gl_before, lens)
        d = dict(logits=dev(x), q=dev(inp["q"]), k_tree=dev(inp["k_tree"]), v_tree=dev(inp["v_tree"]))
        # draft half first: the target tokens depend on the tree
        tg0 = torch.full((base.batch, base.nq_max), -1, dtype=torch.int32, device=DEV)
        vs.set_inputs(d["logits"], d["q"], gk, gv, goff, d["k_tree"], d["v_tree"], tg0,
                      root_token=groot, ctx_lengths=gl, commit=True, next_root=gnext)
        vs.run(stages=td.TD_STEP_DRAFT)
        torch.cuda.synchronize()
        tree = {k: v.cpu().numpy() for k, v in vs.tree.items()}
        np.testing.assert_array_equal(tree["node_token"][:, 0], root)
        orc = oracle_front(cfg, x)
        for b in range(base.batch):
            compare_tree(b, tree, orc, cfg.use_stop)
        tg = targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree)
        vs.set_inputs(d["logits"], d["q"], gk, gv, goff, d["k_tree"], d["v_tree"], dev(tg),
                      root_token=groot, ctx_lengths=gl, commit=True, next_root=gnext)
        vs.run(stages=td.TD_STEP_VERIFY)
        torch.cuda.synchronize()
        # the oracle on the same tree and state
        m = oracle.tree_mask(tree["node_parent"], tree["n_nodes"])
        np.testing.assert_array_equal(vs.mask.cpu().numpy().view(np.uint64), m)
        want = oracle.tree_attn(inp["q"], kc, vc, off, inp["k_tree"], inp["v_tree"], m,
                                tree["n_nodes"], cfg.hq, cfg.hkv, cfg.head_dim, wl.attn_scale(cfg),
                                ctx_lengths=lens)
        if cfg.attn_dtype == "bf16":
            got = wl.bf16_bits_to_f32(host(vs.out)).astype(np.float64)
        else:
            got = host(vs.out).astype(np.float64)
        attn_close(got, want, cfg.attn_dtype, f"{name} step {step}", tree["n_nodes"])
        a_o, p_o, b_o = oracle.accept(tree["node_token"], tree["node_parent"], tree["n_nodes"], tg,
                                      cfg.block)
        np.testing.assert_array_equal(vs.accept_len.cpu().numpy(), a_o)
        np.testing.assert_array_equal(vs.accept_path.cpu().numpy(), p_o)
        np.testing.assert_array_equal(vs.bonus_token.cpu().numpy(), b_o)
        nxt = oracle.kv_commit(inp["k_tree"], inp["v_tree"], a_o, p_o, b_o, kc, vc, off, lens,
                               cfg.hkv, cfg.head_dim)
        np.testing.assert_array_equal(host(gl), lens)
        np.testing.assert_array_equal(host(gnext), nxt)
        np.testing.assert_array_equal(host(gk), kc)
        np.testing.assert_array_equal(host(gv), vc)
        total_accepted += int(a_o.sum())
        root = nxt
        groot.copy_(gnext)
    assert np.all(lens > L0)
    if name == "qwen3_8b_stress":
        assert total_accepted > 0
