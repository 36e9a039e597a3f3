"""GPU: the fused verify step (td_verify_step, three kernels, or two when the
context split runs inside the first kernel) produces exactly what the five
stage calls produce on the same inputs, on every workload (the attention
output within one bf16 rounding step in the two-kernel form), and keeps doing
so over repeated calls on one workspace (its epoch words advance by
themselves).  The stage calls are checked against the oracle in
test_gpu_parity.py; here the oracle also checks the step's attention and
acceptance directly on one workload."""
import numpy as np
import pytest
import torch

import oracle
from helpers import attn_close, cost_of, targets_by_path
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


def modular(td, cfg, d, tg, **kw):
    ids, lq, lse = td.draft_topk(d["logits"], cfg.topk)
    t = td.build_tree(ids, lq, cfg.n_max, cfg.use_stop, cost_of(cfg), cfg.l_ar, cfg.ahat0, **kw)
    mask = td.tree_mask(t["node_parent"], t["n_nodes"])
    out = td.tree_verify_attn(d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["total"], d["maxc"],
                              d["k_tree"], d["v_tree"], mask, t["n_nodes"], wl.attn_scale(cfg))
    res = dict(topk_id=ids, topk_logq=lq, lse=lse, mask=mask, out=out, **t)
    if tg is not None:
        a, p, bo = td.accept(t["node_token"], t["node_parent"], t["n_nodes"], tg, cfg.block)
        res.update(accept_len=a, accept_path=p, bonus_token=bo)
    torch.cuda.synchronize()
    return only_tree_rows({k: v.cpu() for k, v in res.items()})


def make_step(td, cfg, d, **kw):
    s = td.VerifyStep(batch=cfg.batch, block=cfg.block, vocab=cfg.vocab, topk=cfg.topk,
                      n_max=cfg.n_max, use_stop=cfg.use_stop, cost=cost_of(cfg), l_ar=cfg.l_ar,
                      ahat0=cfg.ahat0, hq=cfg.hq, hkv=cfg.hkv, head_dim=cfg.head_dim,
                      scale=wl.attn_scale(cfg),
                      logits_dtype=td.TD_BF16 if cfg.logit_dtype == "bf16" else td.TD_F32,
                      attn_dtype=td.TD_BF16 if cfg.attn_dtype == "bf16" else td.TD_F32,
                      total_ctx=d["total"], max_ctx=d["maxc"], device=DEV, **kw)
    return s


def step_outputs(s):
    res = dict(topk_id=s.topk_id, topk_logq=s.topk_logq, lse=s.lse, mask=s.mask, out=s.out,
               accept_len=s.accept_len, accept_path=s.accept_path, bonus_token=s.bonus_token,
               **s.tree)
    return only_tree_rows({k: v.cpu() for k, v in res.items()})


def only_tree_rows(res):
    """The attention output's rows past each tree are not written: zero
    them in the host copy so two runs compare on the tree rows only."""
    out = res["out"].clone()
    for b, n in enumerate(res["n_nodes"].tolist()):
        out[b, max(n, -1) + 1:] = 0
    res["out"] = out
    return res


def inputs(cfg):
    x = wl.make_logits(cfg)
    inp = wl.make_attn_inputs(cfg)
    return x, inp, dict(logits=dev(x), q=dev(inp["q"]), k_ctx=dev(inp["k_ctx"]),
                        v_ctx=dev(inp["v_ctx"]), k_tree=dev(inp["k_tree"]),
                        v_tree=dev(inp["v_tree"]), off=dev(inp["ctx_offsets"]),
                        total=int(inp["ctx_offsets"][-1]), maxc=int(inp["ctx_len"].max()))


def assert_same(a, b, what, exact_out=True):
    """Every output bit for bit; with exact_out False the attention output
    within two bf16 rounding steps instead: a step whose context split runs
    inside its first kernel sums each chunk's keys in another order, and both
    forms round their chunk partials' O rows to bf16 (2^-9 each), so the two
    can differ by the output's own rounding step plus the partials'."""
    for k in a:
        if k == "out" and not exact_out:
            x, y = a[k].float(), b[k].float()
            assert torch.allclose(x, y, rtol=2.0 ** -6, atol=2e-3), \
                f"{what}: out differs by {(x - y).abs().max().item():.3g}"
        else:
            assert torch.equal(a[k], b[k]), f"{what}: {k} differs"


def split_inside(s):
    """The step runs its context split inside its first kernel."""
    return s.kernels() == 2


@pytest.mark.parametrize("name", ["tiny", "tiny_fixed", "qwen3_8b", "qwen3_8b_stress",
                                  "qwen3_8b_masksens", "llama31_8b", "batched", "long",
                                  "two_seq_k4", "few_slices", "fused_ragged"])
def test_step_equals_stage_calls(td, name):
    cfg = wl.CONFIGS[name]
    print("[case] step vs stages", name, flush=True)
    x, inp, d = inputs(cfg)
    ref = modular(td, cfg, d, None)
    tree_np = {k: ref[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
    tg = dev(targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree_np))
    ref = modular(td, cfg, d, tg)
    s = make_step(td, cfg, d)
    s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"], tg)
    for rep in range(3):  # the workspace must be ready again after every call
        s.run()
        torch.cuda.synchronize()
        assert_same(ref, step_outputs(s), f"{name} call {rep}", not split_inside(s))


def test_step_tied_logits(td):
    """Positions of all-equal or two-valued logits (many tied keys) through
    the fused step at the Qwen3-8B shape, against the stage calls."""
    cfg = wl.CONFIGS["qwen3_8b_stress"]
    print("[case] step tied logits", flush=True)
    x, inp, d = inputs(cfg)
    x = x.copy()
    x[0, 3, :] = 0x3F00                        # bf16 0.5 everywhere
    x[0, 10, :] = 0x4000                       # bf16 2.0 ...
    x[0, 10, 1::3] = 0x4080                    # ... and 4.0 on every third token
    x[0, 15, :cfg.vocab // 2] = 0xBF80         # -1.0 on the first half
    d["logits"] = dev(x)
    ref = modular(td, cfg, d, None)
    tree_np = {k: ref[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
    tg = dev(targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree_np))
    ref = modular(td, cfg, d, tg)
    s = make_step(td, cfg, d)
    s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"], tg)
    for rep in range(2):
        s.run()
        torch.cuda.synchronize()
        assert_same(ref, step_outputs(s), f"tied call {rep}", not split_inside(s))
    ids = ref["topk_id"].numpy().reshape(cfg.block, cfg.topk)
    assert list(ids[3]) == list(range(cfg.topk))                # ties go to the smaller id
    assert list(ids[10]) == [1 + 3 * j for j in range(cfg.topk)]


def test_step_alternating_inputs(td):
    """Two workloads of one shape through one step object, alternating."""
    cfg_a = wl.CONFIGS["qwen3_8b_stress"]
    cfg_b = cfg_a.replace(index=31)
    print("[case] step alternating", flush=True)
    xa, ia, da = inputs(cfg_a)
    xb, ib, db = inputs(cfg_b)
    assert da["total"] == db["total"]
    refs, tgs = [], []
    for cfg, x, d in ((cfg_a, xa, da), (cfg_b, xb, db)):
        r = modular(td, cfg, d, None)
        tree_np = {k: r[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
        tg = dev(targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree_np))
        refs.append(modular(td, cfg, d, tg))
        tgs.append(tg)
    s = make_step(td, cfg_a, da)
    for rep in range(6):
        j = rep % 2
        d = (da, db)[j]
        s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"],
                     d["v_tree"], tgs[j])
        s.run()
        torch.cuda.synchronize()
        assert_same(refs[j], step_outputs(s), f"alternating call {rep}", not split_inside(s))


def test_step_against_oracle(td):
    cfg = wl.CONFIGS["qwen3_8b_stress"]
    print("[case] step vs oracle", flush=True)
    x, inp, d = inputs(cfg)
    ids, lq, _ = oracle.draft_topk(x, cfg.topk)
    tr = oracle.build_tree(ids, lq, cfg.n_max, cfg.use_stop, cost_of(cfg), cfg.l_ar, cfg.ahat0)
    tg_np = wl.target_tokens(cfg, wl.logits_as_f64(x, "bf16"), tr["node_token"], tr["node_parent"],
                             tr["n_nodes"])
    s = make_step(td, cfg, d)
    s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"],
                 dev(tg_np))
    s.run()
    torch.cuda.synchronize()
    out = step_outputs(s)
    for k in ("n_nodes", "node_token", "node_parent", "node_depth"):
        np.testing.assert_array_equal(out[k].numpy(), tr[k])
    m = oracle.tree_mask(tr["node_parent"], tr["n_nodes"])
    np.testing.assert_array_equal(out["mask"].numpy().view(np.uint64), m)
    want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"], inp["k_tree"],
                            inp["v_tree"], m, tr["n_nodes"], cfg.hq, cfg.hkv, cfg.head_dim,
                            wl.attn_scale(cfg))
    got = wl.bf16_bits_to_f32(out["out"].view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    attn_close(got, want, "bf16", "step attention", tr["n_nodes"])
    a_o, p_o, b_o = oracle.accept(tr["node_token"], tr["node_parent"], tr["n_nodes"], tg_np, cfg.block)
    np.testing.assert_array_equal(out["accept_len"].numpy(), a_o)
    np.testing.assert_array_equal(out["accept_path"].numpy(), p_o)
    np.testing.assert_array_equal(out["bonus_token"].numpy(), b_o)


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b_stress", "batched", "two_seq_k4", "fused_ragged"])
def test_step_in_two_calls(td, name):
    """A draft-only call followed by a verify-only call on the same argument
    block and workspace gives the one-call step's results."""
    cfg = wl.CONFIGS[name]
    print("[case] step in two calls", name, flush=True)
    x, inp, d = inputs(cfg)
    ref = modular(td, cfg, d, None)
    tree_np = {k: ref[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
    tg = dev(targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree_np))
    ref = modular(td, cfg, d, tg)
    s = make_step(td, cfg, d)
    s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"], tg)
    for rep in range(2):
        s.out.fill_(0)
        s.accept_len.fill_(-7)
        s.run(stages=td.TD_STEP_DRAFT)
        torch.cuda.synchronize()
        got = step_outputs(s)
        for k in ("topk_id", "topk_logq", "lse", "mask", "n_nodes", "node_token", "node_parent",
                  "node_depth", "node_logrho"):
            assert torch.equal(ref[k], got[k]), f"{name} draft call {rep}: {k} differs"
        assert int(got["accept_len"][0]) == -7      # verify kernels did not run
        s.run(stages=td.TD_STEP_VERIFY)
        torch.cuda.synchronize()
        assert_same(ref, step_outputs(s), f"{name} two calls {rep}")


def test_split_inside_first_kernel_modes(td):
    """One workspace through every way of calling the step: both stages in
    one call (split inside the first kernel), the two stages in two calls
    (split kernel of its own), and a change of the tree size law between
    calls (the trees' sizes reach the split workgroups anew each call)."""
    cfg = wl.CONFIGS["qwen3_8b"]        # S(N) stops at the root; the fixed law fills 64 nodes
    print("[case] split inside kernel 1: call modes", flush=True)
    x, inp, d = inputs(cfg)
    refs, tgs = {}, {}
    for stop in (True, False):
        c = cfg.replace(use_stop=stop)
        r = modular(td, c, d, None)
        tree_np = {k: r[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
        tgs[stop] = dev(targets_by_path(c, wl.logits_as_f64(x, c.logit_dtype), tree_np))
        refs[stop] = modular(td, c, d, tgs[stop])
    assert int(refs[True]["n_nodes"][0]) != int(refs[False]["n_nodes"][0])
    s = make_step(td, cfg, d)
    assert split_inside(s) and s.kernels(td.TD_STEP_DRAFT) == 1
    for rep, (stop, mode) in enumerate([(True, "one"), (True, "two"), (True, "one"), (False, "one"),
                                        (False, "two"), (True, "one"), (False, "one")]):
        s.args.use_stop = int(stop)
        s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"],
                     tgs[stop])
        s.out.fill_(0)
        if mode == "one":
            s.run()
        else:
            s.run(stages=td.TD_STEP_DRAFT)
            s.run(stages=td.TD_STEP_VERIFY)
        torch.cuda.synchronize()
        assert_same(refs[stop], step_outputs(s), f"call {rep} ({mode}, stop {stop})", mode == "two")
    assert s.status() == td.TD_OK


@pytest.mark.parametrize("kw", [dict(logit_dtype="f32"), dict(n_max=100), dict(n_max=200, topk=8),
                                dict(use_stop=True, n_max=64)])
def test_split_inside_first_kernel_variants(td, kw):
    """The two-kernel step beyond the ragged workload's own settings: float32
    logits, 4 and 8 frontier slots per lane (trees of 101 and 201 rows: 26
    and 51 row groups per KV head, most of them after the tree size
    arrives) and the S(N) stop, against the stage calls."""
    cfg = wl.CONFIGS["fused_ragged"].replace(**kw)
    print("[case] split inside kernel 1:", kw, flush=True)
    x, inp, d = inputs(cfg)
    ref = modular(td, cfg, d, None)
    tree_np = {k: ref[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
    tg = dev(targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree_np))
    ref = modular(td, cfg, d, tg)
    s = make_step(td, cfg, d)
    assert split_inside(s)
    s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"], tg)
    for rep in range(2):
        s.run()
        torch.cuda.synchronize()
        assert_same(ref, step_outputs(s), f"{kw} call {rep}", exact_out=False)
    assert s.status() == td.TD_OK


def test_split_inside_first_kernel_ragged_against_oracle(td):
    """Four sequences of ragged short contexts, one of them empty, through
    the two-kernel step: trees, attention and acceptance against the oracle."""
    cfg = wl.CONFIGS["fused_ragged"]
    print("[case] split inside kernel 1: ragged vs oracle", flush=True)
    x, inp, d = inputs(cfg)
    off = inp["ctx_offsets"].copy()
    off[3] = off[2]                      # sequence 2 has no context
    inp = dict(inp, ctx_offsets=off)
    d = dict(d, off=dev(off), maxc=int(np.diff(off).max()))
    ids, lq, _ = oracle.draft_topk(x, cfg.topk)
    tr = oracle.build_tree(ids, lq, cfg.n_max, cfg.use_stop, cost_of(cfg), cfg.l_ar, cfg.ahat0)
    tg_np = wl.target_tokens(cfg, wl.logits_as_f64(x, "bf16"), tr["node_token"], tr["node_parent"],
                             tr["n_nodes"])
    s = make_step(td, cfg, d)
    assert split_inside(s)
    s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"],
                 dev(tg_np))
    m = oracle.tree_mask(tr["node_parent"], tr["n_nodes"])
    want = oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], off, inp["k_tree"], inp["v_tree"],
                            m, tr["n_nodes"], cfg.hq, cfg.hkv, cfg.head_dim, wl.attn_scale(cfg))
    a_o, p_o, b_o = oracle.accept(tr["node_token"], tr["node_parent"], tr["n_nodes"], tg_np, cfg.block)
    for rep in range(2):
        s.run()
        torch.cuda.synchronize()
        out = step_outputs(s)
        for k in ("n_nodes", "node_token", "node_parent", "node_depth"):
            np.testing.assert_array_equal(out[k].numpy(), tr[k])
        np.testing.assert_array_equal(out["mask"].numpy().view(np.uint64), m)
        got = wl.bf16_bits_to_f32(out["out"].view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
        attn_close(got, want, "bf16", f"ragged attention call {rep}", tr["n_nodes"])
        np.testing.assert_array_equal(out["accept_len"].numpy(), a_o)
        np.testing.assert_array_equal(out["accept_path"].numpy(), p_o)
        np.testing.assert_array_equal(out["bonus_token"].numpy(), b_o)
    assert s.status() == td.TD_OK


@pytest.mark.parametrize("name", ["qwen3_8b_stress", "two_seq_k4"])
def test_step_graph_replays(td, name):
    """Steps captured in a HIP graph (input sets A, B, A), replayed several
    times with eager steps on set B between the replays: every replay and
    every eager call gives the stage calls' results (the hand-off words and,
    in the two-kernel form, the tree-size words are left ready by each call
    for the next, captured or not)."""
    from tree_draft_build_amd.binding import StepArgs
    cfg_a = wl.CONFIGS[name]
    cfg_b = cfg_a.replace(index=cfg_a.index + 40)
    print("[case] step graph replays", name, flush=True)
    sets = []
    for cfg in (cfg_a, cfg_b):
        x, inp, d = inputs(cfg)
        r = modular(td, cfg, d, None)
        tree_np = {k: r[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
        tg = dev(targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree_np))
        sets.append((d, tg, modular(td, cfg, d, tg)))
    (da, _, _), (db, _, _) = sets
    assert da["total"] == db["total"]
    s = make_step(td, cfg_a, da)
    exact = not split_inside(s)
    args = []
    for d, tg, _ in sets:
        s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"], tg)
        args.append(StepArgs.from_buffer_copy(s.args))
    keep = [sets[0][0], sets[1][0]]  # the graph reads these buffers
    s.args = StepArgs.from_buffer_copy(args[0])
    s.run()                       # outside the capture first: the workspace is in use
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in (0, 1, 0):
            s.args = StepArgs.from_buffer_copy(args[j])
            s.run()
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert_same(sets[0][2], step_outputs(s), f"{name} replay {rep}", exact)
        s.args = StepArgs.from_buffer_copy(args[1])
        s.run()                   # eager work between replays
        torch.cuda.synchronize()
        assert_same(sets[1][2], step_outputs(s), f"{name} eager after replay {rep}", exact)
    assert s.status() == td.TD_OK
    del keep


def _scramble_epochs(ws, nbytes):
    """Every 8-byte word of the first nbytes (past the 16-byte status header)
    set to its own index: the workgroups' epoch words then all differ, so no
    waiter ever sees the tag it polls for, and every bounded wait gives up.
    Only the library's own polls read these words; no kernel indexes with
    them."""
    n8 = nbytes // 8
    pat = torch.arange(n8, dtype=torch.int64, device=ws.device)
    pat[:2] = 0                                     # the status header stays clear
    ws[:n8 * 8].view(torch.int64).copy_(pat)


def test_handoff_give_up_is_reported(td):
    """A workspace that was not zero-filled (its epoch words disagree) makes
    the kernels' bounded waits give up: the row mergers write lse = NaN and
    the tree builders n_nodes = -1, td_workspace_status reports TD_ESYNC once
    and clears the word, and after re-zeroing the results are right again."""
    print("[case] hand-off give-up", flush=True)
    # stand-alone top-K: 2 rows of 64 slices each
    x = wl.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((1, 2, 65536)).astype(np.float32))
    lg = dev(x)
    ws = td.draft_topk_alloc_workspace(1, 2, 65536, 8, DEV)
    ids0, lq0, lse0 = [t.clone() for t in td.draft_topk(lg, 8, workspace=ws)]
    assert td.workspace_status(ws) == td.TD_OK
    _scramble_epochs(ws, td.draft_topk_workspace(1, 2, 65536, 8))
    _, _, lse = td.draft_topk(lg, 8, workspace=ws)
    assert td.workspace_status(ws) == td.TD_ESYNC
    assert "row merge" in td.last_error()
    assert torch.isnan(lse).all()
    assert td.workspace_status(ws) == td.TD_OK      # the check cleared the word
    ws.zero_()
    ids, lq, lse = td.draft_topk(lg, 8, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids0) and torch.equal(lq, lq0) and torch.equal(lse, lse0)
    assert td.workspace_status(ws) == td.TD_OK

    # the fused step at the Qwen3-8B stress shape
    cfg = wl.CONFIGS["qwen3_8b_stress"]
    xs, inp, d = inputs(cfg)
    ref = modular(td, cfg, d, None)
    tree_np = {k: ref[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
    tg = dev(targets_by_path(cfg, wl.logits_as_f64(xs, cfg.logit_dtype), tree_np))
    ref = modular(td, cfg, d, tg)
    s = make_step(td, cfg, d)
    s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"], tg)
    s.run()
    assert s.status() == td.TD_OK
    assert_same(ref, step_outputs(s), "before scrambling", not split_inside(s))
    _scramble_epochs(s.workspace, td.draft_topk_workspace(cfg.batch, cfg.block, cfg.vocab, cfg.topk))
    s.run()
    assert s.status() == td.TD_ESYNC
    err = td.last_error()
    assert "row merge" in err and "tree build" in err
    got = step_outputs(s)
    assert int(got["n_nodes"][0]) == -1
    assert torch.isnan(got["lse"]).all()
    assert int(got["accept_len"][0]) == 0
    assert int(got["bonus_token"][0]) == int(tg[0, 0])
    # n_nodes -1: no row is a tree row, so the attention wrote none
    s.workspace.zero_()
    s.run()
    assert s.status() == td.TD_OK
    assert_same(ref, step_outputs(s), "after re-zeroing", not split_inside(s))


@pytest.mark.parametrize("name,kw", [("qwen3_8b_stress", dict(branch=3, min_logrho=-6.0)),
                                     ("batched", dict(branch=1)),
                                     ("long", dict(min_logrho=-40.0))])
def test_step_selective_equals_stage_calls(td, name, kw):
    """The fused step with a branch cap and a confidence threshold gives the
    stage calls' results with the same settings."""
    cfg = wl.CONFIGS[name]
    print("[case] step selective", name, kw, flush=True)
    x, inp, d = inputs(cfg)
    ref = modular(td, cfg, d, None, **kw)
    tree_np = {k: ref[k].numpy() for k in ("node_token", "node_parent", "n_nodes")}
    tg = dev(targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree_np))
    ref = modular(td, cfg, d, tg, **kw)
    s = make_step(td, cfg, d, **kw)
    s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"], d["v_tree"], tg)
    s.run()
    torch.cuda.synchronize()
    assert_same(ref, step_outputs(s), f"{name} selective", not split_inside(s))
