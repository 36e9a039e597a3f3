"""GPU: td_verify_step_noalloc (the workspace in the library's static device
scratch array) gives exactly td_verify_step's results, on two calls in a
row, the second with a smaller problem than the first."""
import ctypes

import pytest
import torch

from helpers import cost_of, targets_by_path
from tree_draft_build_amd import workload as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def td():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tree_draft_build_amd import binding
    return binding


def _dev(x):
    import numpy as np
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def _step(td, cfg, total, maxc):
    return td.VerifyStep(batch=cfg.batch, block=cfg.block, vocab=cfg.vocab, topk=cfg.topk,
                         n_max=cfg.n_max, use_stop=cfg.use_stop, cost=cost_of(cfg), l_ar=cfg.l_ar,
                         ahat0=cfg.ahat0, hq=cfg.hq, hkv=cfg.hkv, head_dim=cfg.head_dim,
                         scale=wl.attn_scale(cfg),
                         logits_dtype=td.TD_BF16 if cfg.logit_dtype == "bf16" else td.TD_F32,
                         attn_dtype=td.TD_BF16 if cfg.attn_dtype == "bf16" else td.TD_F32,
                         total_ctx=total, max_ctx=maxc, device=DEV)


def _outputs(s):
    res = dict(topk_id=s.topk_id, topk_logq=s.topk_logq, lse=s.lse, mask=s.mask, out=s.out,
               accept_len=s.accept_len, accept_path=s.accept_path, bonus_token=s.bonus_token,
               **s.tree)
    res = {k: v.cpu() for k, v in res.items()}
    out = res["out"].clone()                       # rows past a tree are not written
    for b, n in enumerate(res["n_nodes"].tolist()):
        out[b, n + 1:] = 0
    res["out"] = out
    return res


@pytest.mark.parametrize("first,second", [("qwen3_8b_stress", "tiny"), ("batched", "two_seq_k4")])
def test_noalloc_matches_workspace_step(td, first, second):
    for name in (first, second):
        cfg = wl.CONFIGS[name]
        print("[case] noalloc", name, flush=True)
        x = wl.make_logits(cfg)
        inp = wl.make_attn_inputs(cfg)
        d = dict(logits=_dev(x), q=_dev(inp["q"]), k_ctx=_dev(inp["k_ctx"]),
                 v_ctx=_dev(inp["v_ctx"]), k_tree=_dev(inp["k_tree"]), v_tree=_dev(inp["v_tree"]),
                 off=_dev(inp["ctx_offsets"]))
        total, maxc = int(inp["ctx_offsets"][-1]), int(inp["ctx_len"].max())
        ref = _step(td, cfg, total, maxc)
        tg0 = torch.full((cfg.batch, cfg.nq_max), -1, dtype=torch.int32, device=DEV)
        ref.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"],
                       d["v_tree"], tg0)
        ref.run()
        torch.cuda.synchronize()
        tree_np = {k: ref.tree[k].cpu().numpy() for k in ("node_token", "node_parent", "n_nodes")}
        tg = _dev(targets_by_path(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tree_np))
        ref.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"],
                       d["v_tree"], tg)
        ref.run()
        torch.cuda.synchronize()
        want = _outputs(ref)
        got_s = _step(td, cfg, total, maxc)          # only its output buffers are used
        got_s.set_inputs(d["logits"], d["q"], d["k_ctx"], d["v_ctx"], d["off"], d["k_tree"],
                         d["v_tree"], tg)
        got_s.args.stages = 0
        st = td.lib.td_verify_step_noalloc(ctypes.byref(got_s.args), td._stream())
        assert st == td.TD_OK, td.last_error()
        torch.cuda.synchronize()
        got = _outputs(got_s)
        for k in want:
            assert torch.equal(want[k], got[k]), f"{name}: {k} differs from td_verify_step"
