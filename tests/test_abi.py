"""The C-ABI library on the host: it loads, exports every function declared
in include/treedraft.h, and its argument validation rejects bad calls before
any GPU work is enqueued (no GPU needed: validation runs first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "treedraft.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(td_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def b():
    from tree_draft_build_amd import binding
    return binding


def test_every_declared_symbol_is_exported(b):
    names = declared_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(b.lib, n), n
    assert sorted(b.EXPORTED) == names


def test_abi_version(b):
    assert b.lib.td_abi_version() == 2


def test_workspace_status_validation(b):
    assert b.lib.td_workspace_status(None, 1 << 20, None) == 1
    assert b.lib.td_workspace_status(P(4097), 1 << 20, None) == 1
    assert b.lib.td_workspace_status(P(4096), 8, None) == 1
    assert "status" in b.last_error()


def test_workspace_queries(b):
    assert b.draft_topk_workspace(1, 16, 151936, 8) > 0
    assert b.draft_topk_workspace(0, 16, 151936, 8) == 0
    w1 = b.tree_verify_attn_workspace(1, 65, 32, 8, 128, 4096, 4096)
    w2 = b.tree_verify_attn_workspace(1, 65, 32, 8, 128, 8192, 8192)
    assert 0 < w1 <= w2
    assert b.tree_verify_attn_workspace(1, 65, 32, 7, 128, 4096, 4096) == 0  # hq % hkv


P = ctypes.c_void_p
FAKE = P(4096)          # never dereferenced: validation fails before any launch
FAKE8 = P(4096 + 8)     # 8-byte but not 16-byte aligned


@pytest.mark.parametrize("args,status,needle", [
    ((None, 1, 1, 16, 1000, 1000, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 1, "null"),
    ((FAKE, 1, 1, 16, 1000, 1000, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 1, "positive"),
    ((FAKE, 1, 1, 16, 1000, 1000, 33, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 2, "TD_MAX_TOPK"),
    ((FAKE, 1, 1, 16, 4, 4, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 1, "exceeds"),
    ((FAKE, 1, 1, 33, 1000, 1000, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 2, "block"),
    ((FAKE, 7, 1, 16, 1000, 1000, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 3, "dtype"),
    ((FAKE, 1, 1, 16, 1000, 999, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 1, "pos_stride"),
    ((P(4097), 1, 1, 16, 1000, 1000, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 1, "element"),
    ((P(4098), 0, 1, 16, 1000, 1000, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), 1, "element"),
    ((FAKE, 1, 1, 16, 1000, 1000, 8, FAKE, FAKE, FAKE, FAKE, 16, None), 1, "workspace"),
])
def test_draft_topk_validation(b, args, status, needle):
    assert b.lib.td_draft_topk(*args) == status
    assert needle in b.last_error()


def test_build_tree_validation(b):
    base = [FAKE, FAKE, 1, 16, 8, 64, 1, 1.0, 0.005, 0.03, 32, 1.0, 1.0, 0, -1e300, None, FAKE, FAKE,
            FAKE, FAKE, FAKE, None, None, None]
    bad = list(base); bad[5] = 256
    assert b.lib.td_build_tree(*bad) == 2 and "capacity" in b.last_error()
    bad = list(base); bad[0] = None
    assert b.lib.td_build_tree(*bad) == 1
    bad = list(base); bad[5] = -1
    assert b.lib.td_build_tree(*bad) == 1


def test_flex_budget_matches_oracle(b):
    import oracle
    for batch in (1, 7, 8, 64):
        for switch in (0, 8, 16):
            for n_max in (4, 64):
                assert b.flex_budget(batch, switch, 8, n_max, 16) == \
                    oracle.flex_budget(batch, switch, 8, n_max, 16)


def test_mask_accept_validation(b):
    assert b.lib.td_tree_mask(FAKE, FAKE, 1, 257, FAKE, None) == 2
    assert b.lib.td_tree_mask(FAKE, FAKE, 1, 65, P(4097), None) == 1     # misaligned mask
    assert b.lib.td_accept(FAKE, FAKE, FAKE, None, 1, 64, 16, FAKE, FAKE, FAKE, None) == 1
    assert b.lib.td_accept(FAKE, FAKE, FAKE, FAKE, 1, 64, 33, FAKE, FAKE, FAKE, None) == 2


def test_attention_validation(b):
    ws = b.tree_verify_attn_workspace(1, 65, 32, 8, 128, 4096, 4096)
    base = [FAKE, FAKE, FAKE, FAKE, None, 4096, 4096, FAKE, FAKE, FAKE, FAKE, 1, 65, 32, 8, 128,
            0.088, 1, FAKE, FAKE, ws, None]
    bad = list(base); bad[14] = 7
    assert b.lib.td_tree_verify_attn(*bad) == 1 and "multiple" in b.last_error()
    bad = list(base); bad[15] = 96
    assert b.lib.td_tree_verify_attn(*bad) == 3
    bad = list(base); bad[20] = ws - 1
    assert b.lib.td_tree_verify_attn(*bad) == 1 and "workspace" in b.last_error()
    bad = list(base); bad[0] = FAKE8
    assert b.lib.td_tree_verify_attn(*bad) == 1
    bad = list(base); bad[12] = 257
    assert b.lib.td_tree_verify_attn(*bad) == 2
    bad = list(base); bad[4] = P(4096 + 4)          # misaligned context lengths
    assert b.lib.td_tree_verify_attn(*bad) == 1


def test_kv_commit_validation(b):
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 65, 16, 8, 128, 1, FAKE, FAKE, FAKE, FAKE, None, None]
    bad = list(base); bad[0] = None
    assert b.lib.td_kv_commit(*bad) == 1 and "null" in b.last_error()
    bad = list(base); bad[9] = 96
    assert b.lib.td_kv_commit(*bad) == 3
    bad = list(base); bad[7] = 33
    assert b.lib.td_kv_commit(*bad) == 2
    bad = list(base); bad[11] = FAKE8
    assert b.lib.td_kv_commit(*bad) == 1 and "misaligned" in b.last_error()


def test_step_args_layout_and_validation(b):
    assert b.lib.td_step_args_bytes() == ctypes.sizeof(b.StepArgs)
    a = b.StepArgs()
    assert b.lib.td_verify_step(None, FAKE, 1 << 20, None) == 1
    assert b.lib.td_verify_step(ctypes.byref(a), FAKE, 1 << 20, None) == 1   # all null
    assert b.lib.td_verify_step_workspace(ctypes.byref(a)) == 0
    a.batch, a.block, a.vocab, a.pos_stride, a.topk = 1, 16, 151936, 151936, 8
    a.n_max, a.hq, a.hkv, a.head_dim, a.total_ctx, a.max_ctx = 64, 32, 8, 128, 4096, 4096
    assert b.lib.td_verify_step_workspace(ctypes.byref(a)) > 0
    for f in ("logits", "q", "k_ctx", "v_ctx", "ctx_offsets", "k_tree", "v_tree", "target_token",
              "topk_id", "topk_logq", "lse", "n_nodes", "node_token", "node_parent", "node_depth",
              "node_logrho", "mask", "out", "accept_len", "accept_path", "bonus_token"):
        setattr(a, f, 4096)
    a.logits_dtype = a.attn_dtype = 1
    a.topk = 33
    assert b.lib.td_verify_step(ctypes.byref(a), FAKE, 1 << 30, None) == 2
    a.topk = 8
    a.n_max = 300
    assert b.lib.td_verify_step(ctypes.byref(a), FAKE, 1 << 30, None) == 2
    a.n_max = 64
    a.hkv = 7
    assert b.lib.td_verify_step(ctypes.byref(a), FAKE, 1 << 30, None) == 1
    a.hkv = 8
    assert b.lib.td_verify_step(ctypes.byref(a), FAKE, 16, None) == 1
    assert "workspace" in b.last_error()
    a.stages = 4
    assert b.lib.td_verify_step(ctypes.byref(a), FAKE, 1 << 30, None) == 1
    assert "stages" in b.last_error()
    # a verify-only call checks only the attention and acceptance fields
    a.stages = b.TD_STEP_VERIFY
    a.topk = 33
    a.hkv = 7
    assert b.lib.td_verify_step(ctypes.byref(a), FAKE, 1 << 30, None) == 1
    assert "hkv" in b.last_error() or "hq" in b.last_error()
    a.hkv = 8
    a.stages = b.TD_STEP_DRAFT
    assert b.lib.td_verify_step(ctypes.byref(a), FAKE, 1 << 30, None) == 2
    # the allocation-free variant validates the same way before anything else
    assert b.lib.td_verify_step_noalloc(ctypes.byref(a), None) == 2
    assert b.lib.td_verify_step_noalloc(None, None) == 1
    a.topk = 8
    a.stages = 0
    a.batch, a.total_ctx, a.max_ctx = 64, 64 * 32768, 32768
    assert b.lib.td_verify_step_noalloc(ctypes.byref(a), None) == 2
    assert "64 MiB" in b.last_error()


@pytest.mark.parametrize("seed", range(6))
def test_fit_cost_matches_oracle(b, seed):
    """The library's fit (normal equations) against the oracle's (library
    least squares per knee) on noisy piecewise-linear measurements."""
    import numpy as np
    from oracle.fit import fit_cost
    rng = np.random.default_rng(seed)
    n = np.repeat(np.array([0, 1, 2, 4, 8, 16, 24, 32, 48, 64, 80, 96, 128], float), 3)
    knee = int(rng.integers(8, 100))
    t = 50 + rng.uniform(0, 0.2) * n + rng.uniform(0.5, 3) * np.maximum(0, n - knee)
    t = t + rng.normal(0, 0.05, len(t))
    got = b.fit_cost(n, t, 0, 128)
    want = fit_cost(n, t, 0, 128)
    assert got[3] == want[3]
    for g, w in zip(got[:3], want[:3]):
        assert g == pytest.approx(w, rel=1e-7, abs=1e-9)
    assert got[4] == pytest.approx(want[4], rel=1e-7)


def test_fit_cost_validation(b):
    import numpy as np
    with pytest.raises(b.TreedraftError):
        b.fit_cost(np.array([1.0, 2.0]), np.array([1.0, 2.0]), 0, 4)
    with pytest.raises(b.TreedraftError):
        b.fit_cost(np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.0, 3.0]), 5, 4)


def test_step_kernel_count(b):
    """td_verify_step_kernels: the context split joins the first kernel for
    short bf16 contexts at head dim 128 with topk <= 8 and few top-K
    workgroups, and only when both stages run (host-side fields only)."""
    a = b.StepArgs()
    assert b.lib.td_verify_step_kernels(None) == 0
    assert b.lib.td_verify_step_kernels(ctypes.byref(a)) == 0  # no shape
    a.batch, a.block, a.vocab, a.pos_stride, a.topk = 1, 16, 151936, 151936, 8
    a.n_max, a.hq, a.hkv, a.head_dim, a.total_ctx, a.max_ctx = 64, 32, 8, 128, 4096, 4096
    a.logits_dtype = a.attn_dtype = b.TD_BF16
    assert b.lib.td_verify_step_kernels(ctypes.byref(a)) == 2
    a.stages = b.TD_STEP_DRAFT
    assert b.lib.td_verify_step_kernels(ctypes.byref(a)) == 1
    a.stages = b.TD_STEP_VERIFY
    assert b.lib.td_verify_step_kernels(ctypes.byref(a)) == 2
    a.stages = 4
    assert b.lib.td_verify_step_kernels(ctypes.byref(a)) == 0
    a.stages = 0
    for field, value in (("total_ctx", 16384), ("batch", 64), ("topk", 16), ("head_dim", 64),
                         ("attn_dtype", b.TD_F32)):
        old = getattr(a, field)
        setattr(a, field, value)
        if field == "batch":
            a.total_ctx = 64 * 4096
        assert b.lib.td_verify_step_kernels(ctypes.byref(a)) == 3, field
        setattr(a, field, old)
        a.total_ctx = 4096
    a.logits_dtype = b.TD_F32  # the logits' type does not matter
    assert b.lib.td_verify_step_kernels(ctypes.byref(a)) == 2
    a.total_ctx = a.max_ctx = 8192  # 128-key chunks up to about 512 work items
    assert b.lib.td_verify_step_kernels(ctypes.byref(a)) == 2


def test_step_kernel_events_validation(b):
    a = b.StepArgs()
    a.batch, a.block, a.vocab, a.pos_stride, a.topk = 1, 16, 151936, 151936, 8
    a.n_max, a.hq, a.hkv, a.head_dim, a.total_ctx, a.max_ctx = 64, 32, 8, 128, 4096, 4096
    a.logits_dtype = a.attn_dtype = b.TD_BF16
    for first, last in ((-1, 0), (1, 0), (0, 2), (2, 2)):
        assert b.lib.td_verify_step_kernel_events(ctypes.byref(a), FAKE, 1 << 30, None, first, last,
                                                  None, None) == 1
        assert "kernel range" in b.last_error()
