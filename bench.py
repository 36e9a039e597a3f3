"""Verify-step throughput of the MI355X path on a synthetic workload.

One step = the whole verify-side path over one batch:
  draft_topk -> build_tree (S(N) stop) -> tree_mask -> tree_verify_attn -> accept
with every input already resident in HBM.  Inputs are rotated over enough
distinct device copies (>= --rotate-mb in total) that the 256 MB Infinity
Cache cannot serve a step from the previous one.

Prints one JSON line (rank 0, one GPU):
  value        verify steps per second over the K timed steps
  roofline     the dominant launch unit's algorithmic bytes (or flops) / its
               average duration, measured with HIP events attached to the
               kernels' own dispatch inside whole steps
               (td_verify_step_kernel_events) over K steps.  Units: kernel 1
               (top-K + tree + mask, plus the context split where it runs
               there) and the rest of the step
  tree_row     the same shape with the tree fixed at N = 64 (65 query rows)
  streaming    64 independent sequences of the headline shape per step
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload,
               on all host cores (and on one thread)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_TFLOPS = 2500.0      # dense bf16 MFMA, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3_8b")
    ap.add_argument("--rotate-mb", type=float, default=1024.0)
    ap.add_argument("--no-graph", action="store_true", help="launch every step eagerly")
    ap.add_argument("--graph-steps", type=int, default=8, help="steps captured per HIP graph")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run plain copies of MIB MiB (profiler byte-counter reference)")
    ap.add_argument("--no-streaming", dest="streaming", action="store_false",
                    help="skip the 64-sequence streaming measurement")
    ap.add_argument("--no-tree-row", dest="tree_row", action="store_false",
                    help="skip the full-tree (N = 64 fixed) measurement")
    ap.add_argument("--no-decode", dest="decode", action="store_false",
                    help="skip the multi-step decode loop with KV commit")
    ap.add_argument("--no-layer", dest="layer", action="store_false",
                    help="skip the one-layer verification pass and the tachometer")
    ap.add_argument("--no-tachometer", dest="tachometer", action="store_false",
                    help="with the one-layer pass, skip the tachometer's sweep over tree sizes")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the all-core oracle baseline (0: every core available)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the verify step runs on one GPU; --gpus {args.gpus} is not supported "
              "(it would shard by sequence, with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from tree_draft_build_amd import workload as wl

    torch.cuda.set_device(torch.device("cuda:0"))
    if args.calibrate_copy:
        copy_calibration(args.calibrate_copy)
        return
    cfg = wl.CONFIGS[args.config]
    result, x, inp = measure(cfg, args, args.steps, args.warmup)
    if args.tree_row and cfg.name == "qwen3_8b":
        # the same shape with a full tree (N = 64 fixed, 65 query rows)
        tcfg = wl.CONFIGS["qwen3_8b_tree"]
        tres, _, _ = measure(tcfg, args, max(10, args.steps // 2), max(2, args.warmup // 2))
        result["tree_row"] = {
            "workload": tcfg.name, "n_nodes": tres["config"]["n_nodes"][:1],
            "value": tres["value"], "unit": "verify steps/s", "ms_per_step": tres["ms_per_step"],
            "steps": tres["steps"], "kernels_us": tres["kernels_us"],
            "kernel_roofline": tres["kernel_roofline"]}
    if args.layer and cfg.name == "qwen3_8b":
        # the one-layer verification pass (Q/K/V + RoPE, attention, LM-head
        # argmax) at the Qwen3-8B shape, and the tachometer fitted to it
        result.update(layer_rows(args))
    if args.decode and cfg.name == "qwen3_8b":
        # the step in a decode loop: the accepted path's K/V committed into
        # the context after each step, the bonus token as the next root
        result["decode"] = decode_row(wl.CONFIGS["qwen3_8b_stress"], args,
                                      max(16, args.steps // 2), max(8, args.warmup))
    if args.streaming and cfg.name == "qwen3_8b":
        # the same per-sequence work, 64 independent sequences per step
        scfg = wl.CONFIGS["qwen3_8b_x64"]
        sres, _, _ = measure(scfg, args, max(10, args.steps // 4), max(2, args.warmup // 4))
        result["streaming"] = {
            "workload": scfg.name, "batch": scfg.batch,
            "value": sres["value"], "unit": "verify steps/s",
            "sequence_steps_per_s": round(sres["value"] * scfg.batch, 1),
            "ms_per_step": sres["ms_per_step"], "steps": sres["steps"],
            "kernels_us": sres["kernels_us"], "roofline": sres["roofline"],
            "stage_roofline": sres["stage_roofline"]}
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg, x, inp, args.cpu_seconds, args.cpu_threads)
    print(json.dumps(result), flush=True)


def measure(cfg, args, steps, warmup):
    import torch

    from tree_draft_build_amd import binding as td
    from tree_draft_build_amd import workload as wl

    dev = torch.device("cuda:0")

    # ---------------- inputs (host generation, one upload, device copies) ----
    x = wl.make_logits(cfg)
    inp = wl.make_attn_inputs(cfg)
    tdt = torch.bfloat16 if cfg.attn_dtype == "bf16" else torch.float32

    def up(a, dtype):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev).to(dtype) if dtype is not None else torch.from_numpy(a).to(dev)

    base = dict(logits=up(x, None), q=up(inp["q"], tdt), k_ctx=up(inp["k_ctx"], tdt),
                v_ctx=up(inp["v_ctx"], tdt), k_tree=up(inp["k_tree"], tdt),
                v_tree=up(inp["v_tree"], tdt))
    off = torch.from_numpy(inp["ctx_offsets"]).to(dev)
    total_ctx = int(inp["ctx_offsets"][-1])
    max_ctx = int(inp["ctx_len"].max())
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    n_sets = max(1, int(math.ceil(args.rotate_mb * 1e6 / set_bytes)))
    if n_sets == 1 and set_bytes < 4 * 256e6:
        n_sets = 2
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_sets - 1)]

    b, B, K, V = cfg.batch, cfg.block, cfg.topk, cfg.vocab
    cost = (cfg.cost_a, cfg.cost_b, cfg.cost_c, cfg.cost_knee)
    scale = wl.attn_scale(cfg)

    # ---------------- stage calls: outputs and workspaces (allocated once) ----
    topk_out = (torch.empty((b, B, K), dtype=torch.int32, device=dev),
                torch.empty((b, B, K), dtype=torch.float64, device=dev),
                torch.empty((b, B), dtype=torch.float64, device=dev))
    ws_topk = td.draft_topk_alloc_workspace(b, B, V, K, dev)
    tree = td.alloc_tree(b, cfg.n_max, dev)
    nq = cfg.nq_max
    mask = torch.empty((b, nq, (nq + 63) // 64), dtype=torch.int64, device=dev)
    attn_out = torch.empty((b, nq, cfg.hq, cfg.head_dim), dtype=tdt, device=dev)
    ws_attn = td.tree_verify_attn_alloc_workspace(b, nq, cfg.hq, cfg.hkv, cfg.head_dim, total_ctx,
                                                  max_ctx, dev)
    acc_out = (torch.empty(b, dtype=torch.int32, device=dev),
               torch.empty((b, B + 1), dtype=torch.int32, device=dev),
               torch.empty(b, dtype=torch.int32, device=dev))
    target = torch.full((b, nq), -1, dtype=torch.int32, device=dev)

    def stage_a(s):
        td.draft_topk(s["logits"], K, out=topk_out, workspace=ws_topk)

    def stage_b():
        td.build_tree(topk_out[0], topk_out[1], cfg.n_max, cfg.use_stop, cost, cfg.l_ar, cfg.ahat0,
                      out=tree)
        td.tree_mask(tree["node_parent"], tree["n_nodes"], out=mask)

    def stage_c(s):
        td.tree_verify_attn(s["q"], s["k_ctx"], s["v_ctx"], off, total_ctx, max_ctx, s["k_tree"],
                            s["v_tree"], mask, tree["n_nodes"], scale, out=attn_out,
                            workspace=ws_attn)

    def stage_d():
        td.accept(tree["node_token"], tree["node_parent"], tree["n_nodes"], target, B, out=acc_out)

    def step(i):
        s = sets[i % n_sets]
        stage_a(s)
        stage_b()
        stage_c(s)
        stage_d()

    # The tree is a deterministic function of the logits: build it once,
    # untimed, and give the acceptance stage the synthetic target's tokens.
    step(0)
    torch.cuda.synchronize()
    tnp = {k: v.cpu().numpy() for k, v in tree.items()}
    tg = wl.target_tokens(cfg, wl.logits_as_f64(x, cfg.logit_dtype), tnp["node_token"],
                          tnp["node_parent"], tnp["n_nodes"])
    target.copy_(torch.from_numpy(tg))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    # ---------------- the timed step: td_verify_step (3 kernels) ----------------
    vs = td.VerifyStep(batch=b, block=B, vocab=V, topk=K, n_max=cfg.n_max, use_stop=cfg.use_stop,
                       cost=cost, l_ar=cfg.l_ar, ahat0=cfg.ahat0, hq=cfg.hq, hkv=cfg.hkv,
                       head_dim=cfg.head_dim, scale=scale,
                       logits_dtype=td.TD_BF16 if cfg.logit_dtype == "bf16" else td.TD_F32,
                       attn_dtype=td.TD_BF16 if cfg.attn_dtype == "bf16" else td.TD_F32,
                       total_ctx=total_ctx, max_ctx=max_ctx, device=dev)
    args_per_set = []
    for st_ in sets:
        vs.set_inputs(st_["logits"], st_["q"], st_["k_ctx"], st_["v_ctx"], off, st_["k_tree"],
                      st_["v_tree"], target)
        args_per_set.append(td.StepArgs.from_buffer_copy(vs.args))
    use_graph = not args.no_graph

    def fused(i, stages=0):
        vs.args = args_per_set[i % n_sets]
        vs.run(stages=stages)

    # HIP graphs of G consecutive steps (cycling the input sets) so that the
    # host's launch cost is paid once per G steps; single-step graphs cover
    # the remainder, so a timed region runs exactly the steps it names
    G = max(1, min(args.graph_steps, n_sets))

    def make_runner(stages):
        multi, single = [], []
        if use_graph:
            for i in range(0, n_sets - G + 1, G):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for j in range(G):
                        fused(i + j, stages)
                multi.append(g)
            for i in range(n_sets):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fused(i, stages)
                single.append(g)
            torch.cuda.synchronize()

        def run_steps(first, count):
            """Steps first .. first+count-1 (input set = step index mod n_sets)."""
            i = first
            end = first + count
            while i < end:
                k = i % n_sets
                if use_graph and k % G == 0 and k // G < len(multi) and i + G <= end:
                    multi[k // G].replay()
                    i += G
                elif use_graph:
                    single[k].replay()
                    i += 1
                else:
                    fused(i, stages)
                    i += 1
        return run_steps

    def timed(run_steps, count):
        run_steps(0, warmup)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        run_steps(warmup, count)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / count

    # ---------------- timed region: whole steps ----------------
    ms_per_step = timed(make_runner(0), steps)
    # the step's results equal the stage calls' (checked by the test-suite);
    # keep one cheap guard here that the timed path ran
    assert int(vs.tree["n_nodes"][0]) == int(tnp["n_nodes"][0])

    # ---------------- the step's kernels, timed apart ----------------
    # Two launch units.  With the context split inside the first kernel
    # (short contexts, few top-K workgroups) the step runs two kernels:
    # kernel 1 (top-K + tree + mask + context split) and kernel 2 (combine +
    # accept); otherwise three: kernel 1 (top-K + tree + mask) and kernels
    # 2-3 (split + combine + accept).  Each unit is timed inside whole steps:
    #  - duration: HIP events attached to the unit's first and last kernels'
    #    own dispatch (td_verify_step_kernel_events), one pair per step,
    #    averaged: the kernels' execution time as a kernel-trace profiler
    #    reports it;
    #  - loop (three-kernel steps only): graph replays of back-to-back
    #    launches of the unit's stage between two events on the launch
    #    stream, divided by the count (includes the launch gaps).
    n_kernels = vs.kernels()
    fused_split = n_kernels == 2

    def kernel_ms(first, last, count):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(count)]
        for a, b_ in evs:            # create the HIP events behind them
            a.record(stream)
            b_.record(stream)
        for i in range(warmup):
            fused(i)
        torch.cuda.synchronize()
        for i, (a, b_) in enumerate(evs):
            vs.args = args_per_set[(warmup + i) % n_sets]
            vs.run_kernels_timed(first, last, a, b_)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b_) for a, b_ in evs]))

    k1_ms = kernel_ms(0, 0, steps)
    k23_ms = kernel_ms(1, n_kernels - 1, steps)
    if fused_split:
        k1_loop_ms = k23_loop_ms = None
    else:
        k1_loop_ms = timed(make_runner(td.TD_STEP_DRAFT), steps)
        k23_loop_ms = timed(make_runner(td.TD_STEP_VERIFY), steps)

    # ---------------- per-stage calls (HIP events, eager) ----------------
    names = ["draft_topk", "build_tree+tree_mask", "tree_verify_attn", "accept"]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in names] for _ in range(steps)]
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    for i in range(steps):
        s = sets[i % n_sets]
        e = ev[i]
        e[0][0].record(stream); stage_a(s); e[0][1].record(stream)
        e[1][0].record(stream); stage_b(); e[1][1].record(stream)
        e[2][0].record(stream); stage_c(s); e[2][1].record(stream)
        e[3][0].record(stream); stage_d(); e[3][1].record(stream)
    torch.cuda.synchronize()
    stage_ms = [float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)]))
                for j in range(len(names))]

    # ---------------- algorithmic work ----------------
    nn = tnp["n_nodes"].astype(np.int64)
    rows = nn + 1
    W = (nq + 63) // 64
    L = inp["ctx_len"].astype(np.int64)
    esz = 2 if cfg.attn_dtype == "bf16" else 4
    lsz = 2 if cfg.logit_dtype == "bf16" else 4
    # (a): logits read once; top-K ids (4 B) + log q (8 B) and lse (8 B) written
    bytes_a = b * B * V * lsz + b * B * K * 12 + b * B * 8
    # (b)+(b'): node arrays (token, parent, depth 4 B; log rho 8 B) + mask rows
    bytes_b = b * nq * (20 + 8 * W)
    # (c): K/V of context and tree read once, q read and out written once
    bytes_kv_ctx = int((2 * cfg.hkv * cfg.head_dim * esz * L).sum())
    bytes_c = int((2 * cfg.hkv * cfg.head_dim * esz * (L + rows)).sum()
                  + 2 * (rows.sum()) * cfg.hq * cfg.head_dim * esz)
    depth = tnp["node_depth"]
    anc = int(sum((depth[i, :rows[i]] + 1).sum() for i in range(b)))
    flops_ctx = int(4 * cfg.hq * cfg.head_dim * (rows * L).sum())
    flops_c = flops_ctx + int(4 * cfg.hq * cfg.head_dim * anc)
    ridge = MFMA_BF16_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)

    def roofline(kernel, ms, loop_ms, nbytes, nflops):
        gbs = nbytes / (ms * 1e-3) / 1e9
        tfs = nflops / (ms * 1e-3) / 1e12
        if nflops / nbytes > ridge:
            r = dict(bound="mfma", achieved=round(tfs, 2), peak=MFMA_BF16_TFLOPS,
                     unit="TFLOP/s", frac=round(tfs / MFMA_BF16_TFLOPS, 4), traffic=None)
        else:
            r = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                     frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None)
        r.update(kernel=kernel, bytes_per_launch=int(nbytes), flops_per_launch=int(nflops),
                 avg_launch_us=round(ms * 1e3, 2), timing="HIP events on the kernels' dispatch",
                 hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                 mfma_frac=round(tfs / MFMA_BF16_TFLOPS, 5) if nflops else None,
                 loop_us_per_launch=None if loop_ms is None else round(loop_ms * 1e3, 2))
        return r

    if fused_split:
        # kernel 1 also reads the context K/V; kernel 2 the tree K/V, q and out
        u1, u2 = "draft+split", "combine+accept"
        k1 = roofline("draft+split (kernel 1: top-K + tree + mask + context split)", k1_ms, k1_loop_ms,
                      bytes_a + bytes_b + bytes_kv_ctx, flops_ctx)
        k23 = roofline("combine + acceptance (kernel 2)", k23_ms, k23_loop_ms,
                       bytes_c - bytes_kv_ctx, flops_c - flops_ctx)
    else:
        u1, u2 = "topk_tree", "attention+accept"
        k1 = roofline("topk_tree (kernel 1: top-K + tree + mask)", k1_ms, k1_loop_ms,
                      bytes_a + bytes_b, 0)
        k23 = roofline("attention + acceptance (kernels 2-3)", k23_ms, k23_loop_ms, bytes_c, flops_c)
    measured = hbm_traffic(cfg.name)
    if measured:
        k1["traffic"] = measured.get(u1)
        k23["traffic"] = measured.get(u2)
    roof = k1 if k1_ms >= k23_ms else k23

    result = {
        "metric": "verify steps/s (logits->tree->tree-attn->accept) + % HBM/MFMA peak, "
                  "Qwen3-8B shape" if cfg.name == "qwen3_8b" else f"verify steps/s ({cfg.name})",
        "value": round(1e3 / ms_per_step, 1),
        "unit": "verify steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.logit_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": b, "block": B, "vocab": V, "topk": K,
                   "n_max": cfg.n_max, "stop": "S(N)" if cfg.use_stop else "fixed",
                   "hq": cfg.hq, "hkv": cfg.hkv, "head_dim": cfg.head_dim,
                   "ctx_total": total_ctx, "n_nodes": [int(v) for v in nn[:8]],
                   "step": f"td_verify_step ({n_kernels} kernels)", "graph": use_graph, "graph_steps": G,
                   "input_sets": n_sets, "parallelism": "single GPU"},
        "roofline": roof,
        "kernels_us": {u1: round(k1_ms * 1e3, 2), u2: round(k23_ms * 1e3, 2)},
        "kernel_roofline": {u1: k1, u2: k23},
        "stages_us": {n: round(t * 1e3, 2) for n, t in zip(names, stage_ms)},
        "stage_roofline": {
            "draft_topk": {"bytes": bytes_a, "GB/s": round(bytes_a / (stage_ms[0] * 1e-3) / 1e9, 1)},
            "tree_verify_attn": {"bytes": bytes_c, "flops": flops_c,
                                 "GB/s": round(bytes_c / (stage_ms[2] * 1e-3) / 1e9, 1),
                                 "TFLOP/s": round(flops_c / (stage_ms[2] * 1e-3) / 1e12, 3)}},
    }
    return result, x, inp


def layer_rows(args):
    """The one-layer verification pass at the Qwen3-8B shape (hidden 4096,
    32/8 heads of 128, vocabulary 151936, random bf16 weights) on a 64-node
    tree over a 4096-token context:
      verify_layer  per call: td_tree_qkv (the 6144 x 4096 projection streams
                    50 MB of weights) and td_lm_head_argmax (151936 x 4096:
                    1.24 GB), each against the HBM roofline, and the whole
                    step (draft kernel, Q/K/V, attention, LM head, acceptance)
                    in a graph;
      tachometer    the pass timed over tree sizes 0 .. 255 and the fit of
                    C(N) = a + b N + c max(0, N - knee); with the fitted cost
                    the S(N) stop picks N* on the headline logits."""
    import torch

    from tree_draft_build_amd import binding as td
    from tree_draft_build_amd import tachometer as tach
    from tree_draft_build_amd import workload as wl

    dev = torch.device("cuda:0")
    cfg = wl.CONFIGS["qwen3_8b_tree"]
    sh = wl.layer_shape(cfg)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    w = {k: up(v) for k, v in wl.layer_weights(cfg, sh).items()}
    x = wl.make_logits(cfg)
    inp = wl.make_attn_inputs(cfg)
    kc, vc, off = up(inp["k_ctx"]), up(inp["v_ctx"]), up(inp["ctx_offsets"])
    ids, lq, _ = td.draft_topk(up(x), cfg.topk)
    stream = torch.cuda.current_stream()
    pass_kw = dict(batch=cfg.batch, hq=sh.hq, hkv=sh.hkv, head_dim=sh.head_dim, vocab=sh.vocab,
                   weights=w, k_ctx=kc, v_ctx=vc, ctx_offsets=off, scale=wl.attn_scale(cfg),
                   rope_base=sh.rope_base, device=dev)

    # ---- per call, at N = 64 ----
    tree = td.build_tree(ids, lq, cfg.n_max, False)
    vp = tach.VerifyPass(nq_max=cfg.nq_max, **pass_kw)
    reps = max(20, args.steps // 4)

    def loop_us(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / reps

    rows = cfg.batch * cfg.nq_max
    qkv_us = loop_us(lambda: td.tree_qkv(w["embed"], w["w_qkv"], tree["node_token"],
                                          tree["node_depth"], tree["n_nodes"], off, sh.hq, sh.hkv,
                                          sh.head_dim, sh.rope_base, out=(vp.q, vp.kt, vp.vt),
                                          workspace=vp.ws_layer))
    lm_us = loop_us(lambda: td.lm_head_argmax(vp.out, w["w_lm"], tree["n_nodes"], out=vp.target,
                                               workspace=vp.ws_layer))
    qkv_bytes = sh.qkv_out * sh.hidden * 2 + rows * sh.hidden * 2 + rows * sh.qkv_out * 2
    lm_bytes = sh.vocab * sh.hidden * 2 + rows * sh.hidden * 2 + rows * 4

    def roof(name, us, nbytes, flops):
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "avg_launch_us": round(us, 2),
                "bytes_per_launch": int(nbytes), "flops_per_launch": int(flops),
                "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_TFLOPS, 5),
                "timing": "HIP events around back-to-back calls"}

    # ---- the whole step with the layer, graph-captured ----
    vs = td.VerifyStep(batch=cfg.batch, block=cfg.block, vocab=cfg.vocab, topk=cfg.topk,
                       n_max=cfg.n_max, use_stop=False,
                       cost=(cfg.cost_a, cfg.cost_b, cfg.cost_c, cfg.cost_knee), l_ar=cfg.l_ar,
                       ahat0=cfg.ahat0, hq=cfg.hq, hkv=cfg.hkv, head_dim=cfg.head_dim,
                       scale=wl.attn_scale(cfg), logits_dtype=td.TD_BF16, attn_dtype=td.TD_BF16,
                       total_ctx=int(inp["ctx_offsets"][-1]), max_ctx=int(inp["ctx_len"].max()),
                       device=dev)
    root = torch.zeros(cfg.batch, dtype=torch.int32, device=dev)
    lg = up(x)
    vs.set_inputs(lg, vp.q, kc, vc, off, vp.kt, vp.vt, vp.target, root_token=root)
    acc = (torch.empty(cfg.batch, dtype=torch.int32, device=dev),
           torch.empty((cfg.batch, cfg.block + 1), dtype=torch.int32, device=dev),
           torch.empty(cfg.batch, dtype=torch.int32, device=dev))

    def full_step():
        vs.run(stages=td.TD_STEP_DRAFT)              # top-K, tree, mask
        t = vs.tree
        td.tree_qkv(w["embed"], w["w_qkv"], t["node_token"], t["node_depth"], t["n_nodes"], off,
                    sh.hq, sh.hkv, sh.head_dim, sh.rope_base, out=(vp.q, vp.kt, vp.vt),
                    workspace=vp.ws_layer)
        td.tree_verify_attn(vp.q, kc, vc, off, vp.total_ctx, vp.total_ctx, vp.kt, vp.vt, vs.mask,
                            t["n_nodes"], wl.attn_scale(cfg), out=vp.out, workspace=vp.ws_attn)
        td.lm_head_argmax(vp.out, w["w_lm"], t["n_nodes"], out=vp.target, workspace=vp.ws_layer)
        td.accept(t["node_token"], t["node_parent"], t["n_nodes"], vp.target, cfg.block, out=acc)

    full_step()
    torch.cuda.synchronize()
    if args.no_graph:
        step_us = loop_us(full_step)
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            full_step()
        step_us = loop_us(g.replay)

    layer = {
        "verify_layer": {
            "workload": "qwen3_8b_tree one-layer verification (hidden 4096, vocab 151936)",
            "rows": rows,
            "step_value": round(1e6 / step_us, 1), "step_unit": "verify steps/s",
            "step_us": round(step_us, 2),
            "step": "kernel 1 (top-K, tree, mask), Q/K/V + RoPE (2 kernels), attention "
                    "(2 kernels), LM-head argmax (2 kernels), acceptance; "
                    + ("eager launches" if args.no_graph else "one graph"),
            "kernel_roofline": {
                "tree_qkv": roof("tree_qkv (projection + RoPE)", qkv_us, qkv_bytes,
                                 2 * rows * sh.hidden * sh.qkv_out),
                "lm_head_argmax": roof("lm_head_argmax", lm_us, lm_bytes,
                                       2 * rows * sh.hidden * sh.vocab)}}}
    if not args.tachometer:
        return layer

    # ---- tachometer ----
    points = tach.measure(ids, lq, reps=10, warmup=2, **pass_kw)
    fit = tach.fit(points)
    # the fitted cost model drives the S(N) stop on the headline logits
    hcfg = wl.CONFIGS["qwen3_8b"]
    hids, hlq, _ = td.draft_topk(up(wl.make_logits(hcfg)), hcfg.topk)
    picked = {}
    for name, cost, lar in (("configured", (hcfg.cost_a, hcfg.cost_b, hcfg.cost_c, hcfg.cost_knee),
                             hcfg.l_ar), ("fitted", fit["cost"], fit["l_ar"])):
        t_ = td.build_tree(hids, hlq, hcfg.n_max, True, cost, lar, hcfg.ahat0)
        picked[name] = {"n_nodes": int(t_["n_nodes"][0]), "ahat": round(float(t_["ahat"][0]), 4),
                        "speedup_estimate": round(float(t_["speedup"][0]), 4)}
    return {
        **layer,
        "tachometer": {
            "what": "the one-layer verification pass (Q/K/V, tree attention, LM-head argmax) "
                    "timed at tree sizes N, fitted to C(N) = a + b N + c max(0, N - knee)",
            "points_us": [[p[1], round(p[2], 2)] for p in points],
            "fit_us": {"a": round(fit["a_us"], 3), "b": round(fit["b_us"], 5),
                       "c": round(fit["c_us"], 5), "knee": fit["knee"], "r2": round(fit["r2"], 5)},
            "cost_normalised": [round(v, 6) for v in fit["cost"][:3]] + [fit["cost"][3]],
            "stop_on_headline_logits": picked}}


def decode_row(cfg, args, steps, warmup):
    """The verify step in a synthetic decode loop: each step is one
    td_verify_step call with the commit fused into its last kernel, so the accepted path's keys and
    values are appended to the context (which grows in place inside a region
    of room steps * (block + 1) rows) and the bonus token becomes the next
    root; per-step inputs (logits, tree queries and K/V) rotate over 8 sets.
    The synthetic target depends on the tree's token paths only, so one
    target array per input set, made before the loop, serves every step."""
    import torch

    from tree_draft_build_amd import binding as td
    from tree_draft_build_amd import workload as wl

    dev = torch.device("cuda:0")
    n_sets = 8
    total = 2 * n_sets + warmup + steps          # every step the loop below can run
    inp0 = wl.make_attn_inputs(cfg)
    L0 = inp0["ctx_len"].astype(np.int64)
    region = L0 + total * (cfg.block + 1)
    off = np.zeros(cfg.batch + 1, np.int64)
    off[1:] = np.cumsum(region)
    tdt = torch.bfloat16 if cfg.attn_dtype == "bf16" else torch.float32

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    kc = torch.zeros((int(off[-1]), cfg.hkv, cfg.head_dim), dtype=tdt, device=dev)
    vc = torch.zeros_like(kc)
    for b in range(cfg.batch):
        o = int(inp0["ctx_offsets"][b])
        kc[int(off[b]):int(off[b]) + int(L0[b])] = up(inp0["k_ctx"][o:o + int(L0[b])])
        vc[int(off[b]):int(off[b]) + int(L0[b])] = up(inp0["v_ctx"][o:o + int(L0[b])])
    goff = torch.from_numpy(off).to(dev)
    lens = torch.from_numpy(L0.copy()).to(dev)
    # kernel 1 reads the root as it starts, the last kernel of the same step writes
    # the bonus into the same array afterwards: the next step's root
    root = torch.zeros(cfg.batch, dtype=torch.int32, device=dev)
    vs = td.VerifyStep(batch=cfg.batch, block=cfg.block, vocab=cfg.vocab, topk=cfg.topk,
                       n_max=cfg.n_max, use_stop=cfg.use_stop,
                       cost=(cfg.cost_a, cfg.cost_b, cfg.cost_c, cfg.cost_knee), l_ar=cfg.l_ar,
                       ahat0=cfg.ahat0, hq=cfg.hq, hkv=cfg.hkv, head_dim=cfg.head_dim,
                       scale=wl.attn_scale(cfg),
                       logits_dtype=td.TD_BF16 if cfg.logit_dtype == "bf16" else td.TD_F32,
                       attn_dtype=td.TD_BF16 if cfg.attn_dtype == "bf16" else td.TD_F32,
                       total_ctx=int(off[-1]), max_ctx=int(region.max()), device=dev)
    sets, accepted_per_set = [], []
    for k in range(n_sets):
        scfg = cfg.replace(index=cfg.index + 100 + k)
        x = wl.make_logits(scfg)
        inp = wl.make_attn_inputs(scfg)
        d = dict(logits=up(x), q=up(inp["q"]), k_tree=up(inp["k_tree"]), v_tree=up(inp["v_tree"]))
        tg = torch.full((cfg.batch, cfg.nq_max), -1, dtype=torch.int32, device=dev)
        vs.set_inputs(d["logits"], d["q"], kc, vc, goff, d["k_tree"], d["v_tree"], tg,
                      root_token=root, ctx_lengths=lens)
        vs.run(stages=td.TD_STEP_DRAFT)
        torch.cuda.synchronize()
        tree = {k_: v.cpu().numpy() for k_, v in vs.tree.items()}
        tg.copy_(torch.from_numpy(wl.target_tokens(scfg, wl.logits_as_f64(x, scfg.logit_dtype),
                                                   tree["node_token"], tree["node_parent"],
                                                   tree["n_nodes"])))
        vs.set_inputs(d["logits"], d["q"], kc, vc, goff, d["k_tree"], d["v_tree"], tg,
                      root_token=root, ctx_lengths=lens, commit=True, next_root=root)
        sets.append((td.StepArgs.from_buffer_copy(vs.args), d, tg))

    def one(i):
        vs.args = sets[i % n_sets][0]
        vs.run()

    G = n_sets
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    for i in range(G):           # warm the kernels before capture (no commit state lost:
        one(i)                   # these steps are part of the loop)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(G):
            one(i)
    stream = torch.cuda.current_stream()
    done = G
    while done < warmup:
        graph.replay()
        done += G
    torch.cuda.synchronize()
    len0 = lens.cpu().numpy().copy()
    reps = max(1, steps // G)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / (reps * G)
    grown = lens.cpu().numpy() - len0
    tokens = float(grown.sum()) / (reps * G)            # committed tokens per step, all sequences
    assert td.workspace_status(vs.workspace) == td.TD_OK
    return {"workload": cfg.name + " decode loop", "batch": cfg.batch, "steps": reps * G,
            "value": round(1e3 / ms, 1), "unit": "decode steps/s", "ms_per_step": round(ms, 5),
            "tokens_per_step": round(tokens, 3),
            "tokens_per_s": round(tokens * 1e3 / ms, 1),
            "context_growth": [int(v) for v in grown[:4]],
            "kernels_per_step": vs.kernels(),
            "note": "one td_verify_step call per step; the KV commit runs in its last kernel, "
                    "which also writes the bonus as the next step's root"}


def _code_tokens(text):
    """C/C++ source with comments removed and runs of whitespace folded, so
    that editing a comment does not change the digest."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest():
    """Digest of the library's code (comments and layout ignored): profiler
    counts are only reported for the kernels they were taken on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "tree_draft_build_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "treedraft.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def hbm_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload (scaled by the plain-copy
    calibration), or None when it is missing or was taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"verify_step_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("traffic_bytes")


def copy_calibration(mib):
    """Plain device-to-device copies of a known size, as the reference point
    for the HBM byte counters of a profiler run: each copy reads and writes
    exactly mib MiB."""
    import torch
    n = int(mib) << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": int(mib), "copies": 5}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, x, inp, budget_s, threads=0):
    """The CPU oracle, as it stands, on whole verify steps of the same
    workload: as many full steps as fit in about budget_s seconds, first on
    every core available to this process (the oracle spreads independent
    outputs over OpenMP threads), then on one thread."""
    import oracle
    avail = len(os.sched_getaffinity(0))
    n = threads if threads > 0 else avail
    before = oracle.set_threads(0)
    try:
        used = oracle.set_threads(n)
        multi = cpu_steps(cfg, x, inp, budget_s)
        oracle.set_threads(1)
        single = cpu_steps(cfg, x, inp, budget_s)
    finally:
        oracle.set_threads(before)
    return {"value": multi["value"], "unit": "verify steps/s", "cores": used, "kind": "oracle",
            "sample": multi["sample"] + f", {used} OpenMP threads",
            "cpu_model": cpu_model(), "cores_available": avail,
            "single_thread": {"value": single["value"], "cores": 1, "sample": single["sample"]}}


def cpu_steps(cfg, x, inp, budget_s):
    import oracle
    from tree_draft_build_amd import workload as wl

    cost = (cfg.cost_a, cfg.cost_b, cfg.cost_c, cfg.cost_knee)
    scale = wl.attn_scale(cfg)
    lf = wl.logits_as_f64(x, cfg.logit_dtype)
    steps = 0
    t0 = time.perf_counter()
    tg = None
    while True:
        ids, lq, lse = oracle.draft_topk(x, cfg.topk)
        tr = oracle.build_tree(ids, lq, cfg.n_max, cfg.use_stop, cost, cfg.l_ar, cfg.ahat0)
        m = oracle.tree_mask(tr["node_parent"], tr["n_nodes"])
        oracle.tree_attn(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"], inp["k_tree"],
                         inp["v_tree"], m, tr["n_nodes"], cfg.hq, cfg.hkv, cfg.head_dim, scale)
        if tg is None:   # target tokens are an input, made once outside the count
            t_pause = time.perf_counter()
            tg = wl.target_tokens(cfg, lf, tr["node_token"], tr["node_parent"], tr["n_nodes"])
            t0 += time.perf_counter() - t_pause
        oracle.accept(tr["node_token"], tr["node_parent"], tr["n_nodes"], tg, cfg.block)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 1000:
            break
    return {"value": round(steps / el, 3),
            "sample": f"{steps} whole verify steps of {cfg.name} in {el:.1f} s"}


if __name__ == "__main__":
    main()
