#!/usr/bin/env python3
"""Throughput of the EAGLE draft-and-verify hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the root distribution from the true feature, every depth's tree expansion and
draft step (embedding gather, [f ; e] FC, one decoder layer with tree
attention, LM head, softmax + top-k), the final expansion and rerank/flatten,
and tree-structured recursive rejection sampling against target logits that
sit in HBM before the timed region starts.

Default workload: the LLaMA2-7B-shaped draft head (d=4096, 32 heads x 128,
ffn 11008, vocab 32000, bf16), batch 1, prefix KV 1024, the static 26-node
tree (depth 5, branching 4/3/2/1).  Weights ~N(0, 0.02), features and prefix
KV ~N(0, 1), target logits = draft logits + N(0, 0.5) (root: exact copy).

Prints one JSON line.  value = drafted tree nodes per second through draft +
verify (whole job, one GPU), from K replays of the round captured as one HIP
graph (--no-graph: K eager rounds; both are reported).  `roofline` covers the dominant kernel, with its
per-launch duration measured by HIP events around each launch on the stream
it runs on; `cpu_baseline` times the fp64 CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
COUNTERS = os.path.join(ROOT, "profiles", "counters_gemm_7b_static26.json")
GEMM_SRC = os.path.join(ROOT, "eagle_feature_level_amd", "csrc", "gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_engine(cid: int):
    import torch
    from eagle_feature_level_amd.engine import EagleRound
    from workloads import (CONFIGS, TEMPLATES, make_prefix_kv, make_prefix_lens, make_root_features, make_root_tokens,
                           make_weights)
    from workloads import device as dev

    cfg = CONFIGS[cid]
    s = cfg.shape
    t0 = time.time()
    w = make_weights(cfg)
    lens = make_prefix_lens(cfg)
    ks, vs = make_prefix_kv(cfg, lens)
    feat = make_root_features(cfg)
    tok = make_root_tokens(cfg)
    log(f"[bench] generated {cfg.name} inputs in {time.time() - t0:.1f}s")
    wt = dev.weights(w, s.dtype)
    pf = dev.prefix(ks, vs, lens, s.dtype)
    kind = "dynamic" if cfg.tree == "dynamic" else "static"
    eng = EagleRound(dev.shape_dict(s), wt, cfg.batch, kind, cfg.topk, cfg.depth, cfg.rerank_m,
                     TEMPLATES.get(cfg.tree), pf)
    host = dict(w=w, lens=lens, ks=ks, vs=vs, feat=feat, tok=tok)
    # root features staged into the engine's own rows (input resident before the round)
    root = eng.root_features()
    root.copy_(torch.from_numpy(feat).cuda())
    return cfg, eng, root, dev.ints(tok), host


def synth_target(cfg, eng):
    """Target logits [B*N, V]: root row = the root draft row (q == p), other
    nodes = tree-wide draft logits + N(0, 0.5) noise."""
    import torch
    from workloads import make_target_noise
    B, N, V = cfg.batch, eng.n_nodes, cfg.shape.vocab
    eng.tree_wide()
    noise = torch.from_numpy(make_target_noise(cfg, B * N)).cuda()
    tgt = torch.empty(B * N, V, device="cuda")
    tw = eng.tw_logits[:B * (N - 1)].view(B, N - 1, V)
    tgt.view(B, N, V)[:, 1:] = tw + noise.view(B, N, V)[:, 1:]
    tgt.view(B, N, V)[:, 0] = eng.logits[:B]
    torch.cuda.synchronize()
    return tgt


def run_steps(eng, feat, tok, tgt, steps, marks=None):
    import torch
    for i in range(steps):
        if marks is not None:
            marks[i][0].record()
        eng.draft_phase(feat, tok)
        if marks is not None:
            marks[i][1].record()
        eng.verify(tgt, 0, i)
        if marks is not None:
            marks[i][2].record()


def cpu_baseline(cfg, host):
    """The fp64 oracle on one full round of the same workload (root head, every
    draft step, expansions, rerank, verify), on the host cores."""
    import numpy as np
    from oracle import pipeline as OP
    from workloads import TEMPLATES, make_target_noise
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    s = cfg.shape
    kind = "dynamic" if cfg.tree == "dynamic" else "static"
    # draft phase: whole rounds, repeated until ~10 s of CPU work (at most 20 rounds)
    t_draft, rounds = 0.0, 0
    while rounds == 0 or (t_draft < 10.0 and rounds < 20):
        t0 = time.perf_counter()
        res = OP.draft_phase(s, host["w"], host["feat"], host["tok"], host["ks"], host["vs"], host["lens"], kind,
                             cfg.topk, cfg.depth, cfg.rerank_m, TEMPLATES.get(cfg.tree), tree_wide=False)
        t_draft += time.perf_counter() - t0
        rounds += 1
    # target logits from the oracle's own tree-wide step (not timed), then verify (timed)
    from oracle import draft as OD
    B = cfg.batch
    rows = {k: [] for k in ("seq", "token", "parent", "pos", "slot", "mask")}
    for b in range(B):
        tr, pool = res["trees"][b], res["pools"][b]
        for t in range(1, len(tr["parent"])):
            pid = int(tr["pool_id"][t])
            rows["seq"].append(b)
            rows["token"].append(int(tr["token"][t]))
            rows["parent"].append(pool.feat_row[pool.parent[pid]])
            rows["pos"].append(int(host["lens"][b]) + int(tr["depth"][t]) - 1)
            rows["slot"].append(t)
            rows["mask"].append(int(tr["mask"][t]))
    tk, tv = OD.new_tree_kv(s, B)
    tw = OD.draft_step(s, host["w"], rows, res["feat_buf"], host["ks"], host["vs"], host["lens"], tk, tv,
                       act_bf16=False)["logits"]
    N = len(res["trees"][0]["parent"])
    noise = make_target_noise(cfg, B * N).reshape(B, N, -1)
    targets = [np.concatenate([res["logits"][b:b + 1], tw[b * (N - 1):(b + 1) * (N - 1)] + noise[b, 1:]])
               for b in range(B)]
    qrow = [OP.q_rows(res, b) for b in range(B)]
    t1 = time.perf_counter()
    for r in range(rounds):
        OP.verify_all(res["trees"], targets, res["logits"], qrow, 0, r)
    t_verify = time.perf_counter() - t1
    drafted = B * (N - 1) * rounds
    total = t_draft + t_verify
    return {"value": drafted / total, "unit": "draft-tree nodes/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rounds} full rounds of the same workload ({B} x {N - 1} drafted nodes each: root head, every "
                      f"draft step, expansions, rerank, verify) in fp64 numpy; draft {t_draft:.2f}s + verify "
                      f"{t_verify:.2f}s"}


def traffic_for(kernel_role: str, config_name: str):
    """HBM bytes per launch of a draft GEMM role from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what
    the counter reads for a plain 1 GiB copy), or None if the summary is missing,
    was taken on another workload, or the GEMM source changed since."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f)
    with open(GEMM_SRC, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    r = c.get("roles", {}).get(kernel_role)
    if c.get("gemm_source_sha256") != sha or c.get("workload") != config_name or r is None:
        return None
    return round(r["fetch_kib_per_dispatch"] * 1024 * c["fetch_factor"] +
                 r["write_kib_per_dispatch"] * 1024 * c["write_factor"])


def round_bench(cid: int, steps: int, warmup: int) -> dict:
    """One full round (draft phase + verify) of workload `cid`, replayed as a
    HIP graph `steps` times after `warmup` replays; draft / verify split from
    as many eager rounds with events between the phases."""
    import torch
    cfg, eng, feat, tok, _ = build_engine(cid)
    B, N = cfg.batch, eng.n_nodes
    eng.draft_phase(feat, tok)
    tgt = synth_target(cfg, eng)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    run_steps(eng, feat, tok, tgt, warmup)
    run_steps(eng, feat, tok, tgt, steps, marks)
    torch.cuda.synchronize()
    ms_draft = sum(m[0].elapsed_time(m[1]) for m in marks) / steps
    ms_verify = sum(m[1].elapsed_time(m[2]) for m in marks) / steps
    eng.capture_round(feat, tok, tgt, 0, 0)
    for _ in range(warmup):
        eng.replay_round()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        eng.replay_round()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    s = cfg.shape
    out = {"workload": cfg.name, "batch": B, "drafted_nodes_per_seq": N - 1, "d": s.d, "vocab": s.vocab,
           "value": round(B * (N - 1) / (ms * 1e-3), 1), "unit": "draft-tree nodes/s", "ms_per_round": round(ms, 4),
           "ms_draft_phase_eager": round(ms_draft, 4), "ms_verify_eager": round(ms_verify, 4),
           "draft_nodes_per_s": round(B * (N - 1) / (ms_draft * 1e-3), 1),
           "verify_nodes_per_s": round(B * N / (ms_verify * 1e-3), 1)}
    del eng, tgt
    torch.cuda.empty_cache()
    return out


def tree_wide_bench(args, cfg, eng, feat, tok):
    """K tree-wide draft steps (B x (N-1) rows in one eagle_draft_step) after one
    draft phase built the tree; per-role time, TFLOP/s and fraction of the
    bf16 MFMA peak from the library's measurement hook."""
    import torch
    import eagle_feature_level_amd as E
    eng.draft_phase(feat, tok)
    for _ in range(args.warmup):
        eng.tree_wide()
    torch.cuda.synchronize()
    rows = cfg.batch * (eng.n_nodes - 1)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        eng.tree_wide()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    E.eagle_profile_enable(args.steps * 200)
    for _ in range(args.steps):
        eng.tree_wide()
    torch.cuda.synchronize()
    kernels = {}
    for role in E._abi.ROLES:
        r = E.eagle_profile_read(role)
        if r["launches"]:
            kernels[role] = dict(avg_us=round(1e3 * r["ms"] / r["launches"], 2),
                                 tflops=round(r["flops"] / (r["ms"] * 1e-3) / 1e12, 1) if r["ms"] > 0 else None,
                                 ms_per_step=round(r["ms"] / args.steps, 4))
    E.eagle_profile_disable()
    gemm = ["fc", "qkv", "o", "gate_up", "down", "lm_head"]
    g_ms = sum(kernels[r]["ms_per_step"] for r in gemm if r in kernels)
    g_fl = sum(kernels[r]["tflops"] * kernels[r]["ms_per_step"] for r in gemm if r in kernels)  # TF/s x ms
    dom = max(gemm, key=lambda r: kernels[r]["ms_per_step"])
    ach = kernels[dom]["tflops"]
    s = cfg.shape
    out = {"metric": "tree-wide draft rows/sec (one draft step over every drafted node)",
           "value": round(rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": s.dtype,
           "data": "synthetic", "config": {"workload": cfg.name, "rows": rows, "d": s.d, "ffn": s.ffn,
                                           "heads": f"{s.n_heads}q/{s.n_kv_heads}kv x {s.head_dim}",
                                           "operands": "split bf16 (hi, lo): two MFMAs per product"},
           "gemm_tflops": round(g_fl / g_ms, 1) if g_ms else None,
           "roofline": {"bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / BF16_PEAK_TFLOPS, 4), "mfma_pipe_frac": round(2 * ach / BF16_PEAK_TFLOPS, 4),
                        "kernel": dom, "avg_launch_us": kernels[dom]["avg_us"]},
           "kernels": kernels}
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = 7B static-26, the bench line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the full-round measurements of the other workloads (7B EAGLE-2, 13B, 70B)")
    ap.add_argument("--tree-wide", action="store_true",
                    help="time only the tree-wide draft step (every drafted node of the flattened tree in one call: "
                         "the matrix-unit bound shape at batch 8 / 16) and print its own JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path here is single-GPU.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "launches": 3}))
        return
    import eagle_feature_level_amd as E

    cfg, eng, feat, tok, host = build_engine(args.config)
    B, N = cfg.batch, eng.n_nodes
    drafted = B * (N - 1)
    if args.tree_wide:
        tree_wide_bench(args, cfg, eng, feat, tok)
        return
    # target logits resident in HBM before timing
    eng.draft_phase(feat, tok)
    tgt = synth_target(cfg, eng)
    run_steps(eng, feat, tok, tgt, args.warmup)
    torch.cuda.synchronize()

    # timed region: exactly K steps
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    run_steps(eng, feat, tok, tgt, args.steps, marks)
    end.record()
    t_submit = time.perf_counter() - t_wall
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    ms_draft = sum(m[0].elapsed_time(m[1]) for m in marks) / args.steps
    ms_verify = sum(m[1].elapsed_time(m[2]) for m in marks) / args.steps
    ms_eager = ms_step

    # the same round captured as one HIP graph (every kernel of the round, the
    # launches pre-recorded): exactly K replays, timed the same way
    ms_graph = None
    if not args.no_graph:
        eng.capture_round(feat, tok, tgt, 0, 0)
        for _ in range(args.warmup):
            eng.replay_round()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_g = time.perf_counter()
        g0.record()
        for _ in range(args.steps):
            eng.replay_round()
        g1.record()
        torch.cuda.synchronize()
        t_g = time.perf_counter() - t_g
        ms_graph = g0.elapsed_time(g1) / args.steps
        ms_step, t_wall = ms_graph, t_g  # the step of record: graph replay

    # per-kernel durations: HIP events around every draft-step launch, same K steps again
    E.eagle_profile_enable(args.steps * 200)
    run_steps(eng, feat, tok, tgt, args.steps)
    torch.cuda.synchronize()
    kernels = {}
    for role in E._abi.ROLES:
        r = E.eagle_profile_read(role)
        if r["launches"]:
            kernels[role] = dict(launches_per_step=r["launches"] / args.steps,
                                 avg_us=1e3 * r["ms"] / r["launches"],
                                 gbs=r["bytes"] / (r["ms"] * 1e-3) / 1e9 if r["ms"] > 0 else None,
                                 tflops=r["flops"] / (r["ms"] * 1e-3) / 1e12 if r["ms"] > 0 else None,
                                 bytes_per_launch=r["bytes"] / r["launches"],
                                 ms_per_step=r["ms"] / args.steps)
    E.eagle_profile_disable()
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    kd = kernels[dom]
    achieved = kd["gbs"]
    traffic = traffic_for(dom, cfg.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                "avg_launch_us": round(kd["avg_us"], 2), "bytes_per_launch": round(kd["bytes_per_launch"])}
    gemm_roles = ["fc", "qkv", "o", "gate_up", "down", "lm_head"]
    g_ms = sum(kernels[r]["ms_per_step"] for r in gemm_roles if r in kernels)
    g_bytes = sum(kernels[r]["bytes_per_launch"] * kernels[r]["launches_per_step"] for r in gemm_roles if r in kernels)

    others = []
    if not args.headline_only and args.config == 2:
        del eng, tgt
        torch.cuda.empty_cache()
        for cid in (3, 4, 5):
            log(f"[bench] full round of workload {cid} ...")
            others.append(round_bench(cid, 10, 2))

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on one round ...")
        cpu = cpu_baseline(cfg, host)

    s = cfg.shape
    out = {
        "metric": "draft-tree nodes/sec + verify nodes/sec at 7B shape; % of MFMA/HBM roofline",
        "value": round(drafted / (ms_step * 1e-3), 1),
        "unit": "draft-tree nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "d": s.d, "heads": f"{s.n_heads}q/{s.n_kv_heads}kv x {s.head_dim}",
                   "ffn": s.ffn, "vocab": s.vocab, "batch": B, "prefix": cfg.prefix[1], "tree": cfg.tree,
                   "drafted_nodes_per_seq": N - 1, "global_batch": B, "seq_len": cfg.prefix[1],
                   "parallelism": "single GPU"},
        "draft_nodes_per_s": round(drafted / (ms_draft * 1e-3), 1),
        "verify_nodes_per_s": round(B * N / (ms_verify * 1e-3), 1),
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_graph": round(ms_graph, 4) if ms_graph is not None else None,
        "ms_draft_phase": round(ms_draft, 4),
        "ms_verify": round(ms_verify, 4),
        "wall_s_timed": round(t_wall, 4),
        "host_submit_ms_per_step": round(1e3 * t_submit / args.steps, 4),
        "gemm_stream_gbs": round(g_bytes / (g_ms * 1e-3) / 1e9, 1) if g_ms else None,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "roofline": roofline,
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
