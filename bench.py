"""Benchmark of the W4A16 routed-expert layer on one MI355X.

A step is one pass of the layer -- route (logits, top-k, grouping), W4A16
gate/up + SiLU*up, W4A16 down, weighted combine -- over one batch of T
synthetic FP16 tokens whose expert rows already sit in HBM.  Steps rotate over
R byte-identical replicas of the layer's expert rows at distinct addresses
(R * layer bytes >= 1 GiB, four times the 256 MB Infinity Cache), so the
weights stream from HBM rather than from the cache, and over a set of fresh
activation batches.  Each step is captured once into a HIP graph (one graph
per replica) and the timed loop replays the graphs.

Per-kernel durations come from HIP events around each kernel of the same steps
run eagerly on the stream the kernels are launched on.  The roofline object
reports the dominant kernel (W4A16 gate/up): algorithmic bytes per launch =
qpacked gate+up bytes of the experts that launch actually reads (active
experts x 2 x (I*H/2 + I*ceil(H/256)*2)), divided by its average duration,
against the 8 TB/s HBM peak.

The CPU baseline times the oracle (single-threaded C, fp64) on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="olmoe", choices=["olmoe", "qwen", "tiny", "prefill"])
    ap.add_argument("--tokens", type=int, default=None, help="batch T (default: largest decode batch of the config)")
    ap.add_argument("--replicas", type=int, default=0, help="weight replicas (0 = enough for >= 1 GiB)")
    ap.add_argument("--inputs", type=int, default=8, help="distinct activation batches per replica")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--kernel-only", default=None, choices=[None, "gateup"],
                    help="profile helper: after setup, launch only this kernel --steps times")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported by this build "
              "(the layer is single-GPU; multi-GPU sharding is described in the design notes, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from w4a16_routed_expert_amd import binding as B
    from w4a16_routed_expert_amd import synth
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    T = args.tokens or max(cfg.batches)
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    row_bytes, _ = B.moe_expert_row_bytes(H, I)
    layer_bytes = row_bytes * E
    R = args.replicas or max(1, -(-(1 << 30) // layer_bytes))
    S = args.inputs

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    rows_np = synth.make_expert_rows(cfg)
    wr_np = synth.make_router(cfg)
    xs_np = [synth.make_x(cfg, T, step=s) for s in range(S)]
    gen_s = time.time() - t0
    rows0 = torch.from_numpy(rows_np).to(dev)
    replicas = [rows0] + [rows0.clone() for _ in range(R - 1)]
    router = torch.from_numpy(wr_np).to(dev)
    xs = [torch.from_numpy(x).to(dev) for x in xs_np]
    lay = RoutedExpertLayer(H, I, E, k, rows0, router, max_T=T, device=dev)
    y = torch.empty((T, H), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()

    # active experts per input batch (sets the algorithmic bytes of each launch)
    n_act = []
    for x in xs:
        lay.route(x)
        torch.cuda.synchronize()
        n_act.append(int(lay.n_active.cpu()[0]))
    gateup_unit = 2 * (I * H // 2 + I * ((H + 255) // 256) * 2)      # gate+up qpacked bytes per expert
    down_unit = H * I // 2 + H * ((I + 255) // 256) * 2

    # step s uses replica s % R and input batch (s // R) % S
    def step_args(s):
        return replicas[s % R], xs[(s // R) % S], n_act[(s // R) % S]

    def run_step(s, ev=None):
        rows, x, _ = step_args(s)
        if ev is not None:
            ev[0].record(stream)
        lay.route(x)
        if ev is not None:
            ev[1].record(stream)
        B.moe_w4a16_gateup(x, T, H, I, E, k, rows, lay.row_stride, None, lay.expert_offsets, lay.sorted_pairs,
                           lay.active_list, lay.n_active, lay.h, lay.status)
        if ev is not None:
            ev[2].record(stream)
        B.moe_w4a16_down(T, H, I, E, k, rows, lay.row_stride, None, lay.expert_offsets, lay.active_list,
                         lay.n_active, lay.h, lay.pair_out, lay.status)
        if ev is not None:
            ev[3].record(stream)
        lay.combine(T, y)
        if ev is not None:
            ev[4].record(stream)

    if args.kernel_only == "gateup":
        lay.route(xs[0])
        for s in range(args.steps):
            rows = replicas[s % R]
            B.moe_w4a16_gateup(xs[0], T, H, I, E, k, rows, lay.row_stride, None, lay.expert_offsets,
                               lay.sorted_pairs, lay.active_list, lay.n_active, lay.h, lay.status)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": "gateup", "launches": args.steps}))
        return

    # ---------------------------------------------------------------- graphs
    n_graph = R * S
    graphs = []
    if not args.no_graph:
        for s in range(n_graph):
            run_step(s)                 # warm the step once eagerly before capture
        torch.cuda.synchronize()
        cap = torch.cuda.Stream()
        for s in range(n_graph):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                run_step(s)
            graphs.append(g)
        torch.cuda.synchronize()

    def replay(s):
        graphs[s % n_graph].replay()

    step_fn = run_step if args.no_graph else replay
    for s in range(args.warmup):
        step_fn(s)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    K = args.steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(K):
        step_fn(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / K
    tokens_per_s = T * K / elapsed

    # ---------------------------------------------------------------- per-kernel events (eager, same steps)
    n_ev = min(K, 400)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_ev)]
    for s in range(n_ev):
        run_step(s, evs[s])
    torch.cuda.synchronize()
    dur = np.array([[evs[s][i].elapsed_time(evs[s][i + 1]) for i in range(4)] for s in range(n_ev)]) * 1e3  # us
    names = ["route", "gateup", "down", "combine"]
    mean_us = {n: float(dur[:, i].mean()) for i, n in enumerate(names)}
    gu_bytes = np.array([gateup_unit * step_args(s)[2] for s in range(n_ev)], dtype=np.float64)
    dn_bytes = np.array([down_unit * step_args(s)[2] for s in range(n_ev)], dtype=np.float64)
    gu_gbs = float(gu_bytes.mean() / (mean_us["gateup"] * 1e-6) / 1e9)
    ffn_gbs = float((gu_bytes.mean() + dn_bytes.mean()) / ((mean_us["gateup"] + mean_us["down"]) * 1e-6) / 1e9)

    # ---------------------------------------------------------------- parity spot check of the timed path
    lay.forward(xs[0], y)
    torch.cuda.synchronize()
    y_gpu = y.cpu().numpy()

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.skip_cpu:
        import oracle
        n_calls, cpu_s, tok = 0, 0.0, 0
        sample_T = T
        while cpu_s < args.cpu_seconds and n_calls < S:
            tc = time.perf_counter()
            ref = oracle.layer(xs_np[n_calls], wr_np, rows_np, H, I, E, k)
            cpu_s += time.perf_counter() - tc
            tok += sample_T
            if n_calls == 0:
                d = np.abs(ref["y"].view(np.float16).astype(np.float64) - y_gpu.astype(np.float64))
                m = np.abs(ref["y"].view(np.float16).astype(np.float64)).max(axis=1, keepdims=True)
                parity_norm = float((d / m).max())
            n_calls += 1
        cpu = {"value": tok / cpu_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_calls} oracle layer call(s) of {sample_T} tokens on the same inputs "
                         f"({cpu_s:.1f} s, single-threaded C, fp64)",
               "gpu_vs_oracle_normwise_err": parity_norm}

    out = {
        "metric": "W4A16 MoE layer tokens/s + HBM GB/s on qpacked bytes (decode)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}_decode_layer_T{T}" if args.config != "prefill" else f"prefill_T{T}",
            "experts": E, "top_k": k, "hidden": H, "intermediate": I, "tokens": T,
            "weights": "int4 qpacked, 256-value blocks, fp16 scales; fp16 activations, fp32 accumulation",
            "replicas": R, "input_batches": S, "graph_replay": not args.no_graph,
            "mean_active_experts": float(np.mean(n_act)),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "w4a16_ffn_kernel<gate/up> (W4A16 gate/up + SiLU*up)",
            "achieved": gu_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gu_gbs / HBM_PEAK_GBS,
            "traffic": None,
            "algorithmic_bytes_per_launch": float(gu_bytes.mean()),
            "avg_launch_us": mean_us["gateup"],
        },
        "ffn_hbm": {"achieved_gbs": ffn_gbs, "frac": ffn_gbs / HBM_PEAK_GBS,
                    "qpacked_bytes_per_step": float(gu_bytes.mean() + dn_bytes.mean())},
        "kernel_us": mean_us,
        "cpu_baseline": cpu,
        "setup_s": {"generate_inputs": gen_s},
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
