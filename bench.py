"""Benchmark of the W4A16 routed-expert layer on one MI355X.

A step is one pass of the layer -- route (logits, top-k, grouping), W4A16
gate/up + SiLU*up, W4A16 down, the FP16 shared expert where the layer has one,
weighted combine -- over one batch of T synthetic FP16 tokens whose expert rows
already sit in HBM.  Steps rotate over R byte-identical replicas of the layer's
weights at distinct addresses (R * layer bytes >= 1 GiB, four times the 256 MB
Infinity Cache), so the weights stream from HBM rather than from the cache,
and over a set of fresh activation batches.  Each (replica, batch) step is
captured once into a HIP graph and the timed loop replays the graphs.

Per-kernel durations (`kernel_us`) come from HIP events around each call of the
same steps run eagerly on the stream the kernels are launched on.  The roofline
object reports the dominant kernel (W4A16 gate/up): its duration is measured
with HIP events around a graph of back-to-back gate/up launches over the
replicas on the launch stream, and its algorithmic bytes per launch are the
qpacked gate+up bytes of the experts that launch reads (active experts x 2 x
(I*H/2 + I*ceil(H/256)*2)), against the 8 TB/s HBM peak.  `traffic` is the
HBM byte count per launch measured with rocprofv3 counters (FETCH_SIZE x 2 +
WRITE_SIZE, the factors calibrated on a plain copy), read from
profiles/gateup_traffic.json when that file was measured on the current
kernel source, else null.  Where the batch is large enough for the grouped
GEMM (T*k >= 64*E, the library's automatic choice; the prefill workload), the
gate/up launch is a matrix-core bound contraction and the roofline reports its
useful FLOPs (2 * T*k * H * 2I per launch) against the 2.5 PFLOP/s dense FP16
MFMA peak instead.

The timed K steps run in three blocks (graph replays of chunks of consecutive
steps); the line reports the pooled rate (all tokens over all block time) and
the blocks' spread.  For the OLMoE-shaped layer the line also carries the
prefill-sized layer on the same expert shape (T = 4096, grouped GEMM): each
phase timed with HIP events over back-to-back launches, the FFN's useful FLOPs
against the FP16 MFMA peak - and what vendor code reaches on the same GPU
(`practical_ceilings`: a 1 GiB device copy, an 8192^3 FP16 matrix product),
beside the published peaks the fractions are taken against.

The CPU baseline times the oracle (C, fp64) on a bounded sample of the same
workload, on one thread and on every host thread (at most 16).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense FP16 matrix peak
# the sources the streaming gate/up kernel is compiled from (the traffic counters are tied to them)
FFN_SOURCE = [os.path.join(ROOT, "w4a16_routed_expert_amd", "csrc", f)
              for f in ("expert_ffn.hip", "ffn_stream.h", "ffn_common.h", "moe_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="olmoe", choices=["olmoe", "qwen", "tiny", "prefill", "olmoe_stack"])
    ap.add_argument("--layers", type=int, default=0, help="olmoe_stack: layers (0 = the config's 16)")
    ap.add_argument("--tokens", type=int, default=None, help="batch T (default: largest decode batch of the config)")
    ap.add_argument("--replicas", type=int, default=0, help="weight replicas (0 = enough for >= 1 GiB)")
    ap.add_argument("--inputs", type=int, default=8, help="distinct activation batches per replica (per layer for "
                                                            "olmoe_stack)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of each batch the CPU baseline routes (0 = all; prefill defaults to 32)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--graph-steps", type=int, default=0,
                    help="consecutive steps captured in one graph (0 = one full rotation over the weight "
                         "replicas and input batches; each graph launch costs about 4.5 us, so one step per "
                         "graph is measurably slower)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed work before the warm-up steps and before the prefill "
                         "sub-measurement (the GPU's clocks rise over the first tenths of a second)")
    ap.add_argument("--fused", action="store_true",
                    help="run each step through the one-call layer (moe_layer_forward) instead of the separate calls")
    ap.add_argument("--ffn-mode", choices=["auto", "stream", "ksplit", "one"], default="auto",
                    help="--fused: the expert-FFN family of the one call (auto: the library's choice; one: the "
                         "whole layer in one persistent launch)")
    ap.add_argument("--one-stream", action="store_true",
                    help="--fused with a shared expert: the layer and its shared expert in one call on one stream "
                         "(moe_layer_forward_shared: the routing launch also runs the shared gate/up pass)")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="olmoe: skip the prefill measurement (T=4096, grouped GEMM) that the line carries")
    ap.add_argument("--prefetch", action="store_true",
                    help="olmoe_stack: load each next layer's predicted experts while the current layer computes")
    ap.add_argument("--staging", type=int, default=2, help="pinned staging rows per table (stack and partial)")
    ap.add_argument("--pinned-source", action="store_true",
                    help="stack and partial: keep the host source page-locked (misses copied directly, no "
                         "staging); the default is a pageable source")
    ap.add_argument("--fp16-slots", action="store_true",
                    help="offload-qpacked profile: experts in FP16 execution slots (dequantized on the GPU).  With "
                         "olmoe/qwen: the decode layer's expert FFN over qpacked rows and over FP16 slots, side by "
                         "side; with olmoe_stack: the tables hold FP16 slots")
    ap.add_argument("--partial", action="store_true",
                    help="qwen: keep only the config's resident experts published (39 of 60) and upload the "
                         "misses of every step before its expert FFN, as olmoe_stack does")
    ap.add_argument("--kernel-only", default=None, choices=[None, "gateup", "down", "copy"],
                    help="profile helper: after setup, launch only this kernel --steps times "
                         "(copy: a 256 MiB device-to-device copy, the counter calibration)")
    ap.add_argument("--traffic-report", nargs=5, metavar=("GU_FETCH", "GU_WRITE", "COPY_FETCH", "COPY_WRITE", "OUT"),
                    default=None,
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output directories of a --kernel-only "
                         "gateup run and a --kernel-only copy run into the traffic file OUT, then exit")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def pmc_per_dispatch(directory: str, kernel_substr: str, counter: str) -> float:
    """Mean counter value (KiB for FETCH_SIZE/WRITE_SIZE) per dispatch of the matching kernel."""
    import csv
    import glob
    vals = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} records for {kernel_substr} under {directory}")
    return sum(vals) / len(vals)


def traffic_report(gu_fetch, gu_write, copy_fetch, copy_write, out_path, config_name, T):
    """HBM bytes per gate/up launch: each counter scaled by its reading on a copy of known size."""
    cf = COPY_BYTES / (pmc_per_dispatch(copy_fetch, "copyBuffer", "FETCH_SIZE") * 1024)
    cw = COPY_BYTES / (pmc_per_dispatch(copy_write, "copyBuffer", "WRITE_SIZE") * 1024)
    fetch = pmc_per_dispatch(gu_fetch, "w4a16_ffn_kernel<true", "FETCH_SIZE") * 1024 * cf
    write = pmc_per_dispatch(gu_write, "w4a16_ffn_kernel<true", "WRITE_SIZE") * 1024 * cw
    d = {"workload": f"{config_name}_T{T}", "source_sha256": source_digest(FFN_SOURCE),
         "bytes_per_launch": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
         "fetch_factor": cf, "write_factor": cw}
    with open(out_path, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(d))


def source_digest(paths) -> str:
    """sha256 over the files' contents in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(config_name: str, T: int):
    """HBM bytes per gate/up launch from the counter file, if it matches this source and workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != source_digest(FFN_SOURCE) or d.get("workload") != f"{config_name}_T{T}":
        return None
    return d.get("bytes_per_launch")


def main():
    args = parse()
    if args.traffic_report:
        from w4a16_routed_expert_amd import synth
        cfg = synth.CONFIGS[args.config]
        traffic_report(*args.traffic_report, cfg.name, args.tokens or max(cfg.batches))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer is single-GPU; multi-GPU sharding is described in the design notes, not built).",
              file=sys.stderr)
        sys.exit(2)
    if args.one_stream and not args.fused:
        print("--one-stream selects the one-call layer with its shared expert: use it with --fused",
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
    if args.config == "olmoe_stack" or (args.config == "qwen" and args.partial):
        run_stack(args, torch, dev)
        return
    if args.fp16_slots:
        run_compact_vs_expanded(args, torch, dev)
        return
    if args.kernel_only == "copy":
        # before any other device copy, so the copy kernels profiled are exactly these
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": "copy", "launches": args.steps, "bytes": COPY_BYTES}))
        return
    cfg = synth.CONFIGS[args.config]
    T = args.tokens or max(cfg.batches)
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    Is = cfg.shared_I
    row_bytes, _ = B.moe_expert_row_bytes(H, I)
    shared_bytes = 3 * Is * H * 2 + H * 2 if Is else 0
    layer_bytes = row_bytes * E + shared_bytes
    R = args.replicas or max(1, -(-(1 << 30) // layer_bytes))
    S = args.inputs

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    rows_np = synth.make_expert_rows(cfg)
    wr_np = synth.make_router(cfg)
    xs_np = [synth.make_x(cfg, T, step=s) for s in range(S)]
    shared_np = synth.make_shared(cfg) if Is else None
    gen_s = time.time() - t0
    rows0 = torch.from_numpy(rows_np).to(dev)
    replicas = [rows0] + [rows0.clone() for _ in range(R - 1)]
    shared_reps = None
    if Is:
        # gate/up/down in the tile8 layout the shared-expert kernels read (packed on the device)
        sh0 = [B.pack_tile8(torch.from_numpy(np.ascontiguousarray(m)).to(dev)) for m in shared_np[:3]]
        sh0.append(torch.from_numpy(np.ascontiguousarray(shared_np[3])).to(dev))
        shared_reps = [sh0] + [[m.clone() for m in sh0] for _ in range(R - 1)]
    router = torch.from_numpy(wr_np).to(dev)
    xs = [torch.from_numpy(x).to(dev) for x in xs_np]
    lay = RoutedExpertLayer(H, I, E, k, rows0, router, max_T=T, device=dev)
    y = torch.empty((T, H), dtype=torch.float16, device=dev)
    if Is:
        sh_out = torch.empty((T, H), dtype=torch.float32, device=dev)
        sh_gate = torch.empty(T, dtype=torch.float32, device=dev)
        sh_ws_bytes = B.moe_shared_ffn_workspace_size(T, H, Is)
        sh_ws = torch.empty(sh_ws_bytes, dtype=torch.uint8, device=dev)
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
        return s % R, xs[(s // R) % S], n_act[(s // R) % S]

    side = torch.cuda.Stream(device=dev) if Is else None

    def run_step(s, ev=None):
        r, x, _ = step_args(s)
        rows = replicas[r]
        marks = iter(ev) if ev is not None else None
        # The shared expert needs x only: the timed steps fork it onto a second
        # stream beside the routing and the routed experts; the per-kernel event
        # steps keep everything on one stream so each phase has its own time.
        concurrent = bool(Is) and ev is None
        main = torch.cuda.current_stream()
        if concurrent:
            side.wait_stream(main)
            Wsg, Wsu, Wsd, wg = shared_reps[r]
            B.moe_shared_ffn(x, Wsg, Wsu, Wsd, wg, T, H, Is, sh_out, sh_gate, sh_ws, sh_ws_bytes, side)

        def mark():
            if marks is not None:
                next(marks).record(stream)
        mark()
        lay.route(x)
        mark()
        B.moe_w4a16_gateup(x, T, H, I, E, k, rows, lay.row_stride, None, lay.expert_offsets, lay.sorted_pairs,
                           lay.active_list, lay.n_active, lay.h, lay.status)
        mark()
        B.moe_w4a16_down(T, H, I, E, k, rows, lay.row_stride, None, lay.expert_offsets, lay.active_list,
                         lay.n_active, lay.h, lay.pair_out, lay.status)
        mark()
        if Is:
            if concurrent:
                main.wait_stream(side)
            else:
                Wsg, Wsu, Wsd, wg = shared_reps[r]
                B.moe_shared_ffn(x, Wsg, Wsu, Wsd, wg, T, H, Is, sh_out, sh_gate, sh_ws, sh_ws_bytes)
                mark()
            lay.combine(T, y, sh_out, sh_gate)
        else:
            lay.combine(T, y)
        mark()

    names = ["route", "gateup", "down"] + (["shared"] if Is else []) + ["combine"]

    shared_done = torch.cuda.Event() if Is else None

    fused_mode = {"auto": B.MOE_FFN_PATH_AUTO, "stream": B.MOE_FFN_PATH_STREAM,
                  "ksplit": B.MOE_FFN_PATH_KSPLIT, "one": B.MOE_FFN_PATH_ONE_LAUNCH}[args.ffn_mode]

    def run_step_fused(s, ev=None):
        """One step through the one-call layer (moe_layer_forward); the shared expert, where
        the layer has one, runs on the second stream and the call's combine waits for it."""
        r, x, _ = step_args(s)
        rows = replicas[r]
        main = torch.cuda.current_stream()
        if ev is not None:
            ev[0].record(stream)
        if Is and args.one_stream:
            Wsg, Wsu, Wsd, wg = shared_reps[r]
            B.moe_layer_forward_shared(x, router, None, T, H, I, E, k, rows, lay.row_stride, None, Wsg, Wsu, Wsd,
                                       wg, Is, sh_out, sh_gate, sh_ws, sh_ws_bytes, y, lay._bufs, fused_mode, main)
            if ev is not None:
                ev[1].record(stream)
            return
        if Is:
            side.wait_stream(main)
            Wsg, Wsu, Wsd, wg = shared_reps[r]
            B.moe_shared_ffn(x, Wsg, Wsu, Wsd, wg, T, H, Is, sh_out, sh_gate, sh_ws, sh_ws_bytes, side)
            shared_done.record(side)
        B.moe_layer_forward(x, router, None, T, H, I, E, k, rows, lay.row_stride, None, sh_out if Is else None,
                            sh_gate if Is else None, shared_done, y, lay._bufs, fused_mode, main)
        if Is:
            main.wait_stream(side)
        if ev is not None:
            ev[1].record(stream)

    if args.fused:
        run_step = run_step_fused       # noqa: F811 (the timed steps and the event steps use the one call)
        names = ["layer"]

    if args.kernel_only in ("gateup", "down"):
        lay.route(xs[0])

        def gateup(rows):
            B.moe_w4a16_gateup(xs[0], T, H, I, E, k, rows, lay.row_stride, None, lay.expert_offsets,
                               lay.sorted_pairs, lay.active_list, lay.n_active, lay.h, lay.status)
        if args.kernel_only == "down":
            gateup(replicas[0])
        for s in range(args.steps):
            rows = replicas[s % R]
            if args.kernel_only == "gateup":
                gateup(rows)
            else:
                B.moe_w4a16_down(T, H, I, E, k, rows, lay.row_stride, None, lay.expert_offsets, lay.active_list,
                                 lay.n_active, lay.h, lay.pair_out, lay.status)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": args.kernel_only, "launches": args.steps}))
        return

    # ---------------------------------------------------------------- graphs
    # Steps repeat with period R*S (replica, input batch).  The K timed steps
    # run in three blocks (their spread is reported); each block is cut into
    # chunks of at most G consecutive steps and each chunk is one graph launch
    # (one graph per distinct first step modulo the period and length).  The
    # warm-up replays the same kind of chunks.
    n_graph = R * S
    K = args.steps
    G = args.graph_steps if args.graph_steps > 0 else n_graph
    nb = 3 if K >= 3 else 1
    blocks = [(args.warmup + K * b // nb, K * (b + 1) // nb - K * b // nb) for b in range(nb)]

    def chunks(s0, count):
        out, s = [], s0
        while s < s0 + count:
            n = min(G, s0 + count - s)
            out.append((s, n))
            s += n
        return out

    graphs = {}
    if not args.no_graph:
        for s in range(n_graph):
            run_step(s)                 # warm every step once eagerly before capture
        torch.cuda.synchronize()
        cap = torch.cuda.Stream()
        spans = [(0, n_graph), (0, args.warmup)] + blocks      # settle, warm-up, timed blocks
        keys = sorted({(s % n_graph, n) for b0, bn in spans for s, n in chunks(b0, bn)})
        for s0, n in keys:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for j in range(n):
                    run_step(s0 + j)
            graphs[(s0, n)] = g
        torch.cuda.synchronize()

    def run_steps(s_begin, count):
        """Steps s_begin .. s_begin + count - 1."""
        if args.no_graph:
            for s in range(s_begin, s_begin + count):
                run_step(s)
            return
        for s, n in chunks(s_begin, count):
            graphs[(s % n_graph, n)].replay()

    # The GPU's clocks rise over the first tenths of a second of sustained work: untimed
    # replays of whole rotations bring it to its steady state before the warm-up steps.
    settle_s = settle(lambda: run_steps(0, n_graph), torch, args.settle)
    run_steps(0, args.warmup)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    # One region, synchronized on both sides; HIP events between its blocks give the
    # per-block rates without host synchronizations inside the region.
    bev = [torch.cuda.Event(enable_timing=True) for _ in range(len(blocks) + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    bev[0].record(stream)
    for i, (b0, bn) in enumerate(blocks):
        run_steps(b0, bn)
        bev[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    block_s = [bev[i].elapsed_time(bev[i + 1]) * 1e-3 for i in range(len(blocks))]
    ms_per_step = elapsed * 1e3 / K
    tokens_per_s = T * K / elapsed
    block_rates = [T * bn / t for (_, bn), t in zip(blocks, block_s)]
    block_spread = (max(block_rates) - min(block_rates)) / (sum(block_rates) / len(block_rates))
    graph_chunks = [n for b0, bn in blocks for _, n in chunks(b0, bn)] if not args.no_graph else []

    # ---------------------------------------------------------------- per-kernel events (eager, same steps)
    n_ev = min(K, 400)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(n_ev)]
    for s in range(n_ev):
        run_step(s, evs[s])
    torch.cuda.synchronize()
    dur = np.array([[evs[s][i].elapsed_time(evs[s][i + 1]) for i in range(len(names))] for s in range(n_ev)]) * 1e3
    mean_us = {n: float(dur[:, i].mean()) for i, n in enumerate(names)}
    gu_bytes_step = np.array([gateup_unit * step_args(s)[2] for s in range(n_ev)], dtype=np.float64)
    dn_bytes_step = np.array([down_unit * step_args(s)[2] for s in range(n_ev)], dtype=np.float64)
    ffn_us = mean_us["layer"] if args.fused else mean_us["gateup"] + mean_us["down"]
    ffn_gbs = float((gu_bytes_step.mean() + dn_bytes_step.mean()) / (ffn_us * 1e-6) / 1e9)

    # ---------------------------------------------------------------- gate/up roofline: back-to-back launches
    lay.route(xs[0])
    torch.cuda.synchronize()
    n_b2b = 2 * R

    def gateup_burst():
        for i in range(n_b2b):
            rows = replicas[i % R]
            B.moe_w4a16_gateup(xs[0], T, H, I, E, k, rows, lay.row_stride, None, lay.expert_offsets,
                               lay.sorted_pairs, lay.active_list, lay.n_active, lay.h, lay.status)
    gateup_burst()
    torch.cuda.synchronize()
    if args.no_graph:
        burst = gateup_burst
    else:
        gb = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(gb, stream=cap):
            gateup_burst()
        burst = gb.replay
    burst()
    torch.cuda.synchronize()
    reps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        burst()
    e1.record(stream)
    torch.cuda.synchronize()
    gu_us = e0.elapsed_time(e1) * 1e3 / (reps * n_b2b)
    gu_bytes = float(gateup_unit * n_act[0])
    gu_gbs = gu_bytes / (gu_us * 1e-6) / 1e9
    # The library's automatic choice (T*k >= 64*E: the grouped GEMM, a matrix-core
    # bound contraction) decides which roofline applies.
    gemm_path = T * k >= 64 * E
    gu_flops = 2.0 * T * k * H * 2 * I                      # useful FLOPs of one gate/up launch
    gu_tflops = gu_flops / (gu_us * 1e-6) / 1e12

    # ---------------------------------------------------------------- parity spot check of the timed path
    if Is:
        Wsg, Wsu, Wsd, wg = shared_reps[0]
        B.moe_shared_ffn(xs[0], Wsg, Wsu, Wsd, wg, T, H, Is, sh_out, sh_gate, sh_ws, sh_ws_bytes)
        lay.forward(xs[0], y, shared_out=sh_out, shared_gate=sh_gate)
    else:
        lay.forward(xs[0], y)
    torch.cuda.synchronize()
    y_gpu = y.cpu().numpy()

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = cpu_all = None
    if not args.skip_cpu:
        cpu, cpu_all = cpu_baselines(args, xs_np, wr_np, rows_np, shared_np, H, I, E, k, T, S, y_gpu)

    # ---------------------------------------------------------------- prefill, same expert shape
    prefill = None
    if args.config == "olmoe" and not args.no_prefill:
        prefill = measure_prefill(torch, B, synth, RoutedExpertLayer, replicas, dev, args.settle)

    ceilings = None
    if args.config == "olmoe" and not args.no_prefill:
        ceilings = measure_ceilings(torch, dev)

    workload = f"{cfg.name}_decode_layer_T{T}" if args.config != "prefill" else f"prefill_T{T}"
    out = {
        "metric": "W4A16 MoE layer tokens/s + HBM GB/s on qpacked bytes (decode) / MFMA % (prefill)",
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
            "workload": workload,
            "experts": E, "top_k": k, "hidden": H, "intermediate": I, "tokens": T,
            "shared_expert_intermediate": Is,
            "shared_expert_stream": (None if not Is else
                                     "one stream, gate/up pass in the routing launch"
                                     if args.fused and args.one_stream else
                                     "second stream, concurrent with routing and the routed experts"),
            "layer_call": f"moe_layer_forward (one call, expert FFN {args.ffn_mode})" if args.fused else "separate calls",
            "weights": "int4 qpacked, 256-value blocks, fp16 scales; fp16 activations, fp32 accumulation",
            "replicas": R, "input_batches": S, "graph_replay": not args.no_graph,
            "steps_per_graph": None if args.no_graph else G,
            "graph_chunks_timed": graph_chunks,
            "mean_active_experts": float(np.mean(n_act)),
        },
        "blocks": {"steps": [bn for _, bn in blocks], "tokens_per_s": block_rates,
                   "spread": block_spread, "pooled_tokens_per_s": tokens_per_s,
                   "spread_definition": "(max - min) / mean of the blocks' rates",
                   "timing": "one host-timed region; HIP events on the launch stream between its blocks"},
        "settle_s": settle_s,
        "roofline": ({
            "bound": "hbm",
            "kernel": "w4a16_ffn_kernel<gate/up> (W4A16 gate/up + SiLU*up)",
            "achieved": gu_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gu_gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic(cfg.name, T),
            "algorithmic_bytes_per_launch": gu_bytes,
            "avg_launch_us": gu_us,
            "timing": f"HIP events around {reps} replays of a graph of {n_b2b} back-to-back launches",
        } if not gemm_path else {
            "bound": "mfma",
            "kernel": "w4a16_gemm_kernel<gate/up> (grouped W4A16 GEMM + SiLU*up)",
            "achieved": gu_tflops,
            "peak": FP16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gu_tflops / FP16_MFMA_PEAK_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": gu_flops,
            "avg_launch_us": gu_us,
            "timing": f"HIP events around {reps} replays of a graph of {n_b2b} back-to-back launches",
        }),
        "ffn_hbm": {"achieved_gbs": ffn_gbs, "frac": ffn_gbs / HBM_PEAK_GBS,
                    "qpacked_bytes_per_step": float(gu_bytes_step.mean() + dn_bytes_step.mean()),
                    "timing": ("HIP events around whole one-call layer steps (routing and combine included), "
                               "eager" if args.fused else "per-kernel HIP events, eager steps")},
        "kernel_us": mean_us,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "prefill": prefill,
        "practical_ceilings": ceilings,
        "setup_s": {"generate_inputs": gen_s},
    }
    if Is and not args.fused:
        out["shared_hbm"] = {"bytes_per_step": shared_bytes,
                             "achieved_gbs": shared_bytes / (mean_us["shared"] * 1e-6) / 1e9}
    print(json.dumps(out))


def settle(run_once, torch, seconds: float) -> float:
    """Repeat run_once (GPU work) until `seconds` of wall time have passed; returns the time spent."""
    t0 = time.perf_counter()
    while True:
        run_once()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return time.perf_counter() - t0


def host_threads() -> int:
    """Host threads the baselines use: the CPUs this process may run on, at most 16 (the
    CPU share of one GPU on the benchmark machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baselines(args, xs_np, wr_np, rows_np, shared_np, H, I, E, k, T, S, y_gpu):
    """The oracle (plain C, fp64) on a bounded sample of the workload's input batches: one
    thread, then every host thread on the same batches (each thread runs whole tokens; a
    token's output depends on that token only, so the arithmetic is the same)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    n_calls, cpu_s, tok = 0, 0.0, 0
    parity_norm = None
    Tc = args.cpu_tokens or (32 if args.config == "prefill" else T)
    Tc = min(Tc, T)
    while cpu_s < args.cpu_seconds and n_calls < S:
        tc = time.perf_counter()
        ref = oracle.layer(xs_np[n_calls][:Tc], wr_np, rows_np, H, I, E, k, shared=shared_np)
        cpu_s += time.perf_counter() - tc
        tok += Tc
        if n_calls == 0:
            # every token's output depends on that token only: compare the sampled rows
            yr = ref["y"].view(np.float16).astype(np.float64)
            d = np.abs(yr - y_gpu[:Tc].astype(np.float64))
            parity_norm = float((d / np.abs(yr).max(axis=1, keepdims=True)).max())
        n_calls += 1
    one = {"value": tok / cpu_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"{n_calls} oracle layer call(s) of {Tc} of the batch's {T} tokens on the same inputs "
                     f"({cpu_s:.1f} s, single-threaded C, fp64)",
           "gpu_vs_oracle_normwise_err": parity_norm}
    nt = host_threads()
    per = max(1, -(-Tc // nt))
    tasks = [(b, a, min(Tc, a + per)) for b in range(n_calls) for a in range(0, Tc, per)]

    def run(task):
        b, a, e = task
        oracle.layer(xs_np[b][a:e], wr_np, rows_np, H, I, E, k, shared=shared_np)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nt) as ex:
        list(ex.map(run, tasks))
    wall = time.perf_counter() - t0
    allc = {"value": tok / wall, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"the same {n_calls} batch(es) of {Tc} tokens, {len(tasks)} token chunks on {nt} host "
                      f"threads ({wall:.1f} s wall)"}
    return one, allc


def stack_cpu_baselines(args, synth, cfg, host_rows, x_np, T, L):
    """The oracle on the stack workload: whole layers of one step (layer l's rows, router, bias and
    shared expert) until about --cpu-seconds of CPU time, scaled to tokens/s of the L-layer stack;
    then every host thread on the same layers (whole tokens per thread)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k

    def args_of(l):
        return (synth.make_router(cfg, layer=l), host_rows[l],
                synth.make_zipf_bias(cfg, layer=l) if cfg.zipf_s else None,
                synth.make_shared(cfg, layer=l) if cfg.shared_I else None)
    done, cpu_s = [], 0.0
    while cpu_s < args.cpu_seconds and len(done) < L:
        l = len(done)
        wr, rows, bias, shared = args_of(l)
        tc = time.perf_counter()
        oracle.layer(x_np, wr, rows, H, I, E, k, bias=bias, shared=shared)
        cpu_s += time.perf_counter() - tc
        done.append(l)
    per_layer = cpu_s / len(done)
    one = {"value": T / (per_layer * L), "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"{len(done)} of the {L} layers of one step, {T} tokens each ({cpu_s:.1f} s, "
                     f"single-threaded C, fp64), scaled to the {L}-layer stack"}
    nt = host_threads()
    per = max(1, -(-T // nt))
    tasks = [(l, a, min(T, a + per)) for l in done for a in range(0, T, per)]
    cache = {l: args_of(l) for l in done}

    def run(task):
        l, a, e = task
        wr, rows, bias, shared = cache[l]
        oracle.layer(x_np[a:e], wr, rows, H, I, E, k, bias=bias, shared=shared)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nt) as ex:
        list(ex.map(run, tasks))
    wall = time.perf_counter() - t0
    allc = {"value": T * len(done) / (wall * L), "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"the same {len(done)} layers, {len(tasks)} token chunks on {nt} host threads "
                      f"({wall:.1f} s wall), scaled to the {L}-layer stack"}
    return one, allc


def measure_ceilings(torch, dev, settle_s=0.3):
    """What vendor code reaches on this GPU, beside the published peaks the fractions use: a
    1 GiB device-to-device copy (torch copy_, HBM read + write bytes per second) and an
    8192^3 FP16 matrix product (torch.mm, the ROCm BLAS libraries), each timed with HIP events
    around 10 calls after a settle."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    a = torch.randn((8192, 8192), dtype=torch.float16, device=dev)
    b = torch.randn((8192, 8192), dtype=torch.float16, device=dev)
    c = torch.empty((8192, 8192), dtype=torch.float16, device=dev)

    def timed(f, reps=10):
        settle(f, torch, settle_s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_copy = timed(lambda: dst.copy_(src))
    t_mm = timed(lambda: torch.mm(a, b, out=c))
    copy_gbs = 2 * n / t_copy / 1e9
    mm_tflops = 2 * 8192 ** 3 / t_mm / 1e12
    del src, dst, a, b, c
    return {"hbm_copy_gbs": copy_gbs, "hbm_copy_frac": copy_gbs / HBM_PEAK_GBS,
            "fp16_gemm_tflops": mm_tflops, "fp16_gemm_frac": mm_tflops / FP16_MFMA_PEAK_TFLOPS,
            "what": "torch copy_ of 1 GiB (read + write bytes) and torch.mm of 8192^3 FP16, HIP events "
                    "around 10 calls after a settle"}


def measure_prefill(torch, B, synth, RoutedExpertLayer, replicas, dev, settle_s, rounds=3):
    """Prefill-sized layer on the same expert shape (T = 4096, uniform router init, the
    grouped-GEMM path): each phase captured as one graph of back-to-back launches over the
    weight replicas, every graph replayed for `settle_s` seconds first (steady clocks), then
    HIP events around `rounds` replays per phase on the launch stream.  Useful FLOPs: gate/up
    2*T*k*H*2I, down 2*T*k*I*H."""
    cfg = synth.CONFIGS["prefill"]
    T, H, I, E, k = max(cfg.batches), cfg.H, cfg.I, cfg.E, cfg.k
    router = torch.from_numpy(synth.make_router(cfg)).to(dev)
    x = torch.from_numpy(synth.make_x(cfg, T)).to(dev)
    lay = RoutedExpertLayer(H, I, E, k, replicas[0], router, max_T=T, device=dev)
    y = torch.empty((T, H), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()
    R = len(replicas)

    def gateup(r):
        B.moe_w4a16_gateup(x, T, H, I, E, k, replicas[r], lay.row_stride, None, lay.expert_offsets,
                           lay.sorted_pairs, lay.active_list, lay.n_active, lay.h, lay.status)

    def down(r):
        B.moe_w4a16_down(T, H, I, E, k, replicas[r], lay.row_stride, None, lay.expert_offsets, lay.active_list,
                         lay.n_active, lay.h, lay.pair_out, lay.status)

    phases = {"route": lambda r: lay.route(x), "gateup": gateup, "down": down,
              "combine": lambda r: lay.combine(T, y)}
    for f in phases.values():           # warm each phase (and leave valid routing behind)
        f(0)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    graphs = {}
    for name, f in phases.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for i in range(R):
                f(i)
        graphs[name] = g
    torch.cuda.synchronize()
    settled = settle(lambda: [g.replay() for g in graphs.values()], torch, settle_s)
    us = {}
    for name, g in graphs.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(rounds):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us[name] = e0.elapsed_time(e1) * 1e3 / (rounds * R)
    lay.check_status()
    fl_gu, fl_dn = 2.0 * T * k * H * 2 * I, 2.0 * T * k * I * H
    tf = lambda fl, t: fl / (t * 1e-6) / 1e12
    layer_us = sum(us.values())
    return {
        "workload": f"prefill_T{T} (E {E}, top-{k}, H {H}, I {I})",
        "kernel_us": us,
        "gateup": {"tflops": tf(fl_gu, us["gateup"]), "frac": tf(fl_gu, us["gateup"]) / FP16_MFMA_PEAK_TFLOPS},
        "down": {"tflops": tf(fl_dn, us["down"]), "frac": tf(fl_dn, us["down"]) / FP16_MFMA_PEAK_TFLOPS},
        "ffn": {"us": us["gateup"] + us["down"], "tflops": tf(fl_gu + fl_dn, us["gateup"] + us["down"]),
                "frac": tf(fl_gu + fl_dn, us["gateup"] + us["down"]) / FP16_MFMA_PEAK_TFLOPS},
        "peak_tflops": FP16_MFMA_PEAK_TFLOPS,
        "layer_us": layer_us, "layer_tokens_per_s": T / (layer_us * 1e-6),
        "settle_s": settled,
        "timing": f"HIP events around {rounds} replays per phase of a graph of {R} back-to-back launches "
                  f"over {R} weight replicas",
    }


def run_compact_vs_expanded(args, torch, dev):
    """The decode layer's expert FFN over qpacked rows (W4A16, converted in registers) and over
    FP16 execution slots (the offload-qpacked profile: the same experts dequantized on the GPU
    into FP16, read as stored), side by side on the same routing.  Each format rotates over enough
    replicas for >= 1 GiB, so the weights stream from HBM; HIP events around each FFN call, and
    around whole steps (route, FFN, combine) eager."""
    from w4a16_routed_expert_amd import binding as B
    from w4a16_routed_expert_amd import synth
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer
    cfg = synth.CONFIGS[args.config]
    T = args.tokens or max(cfg.batches)
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    S = args.inputs
    rows_np = synth.make_expert_rows(cfg)
    router = torch.from_numpy(synth.make_router(cfg)).to(dev)
    xs = [torch.from_numpy(synth.make_x(cfg, T, step=s)).to(dev) for s in range(S)]
    rows0 = torch.from_numpy(rows_np).to(dev)
    qb, _ = B.moe_expert_row_bytes(H, I)
    fb = B.moe_expert_row_bytes_fp16(H, I)
    fstride = (fb + 255) // 256 * 256
    slots0 = torch.empty((E, fstride), dtype=torch.uint8, device=dev)
    B.moe_dequant_expert_rows(rows0, rows0.stride(0), slots0, fstride, E, H, I)
    fmts = {"qpacked": (rows0, qb), "fp16_slots": (slots0, fb)}
    reps = {}
    for name, (r0, per) in fmts.items():
        R = max(1, -(-(1 << 30) // (per * E)))
        reps[name] = [r0] + [r0.clone() for _ in range(R - 1)]
    lay = RoutedExpertLayer(H, I, E, k, rows0, router, max_T=T, device=dev)
    y = torch.empty((T, H), dtype=torch.float16, device=dev)
    n_act = []
    for x in xs:
        lay.route(x)
        n_act.append(int(lay.n_active.cpu()[0]))
    steps = max(args.steps // 10, 50)
    out_f = {}
    for name, rr in reps.items():
        f16 = name == "fp16_slots"
        e = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for s in range(args.warmup + steps):
            x = xs[s % S]
            ev = e[s - args.warmup] if s >= args.warmup else None
            if ev:
                ev[0].record()
            lay.route(x)
            if ev:
                ev[1].record()
            lay.ffn(x, rows=rr[s % len(rr)], fp16_slots=f16, mode=B.MOE_FFN_PATH_STREAM)
            if ev:
                ev[2].record()
            lay.combine(T, y)
            if ev:
                ev[3].record()
        torch.cuda.synchronize()
        lay.check_status()
        ffn_us = float(np.mean([v[1].elapsed_time(v[2]) for v in e])) * 1e3
        step_us = float(np.mean([v[0].elapsed_time(v[3]) for v in e])) * 1e3
        act = float(np.mean([n_act[(args.warmup + i) % S] for i in range(steps)]))
        per = fmts[name][1]
        out_f[name] = {"ffn_us": ffn_us, "step_us_eager": step_us, "tokens_per_s_eager": T / (step_us * 1e-6),
                       "bytes_per_active_expert": per, "ffn_bytes_per_step": act * per,
                       "ffn_gbs": act * per / (ffn_us * 1e-6) / 1e9,
                       "ffn_frac_of_hbm_peak": act * per / (ffn_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                       "replicas": len(rr), "device_bytes_per_expert": per}
    q, f = out_f["qpacked"], out_f["fp16_slots"]
    out = {
        "metric": "W4A16 MoE layer tokens/s + HBM GB/s on qpacked bytes (decode) / MFMA % (prefill)",
        "value": q["tokens_per_s_eager"], "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": q["step_us_eager"] * 1e-3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}_decode_layer_T{T}_compact_vs_expanded", "experts": E, "top_k": k,
                   "hidden": H, "intermediate": I, "tokens": T, "mean_active_experts": float(np.mean(n_act))},
        "compact_vs_expanded": {"qpacked": q, "fp16_slots": f,
                                "bytes_ratio": f["bytes_per_active_expert"] / q["bytes_per_active_expert"],
                                "ffn_time_ratio": f["ffn_us"] / q["ffn_us"],
                                "timing": f"HIP events, {steps} eager steps per format (route, expert FFN, combine)"},
    }
    print(json.dumps(out))


def pinned_h2d_gbs(torch, dev, nbytes=256 << 20, reps=8):
    """Host-to-device rate from a pinned host buffer (hipMemcpyAsync of 256 MiB, HIP events): the
    link ceiling the miss uploads are judged against."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def run_stack(args, torch, dev):
    """Decode with partial residency: each layer keeps `resident` of its E experts published in a
    resident expert table.  Workloads: the OLMoE-shaped 16-layer stack with a Zipf-skewed router,
    its layers chained by the residual stream (x_{l+1} = x_l + y_l), and the Qwen-shaped layer with
    39 of 60 experts resident and its shared expert (--config qwen --partial).  A step routes each
    layer, brings the active experts to the host, runs one miss transaction (the table's copy
    stream), a lease on the new generation, the expert FFN on its rows, and the combine (layer.py
    DecodeStack).  With --prefetch, layer l+1's router is also applied to x_l and its predicted
    experts are loaded while layer l computes.  No graphs: every layer of every step has a host
    round trip."""
    from w4a16_routed_expert_amd import binding as B
    from w4a16_routed_expert_amd import synth
    from w4a16_routed_expert_amd.layer import DecodeStack, ResidentExpertTable, RoutedExpertLayer, SharedExpert
    cfg = synth.CONFIGS[args.config]
    T = args.tokens or max(cfg.batches)
    L = args.layers or cfg.n_layers
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    Is = cfg.shared_I
    spare = min(E - cfg.resident, T * k)
    S = max(1, args.inputs)
    t0 = time.time()
    host = [synth.make_expert_rows(cfg, layer=l) for l in range(L)]
    layers, tables, shared = [], [], []
    for l in range(L):
        wr = torch.from_numpy(synth.make_router(cfg, layer=l)).to(dev)
        bias = torch.from_numpy(synth.make_zipf_bias(cfg, layer=l)).to(dev) if cfg.zipf_s else None
        if Is:
            shared.append(SharedExpert(*(torch.from_numpy(np.ascontiguousarray(m)).to(dev)
                                         for m in synth.make_shared(cfg, layer=l)), max_T=T, device=dev))
        tab = ResidentExpertTable(host[l], H, I, cfg.resident, spare, staging_rows=args.staging, top_k=k,
                                  max_tokens=T, fp16_slots=args.fp16_slots, pinned_source=args.pinned_source)
        rows_dev, stride, _ = tab.device()
        lay = RoutedExpertLayer(H, I, E, k, torch.empty((1, stride), dtype=torch.uint8, device=dev), wr, bias,
                                max_T=T, device=dev)
        layers.append(lay)
        tables.append(tab)
    x0s = [torch.from_numpy(synth.make_x(cfg, T, step=s)).to(dev) for s in range(S)]
    gen_s = time.time() - t0
    stack = DecodeStack(layers, tables, shared=shared if Is else None, prefetch=args.prefetch)
    row_bytes, _ = B.moe_expert_row_bytes(H, I)
    if args.fp16_slots:
        row_bytes = B.moe_expert_row_bytes_fp16(H, I)           # what the FFN reads per active expert
    ffn_ev = []

    def timer(l, phase):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        ffn_ev.append((l, phase, e))

    for s in range(args.warmup):
        stack.step(x0s[s % S])
    torch.cuda.synchronize()
    base = [t.stats() for t in tables]
    K = args.steps
    t_start = time.perf_counter()
    for s in range(K):
        stack.step(x0s[(args.warmup + s) % S])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    after = [t.stats() for t in tables]
    delta = {n: sum(a[n] - b[n] for a, b in zip(after, base)) for n in after[0]}
    # a separate pass with the expert FFN of every layer timed by events
    n_ffn = min(K, 8)
    ffn_us = ffn_bytes = 0.0
    for s in range(n_ffn):
        ffn_ev.clear()
        stack.step(x0s[s % S], timer=timer)
        torch.cuda.synchronize()
        for l in range(L):
            b = [e for (ll, ph, e) in ffn_ev if ll == l]
            ffn_us += b[0].elapsed_time(b[1]) * 1e3
            ffn_bytes += int(layers[l].n_active.cpu()[0]) * row_bytes
    ffn_gbs = ffn_bytes / (ffn_us * 1e-6) / 1e9
    for lay in layers:
        lay.check_status()
    h2d_ceiling = pinned_h2d_gbs(torch, dev)
    demand = delta["hits"] + delta["misses"]
    cpu = cpu_all = None
    if not args.skip_cpu:
        cpu, cpu_all = stack_cpu_baselines(args, synth, cfg, host, x0s[0].cpu().numpy(), T, L)
    out = {
        "metric": "W4A16 MoE layer tokens/s + HBM GB/s on qpacked bytes (decode) / MFMA % (prefill)",
        "value": T * K / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": (f"olmoe_stack{L}" if args.config == "olmoe_stack" else f"{args.config}_decode_layer")
                               + f"_T{T}_resident{cfg.resident}of{E}" + ("_prefetch" if args.prefetch else ""),
                   "layers": L, "tokens": T, "experts": E, "top_k": k, "hidden": H, "intermediate": I,
                   "resident": cfg.resident, "spare_rows": spare, "staging_rows": args.staging,
                   "host_source": "page-locked (direct copies)" if args.pinned_source else "pageable (staged)",
                   "zipf_s": cfg.zipf_s,
                   "shared_expert_intermediate": Is, "input_batches": S,
                   "chain": "residual stream x_{l+1} = RN16(x_l + y_l)" if L > 1 else None,
                   "prefetch": "next layer's router on x_l, loaded while layer l computes" if args.prefetch else None,
                   "device_rows": "FP16 execution slots (offload-qpacked)" if args.fp16_slots else "qpacked"},
        "residency": {
            "hit_rate": delta["hits"] / max(1, demand),
            "misses_per_step": delta["misses"] / K,
            "h2d_bytes_per_step": delta["h2d_bytes"] / K,
            "h2d_gbs": delta["h2d_bytes"] / elapsed / 1e9,
            "evictions_per_step": delta["evictions"] / K,
            "prefetched_per_step": delta["prefetched"] / K,
            "prefetch_hits_per_step": delta["prefetch_hits"] / K,
            "prefetch_unused_per_step": delta["prefetch_unused"] / K,
            "staging_waits": delta["staging_waits"],
            "direct_copies_per_step": delta["direct_copies"] / K,
            "expert_d2h_bytes": delta["expert_d2h_bytes"], "host_writes": delta["host_writes"],
            "pinned_h2d_ceiling_gbs": h2d_ceiling,
            "h2d_frac_of_pinned_ceiling": delta["h2d_bytes"] / elapsed / 1e9 / h2d_ceiling,
        },
        "roofline": {"bound": "hbm", "kernel": "expert FFN (gate/up + down launches of each layer)",
                     "achieved": ffn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ffn_gbs / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": ffn_bytes / (n_ffn * L),
                     "avg_launch_us": ffn_us / (n_ffn * L),
                     "timing": f"HIP events around the expert FFN of {n_ffn} steps x {L} layers (eager); the "
                               "step itself is bound by the host-to-device misses (residency)"},
        "ffn_hbm": {"achieved_gbs": ffn_gbs, "frac": ffn_gbs / HBM_PEAK_GBS,
                    "timing": f"HIP events around the expert FFN of {n_ffn} steps x {L} layers"},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "setup_s": {"generate_inputs": gen_s},
    }
    for t in tables:
        t.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
