"""Decode weight-stream benchmark (one MI355X).

One step = one batch-1 decode pass over the full synthetic weight stream of a
36-layer model: per layer the Q4_K stages {q,k,v} (2048x2048, 512x2048,
512x2048), {o} (2048x2048), {gate,up} (11008x2048 each), {down} (2048x11008),
then the 128256x2048 Q8_0 output head. Stages run in order on one stream (a
stage's multiplies start after the previous stage's outputs are complete);
the pass is captured once into a HIP graph and replayed. Inputs are seeded
synthetic blocks shaped like the SmolLM3-3B tensors; all weights (1.86 GB)
are resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints one JSON line: weight-stream GB/s (whole pass), % of the 8 TB/s HBM
peak, tokens/s-equivalent (1 / pass time), a roofline record for the dominant
kernel (the Q4_K GEMV group kernel) and the CPU oracle timed on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=36, help="layers in the stream (36 = the workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="eager launches instead of a HIP graph")
    return ap.parse_args()


def build_stream(torch, g, synth, n_layers):
    """Upload the seeded stream; returns (batch, steps meta, total bytes, q4k bytes)."""
    dev = "cuda:0"
    t0 = time.time()
    stages = synth.decode_stream(n_layers=n_layers, head=True, threads=16)
    log(f"generated {len(stages)} stages in {time.time() - t0:.1f} s")
    entries, meta = [], []
    total = q4k = 0
    for si, st in enumerate(stages):
        x = torch.from_numpy(st.x).to(dev)
        step_bytes = 0
        for gm, w in zip(st.gemvs, st.weights):
            W = torch.from_numpy(w).to(dev)
            y = torch.empty(gm.rows, dtype=torch.float32, device=dev)
            tid = g.TYPE_Q8_0 if gm.fmt == synth.Q8_0 else g.TYPE_Q4_K
            entries.append((tid, W, x, y, si))
            step_bytes += w.nbytes
            if gm.fmt == synth.Q4_K:
                q4k += w.nbytes
        total += step_bytes
        meta.append((st.layer, tuple(gm.name for gm in st.gemvs), step_bytes))
    del stages
    torch.cuda.synchronize()
    log(f"uploaded {total / 1e9:.3f} GB in {time.time() - t0:.1f} s")
    return g.GemvBatch(entries), entries, meta, total, q4k


def per_step_times(torch, g, entries, meta, reps=5):
    """Event-timed durations of each step of the pass (eager launches, one
    event pair per step on the launch stream), averaged over `reps` passes."""
    s = torch.cuda.current_stream()
    steps = []
    i = 0
    for layer, names, nbytes in meta:
        n = len(names)
        steps.append(g.GemvBatch(entries[i:i + n]))
        i += n
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in steps]
    acc = [0.0] * len(steps)
    for _ in range(reps):
        for b, (e0, e1) in zip(steps, evs):
            e0.record(s)
            g.gguf_qmatvec_batch(b, s)
            e1.record(s)
        torch.cuda.synchronize()
        for k, (e0, e1) in enumerate(evs):
            acc[k] += e0.elapsed_time(e1) / reps
    return acc   # ms per step


def probe_ceiling(torch, g):
    buf = torch.zeros(2 << 30, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    for _ in range(3):
        g.gguf_qk_probe_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        g.gguf_qk_probe_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 10 / 1e3
    del buf
    return buf_bytes_gbps(2 << 30, t)


def buf_bytes_gbps(nbytes, seconds):
    return nbytes / seconds / 1e9


def cpu_baseline():
    """The oracle as it stands, on a bounded sample of the same workload:
    layer 0's seven Q4_K GEMVs and the first 8192 rows of the Q8_0 head,
    decoded to fp32 and multiplied in fp64 with NumPy, one BLAS thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    stages = synth.decode_stream(n_layers=1, head=False, threads=4)
    head_rows = 8192
    hw = synth.q8_0_weights(synth.rng_for(synth.DECODE_CFG_ID, 1000, synth.TENSOR_IDS["head"]),
                            head_rows, synth.HIDDEN)
    hx = synth.activations_f32(synth.rng_for(synth.DECODE_CFG_ID, 1000, 100), synth.HIDDEN)
    nbytes = sum(w.nbytes for st in stages for w in st.weights) + hw.nbytes
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for st in stages:
            for gm, w in zip(st.gemvs, st.weights):
                oracle.matvec_f64(oracle.dequant_q4_k_f32(w, gm.rows, gm.cols), st.x)
        oracle.matvec_f64(oracle.dequant_q8_0_f32(hw, head_rows, synth.HIDDEN), hx)
        dt = time.perf_counter() - t0
    gbps = nbytes / dt / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 q,k,v,o,gate,up,down (Q4_K) + head rows 0..{head_rows - 1} (Q8_0): "
                      f"{nbytes} weight bytes in {dt:.2f} s; tokens/s-equiv "
                      f"{gbps * 1e9 / synth.decode_stream_bytes():.4f}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the workload fits one MI355X); --gpus {args.gpus} "
              "is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    import gguf_block_quant_dequant_amd as g
    import synth

    torch.cuda.set_device(0)
    batch, entries, meta, total_bytes, q4k_bytes = build_stream(torch, g, synth, args.layers)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    if args.no_graph:
        def step():
            g.gguf_qmatvec_batch(batch, stream)
    else:
        with torch.cuda.stream(stream):
            g.gguf_qmatvec_batch(batch, stream)          # untimed first pass outside the graph
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            g.gguf_qmatvec_batch(batch, stream)

        def step():
            graph.replay()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    gbps = total_bytes / (ms / 1e3) / 1e9

    # per-step durations (eager, event-timed) for the roofline record
    with torch.cuda.stream(stream):
        step_ms = per_step_times(torch, g, entries, meta)
    q4k_ms = sum(t for (layer, names, b), t in zip(meta, step_ms) if layer >= 0)
    q4k_launches = sum(1 for (layer, names, b) in meta if layer >= 0)
    head_ms = sum(t for (layer, names, b), t in zip(meta, step_ms) if layer < 0)
    achieved = q4k_bytes / (q4k_ms / 1e3) / 1e9
    ceiling = probe_ceiling(torch, g)

    rec = {
        "metric": "weight-stream GB/s + % of HBM peak; decode tokens/s-equiv (36-layer Q4_K)",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Q4_K/Q8_0 blocks shaped like SmolLM3-3B tensors)",
        "config": {"workload": f"decode weight stream: {args.layers} layers x Q4_K {{q 2048x2048, "
                               "k 512x2048, v 512x2048, o 2048x2048, gate 11008x2048, up 11008x2048, "
                               "down 2048x11008}} + Q8_0 head 128256x2048, batch 1, stage-ordered",
                   "weight_bytes": total_bytes, "layers": args.layers,
                   "launch": "eager" if args.no_graph else "hip-graph"},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s_equiv": round(1e3 / ms, 2),
        "read_probe_GBps": round(ceiling, 1),
        "pct_of_read_probe": round(100 * gbps / ceiling, 2),
        "head_ms": round(head_ms, 4),
        "roofline": {"bound": "hbm", "kernel": "gemv_group_kernel<1, Q4_K>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "launches": q4k_launches, "bytes_per_launch_avg": q4k_bytes / q4k_launches,
                     "avg_launch_us": round(1e3 * q4k_ms / q4k_launches, 3)},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
