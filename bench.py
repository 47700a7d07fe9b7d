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
peak, tokens/s-equivalent (1 / pass time), a roofline record for the
dominant kernel (the Q4_K lanes-along-K GEMV), the CPU oracle timed on a bounded
sample of the same workload, and labelled extras: the pass time distribution,
an unordered upper bound (all GEMVs of the pass as one step), the bf16
MFMA prefill pass over the same 36-layer weights (N = 512 tokens), and the
fp32 small-batch passes (the same 253 matrices times 8, 32 and 64 activation
vectors), batch-1 GEMV passes over the same shapes stored as Q4_0 and Q6_K,
and the 36 layers as decode layers with RMSN, SiLU(gate) * up and the
residual adds fused into the GEMVs against the same steps as separate kernels.

    python bench.py --copy-calibration

only copies 1 GiB device to device three times (the plain copy whose HBM
counter readings scale the GEMV kernel's counter readings).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2500.0
DOMINANT_KERNEL = "gemv_lk_kernel"
KERNEL_SOURCES = ["gguf_block_quant_dequant_amd/csrc/gemv_lk.hpp",
                  "gguf_block_quant_dequant_amd/csrc/device_common.hpp"]
SMALL_BATCH_TOKENS = (8, 32, 64)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_lk_kernel_decode_stream_traffic.md")


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
    ap.add_argument("--quick", action="store_true",
                    help="only the stage-ordered pass (for counter runs): no extras, no CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="copy 1 GiB device to device three times and exit")
    ap.add_argument("--small-batch-only", action="store_true",
                    help="only the small-batch passes (8, 32, 64 tokens) over the weight stream")
    ap.add_argument("--fused-only", action="store_true",
                    help="only the fused / unfused decode-layer passes")
    ap.add_argument("--other-types-only", action="store_true",
                    help="only the Q4_0 and Q6_K GEMV passes")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill pass over the 36-layer weights (for counter runs)")
    return ap.parse_args()


def kernel_source_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    kv = dict(re.findall(r"^([a-z_0-9]+):\s*(\S+)\s*$", text, flags=re.M))
    if kv.get("source_sha256") != kernel_source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_stream(torch, g, synth, n_layers):
    """Upload the seeded stream; returns (batch, entries, meta, total bytes, q4k bytes)."""
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


def capture(torch, fn, stream):
    """One untimed eager call, then a HIP graph of `fn` on `stream`."""
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    return graph


def time_replays(torch, graph, stream, reps, warm=2):
    """Per-replay durations (ms) from events on the replay stream."""
    with torch.cuda.stream(stream):
        for _ in range(warm):
            graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for i in range(reps):
            graph.replay()
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]


def pct(v, q):
    s = sorted(v)
    k = min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))
    return s[k]


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
    return (2 << 30) / t / 1e9


def prefill_pass(torch, g, synth, entries, meta, stream, n_tokens=512, reps=3):
    """36 layers x 7 Q4_K GEMMs (Y = X W^T, X bf16 [n_tokens x K]) over the
    resident decode weights, as one HIP graph: the matrices of a stage that
    share X ({q, k, v}, {gate, up}) in one launch, o and down alone; returns
    the labelled record."""
    dev = "cuda:0"
    gen = torch.Generator().manual_seed(synth.ROOT_SEED * 1000 + synth.PREFILL_CFG_ID)
    xs, ys, stages = {}, {}, {}
    flops, gemms = 0.0, 0
    for tid, W, x, y, si in entries:
        if tid != g.TYPE_Q4_K:
            continue
        cols, rows = x.numel(), y.numel()
        if cols not in xs:
            xs[cols] = torch.randn(n_tokens, cols, generator=gen).to(torch.bfloat16).to(dev)
        stages.setdefault(si, []).append((W, cols, rows))
        flops += 2.0 * n_tokens * rows * cols
        gemms += 1
    calls = []
    for si in sorted(stages):
        mats = stages[si]
        Ys = [ys.setdefault((r, j), torch.empty(n_tokens, r, dtype=torch.bfloat16, device=dev))
              for j, (_, _, r) in enumerate(mats)]
        calls.append(([m[0] for m in mats], xs[mats[0][1]], Ys, [m[2] for m in mats]))

    def run():
        for Ws, X, Ys, rows in calls:
            if len(Ws) == 1:
                g.gguf_qmatmul_q4_k(Ws[0], X, Ys[0], rows=rows[0], stream=stream)
            else:
                g.gguf_qmatmul_q4_k_multi(Ws, X, Ys, rows=rows, stream=stream)

    graph = capture(torch, run, stream)
    t = time_replays(torch, graph, stream, reps)
    ms = sorted(t)[len(t) // 2]
    tflops = flops / (ms / 1e3) / 1e12
    return {"label": "prefill: 36 layers x 7 Q4_K GEMMs, X bf16 [512 x K], Y bf16, bf16 MFMA, "
                     "fp32 accumulate; q/k/v and gate/up one launch each (HIP graph)",
            "gemms": gemms, "launches": len(calls), "flop": flops, "ms_per_pass": round(ms, 4),
            "roofline": {"bound": "mfma", "kernel": "gemm_q4_k_db_kernel", "achieved": round(tflops, 1),
                         "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_DENSE_PEAK_TFLOPS, 4), "traffic": None}}


def small_batch_pass(torch, g, synth, entries, stream, n_tokens, reps=5):
    """The whole weight stream (36 x 7 Q4_K + the Q8_0 head) multiplied by
    n_tokens fp32 activation vectors each (Y = X W^T, fp32), in pass order,
    the matrices of a stage that share X ({q, k, v}, {gate, up}) in one
    launch, as one HIP graph; returns the labelled record."""
    dev = "cuda:0"
    gen = torch.Generator().manual_seed(synth.ROOT_SEED * 1000 + 60 + n_tokens)
    xs, ys, stages = {}, {}, {}
    wbytes = 0
    for tid, W, x, y, si in entries:
        cols, rows = x.numel(), y.numel()
        if cols not in xs:
            xs[cols] = torch.randn(n_tokens, cols, generator=gen).to(dev)
        stages.setdefault(si, []).append((tid, W, cols, rows))
        wbytes += W.numel()
    calls = []
    for si in sorted(stages):
        mats = stages[si]
        Ys = [ys.setdefault((r, j), torch.empty(n_tokens, r, dtype=torch.float32, device=dev))
              for j, (_, _, _, r) in enumerate(mats)]
        calls.append((mats[0][0], [m[1] for m in mats], xs[mats[0][2]], Ys, [m[3] for m in mats]))

    def run():
        for tid, Ws, X, Ys, rows in calls:
            if len(Ws) == 1:
                f = g.gguf_qmatmul_f32_q4_k if tid == g.TYPE_Q4_K else g.gguf_qmatmul_f32_q8_0
                f(Ws[0], X, Ys[0], rows=rows[0], stream=stream)
            else:
                f = g.gguf_qmatmul_f32_q4_k_multi if tid == g.TYPE_Q4_K else g.gguf_qmatmul_f32_q8_0_multi
                f(Ws, X, Ys, rows=rows, stream=stream)

    graph = capture(torch, run, stream)
    t = time_replays(torch, graph, stream, reps)
    ms = sorted(t)[len(t) // 2]
    gbps = wbytes / (ms / 1e3) / 1e9
    del graph
    return {"label": f"small batch: the {sum(len(c[1]) for c in calls)} matrices of the pass x {n_tokens} "
                     "fp32 activation vectors, fp32 Y, bf16 hi/lo MFMA; q/k/v and gate/up one launch "
                     "each (HIP graph)",
            "tokens": n_tokens, "launches": len(calls), "ms_per_pass": round(ms, 4),
            "weight_GBps": round(gbps, 1),
            "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
            "tokens_per_s": round(n_tokens * 1e3 / ms, 1),
            "roofline": {"bound": "hbm", "kernel": "gemv_small_batch_kernel",
                         "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None}}


def fused_layer_pass(torch, g, synth, entries, stream, reps=10):
    """The 36 resident Q4_K layers as decode layers with the neighbouring steps
    (RMSN before q/k/v and before gate/up, SiLU(gate) * up, the two residual
    adds) fused into the GEMVs (4 launches per layer) and, for comparison, as
    separate kernels between plain GEMV launches (9 per layer). The attention
    result, out of scope, is stood in by the q projection's output. Both as
    HIP graphs; returns the labelled record."""
    dev = "cuda:0"
    H, F, KV, EPS = synth.HIDDEN, synth.FFN, synth.KV, 1e-6
    q4 = [e for e in entries if e[0] == g.TYPE_Q4_K]
    layers = [dict(zip(("q", "k", "v", "o", "gate", "up", "down"), (e[1] for e in q4[7 * i:7 * i + 7])))
              for i in range(len(q4) // 7)]
    gen = torch.Generator().manual_seed(80)
    norms = [(torch.rand(H, generator=gen) + 0.5).to(dev) for _ in range(2 * len(layers))]
    e_ = lambda n: torch.empty(n, dtype=torch.float32, device=dev)
    h0 = torch.randn(H, generator=gen).to(dev)
    # fused
    hw, ss = e_(H), e_(H // 64)
    ents, eps, h = [], [], h0
    for li, L in enumerate(layers):
        st = 4 * li
        q, k, v = e_(H), e_(KV), e_(KV)
        h1, hw2, ss2, gg, uu, act = e_(H), e_(H), e_(H // 64), e_(F), e_(F), e_(F)
        h2, hw3, ss3 = e_(H), e_(H), e_(H // 64)
        for name, y in (("q", q), ("k", k), ("v", v)):
            ents.append((g.TYPE_Q4_K, L[name], hw, y, st))
            eps.append({"scale_ss": ss, "eps": EPS})
        ents.append((g.TYPE_Q4_K, L["o"], q, h1, st + 1))
        eps.append({"residual": h, "norm_w": norms[2 * li + 1], "norm_out": hw2, "ss_out": ss2})
        ents.append((g.TYPE_Q4_K, L["gate"], hw2, gg, st + 2))
        eps.append({"scale_ss": ss2, "eps": EPS, "pair": 1, "act": act})
        ents.append((g.TYPE_Q4_K, L["up"], hw2, uu, st + 2))
        eps.append({"scale_ss": ss2, "eps": EPS, "pair": 2, "act": act})
        nxt = norms[2 * (li + 1)] if li + 1 < len(layers) else norms[0]
        ents.append((g.TYPE_Q4_K, L["down"], act, h2, st + 3))
        eps.append({"residual": h1, "norm_w": nxt, "norm_out": hw3, "ss_out": ss3})
        h, hw, ss = h2, hw3, ss3
    fb = g.GemvBatch(ents, eps)
    hw0, ss0 = ents[0][2], eps[0]["scale_ss"]

    def fused():
        g.gguf_rmsnorm_prep_f32(h0, norms[0], hw0, ss0, stream=stream)
        g.gguf_qmatvec_batch(fb, stream)

    # unfused: plain grouped GEMV steps with standalone steps between them
    plan, h = [], h0
    for li, L in enumerate(layers):
        x1, q, k, v, o, h1 = e_(H), e_(H), e_(KV), e_(KV), e_(H), e_(H)
        x2, gg, uu, act, d, h2 = e_(H), e_(F), e_(F), e_(F), e_(H), e_(H)
        qkv = g.GemvBatch([(g.TYPE_Q4_K, L["q"], x1, q, 0), (g.TYPE_Q4_K, L["k"], x1, k, 0),
                           (g.TYPE_Q4_K, L["v"], x1, v, 0)])
        ob = g.GemvBatch([(g.TYPE_Q4_K, L["o"], q, o, 0)])
        gu = g.GemvBatch([(g.TYPE_Q4_K, L["gate"], x2, gg, 0), (g.TYPE_Q4_K, L["up"], x2, uu, 0)])
        db = g.GemvBatch([(g.TYPE_Q4_K, L["down"], act, d, 0)])
        plan.append((h, x1, norms[2 * li], qkv, ob, o, h1, x2, norms[2 * li + 1], gu, gg, uu, act, db, d, h2))
        h = h2

    def unfused():
        for (hh, x1, n1, qkv, ob, o, h1, x2, n2, gu, gg, uu, act, db, d, h2) in plan:
            g.gguf_rmsnorm_f32(hh, n1, EPS, x1, stream=stream)
            g.gguf_qmatvec_batch(qkv, stream)
            g.gguf_qmatvec_batch(ob, stream)
            g.gguf_add_f32(hh, o, h1, stream=stream)
            g.gguf_rmsnorm_f32(h1, n2, EPS, x2, stream=stream)
            g.gguf_qmatvec_batch(gu, stream)
            g.gguf_swiglu_f32(gg, uu, act, stream=stream)
            g.gguf_qmatvec_batch(db, stream)
            g.gguf_add_f32(h1, d, h2, stream=stream)

    out = {"label": f"{len(layers)} decode layers (Q4_K, SmolLM3-3B shapes) with RMSN, SiLU(gate)*up "
                    "and the residual adds; attention stood in by q (not measured); HIP graphs",
           "layers": len(layers)}
    wbytes = sum(e[1].numel() for e in q4)
    for name, fn, launches in (("fused", fused, 4 * len(layers) + 1), ("unfused", unfused, 9 * len(layers))):
        graph = capture(torch, fn, stream)
        t = time_replays(torch, graph, stream, reps)
        ms = sorted(t)[len(t) // 2]
        out[name] = {"ms_per_pass": round(ms, 4), "launches": launches,
                     "weight_GBps": round(wbytes / (ms / 1e3) / 1e9, 1)}
        del graph
    return out


def other_types_pass(torch, g, synth, reps=5):
    """Batch-1 GEMV passes over the 36-layer shapes stored as Q4_0 and as Q6_K:
    one layer's seven tensors generated per type, cloned to 36 distinct device
    copies (so each pass streams every byte from HBM), as one decode batch in
    the Q4_K pass's stages ({q,k,v}, {o}, {gate,up}, {down} per layer; the
    GEMVs of a stage share a lanes-along-K launch), as a HIP graph.
    Returns one labelled record per type."""
    dev = "cuda:0"
    out = []
    for name, gen in (("q4_0", synth.q4_0_weights), ("q6_k", synth.q6_k_weights)):
        layer = []
        for gm in [gm for st in synth.LAYER_STAGES for gm in st]:
            w = gen(synth.rng_for(70, 0, synth.TENSOR_IDS[gm.name]), gm.rows, gm.cols)
            layer.append((gm, torch.from_numpy(w).to(dev)))
        xs = {c: torch.randn(c, generator=torch.Generator().manual_seed(c)).to(dev)
              for c in {gm.cols for gm, _ in layer}}
        tcode = g.TYPE_Q4_0 if name == "q4_0" else g.TYPE_Q6_K
        stage_of = {gm.name: si for si, st in enumerate(synth.LAYER_STAGES) for gm in st}
        ents, keep, wbytes = [], [], 0
        for li in range(synth.N_LAYERS):
            for gm, W in layer:
                Wc = W if li == 0 else W.clone()
                y = torch.empty(gm.rows, dtype=torch.float32, device=dev)
                keep.append((Wc, y))
                ents.append((tcode, Wc, xs[gm.cols], y, len(synth.LAYER_STAGES) * li + stage_of[gm.name]))
                wbytes += Wc.numel()
        batch = g.GemvBatch(ents)
        stream = torch.cuda.Stream()

        def run():
            g.gguf_qmatvec_batch(batch, stream)

        graph = capture(torch, run, stream)
        t = time_replays(torch, graph, stream, reps)
        ms = sorted(t)[len(t) // 2]
        gbps = wbytes / (ms / 1e3) / 1e9
        out.append({"label": f"batch-1 GEMV pass, 36 layers x 7 {name.upper()} tensors "
                             "(SmolLM3-3B shapes), stage-ordered decode batch (HIP graph)",
                    "type": name, "weight_bytes": wbytes, "ms_per_pass": round(ms, 4),
                    "GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
                    "roofline": {"bound": "hbm",
                                 "kernel": f"gemv_lk_kernel ({name.upper()})",
                                 "achieved": round(gbps, 1),
                                 "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                 "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None}})
        del graph, batch, ents, keep, layer
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def cpu_baseline():
    """The oracle as it stands, on a bounded sample of the same workload:
    layers 0..7's seven Q4_K GEMVs each and the first 32768 rows of the Q8_0
    head (about 13 s of work on one core), decoded to fp32 and multiplied in
    fp64 with NumPy, one BLAS thread."""
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    n_layers = 8
    stages = synth.decode_stream(n_layers=n_layers, head=False, threads=4)
    head_rows = 32768
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
            "sample": f"layers 0..{n_layers - 1} q,k,v,o,gate,up,down (Q4_K) + head rows 0..{head_rows - 1} "
                      f"(Q8_0): "
                      f"{nbytes} weight bytes in {dt:.2f} s; tokens/s-equiv "
                      f"{gbps * 1e9 / synth.decode_stream_bytes():.4f}"}


def copy_calibration():
    import torch
    torch.cuda.set_device(0)
    a = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the workload fits one MI355X); --gpus {args.gpus} "
              "is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    import gguf_block_quant_dequant_amd as g
    import synth

    torch.cuda.set_device(0)
    batch, entries, meta, total_bytes, q4k_bytes = build_stream(torch, g, synth, args.layers)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    if args.prefill_only:
        print(json.dumps(prefill_pass(torch, g, synth, entries, meta, stream)), flush=True)
        return
    if args.fused_only:
        print(json.dumps(fused_layer_pass(torch, g, synth, entries, stream)), flush=True)
        return
    if args.other_types_only:
        print(json.dumps(other_types_pass(torch, g, synth)), flush=True)
        return
    if args.small_batch_only:
        print(json.dumps([small_batch_pass(torch, g, synth, entries, stream, n)
                          for n in SMALL_BATCH_TOKENS]), flush=True)
        return
    if args.no_graph:
        def step():
            g.gguf_qmatvec_batch(batch, stream)
    else:
        graph = capture(torch, lambda: g.gguf_qmatvec_batch(batch, stream), stream)

        def step():
            graph.replay()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    gbps = total_bytes / (ms / 1e3) / 1e9

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
        "ms_per_step_p10_p50_p90": [round(pct(per, 0.1), 5), round(pct(per, 0.5), 5),
                                    round(pct(per, 0.9), 5)],
        "wall_s_timed": round(wall, 3),
    }
    if args.quick:
        print(json.dumps(rec), flush=True)
        return

    # Roofline of the dominant kernel: the Q4_K lanes-along-K GEMV launches of
    # the pass (all stages but the head; the down stage's long rows run the
    # same kernel family's long-row variant) replayed alone as a graph, so that
    # the average launch duration is the kernels' own, back to back as in the
    # pass.
    q4k_entries = [e for e in entries if e[0] == g.TYPE_Q4_K]
    q4k_launches = sum(1 for (layer, names, b) in meta if layer >= 0)
    q4k_batch = g.GemvBatch(q4k_entries)
    gq = capture(torch, lambda: g.gguf_qmatvec_batch(q4k_batch, stream), stream)
    tq = time_replays(torch, gq, stream, 10)
    q4k_ms = sorted(tq)[len(tq) // 2]
    avg_launch_s = q4k_ms / 1e3 / q4k_launches
    bytes_per_launch = q4k_bytes / q4k_launches
    achieved = bytes_per_launch / avg_launch_s / 1e9
    traffic = recorded_traffic()
    rec["roofline"] = {"bound": "hbm", "kernel": DOMINANT_KERNEL, "achieved": round(achieved, 1),
                       "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": round(achieved / HBM_PEAK_GBPS, 4),
                       "traffic": round(traffic) if traffic is not None else None,
                       "launches": q4k_launches, "bytes_per_launch_avg": bytes_per_launch,
                       "avg_launch_us": round(avg_launch_s * 1e6, 3)}
    del gq

    head_entries = [e for e in entries if e[0] == g.TYPE_Q8_0]
    hb = g.GemvBatch(head_entries)
    gh = capture(torch, lambda: g.gguf_qmatvec_batch(hb, stream), stream)
    th = time_replays(torch, gh, stream, 10)
    head_ms = sorted(th)[len(th) // 2]
    head_bytes = sum(e[1].numel() for e in head_entries)
    rec["head"] = {"ms": round(head_ms, 4), "GBps": round(head_bytes / (head_ms / 1e3) / 1e9, 1)}
    del gh

    # Labelled upper bound: every GEMV of the pass in one step (no stage order),
    # grouped four to a launch.
    ub = g.GemvBatch([(tid, W, x, y, 0) for tid, W, x, y, si in entries])
    gu = capture(torch, lambda: g.gguf_qmatvec_batch(ub, stream), stream)
    tu = time_replays(torch, gu, stream, 10)
    ums = sorted(tu)[len(tu) // 2]
    rec["unordered_upper_bound"] = {
        "label": "all 253 GEMVs of the pass as one unordered step (not the headline)",
        "ms": round(ums, 4), "GBps": round(total_bytes / (ums / 1e3) / 1e9, 1),
        "pct_hbm_peak": round(100 * total_bytes / (ums / 1e3) / 1e9 / HBM_PEAK_GBPS, 2)}
    del gu

    ceiling = probe_ceiling(torch, g)
    rec["read_probe_GBps"] = round(ceiling, 1)
    rec["pct_of_read_probe"] = round(100 * gbps / ceiling, 2)
    rec["prefill"] = prefill_pass(torch, g, synth, entries, meta, stream)
    rec["small_batch"] = [small_batch_pass(torch, g, synth, entries, stream, n)
                          for n in SMALL_BATCH_TOKENS]
    rec["fused_layers"] = fused_layer_pass(torch, g, synth, entries, stream)
    rec["other_types"] = other_types_pass(torch, g, synth)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
