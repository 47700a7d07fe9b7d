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
dominant kernel (the Q4_K lanes-along-K GEMV), the CPU oracle timed on bounded
samples of the same workloads, and labelled extras: the pass time
distribution, the streaming-read probe (whole-device read ceiling) and the
same probe run as the pass runs (one launch per stage: the floor of a
launch-per-stage pass), the single-matrix GEMVs (256x512, 2048x2048,
11008x2048 Q8_0; 11008x2048, 2048x11008 Q4_K) streamed from HBM, the bf16
MFMA prefill pass over the same 36-layer weights (N = 512 tokens), the fp32
small-batch passes (the same 253 matrices times 8, 32 and 64 activation
vectors), batch-1 GEMV passes over the same shapes stored as Q4_0 and Q6_K,
and the 36 layers as decode layers with RMSN, SiLU(gate) * up and the
residual adds fused into the GEMVs against the same steps as separate kernels.

    python bench.py --timeline

prints per-stage wave timelines of the decode pass instead (the instrumented
library libgguf_qk_timeline.so, built with `build --timeline`).

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
_CSRC = "gguf_block_quant_dequant_amd/csrc/"
# Counter summaries under profiles/ that bench.py reads HBM traffic from, and
# the sources each was measured on: a summary counts only while their hash
# matches (its "source_sha256:" line), else the traffic field is null.
PROFILES = {
    "decode": ("gemv_lk_kernel_decode_stream_traffic.md",
               ["gemv_lk.hpp", "device_common.hpp", "lk.hip", "lk_typed.hip"]),
    "other": ("other_types_lk_traffic.md",
              ["gemv_lk.hpp", "device_common.hpp", "lk.hip", "lk_typed.hip"]),
    "small_batch": ("small_batch_traffic.md",
                    ["gemv_sbw.hpp", "gemv_small_batch.hpp", "device_common.hpp", "gguf_qk.hip"]),
    "prefill": ("gemm_q4_k_db_kernel_prefill_mfma.md", ["gemm.hpp", "device_common.hpp", "gguf_qk.hip", "launch.hpp"]),
}
SMALL_BATCH_TOKENS = (8, 32, 64)


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
    ap.add_argument("--single-only", action="store_true",
                    help="only the single-matrix GEMVs (256x512, 2048x2048, 11008x2048 Q8_0; "
                         "11008x2048, 2048x11008 Q4_K)")
    ap.add_argument("--timeline", action="store_true",
                    help="per-wave stage timeline of the decode pass (needs the instrumented "
                         "library, libgguf_qk_timeline.so)")
    ap.add_argument("--stage-times", action="store_true",
                    help="per stage kind (q+k+v, o, gate+up, down, head): the 36 launches of that kind "
                         "alone, back to back in a HIP graph, microseconds per launch")
    ap.add_argument("--timeline-raw", default=None,
                    help="with --timeline: also save the raw per-wave records of the pass (.npz)")
    return ap.parse_args()


def kernel_source_sha(sources):
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, _CSRC + p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(profile, key):
    """HBM bytes (`key` of the committed counter summary of `profile`), if the
    summary was taken on the current sources; else None."""
    name, sources = PROFILES[profile]
    try:
        text = open(os.path.join(ROOT, "profiles", name)).read()
    except OSError:
        return None
    kv = dict(re.findall(r"^([a-z_0-9]+):\s*(\S+)\s*$", text, flags=re.M))
    if kv.get("source_sha256") != kernel_source_sha(sources):
        return None
    try:
        return float(kv[key])
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


def latency_probe(torch, g):
    """Dependent-load latency (gguf_qk_probe_latency): one wave whose lanes each
    follow a chain i -> (A i + C) mod n (a single cycle over the whole buffer:
    A = 1 mod 4, C odd, n a power of two), over buffers sized for the L2 and
    the Infinity Cache (timed after an untimed chase over the same lines), and
    over 2 GiB for HBM (timed cold, after a streaming read of another 2 GiB has
    pushed the chain's lines out of the caches); then the HBM chase on a second
    stream while streaming-read probes run on the first. ns per dependent load
    from the kernel's own clock (100 MHz)."""
    dev = "cuda:0"
    A, C = 0x9E3779B1, 0x7F4A7C15

    def chain(n):
        i = torch.arange(n, dtype=torch.int64, device=dev)
        return ((i * A + C) & (n - 1)).to(torch.int32)

    def ns(out, steps):
        torch.cuda.synchronize()
        return round(int(out[0].item()) * 10.0 / steps, 1)

    levels = []
    for label, nbytes, steps in (("1 MiB (L2)", 1 << 20, 4096), ("64 MiB (Infinity Cache)", 64 << 20, 4096)):
        nxt = chain(nbytes // 4)
        g.gguf_qk_probe_latency(nxt, steps)
        levels.append({"label": label, "bytes": nbytes, "steps": steps,
                       "ns_per_load": ns(g.gguf_qk_probe_latency(nxt, steps), steps)})
        del nxt
    nbytes = 2 << 30
    nxt = chain(nbytes // 4)
    other = torch.zeros(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    g.gguf_qk_probe_read(other, sink)
    levels.append({"label": "2 GiB (HBM), cold", "bytes": nbytes, "steps": 2048,
                   "ns_per_load": ns(g.gguf_qk_probe_latency(nxt, 2048), 2048)})
    # loaded: 24 read probes over the other 2 GiB on one stream, then the chase
    # (further along the chain) on a second stream (both default priority)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(24):
        g.gguf_qk_probe_read(other, sink, stream=s1)
    out = g.gguf_qk_probe_latency(nxt, 512, stream=s2)
    levels.append({"label": "2 GiB (HBM) while streaming reads run on another stream", "bytes": nbytes,
                   "steps": 512, "ns_per_load": ns(out, 512)})
    del nxt, other
    return {"label": "dependent-load latency: one wave, 64 independent chains, each load waiting for the one "
                     "before (the kernel's 100 MHz clock)", "levels": levels}


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
                         "frac": round(tflops / BF16_DENSE_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic("prefill", "hbm_bytes_per_launch")}}


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
            # (per pass: achieved = the pass's weight bytes / its time, traffic =
            # the pass's HBM bytes)
            "roofline": {"bound": "hbm",
                         "kernel": "gemv_sbw_kernel" if n_tokens <= 32 else "gemv_small_batch_kernel",
                         "basis": "pass",
                         "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "traffic": recorded_traffic("small_batch", f"hbm_bytes_per_pass_{n_tokens}")}}


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
    # fused: each RMSN scale from the producer's partial sums of squares
    # (mode "ss": ss_out -> scale_ss) or from the producer's output itself
    # (mode "v": scale_v, no ss_out and no row-group completion)
    def build_fused(mode):
        hw, ss = e_(H), e_(H // 64)
        ents, eps, h = [], [], h0
        for li, L in enumerate(layers):
            st = 4 * li
            q, k, v = e_(H), e_(KV), e_(KV)
            h1, hw2, ss2, gg, uu, act = e_(H), e_(H), e_(H // 64), e_(F), e_(F), e_(F)
            h2, hw3, ss3 = e_(H), e_(H), e_(H // 64)
            sc = {"scale_ss": ss, "eps": EPS} if mode == "ss" else {"scale_v": h, "eps": EPS}
            for name, y in (("q", q), ("k", k), ("v", v)):
                ents.append((g.TYPE_Q4_K, L[name], hw, y, st))
                eps.append(dict(sc))
            ents.append((g.TYPE_Q4_K, L["o"], q, h1, st + 1))
            eps.append({"residual": h, "norm_w": norms[2 * li + 1], "norm_out": hw2,
                        **({"ss_out": ss2} if mode == "ss" else {})})
            sc2 = {"scale_ss": ss2, "eps": EPS} if mode == "ss" else {"scale_v": h1, "eps": EPS}
            ents.append((g.TYPE_Q4_K, L["gate"], hw2, gg, st + 2))
            eps.append({**sc2, "pair": 1, "act": act})
            ents.append((g.TYPE_Q4_K, L["up"], hw2, uu, st + 2))
            eps.append({**sc2, "pair": 2, "act": act})
            nxt = norms[2 * (li + 1)] if li + 1 < len(layers) else norms[0]
            ents.append((g.TYPE_Q4_K, L["down"], act, h2, st + 3))
            eps.append({"residual": h1, "norm_w": nxt, "norm_out": hw3,
                        **({"ss_out": ss3} if mode == "ss" else {})})
            h, hw, ss = h2, hw3, ss3
        fb = g.GemvBatch(ents, eps)
        hw0, ss0 = ents[0][2], e_(H // 64) if mode == "v" else eps[0]["scale_ss"]

        def fused():
            g.gguf_rmsnorm_prep_f32(h0, norms[0], hw0, ss0, stream=stream)
            g.gguf_qmatvec_batch(fb, stream)
        return fused

    fused, fused_v = build_fused("ss"), build_fused("v")

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
                    "and the residual adds; attention stood in by q (not measured); HIP graphs; fused: "
                    "RMSN scales from the producers' partial sums (ss_out), fused_scale_v: from the "
                    "producers' output vectors (scale_v)",
           "layers": len(layers)}
    wbytes = sum(e[1].numel() for e in q4)
    for name, fn, launches in (("fused", fused, 4 * len(layers) + 1), ("fused_scale_v", fused_v, 4 * len(layers) + 1),
                               ("unfused", unfused, 9 * len(layers))):
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
                                 "frac": round(gbps / HBM_PEAK_GBPS, 4), "basis": "pass",
                                 "traffic": recorded_traffic("other", f"hbm_bytes_per_pass_{name}")}})
        del graph, batch, ents, keep, layer
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def stage_floor(torch, g, meta, total_bytes, stream, reps=10):
    """The streaming-read probe run as the pass runs: one probe launch per
    stage over that stage's weight bytes (distinct ranges of one buffer as
    large as the whole stream), in pass order, as a HIP graph. It bounds what
    a pass of one launch per stage can reach on this device: launch gaps and
    each launch's ramp-up and tail with no decoding or arithmetic at all."""
    buf = torch.zeros(total_bytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    ranges, off = [], 0
    for (_, _, nb) in meta:
        ranges.append((off, nb))
        off += nb

    def run():
        for o, nb in ranges:
            g.gguf_qk_probe_read(buf[o:o + nb], sink, stream=stream)

    graph = capture(torch, run, stream)
    t = time_replays(torch, graph, stream, reps)
    ms = sorted(t)[len(t) // 2]
    del graph, buf
    gbps = total_bytes / (ms / 1e3) / 1e9
    return {"label": "read probe over the pass's stage sizes (36 x {3.5, 2.4, 25.4, 12.7} MB + the "
                     "279 MB head), one launch per stage, HIP graph: the floor of a launch-per-stage pass",
            "launches": len(ranges), "ms_per_pass": round(ms, 4), "GBps": round(gbps, 1),
            "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)}


def single_matrix_pass(torch, g, synth, reps=5):
    """Single GEMVs (256x512, 2048x2048, 11008x2048 Q8_0; 11008x2048 and
    2048x11008 Q4_K): each matrix copied to enough byte-identical copies at
    distinct addresses to pass 1 GiB (at most 4096 copies, always more than the
    256 MB Infinity Cache), one launch per copy back to back in a HIP graph, so
    every launch streams its matrix from HBM. Also a labelled cache-resident
    figure (one copy, launched repeatedly). Returns (records, outputs of copy 0
    with their inputs, for the CPU leg's error check)."""
    dev = "cuda:0"
    recs, outs = [], []
    stream = torch.cuda.Stream()
    for m in synth.SINGLE_MATRICES:
        w, x = synth.single_matrix(m)
        nb = w.nbytes
        copies = min(4096, -(-(1 << 30) // nb))
        big = torch.empty(copies * nb, dtype=torch.uint8, device=dev)
        W0 = torch.from_numpy(w.reshape(-1)).to(dev)
        big.view(copies, nb).copy_(W0.unsqueeze(0).expand(copies, nb))
        X = torch.from_numpy(x).to(dev)
        Y = torch.empty(m.rows, dtype=torch.float32, device=dev)
        f = g.gguf_qmatvec_q8_0 if m.fmt == synth.Q8_0 else g.gguf_qmatvec_q4_k
        views = [big[i * nb:(i + 1) * nb].view(m.rows, nb // m.rows) for i in range(copies)]

        def run_cold():
            for V in views:
                f(V, X, Y, stream=stream)

        gc = capture(torch, run_cold, stream)
        tc = time_replays(torch, gc, stream, reps)
        us = sorted(tc)[len(tc) // 2] * 1e3 / copies
        del gc
        hot_n = 256

        def run_hot():
            for _ in range(hot_n):
                f(views[0], X, Y, stream=stream)

        gh = capture(torch, run_hot, stream)
        th = time_replays(torch, gh, stream, reps)
        hot_us = sorted(th)[len(th) // 2] * 1e3 / hot_n
        del gh
        f(views[0], X, Y, stream=stream)
        torch.cuda.synchronize()
        outs.append((m, w, x, Y.cpu().numpy()))
        gbps = nb / (us / 1e6) / 1e9
        recs.append({"label": m.label, "bytes": nb, "copies": copies, "us_per_gemv": round(us, 3),
                     "GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
                     "tokens_per_s_equiv_note": "single matrix: 1 / us_per_gemv",
                     "cache_resident": {"label": "one copy launched repeatedly (L2 / Infinity Cache)",
                                        "us_per_gemv": round(hot_us, 3),
                                        "GBps": round(nb / (hot_us / 1e6) / 1e9, 1)}})
        del big, views, W0
        torch.cuda.empty_cache()
    return recs, outs


def stage_times(torch, g, entries, meta, stream, reps=10):
    """Microseconds per launch of each stage kind, its launches of the pass
    alone back to back in a HIP graph (events on the replay stream), beside
    the streaming-read probe over the same stage sizes (the floor of a launch
    of that size)."""
    kinds = {}
    for tid, W, x, y, si in entries:
        layer, names, nb = meta[si]
        kind = "head" if layer < 0 else "+".join(names)
        kinds.setdefault(kind, {}).setdefault(si, []).append((tid, W, x, y, si))
    out = {}
    for kind, stages in kinds.items():
        ents = [e for si in sorted(stages) for e in stages[si]]
        batch = g.GemvBatch(ents)
        graph = capture(torch, lambda: g.gguf_qmatvec_batch(batch, stream), stream)
        t = time_replays(torch, graph, stream, reps)
        ms = sorted(t)[len(t) // 2]
        nb = sum(e[1].numel() for e in ents)
        # the read probe over the same stage sizes, one launch per stage
        sizes = [sum(e[1].numel() for e in stages[si]) for si in sorted(stages)]
        buf = torch.zeros(sum(sizes), dtype=torch.uint8, device="cuda:0")
        sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
        offs = [sum(sizes[:i]) for i in range(len(sizes))]

        def probe():
            for o, n in zip(offs, sizes):
                g.gguf_qk_probe_read(buf[o:o + n], sink, stream=stream)

        pg = capture(torch, probe, stream)
        tp = time_replays(torch, pg, stream, reps)
        pms = sorted(tp)[len(tp) // 2]
        out[kind] = {"launches": len(stages), "us_per_launch": round(ms * 1e3 / len(stages), 3),
                     "GBps": round(nb / (ms / 1e3) / 1e9, 1),
                     "probe_us_per_launch": round(pms * 1e3 / len(stages), 3)}
        del graph, pg, buf
    return out


def stage_timeline(torch, g, entries, meta, stream, reps=3, raw_path=None):
    """Per-wave time stamps of the decode pass's kernels (instrumented build):
    per stage kind, medians over the layers of the launch gap, the wave start
    skew and the times (from the kernel's first wave) at which the waves had
    issued their loads, staged x, stored their first row step, computed their
    last one, and ended."""
    import numpy as np
    first_w = {}
    for tid, W, x, y, si in entries:
        first_w.setdefault(si, W.data_ptr())
    slot = g.gguf_qk_timeline_setup(first_w.values())
    batch = g.GemvBatch(entries)
    graph = capture(torch, lambda: g.gguf_qmatvec_batch(batch, stream), stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            graph.replay()
    torch.cuda.synchronize()
    recs_u32 = g.gguf_qk_timeline_fetch()
    if raw_path:
        order = sorted(first_w)
        np.savez_compressed(raw_path, recs=recs_u32[[slot[first_w[si]] for si in order]],
                            stage=np.array(order), layer=np.array([meta[si][0] for si in order]),
                            kind=np.array(["head" if meta[si][0] < 0 else "+".join(meta[si][1]) for si in order]))
    recs = recs_u32.astype(np.int64)
    del graph
    base = None
    rows = []
    for si in sorted(first_w):
        r = recs[slot[first_w[si]]]
        live = r[:, 0] != 0
        t = r[live][:, :6]
        if base is None:
            base = int(t[:, 0].min())
        t = (t - base) % (1 << 32)
        start, end = int(t[:, 0].min()), int(t[:, 5].max())
        layer, names, nb = meta[si]
        kind = "head" if layer < 0 else "+".join(names)
        rows.append((si, kind, start, end, t, int(live.sum()), nb))
    out = {}
    for i, (si, kind, start, end, t, waves, nb) in enumerate(rows):
        prev_end = rows[i - 1][3] if i else None
        rel = t - start
        d = out.setdefault(kind, {"waves": waves, "weight_bytes": nb, "gap": [], "span": [], "skew_p50": [],
                                  "skew_max": [], "issued": [], "staged": [], "first": [], "last": [],
                                  "last_max": [], "end": []})
        if prev_end is not None:
            d["gap"].append(start - prev_end)
        d["span"].append(end - start)
        d["skew_p50"].append(np.median(rel[:, 0]))
        d["skew_max"].append(rel[:, 0].max())
        d["issued"].append(np.median(rel[:, 1]))
        d["staged"].append(np.median(rel[:, 2]))
        d["first"].append(np.median(rel[:, 3]))
        d["last"].append(np.median(rel[:, 4]))
        d["last_max"].append(rel[:, 4].max())
        d["end"].append(rel[:, 5].max())
    res = {}
    for kind, d in out.items():
        res[kind] = {"waves": d["waves"], "weight_bytes": d["weight_bytes"], "launches": len(d["span"])}
        for k, v in d.items():
            if isinstance(v, list) and v:
                res[kind][k + "_us"] = round(float(np.median(v)) * 0.01, 3)   # 100 MHz clock
    return {"timeline": res, "unit": "us from the kernel's first wave (gap: from the previous "
                                      "kernel's last wave); medians over the launches of each kind",
            "clock": "s_memrealtime, 100 MHz"}


def cpu_baseline(single_outs=None):
    """The oracle as it stands (oracle/: NumPy, weights decoded to fp64, fp64
    products; not tuned) on this host's cores, on bounded samples:
    - decode (the headline workload): layers 0..3's seven Q4_K GEMVs and head
      rows 0..16383 (Q8_0), once on one thread and once spread over every core
      this process may use (one GEMV per task, one BLAS thread per task);
      weight bytes per second, and tokens/s-equivalent of the whole pass at
      that rate;
    - the single matrices in full on one thread, with the GPU result's
      floored error against the oracle's;
    - prefill: rows 0..255 of layer 0's seven tensors times 512 bf16 tokens on
      every core, linearly extrapolated to the 36-layer pass (labelled)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    import synth

    ncpu = os.cpu_count()
    cores = len(os.sched_getaffinity(0))
    blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    n_layers, head_rows = 4, 16384
    stages = synth.decode_stream(n_layers=n_layers, head=False, threads=4)
    hw = synth.q8_0_weights(synth.rng_for(synth.DECODE_CFG_ID, 1000, synth.TENSOR_IDS["head"]),
                            head_rows, synth.HIDDEN)
    hx = synth.activations_f32(synth.rng_for(synth.DECODE_CFG_ID, 1000, 100), synth.HIDDEN)
    tasks = [(gm.fmt, w, gm.rows, gm.cols, st.x) for st in stages for gm, w in zip(st.gemvs, st.weights)]
    tasks.append((synth.Q8_0, hw, head_rows, synth.HIDDEN, hx))
    nbytes = sum(t[1].nbytes for t in tasks)

    def one(t):
        fmt, w, rows, cols, x = t
        deq = oracle.dequant_q8_0_f32 if fmt == synth.Q8_0 else oracle.dequant_q4_k_f32
        return oracle.matvec_f64(deq(w, rows, cols), x)

    with threadpool_limits(1):
        t0 = time.perf_counter()
        for t in tasks:
            one(t)
        dt1 = time.perf_counter() - t0
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=cores) as ex:
            list(ex.map(one, sorted(tasks, key=lambda t: -t[1].nbytes)))
        dtn = time.perf_counter() - t0
    pass_bytes = synth.decode_stream_bytes()
    g1, gn = nbytes / dt1 / 1e9, nbytes / dtn / 1e9

    singles = []
    if single_outs:
        with threadpool_limits(1):
            for m, w, x, y_gpu in single_outs:
                t0 = time.perf_counter()
                ref = one((m.fmt, w, m.rows, m.cols, x))
                dt = time.perf_counter() - t0
                err, finite = oracle.floored_rel_err(y_gpu, ref)
                singles.append({"label": m.label, "oracle_s_1thread": round(dt, 3),
                                "oracle_GBps_1thread": round(w.nbytes / dt / 1e9, 4),
                                "gpu_max_floored_err": float(f"{err:.3e}"), "gpu_finite": bool(finite)})

    # prefill sample: 256 rows of each of layer 0's tensors x 512 bf16 tokens
    pf_rows, pf_tokens = 256, 512
    gen_rows = {}
    for st in stages[:4]:
        for gm, w in zip(st.gemvs, st.weights):
            gen_rows[gm.name] = (gm, w[:pf_rows])
    xb = {c: synth.activations_bf16_bits(synth.rng_for(synth.PREFILL_CFG_ID, 0, c), pf_tokens, c)
          for c in (synth.HIDDEN, synth.FFN)}

    def pf(item):
        gm, w = item
        return oracle.matmul_bf16_x_f64(xb[gm.cols], oracle.dequant_q4_k_f32(w, pf_rows, gm.cols))

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as ex:
        list(ex.map(pf, gen_rows.values()))
    dtp = time.perf_counter() - t0
    sample_flop = sum(2.0 * pf_tokens * pf_rows * gm.cols for gm, _ in gen_rows.values())
    pass_flop = 2.0 * pf_tokens * synth.N_LAYERS * sum(gm.rows * gm.cols for st in synth.LAYER_STAGES
                                                        for gm in st)
    pf_s = dtp * pass_flop / sample_flop
    return {"value": round(gn, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"decode: layers 0..{n_layers - 1} q,k,v,o,gate,up,down (Q4_K) + head rows "
                      f"0..{head_rows - 1} (Q8_0), {nbytes} weight bytes, one GEMV per task over {cores} "
                      f"threads in {dtn:.2f} s",
            "tokens_per_s_equiv": round(gn * 1e9 / pass_bytes, 5),
            "one_thread": {"GBps": round(g1, 4), "s": round(dt1, 2),
                           "tokens_per_s_equiv": round(g1 * 1e9 / pass_bytes, 5)},
            "host": {"os_cpu_count": ncpu, "sched_getaffinity": cores, "blas": blas},
            "single_matrices": singles,
            "prefill": {"label": f"oracle prefill, rows 0..{pf_rows - 1} of layer 0's 7 tensors x "
                                 f"{pf_tokens} bf16 tokens on {cores} threads, linearly extrapolated to "
                                 "the 36-layer pass (extrapolated, not measured whole)",
                        "sample_s": round(dtp, 3), "pass_s_extrapolated": round(pf_s, 1),
                        "TFLOPs": round(pass_flop / pf_s / 1e12, 5)}}


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
    if args.timeline:
        os.environ["GGUF_QK_TIMELINE"] = "1"   # the instrumented library
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
    if args.single_only:
        recs, _ = single_matrix_pass(torch, g, synth)
        print(json.dumps(recs), flush=True)
        return
    if args.timeline:
        print(json.dumps(stage_timeline(torch, g, entries, meta, stream, raw_path=args.timeline_raw)), flush=True)
        return
    if args.stage_times:
        print(json.dumps(stage_times(torch, g, entries, meta, stream)), flush=True)
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
    traffic = recorded_traffic("decode", "hbm_bytes_per_launch")
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

    ceiling = probe_ceiling(torch, g)
    rec["read_probe_GBps"] = round(ceiling, 1)
    rec["pct_of_read_probe"] = round(100 * gbps / ceiling, 2)
    rec["latency_probe"] = latency_probe(torch, g)
    rec["stage_floor"] = stage_floor(torch, g, meta, total_bytes, stream)
    rec["pct_of_stage_floor"] = round(100 * rec["stage_floor"]["ms_per_pass"] / ms, 2)
    singles, single_outs = single_matrix_pass(torch, g, synth)
    rec["single_matrices"] = singles
    rec["prefill"] = prefill_pass(torch, g, synth, entries, meta, stream)
    rec["small_batch"] = [small_batch_pass(torch, g, synth, entries, stream, n)
                          for n in SMALL_BATCH_TOKENS]
    rec["fused_layers"] = fused_layer_pass(torch, g, synth, entries, stream)
    rec["other_types"] = other_types_pass(torch, g, synth)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(single_outs)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
