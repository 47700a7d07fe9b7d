"""The decode GEMVs with the neighbouring steps fused (gguf_qmatvec_batch_ep)
and the standalone layer steps, through the C ABI, against the oracle.

Each fused part is checked where it is computed: the residual add and the
norm-preparation outputs of a producing GEMV (bit-identical to the standalone
preparation kernel run on the same y), the RMSN scale of a consuming GEMV (y
against W RMSN(v) of the oracle), the gate/up pair (act against SiLU(g) u of
the GPU's own g and u). Then two chained layers, fused and unfused, stage by
stage against the oracle, agreeing with each other, repeatable and identical
under HIP-graph replay. Bar: floored relative error 1e-3 (the fp32 GEMV bar)."""

import numpy as np
import pytest
import torch

import gguf_block_quant_dequant_amd as g
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-3
EPS = 1e-6


def say(*a):
    print(*a, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def empty(n):
    return torch.empty(n, dtype=torch.float32, device=DEV)


def check(got, ref, what, tol=TOL):
    e, ok = oracle.floored_rel_err(got, ref)
    assert ok and e <= tol, (what, e)
    return e


def weights(fmt, rng, rows, cols):
    if fmt == "q4_k":
        w = synth.q4_k_weights(rng, rows, cols)
        return g.TYPE_Q4_K, w, oracle.dequant_q4_k_f32(w, rows, cols)
    w = synth.q8_0_weights(rng, rows, cols)
    return g.TYPE_Q8_0, w, oracle.dequant_q8_0_f32(w, rows, cols)


@pytest.mark.parametrize("fmt,rows,cols", [("q4_k", 2048, 2048), ("q4_k", 2048, 11008),
                                           ("q4_k", 300, 11008), ("q4_k", 130, 2304),
                                           ("q4_k", 100, 512), ("q8_0", 2048, 2048),
                                           ("q8_0", 777, 4096)])
def test_residual_and_norm_outputs(fmt, rows, cols):
    rng = np.random.default_rng([rows, cols, 5])
    tid, w, w32 = weights(fmt, rng, rows, cols)
    x = synth.activations_f32(rng, cols)
    r = synth.activations_f32(rng, rows)
    nw = rng.uniform(0.5, 1.5, rows).astype(np.float32)
    say("residual + norm", fmt, rows, cols)
    y, no, ss = empty(rows), empty(rows), empty((rows + 63) // 64)
    b = g.GemvBatch([(tid, dev(w), dev(x), y, 0)],
                    [{"residual": dev(r), "norm_w": dev(nw), "norm_out": no, "ss_out": ss}])
    g.gguf_qmatvec_batch(b)
    if fmt == "q4_k" and cols // 256 not in (1, 2, 4, 8, 16):
        # rows of other super-block counts: the split-K-in-block kernel with
        # the epilogue, its 64-row groups spanning blocks
        assert g.gguf_qk_last_launch() == g.LAUNCH_LKS
    yg = host(y)
    check(yg, r.astype(np.float64) + oracle.matvec_f64(w32, x), "y")
    vw, ss2 = g.gguf_rmsnorm_prep_f32(y, dev(nw))
    assert np.array_equal(host(no).view(np.uint32), host(vw).view(np.uint32))
    assert np.array_equal(host(ss).view(np.uint32), host(ss2).view(np.uint32))
    y64 = yg.astype(np.float64)
    want = np.add.reduceat(y64 * y64, np.arange(0, rows, 64))
    assert np.allclose(host(ss), want, rtol=1e-5, atol=0)


@pytest.mark.parametrize("fmt,rows,cols", [("q4_k", 2048, 2048), ("q4_k", 512, 11008),
                                           ("q8_0", 1000, 2048)])
def test_rmsnorm_scale_of_the_input(fmt, rows, cols):
    rng = np.random.default_rng([rows, cols, 6])
    tid, w, w32 = weights(fmt, rng, rows, cols)
    v = (3.0 * rng.standard_normal(cols)).astype(np.float32)
    nw = rng.uniform(0.5, 1.5, cols).astype(np.float32)
    vw, ss = g.gguf_rmsnorm_prep_f32(dev(v), dev(nw))
    y = empty(rows)
    b = g.GemvBatch([(tid, dev(w), vw, y, 0)], [{"scale_ss": ss, "eps": EPS}])
    g.gguf_qmatvec_batch(b)
    check(host(y), oracle.matvec_f64(w32, oracle.rmsnorm_f64(v, nw, EPS)), "scaled y")


@pytest.mark.parametrize("rows,cols", [((2048, 512, 512), 2048), ((300, 100, 37), 2048),
                                       ((64, 1, 130), 512), ((200, 70, 90), 2304)])
def test_rmsnorm_scale_of_three_gemvs_of_one_input(rows, cols):
    # the fused q/k/v: three matrices of one scaled x in one launch
    rng = np.random.default_rng([sum(rows), cols, 9])
    v = (3.0 * rng.standard_normal(cols)).astype(np.float32)
    nw = rng.uniform(0.5, 1.5, cols).astype(np.float32)
    vw, ss = g.gguf_rmsnorm_prep_f32(dev(v), dev(nw))
    xn = oracle.rmsnorm_f64(v, nw, EPS)
    ws = [synth.q4_k_weights(rng, r, cols) for r in rows]
    ys = [empty(r) for r in rows]
    say("three scaled GEMVs", rows, cols)
    b = g.GemvBatch([(g.TYPE_Q4_K, dev(w), vw, y, 0) for w, y in zip(ws, ys)],
                    [{"scale_ss": ss, "eps": EPS}] * 3)
    g.gguf_qmatvec_batch(b)
    if cols // 256 in (1, 2, 4, 8, 16):
        assert g.gguf_qk_last_launch() == g.LAUNCH_LK_THREE
    for w, y, r in zip(ws, ys, rows):
        check(host(y), oracle.matvec_f64(oracle.dequant_q4_k_f32(w, r, cols), xn), ("scaled y", r))


@pytest.mark.parametrize("rows,cols", [(11008, 2048), (100, 512), (300, 11008)])
def test_gate_up_pair_writes_the_activation(rows, cols):
    rng = np.random.default_rng([rows, cols, 7])
    wg = synth.q4_k_weights(rng, rows, cols)
    wu = synth.q4_k_weights(rng, rows, cols)
    x = synth.activations_f32(rng, cols) * np.float32(0.05)
    yg_, yu_, act = empty(rows), empty(rows), empty(rows)
    X = dev(x)
    b = g.GemvBatch([(g.TYPE_Q4_K, dev(wg), X, yg_, 0), (g.TYPE_Q4_K, dev(wu), X, yu_, 0)],
                    [{"pair": 1, "act": act}, {"pair": 2, "act": act}])
    for rep in range(2):   # the pair counters are left at zero for the next call
        act.fill_(float("nan"))
        g.gguf_qmatvec_batch(b)
        if cols <= 4096:   # both rows of an index in one wave, descriptors preloaded
            assert g.gguf_qk_last_launch() == g.LAUNCH_LK_TWO
        gv, uv = host(yg_), host(yu_)
        check(gv, oracle.matvec_f64(oracle.dequant_q4_k_f32(wg, rows, cols), x), "gate")
        check(uv, oracle.matvec_f64(oracle.dequant_q4_k_f32(wu, rows, cols), x), "up")
        check(host(act), oracle.swiglu_f64(gv, uv), "act", tol=1e-5)


def test_standalone_layer_steps():
    rng = np.random.default_rng(8)
    n = 11008
    a = (2.0 * rng.standard_normal(n)).astype(np.float32)
    b = rng.standard_normal(n).astype(np.float32)
    nw = rng.uniform(0.5, 1.5, n).astype(np.float32)
    A, B, NW = dev(a), dev(b), dev(nw)
    check(host(g.gguf_rmsnorm_f32(A, NW, EPS)), oracle.rmsnorm_f64(a, nw, EPS), "rmsnorm", tol=1e-5)
    check(host(g.gguf_swiglu_f32(A, B)), oracle.swiglu_f64(a, b), "swiglu", tol=1e-5)
    assert np.array_equal(host(g.gguf_add_f32(A, B)), a + b)
    vw, ss = g.gguf_rmsnorm_prep_f32(A, NW)
    assert np.array_equal(host(vw), a * nw)
    a64 = a.astype(np.float64)
    assert np.allclose(host(ss), np.add.reduceat(a64 * a64, np.arange(0, n, 64)), rtol=1e-5, atol=0)
    # in place
    C = A.clone()
    g.gguf_add_f32(C, B, C)
    assert np.array_equal(host(C), a + b)


class Layer:
    """Seeded Q4_K weights of one layer at small shapes (H hidden, F ffn) and its
    two norm weight vectors."""

    def __init__(self, rng, H, F, KV):
        self.shapes = {"q": (H, H), "k": (KV, H), "v": (KV, H), "o": (H, H),
                       "gate": (F, H), "up": (F, H), "down": (H, F)}
        self.w = {k: synth.q4_k_weights(rng, r, c) for k, (r, c) in self.shapes.items()}
        self.w32 = {k: oracle.dequant_q4_k_f32(self.w[k], *self.shapes[k]) for k in self.w}
        self.d = {k: dev(v) for k, v in self.w.items()}
        self.attn_norm = rng.uniform(0.5, 1.5, H).astype(np.float32)
        self.ffn_norm = rng.uniform(0.5, 1.5, H).astype(np.float32)


def _layers(n_layers=2, H=2048, F=5632, KV=512):
    rng = np.random.default_rng(99)
    return [Layer(rng, H, F, KV) for _ in range(n_layers)], rng


def _fused_entries(layers, h0, H, F, KV, mode="ss"):
    """The fused chain as one batch: per layer 4 steps. The attention result
    (out of scope) is stood in by the q projection's output. mode "ss": each
    RMSN's scale from the producer's partial sums of squares (ss_out ->
    scale_ss); "v": from the producer's output vector itself (scale_v), the
    producers writing no ss_out."""
    T = {}
    ents, eps = [], []
    h = h0
    hw, ss = empty(H), empty(H // 64)
    T["h0"] = h0
    stage = 0
    first = True
    for li, L in enumerate(layers):
        q, k, v = empty(H), empty(KV), empty(KV)
        h1, hw2, ss2 = empty(H), empty(H), empty(H // 64)
        gg, uu, act = empty(F), empty(F), empty(F)
        h2, hw3, ss3 = empty(H), empty(H), empty(H // 64)
        if first:
            T["prep"] = (dev(L.attn_norm), hw, ss)
            first = False
        sc = {"scale_ss": ss, "eps": EPS} if mode == "ss" else {"scale_v": h, "eps": EPS}
        for name, y in (("q", q), ("k", k), ("v", v)):
            ents.append((g.TYPE_Q4_K, L.d[name], hw, y, stage))
            eps.append(dict(sc))
        stage += 1
        ents.append((g.TYPE_Q4_K, L.d["o"], q, h1, stage))
        eps.append({"residual": h, "norm_w": dev(L.ffn_norm), "norm_out": hw2,
                    **({"ss_out": ss2} if mode == "ss" else {})})
        sc2 = {"scale_ss": ss2, "eps": EPS} if mode == "ss" else {"scale_v": h1, "eps": EPS}
        stage += 1
        ents.append((g.TYPE_Q4_K, L.d["gate"], hw2, gg, stage))
        eps.append({**sc2, "pair": 1, "act": act})
        ents.append((g.TYPE_Q4_K, L.d["up"], hw2, uu, stage))
        eps.append({**sc2, "pair": 2, "act": act})
        stage += 1
        nxt = layers[li + 1].attn_norm if li + 1 < len(layers) else layers[li].attn_norm
        ents.append((g.TYPE_Q4_K, L.d["down"], act, h2, stage))
        eps.append({"residual": h1, "norm_w": dev(nxt), "norm_out": hw3,
                    **({"ss_out": ss3} if mode == "ss" else {})})
        stage += 1
        T[li] = dict(q=q, k=k, v=v, h1=h1, g=gg, u=uu, act=act, h2=h2)
        h, hw, ss = h2, hw3, ss3
    return g.GemvBatch(ents, eps), T


def _unfused(layers, h0, H, F, KV):
    """The same chain with standalone steps between plain GEMV launches."""
    out = {}
    h = h0
    for li, L in enumerate(layers):
        x1 = g.gguf_rmsnorm_f32(h, dev(L.attn_norm), EPS)
        q = g.gguf_qmatvec_q4_k(L.d["q"], x1, rows=H, cols=H)
        h1 = g.gguf_add_f32(h, g.gguf_qmatvec_q4_k(L.d["o"], q, rows=H, cols=H))
        x2 = g.gguf_rmsnorm_f32(h1, dev(L.ffn_norm), EPS)
        gg = g.gguf_qmatvec_q4_k(L.d["gate"], x2, rows=F, cols=H)
        uu = g.gguf_qmatvec_q4_k(L.d["up"], x2, rows=F, cols=H)
        act = g.gguf_swiglu_f32(gg, uu)
        h2 = g.gguf_add_f32(h1, g.gguf_qmatvec_q4_k(L.d["down"], act, rows=H, cols=F))
        out[li] = dict(q=q, h1=h1, g=gg, u=uu, act=act, h2=h2)
        h = h2
    return out


@pytest.mark.parametrize("n_layers,F,mode", [(2, 5632, "ss"), (1, 11008, "ss"), (2, 5632, "v"), (1, 11008, "v")])
def test_fused_layers_stage_by_stage(n_layers, F, mode):
    """Two chained layers at a narrower FFN, and one at the workload's FFN
    width (gate/up rows and down columns of 11008); each RMSN scale from the
    producer's partial sums (ss) or from the producer's output (v)."""
    H, KV = 2048, 512
    layers, rng = _layers(n_layers, H, F, KV)
    h0 = dev(synth.activations_f32(rng, H))
    batch, T = _fused_entries(layers, h0, H, F, KV, mode)
    nw0, hw, ss = T["prep"]
    say("fused chain:", batch.n, "GEMVs")
    g.gguf_rmsnorm_prep_f32(h0, nw0, hw, ss)
    g.gguf_qmatvec_batch(batch)
    h = host(h0)
    for li, L in enumerate(layers):
        t = {k: host(v) for k, v in T[li].items()}
        x1 = oracle.rmsnorm_f64(h, L.attn_norm, EPS)
        for name in ("q", "k", "v"):
            check(t[name], oracle.matvec_f64(L.w32[name], x1), f"L{li} {name}")
        check(t["h1"], h.astype(np.float64) + oracle.matvec_f64(L.w32["o"], t["q"]), f"L{li} h1")
        x2 = oracle.rmsnorm_f64(t["h1"], L.ffn_norm, EPS)
        check(t["g"], oracle.matvec_f64(L.w32["gate"], x2), f"L{li} gate")
        check(t["u"], oracle.matvec_f64(L.w32["up"], x2), f"L{li} up")
        check(t["act"], oracle.swiglu_f64(t["g"], t["u"]), f"L{li} act", tol=1e-5)
        check(t["h2"], t["h1"].astype(np.float64) + oracle.matvec_f64(L.w32["down"], t["act"]), f"L{li} h2")
        h = t["h2"]
    # the unfused chain gives the same layer outputs (to the fp32 bar)
    U = _unfused(layers, h0, H, F, KV)
    for li in range(len(layers)):
        for k in ("q", "h1", "g", "u", "act", "h2"):
            check(host(U[li][k]), host(T[li][k]).astype(np.float64), f"fused vs unfused L{li} {k}")
    # repeat: bit-identical; graph replays: identical
    last = n_layers - 1
    first = {k: host(v).copy() for k, v in T[last].items()}
    g.gguf_rmsnorm_prep_f32(h0, nw0, hw, ss)
    g.gguf_qmatvec_batch(batch)
    for k, v in T[last].items():
        assert np.array_equal(host(v).view(np.uint32), first[k].view(np.uint32)), k
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.gguf_rmsnorm_prep_f32(h0, nw0, hw, ss, stream=s)
        g.gguf_qmatvec_batch(batch, s)
    for _ in range(2):
        for v in T[last].values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in T[last].items():
            assert np.array_equal(host(v).view(np.uint32), first[k].view(np.uint32)), k
    g.gguf_qk_stream_release(s)
