"""Q4_0 and Q6_K through the C ABI against the oracle: dequantization
bit-exact, GEMV within the fp32 bar (1e-3 floored), exact where every partial
sum is an integer, repeat calls bit-identical. Row lengths with an odd number
of blocks put every other row (and, for Q4_0, every other block) at a 2-byte
offset from a 4-byte boundary, the realignment case."""

import numpy as np
import pytest
import torch

import gguf_block_quant_dequant_amd as g
import oracle
import synth
from oracle.formats import pack_q4_0_block, pack_q6_k_block

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_F32 = 1e-3


def say(*a):
    print(*a, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same_bits(a, b):
    a = np.asarray(a, np.float32).ravel()
    b = np.asarray(b, np.float32).ravel()
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (a.view(np.uint32) == b.view(np.uint32))))


FMTS = {"q4_0": (synth.q4_0_weights, oracle.dequant_q4_0_f32, g.dequant_q4_0, g.gguf_qmatvec_q4_0),
        "q6_k": (synth.q6_k_weights, oracle.dequant_q6_k_f32, g.dequant_q6_k, g.gguf_qmatvec_q6_k)}


@pytest.mark.parametrize("fmt,rows,cols", [("q4_0", 1, 32), ("q4_0", 7, 96), ("q4_0", 33, 160),
                                           ("q4_0", 300, 2048), ("q4_0", 64, 11008),
                                           ("q6_k", 1, 256), ("q6_k", 5, 768), ("q6_k", 9, 2816),
                                           ("q6_k", 40, 11008), ("q6_k", 200, 2048)])
def test_dequant_bit_exact(fmt, rows, cols):
    gen, ref, fn, _ = FMTS[fmt]
    w = gen(np.random.default_rng([rows, cols, 1]), rows, cols)
    say("dequant", fmt, rows, cols)
    got = host(fn(dev(w), rows=rows, cols=cols))
    assert same_bits(got, ref(w, rows, cols))


def test_dequant_q4_0_every_scale_and_code():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    q = [(i * 7) % 16 for i in range(32)]
    proto = np.frombuffer(pack_q4_0_block(0, q), np.uint8)
    blk = np.tile(proto, (65536, 1))
    blk[:, 0] = bits & 255
    blk[:, 1] = bits >> 8
    raw = blk.reshape(65536 // 2, 36)        # two blocks per row: rows 36 bytes, odd blocks at +2 mod 4
    got = host(g.dequant_q4_0(dev(raw), rows=65536 // 2, cols=64))
    assert same_bits(got, oracle.dequant_q4_0_f32(raw, 65536 // 2, 64))


def test_dequant_q6_k_extreme_fields():
    rng = np.random.default_rng(9)
    blocks = []
    for d_bits in (0x0001, 0x03FF, 0x3C00, 0x7BFF, 0xFBFF, 0x8000):
        sc = [int(v) for v in rng.integers(-128, 128, 16)]
        sc[0], sc[1] = -128, 127
        code = [int(v) for v in rng.integers(0, 64, 256)]
        code[0], code[1] = 0, 63
        blocks.append(pack_q6_k_block(d_bits, sc, code))
    raw = np.frombuffer(b"".join(blocks), np.uint8)
    got = host(g.dequant_q6_k(dev(raw), rows=3, cols=512))
    assert same_bits(got, oracle.dequant_q6_k_f32(raw, 3, 512))


@pytest.mark.parametrize("fmt,rows,cols", [("q4_0", 1, 32), ("q4_0", 5, 96), ("q4_0", 300, 2048),
                                           ("q4_0", 3, 4128), ("q4_0", 70, 4608), ("q4_0", 9, 12288),
                                           ("q4_0", 9, 12544),
                                           ("q4_0", 2048, 11008), ("q4_0", 11008, 2048),
                                           ("q6_k", 1, 256), ("q6_k", 7, 768), ("q6_k", 333, 2816),
                                           ("q6_k", 2048, 11008), ("q6_k", 11008, 2048)])
def test_gemv_matches_oracle(fmt, rows, cols):
    gen, ref, _, fn = FMTS[fmt]
    rng = np.random.default_rng([rows, cols, 2])
    w = gen(rng, rows, cols)
    x = synth.activations_f32(rng, cols)
    say("gemv", fmt, rows, cols)
    Wd, xd = dev(w), dev(x)
    y = host(fn(Wd, xd, rows=rows, cols=cols))
    yref = oracle.matvec_f64(ref(w, rows, cols), x)
    e, ok = oracle.floored_rel_err(y, yref)
    assert ok and e <= TOL_F32, e
    y2 = host(fn(Wd, xd, rows=rows, cols=cols))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


# Q4_0 rows of 256 .. 4096 weights take the lanes-along-K kernel (two 18-byte
# blocks per lane); row counts leave partial steps; integer weights and x make
# every partial sum exact.
@pytest.mark.parametrize("cols", [256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("rows", [1, 5, 130])
def test_gemv_q4_0_lanes_along_k(rows, cols):
    gen, ref, _, fn = FMTS["q4_0"]
    rng = np.random.default_rng([rows, cols, 9])
    w = gen(rng, rows, cols)
    x = synth.activations_f32(rng, cols)
    y = host(fn(dev(w), dev(x), rows=rows, cols=cols))
    e, ok = oracle.floored_rel_err(y, oracle.matvec_f64(ref(w, rows, cols), x))
    assert ok and e <= TOL_F32, e
    q4 = b"".join(pack_q4_0_block(0x3C00, [int(v) for v in rng.integers(0, 16, 32)])
                  for _ in range(rows * cols // 32))
    w4 = np.frombuffer(q4, np.uint8)
    xi = rng.integers(-8, 9, cols).astype(np.float32)
    yi = host(fn(dev(w4), dev(xi), rows=rows, cols=cols))
    assert np.array_equal(yi.astype(np.float64), oracle.dequant_q4_0_f64(w4, rows, cols) @ xi.astype(np.float64))


# Q6_K rows of 256 .. 12288 weights (multiples of 256) take the lanes-along-K
# kernels: a lane's 64 weights are 16 bytes of each low-bit field and of the
# high-bit field of one half super-block, 2 bytes off a word boundary in every
# other super-block (odd super-block counts also shift every other row); 12544
# is past them (lane-quad kernel). Integer weights and x make every partial
# sum exact.
@pytest.mark.parametrize("cols", [256, 512, 1024, 2048, 4096, 4352, 8192, 11008, 12288, 12544])
@pytest.mark.parametrize("rows", [1, 5, 130])
def test_gemv_q6_k_lanes_along_k(rows, cols):
    gen, ref, _, fn = FMTS["q6_k"]
    rng = np.random.default_rng([rows, cols, 10])
    w = gen(rng, rows, cols)
    x = synth.activations_f32(rng, cols)
    say("q6_k lanes along K", rows, cols)
    y = host(fn(dev(w), dev(x), rows=rows, cols=cols))
    e, ok = oracle.floored_rel_err(y, oracle.matvec_f64(ref(w, rows, cols), x))
    assert ok and e <= TOL_F32, e
    q6 = b"".join(pack_q6_k_block(0x3C00, [int(v) for v in rng.integers(-4, 5, 16)],
                                  [int(v) for v in rng.integers(0, 64, 256)])
                  for _ in range(rows * cols // 256))
    w6 = np.frombuffer(q6, np.uint8)
    xi = rng.integers(-8, 9, cols).astype(np.float32)
    yi = host(fn(dev(w6), dev(xi), rows=rows, cols=cols))
    assert np.array_equal(yi.astype(np.float64), oracle.dequant_q6_k_f64(w6, rows, cols) @ xi.astype(np.float64))


def test_gemv_integer_cases_are_exact():
    rng = np.random.default_rng(12)
    rows, cols = 70, 96 * 32
    q4 = b"".join(pack_q4_0_block(0x3C00, [int(v) for v in rng.integers(0, 16, 32)])
                  for _ in range(rows * cols // 32))
    w4 = np.frombuffer(q4, np.uint8)
    x = rng.integers(-8, 9, cols).astype(np.float32)
    y = host(g.gguf_qmatvec_q4_0(dev(w4), dev(x), rows=rows, cols=cols))
    assert np.array_equal(y.astype(np.float64), oracle.dequant_q4_0_f64(w4, rows, cols) @ x.astype(np.float64))
    rows, cols = 50, 2816
    q6 = b"".join(pack_q6_k_block(0x3C00, [int(v) for v in rng.integers(-4, 5, 16)],
                                  [int(v) for v in rng.integers(0, 64, 256)])
                  for _ in range(rows * cols // 256))
    w6 = np.frombuffer(q6, np.uint8)
    x = rng.integers(-8, 9, cols).astype(np.float32)
    y = host(g.gguf_qmatvec_q6_k(dev(w6), dev(x), rows=rows, cols=cols))
    assert np.array_equal(y.astype(np.float64), oracle.dequant_q6_k_f64(w6, rows, cols) @ x.astype(np.float64))


def test_mixed_types_in_one_decode_batch():
    """A Q4_K_M-like step list: q/k/o/gate/up Q4_K, v and down Q6_K, an extra
    Q4_0 projection, the head Q8_0; stages in order, each GEMV against the
    oracle, a later stage reading an earlier stage's output."""
    rng = np.random.default_rng(44)
    H, F, KV = 2048, 2816, 512
    mats = {"q": ("q4_k", H, H), "k": ("q4_k", KV, H), "v": ("q6_k", KV, H), "o": ("q4_k", H, H),
            "gate": ("q4_k", F, H), "up": ("q4_k", F, H), "down": ("q6_k", H, F), "extra": ("q4_0", 300, H),
            "head": ("q8_0", 4000, H)}
    gen = {"q4_k": (synth.q4_k_weights, oracle.dequant_q4_k_f32, g.TYPE_Q4_K),
           "q6_k": (synth.q6_k_weights, oracle.dequant_q6_k_f32, g.TYPE_Q6_K),
           "q4_0": (synth.q4_0_weights, oracle.dequant_q4_0_f32, g.TYPE_Q4_0),
           "q8_0": (synth.q8_0_weights, oracle.dequant_q8_0_f32, g.TYPE_Q8_0)}
    W, W32, Y = {}, {}, {}
    for name, (fmt, r, c) in mats.items():
        fn, ref, _ = gen[fmt]
        w = fn(rng, r, c)
        W[name], W32[name] = dev(w), ref(w, r, c)
        Y[name] = torch.empty(r, dtype=torch.float32, device=DEV)
    x = dev(synth.activations_f32(rng, H))
    t = lambda n: gen[mats[n][0]][2]
    ents = [(t("q"), W["q"], x, Y["q"], 0), (t("k"), W["k"], x, Y["k"], 0), (t("v"), W["v"], x, Y["v"], 0),
            (t("extra"), W["extra"], x, Y["extra"], 0),
            (t("o"), W["o"], Y["q"], Y["o"], 1),
            (t("gate"), W["gate"], Y["o"], Y["gate"], 2), (t("up"), W["up"], Y["o"], Y["up"], 2),
            (t("down"), W["down"], Y["gate"], Y["down"], 3),
            (t("head"), W["head"], Y["down"], Y["head"], 4)]
    say("mixed batch", len(ents))
    g.gguf_qmatvec_batch(g.GemvBatch(ents))
    inputs = {"q": x, "k": x, "v": x, "extra": x, "o": Y["q"], "gate": Y["o"], "up": Y["o"],
              "down": Y["gate"], "head": Y["down"]}
    for name in mats:
        xin = host(inputs[name])
        e, ok = oracle.floored_rel_err(host(Y[name]), oracle.matvec_f64(W32[name], xin))
        assert ok and e <= TOL_F32, (name, e)


@pytest.mark.parametrize("fmt", ["q4_0", "q6_k"])
def test_decode_batch_ragged_stages(fmt):
    """Stages of 1 to 4 Q4_0 or Q6_K GEMVs sharing x (grouped lanes-along-K
    launches, two-GEMV launches with scalar descriptors, long rows), ragged
    row counts, a later stage reading an earlier output; every row against
    the oracle."""
    gen, ref, _, _ = FMTS[fmt]
    tcode = g.TYPE_Q4_0 if fmt == "q4_0" else g.TYPE_Q6_K
    rng = np.random.default_rng(52)
    row_choices = [1, 7, 64, 65, 300, 1031]
    k_choices = [256, 2048, 4096, 5120, 11008]
    ents, checks, prev = [], [], None
    for si in range(14):
        m = int(rng.integers(1, 5))
        cols = int(rng.choice(k_choices))
        if prev is not None and prev[1].numel() == cols:
            xin, xh = prev[1], None   # read the previous stage's output
        else:
            xh = synth.activations_f32(rng, cols)
            xin = dev(xh)
        last = None
        for _ in range(m):
            rows = int(rng.choice(row_choices))
            w = gen(rng, rows, cols)
            y = torch.empty(rows, dtype=torch.float32, device=DEV)
            ents.append((tcode, dev(w), xin, y, si))
            checks.append((si, w, rows, cols, xin, y))
            last = (rows, y)
        prev = last
    say(fmt, "ragged batch:", len(ents), "GEMVs in 14 stages")
    g.gguf_qmatvec_batch(g.GemvBatch(ents))
    for si, w, rows, cols, xin, y in checks:
        yref = oracle.matvec_f64(ref(w, rows, cols), host(xin))
        e, ok = oracle.floored_rel_err(host(y), yref)
        assert ok and e <= TOL_F32, (si, rows, cols, e)
