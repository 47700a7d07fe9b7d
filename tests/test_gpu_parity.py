"""GPU parity: the HIP library (through its C ABI and the thin binding) against
the CPU oracle, on seeded synthetic inputs.

Bars: dequantization bit-exact in fp32 (uint32 views, all NaNs equal); the
bf16 tiles bit-exact to the oracle's nearest-even rounding of its fp32 value;
fp32 matvec within floored relative error 1e-3 per output vector; bf16 prefill
within 2e-2 per token row; exact equality where every partial sum is exactly
representable (integer weights and activations, one-hot activations).
"""

import numpy as np
import pytest
import torch

import gguf_block_quant_dequant_amd as g
import oracle
import synth
from oracle.formats import pack_q4_k_block
from tests.pins import load_golden, q4_k_hand_bytes

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_F32 = 1e-3
TOL_BF16 = 2e-2


def say(*a):
    print(*a, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same_bits_f32(a, b):
    a = np.asarray(a, np.float32).ravel()
    b = np.asarray(b, np.float32).ravel()
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (a.view(np.uint32) == b.view(np.uint32))))


def same_bits_bf16(a_bits, b_bits):
    a = np.asarray(a_bits, np.uint16).ravel()
    b = np.asarray(b_bits, np.uint16).ravel()
    nan = ((a & 0x7FFF) > 0x7F80) & ((b & 0x7FFF) > 0x7F80)
    return bool(np.all(nan | (a == b)))


def bf16_tensor(bits):
    return dev(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def bf16_bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


# ----------------------------------------------------------------- dequant --

def test_dequant_q8_0_hand_blocks():
    doc = load_golden("q8_0_hand_blocks.json")
    raw = np.concatenate([np.frombuffer(bytes.fromhex(b["hex"]), np.uint8) for b in doc["blocks"]])
    n = len(doc["blocks"])
    say("dequant_q8_0 hand blocks", n)
    got = host(g.dequant_q8_0(dev(raw), rows=n, cols=32))
    assert same_bits_f32(got, oracle.dequant_q8_0_f32(raw, n, 32))


def test_dequant_q8_0_every_scale_times_every_int8():
    # 65536 fp16 scales x 256 int8 values = 524288 blocks
    scales = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    q = np.arange(256, dtype=np.uint32).astype(np.uint8).reshape(8, 32)
    blk = np.empty((65536, 8, 34), np.uint8)
    blk[:, :, 0] = (scales & 0xFF)[:, None]
    blk[:, :, 1] = (scales >> 8)[:, None]
    blk[:, :, 2:] = q[None]
    raw = blk.reshape(65536, 8 * 34)
    say("dequant_q8_0 exhaustive 65536 x 256")
    got = host(g.dequant_q8_0(dev(raw)))
    assert same_bits_f32(got, oracle.dequant_q8_0_f32(raw, 65536, 256))


def test_dequant_q4_k_hand_superblock():
    raw = np.frombuffer(q4_k_hand_bytes(), np.uint8)
    got = host(g.dequant_q4_k(dev(raw), rows=1, cols=256))
    assert same_bits_f32(got, oracle.dequant_q4_k_f32(raw, 1, 256))
    assert got[0, 255] == 371.5 and got[0, 32] == -30.5


def _q4k_blocks(d_bits, dmin_bits, sc, m, q):
    """Vectorised assembly of many super-blocks from field arrays via the
    oracle's packer applied to one prototype per distinct field set."""
    n = len(d_bits)
    out = np.empty((n, 144), np.uint8)
    proto = np.frombuffer(pack_q4_k_block(0, 0, sc, m, q), np.uint8)
    out[:] = proto
    out[:, 0] = d_bits & 0xFF
    out[:, 1] = d_bits >> 8
    out[:, 2] = dmin_bits & 0xFF
    out[:, 3] = dmin_bits >> 8
    return out


Q_ALL = [(i % 16) for i in range(256)]


@pytest.mark.parametrize("sc", [[0, 1, 2, 3, 7, 31, 32, 63], [63, 62, 48, 33, 17, 16, 15, 5]])
def test_dequant_q4_k_every_d_times_scale_and_quant(sc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    raw = _q4k_blocks(bits, np.zeros_like(bits), sc, [0] * 8, Q_ALL)
    say("dequant_q4_k every d x", sc)
    got = host(g.dequant_q4_k(dev(raw), rows=65536, cols=256))
    assert same_bits_f32(got, oracle.dequant_q4_k_f32(raw, 65536, 256))


@pytest.mark.parametrize("m", [[0, 1, 2, 3, 7, 31, 32, 63], [63, 62, 48, 33, 17, 16, 15, 5]])
def test_dequant_q4_k_every_dmin_times_min(m):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    raw = _q4k_blocks(np.zeros_like(bits), bits, [1] * 8, m, Q_ALL)
    say("dequant_q4_k every dmin x", m)
    got = host(g.dequant_q4_k(dev(raw), rows=65536, cols=256))
    assert same_bits_f32(got, oracle.dequant_q4_k_f32(raw, 65536, 256))


def test_dequant_q4_k_random_bytes_all_fields():
    rng = np.random.default_rng(21)
    raw = rng.integers(0, 256, size=(4096, 4 * 144), dtype=np.uint8)
    say("dequant_q4_k random bytes 4096 x 1024")
    got = host(g.dequant_q4_k(dev(raw)))
    assert same_bits_f32(got, oracle.dequant_q4_k_f32(raw, 4096, 1024))
    gb = bf16_bits(g.dequant_q4_k_bf16(dev(raw)))
    assert same_bits_bf16(gb, oracle.dequant_q4_k_bf16_bits(raw, 4096, 1024))


@pytest.mark.parametrize("fmt,rows,cols", [("q8_0", 256, 512), ("q8_0", 2048, 2048),
                                           ("q8_0", 11008, 2048), ("q4_k", 11008, 2048),
                                           ("q4_k", 2048, 11008)])
def test_dequant_workload_tensors(fmt, rows, cols):
    rng = synth.rng_for(2 if rows > 256 else 1, 0, rows + cols)
    w = synth.q8_0_weights(rng, rows, cols) if fmt == "q8_0" else synth.q4_k_weights(rng, rows, cols)
    say("dequant", fmt, rows, cols)
    if fmt == "q8_0":
        got = host(g.dequant_q8_0(dev(w)))
        assert same_bits_f32(got, oracle.dequant_q8_0_f32(w, rows, cols))
    else:
        W = dev(w)
        got = host(g.dequant_q4_k(W))
        ref = oracle.dequant_q4_k_f32(w, rows, cols)
        assert same_bits_f32(got, ref)
        assert same_bits_bf16(bf16_bits(g.dequant_q4_k_bf16(W)), oracle.f32_to_bf16_bits(ref))


# ------------------------------------------------------------------ matvec --

def _matvec_case(fmt, rows, cols, seed, x=None):
    rng = synth.rng_for(seed, 0, 0)
    w = synth.q8_0_weights(rng, rows, cols) if fmt == "q8_0" else synth.q4_k_weights(rng, rows, cols)
    if x is None:
        x = synth.activations_f32(rng, cols)
    f = g.gguf_qmatvec_q8_0 if fmt == "q8_0" else g.gguf_qmatvec_q4_k
    say("matvec", fmt, rows, cols, "seed", seed)
    y = host(f(dev(w), dev(x)))
    deq = oracle.dequant_q8_0_f32 if fmt == "q8_0" else oracle.dequant_q4_k_f32
    ref = oracle.matvec_f64(deq(w, rows, cols), x)
    return y, ref, w, x


def test_matvec_q8_0_small_config_seed0():
    # 256 x 512 Q8_0, seed 0 (the generator of the small configuration)
    rng = np.random.default_rng(0)
    w = synth.q8_0_weights(rng, 256, 512)
    x = synth.activations_f32(rng, 512)
    y = host(g.gguf_qmatvec_q8_0(dev(w), dev(x)))
    ref = oracle.matvec_f64(oracle.dequant_q8_0_f32(w, 256, 512), x)
    e, ok = oracle.floored_rel_err(y, ref)
    say("q8_0 256x512 err", e)
    assert ok and e <= TOL_F32


@pytest.mark.parametrize("fmt,rows,cols", [("q8_0", 2048, 2048), ("q8_0", 11008, 2048),
                                           ("q4_k", 11008, 2048), ("q4_k", 2048, 11008),
                                           ("q4_k", 2048, 2048), ("q4_k", 512, 2048)])
def test_matvec_decode_shapes(fmt, rows, cols):
    y, ref, _, _ = _matvec_case(fmt, rows, cols, 3)
    e, ok = oracle.floored_rel_err(y, ref)
    say("err", e, oracle.linalg.literal_rel_err_stats(y, ref, TOL_F32))
    assert ok and e <= TOL_F32


@pytest.mark.parametrize("rows", [1, 63, 64, 65, 300])
@pytest.mark.parametrize("cols", [256, 512, 11008])
def test_matvec_q4_k_ragged(rows, cols):
    y, ref, _, _ = _matvec_case("q4_k", rows, cols, 5)
    e, ok = oracle.floored_rel_err(y, ref)
    assert ok and e <= TOL_F32, e


@pytest.mark.parametrize("rows", [1, 65, 300])
@pytest.mark.parametrize("cols", [32, 96, 256, 288, 2048])
def test_matvec_q8_0_ragged(rows, cols):
    y, ref, _, _ = _matvec_case("q8_0", rows, cols, 6)
    e, ok = oracle.floored_rel_err(y, ref)
    assert ok and e <= TOL_F32, e


# Row lengths of every kernel form: 1, 2, 4, 8, 16 super-blocks (lanes hold
# x), other lengths up to 128 super-blocks (K split over the waves of a block:
# 3, 9, 17, 20, 32, 48, 49 and 128, i.e. 1 to 16 waves) and the first past
# them (129: the lane-per-row kernel), with row counts that leave a partial
# step.
@pytest.mark.parametrize("cols", [256, 768, 1024, 2304, 4096, 4352, 5120, 8192, 12288, 12544, 32768, 33024])
@pytest.mark.parametrize("rows", [1, 3, 130])
def test_matvec_q4_k_every_row_length(rows, cols):
    y, ref, _, _ = _matvec_case("q4_k", rows, cols, 11)
    e, ok = oracle.floored_rel_err(y, ref)
    assert ok and e <= TOL_F32, e


@pytest.mark.parametrize("cols", [1024, 4608, 11008])
def test_matvec_q4_k_integer_exact_long_rows(cols):
    # d = 1, dmin = 0, sc = 1: integer weights 0..15 and integer x, every
    # partial sum exact in fp32, so the result is exact whatever the order
    rng = np.random.default_rng(17)
    rows = 67
    q = rng.integers(0, 16, size=(rows, cols))
    raw = bytearray()
    for r in range(rows):
        for s in range(cols // 256):
            raw += pack_q4_k_block(0x3C00, 0x0000, [1] * 8, [int(v) for v in rng.integers(0, 64, 8)],
                                   [int(v) for v in q[r, s * 256:(s + 1) * 256]])
    w = np.frombuffer(bytes(raw), np.uint8).reshape(rows, -1)
    x = rng.integers(-8, 9, size=cols).astype(np.float32)
    y = host(g.gguf_qmatvec_q4_k(dev(w), dev(x)))
    assert np.array_equal(y.astype(np.float64), (q @ x.astype(np.int64)).astype(np.float64))


# Every Q8_0 row length the lanes-along-K kernels take (4 to 64 lanes per
# row) and the first past them (lane-per-row kernel), with partial steps.
@pytest.mark.parametrize("cols", [256, 512, 1024, 2048, 4096, 4352])
@pytest.mark.parametrize("rows", [1, 3, 130])
def test_matvec_q8_0_every_row_length(rows, cols):
    y, ref, _, _ = _matvec_case("q8_0", rows, cols, 12)
    e, ok = oracle.floored_rel_err(y, ref)
    assert ok and e <= TOL_F32, e


@pytest.mark.parametrize("cols", [256, 2048, 4096])
def test_matvec_q8_0_integer_exact(cols):
    # d = 1 (fp16 0x3C00), codes -128..127, integer x in [-8, 8]: every
    # partial sum is an integer below 2^24, so the result is exact in any order
    rng = np.random.default_rng(23)
    rows = 37
    q = rng.integers(-128, 128, size=(rows, cols))
    blocks = q.reshape(rows, cols // 32, 32).astype(np.int8).view(np.uint8)
    d = np.full((rows, cols // 32, 2), [0x00, 0x3C], np.uint8)
    w = np.concatenate([d, blocks], axis=2).reshape(rows, -1)
    x = rng.integers(-8, 9, size=cols).astype(np.float32)
    y = host(g.gguf_qmatvec_q8_0(dev(w), dev(x)))
    assert np.array_equal(y.astype(np.float64), (q @ x.astype(np.int64)).astype(np.float64))


def test_matvec_q4_k_integer_exact():
    rng = np.random.default_rng(7)
    rows, cols = 130, 1024
    q = rng.integers(0, 16, size=(rows, cols))
    raw = bytearray()
    for r in range(rows):
        for s in range(cols // 256):
            raw += pack_q4_k_block(0x3C00, 0x0000, [1] * 8, [int(v) for v in rng.integers(0, 64, 8)],
                                   [int(v) for v in q[r, s * 256:(s + 1) * 256]])
    w = np.frombuffer(bytes(raw), np.uint8).reshape(rows, -1)
    x = rng.integers(-8, 9, size=cols).astype(np.float32)
    y = host(g.gguf_qmatvec_q4_k(dev(w), dev(x)))
    assert np.array_equal(y.astype(np.float64), (q @ x.astype(np.int64)).astype(np.float64))


def test_matvec_q8_0_integer_exact():
    rng = np.random.default_rng(8)
    rows, cols = 130, 2048
    qv = rng.integers(-127, 128, size=(rows, cols // 32, 32)).astype(np.int8)
    blk = np.empty((rows, cols // 32, 34), np.uint8)
    blk[..., 0] = 0x00
    blk[..., 1] = 0x3C   # d = 1.0
    blk[..., 2:] = qv.view(np.uint8)
    w = blk.reshape(rows, -1)
    x = rng.integers(-4, 5, size=cols).astype(np.float32)
    y = host(g.gguf_qmatvec_q8_0(dev(w), dev(x)))
    exact = qv.reshape(rows, cols).astype(np.int64) @ x.astype(np.int64)
    assert np.array_equal(y.astype(np.float64), exact.astype(np.float64))


@pytest.mark.parametrize("fmt,rows,cols", [("q4_k", 300, 2048), ("q4_k", 100, 11008),
                                           ("q8_0", 300, 2048)])
def test_matvec_one_hot_returns_dequant_column(fmt, rows, cols):
    rng = synth.rng_for(9, 0, 0)
    w = synth.q8_0_weights(rng, rows, cols) if fmt == "q8_0" else synth.q4_k_weights(rng, rows, cols)
    deq = (oracle.dequant_q8_0_f32 if fmt == "q8_0" else oracle.dequant_q4_k_f32)(w, rows, cols)
    f = g.gguf_qmatvec_q8_0 if fmt == "q8_0" else g.gguf_qmatvec_q4_k
    W = dev(w)
    for k in (0, 31, 32, 255, cols // 2 + 7, cols - 1):
        x = np.zeros(cols, np.float32)
        x[k] = 1.0
        y = host(f(W, dev(x)))
        assert same_bits_f32(y, deq[:, k]), k


@pytest.mark.parametrize("fmt,rows,cols", [("q4_k", 11008, 2048), ("q8_0", 2048, 2048)])
def test_matvec_deterministic(fmt, rows, cols):
    rng = synth.rng_for(10, 0, 0)
    w = synth.q8_0_weights(rng, rows, cols) if fmt == "q8_0" else synth.q4_k_weights(rng, rows, cols)
    x = synth.activations_f32(rng, cols)
    f = g.gguf_qmatvec_q8_0 if fmt == "q8_0" else g.gguf_qmatvec_q4_k
    W, X = dev(w), dev(x)
    a = host(f(W, X))
    b = host(f(W, X))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_matvec_output_is_overwritten():
    rng = synth.rng_for(11, 0, 0)
    w = synth.q4_k_weights(rng, 200, 512)
    x = synth.activations_f32(rng, 512)
    y = torch.full((200,), float("nan"), device=DEV)
    g.gguf_qmatvec_q4_k(dev(w), dev(x), y)
    ref = oracle.matvec_f64(oracle.dequant_q4_k_f32(w, 200, 512), x)
    e, ok = oracle.floored_rel_err(host(y), ref)
    assert ok and e <= TOL_F32


# ------------------------------------------------------------------ matmul --

def _matmul_case(n, rows, cols, seed):
    rng = synth.rng_for(seed, 0, 0)
    w = synth.q4_k_weights(rng, rows, cols)
    xb = synth.activations_bf16_bits(rng, n, cols)
    say("matmul", n, rows, cols)
    Y = bf16_bits(g.gguf_qmatmul_q4_k(dev(w), bf16_tensor(xb)))
    ref = oracle.matmul_bf16_x_f64(xb, oracle.dequant_q4_k_f32(w, rows, cols))
    return oracle.bf16_bits_to_f64(Y), ref


@pytest.mark.parametrize("n,rows,cols", [(512, 256, 512), (1, 200, 256), (100, 129, 768),
                                         (129, 300, 2048), (512, 2048, 2048), (512, 512, 2048),
                                         (512, 2048, 11008), (512, 11008, 2048),
                                         (64, 128, 7 * 256), (129, 33000, 256), (512, 16684, 768)])
def test_matmul_q4_k(n, rows, cols):
    """Includes the prefill shapes at N = 512 and a K of 7 super-blocks, which
    the K split cuts into unequal ranges. The last two take 256-token blocks:
    129 tokens over 258 row tiles of one super-block (127 token rows of the
    tile past the end, every tile whole), and 512 tokens over 262 tiles of
    three super-blocks (256 whole, the last 6 split into three ranges)."""
    Y, ref = _matmul_case(n, rows, cols, 12)
    e, ok = oracle.floored_rel_err(Y, ref)
    say("err", e)
    assert ok and e <= TOL_BF16


def test_matmul_q4_k_integer_exact():
    rng = np.random.default_rng(13)
    rows, cols, n = 160, 512, 136
    q = rng.integers(0, 16, size=(rows, cols))
    raw = bytearray()
    for r in range(rows):
        for s in range(cols // 256):
            raw += pack_q4_k_block(0x3C00, 0x0000, [1] * 8, [0] * 8,
                                   [int(v) for v in q[r, s * 256:(s + 1) * 256]])
    w = np.frombuffer(bytes(raw), np.uint8).reshape(rows, -1)
    X = np.zeros((n, cols), np.float32)
    for i in range(n):                       # at most 8 entries of +-1: |Y| <= 120, exact in bf16
        idx = rng.choice(cols, size=8, replace=False)
        X[i, idx] = rng.choice([-1.0, 1.0], size=8)
    xb = oracle.f32_to_bf16_bits(X)
    Y = bf16_bits(g.gguf_qmatmul_q4_k(dev(w), bf16_tensor(xb)))
    exact = X.astype(np.int64) @ q.T
    assert np.array_equal(oracle.bf16_bits_to_f64(Y), exact.astype(np.float64))


def test_matmul_deterministic_across_calls():
    """Split-K tiles are summed in range order by whichever block arrives last:
    repeated calls give identical bits, also after a call of another shape
    (tile counters return to zero)."""
    rng = synth.rng_for(15, 0, 0)
    W1 = dev(synth.q4_k_weights(rng, 2048, 11008))
    X1 = bf16_tensor(synth.activations_bf16_bits(rng, 512, 11008))
    W2 = dev(synth.q4_k_weights(rng, 300, 2048))
    X2 = bf16_tensor(synth.activations_bf16_bits(rng, 129, 2048))
    a = bf16_bits(g.gguf_qmatmul_q4_k(W1, X1))
    b2 = bf16_bits(g.gguf_qmatmul_q4_k(W2, X2))
    b = bf16_bits(g.gguf_qmatmul_q4_k(W1, X1))
    c2 = bf16_bits(g.gguf_qmatmul_q4_k(W2, X2))
    assert np.array_equal(a, b)
    assert np.array_equal(b2, c2)


def test_matmul_single_token_agrees_with_matvec():
    rng = synth.rng_for(14, 0, 0)
    rows, cols = 300, 2048
    w = synth.q4_k_weights(rng, rows, cols)
    xb = synth.activations_bf16_bits(rng, 1, cols)
    W = dev(w)
    Y = oracle.bf16_bits_to_f64(bf16_bits(g.gguf_qmatmul_q4_k(W, bf16_tensor(xb))))[0]
    y = host(g.gguf_qmatvec_q4_k(W, dev(oracle.bf16_bits_to_f64(xb[0]).astype(np.float32))))
    e, ok = oracle.floored_rel_err(Y, y)
    assert ok and e <= TOL_BF16


# ------------------------------------------------------------ decode batch --

def test_batch_one_layer_and_head_matches_oracle():
    """One decode layer's seven Q4_K GEMVs in four steps, then the Q8_0 head
    (full sizes), through gguf_qmatvec_batch."""
    stages = synth.decode_stream(n_layers=1, head=True, threads=8)
    entries, refs = [], []
    for si, st in enumerate(stages):
        X = dev(st.x)
        for gm, w in zip(st.gemvs, st.weights):
            y = torch.empty(gm.rows, dtype=torch.float32, device=DEV)
            tid = g.TYPE_Q8_0 if gm.fmt == synth.Q8_0 else g.TYPE_Q4_K
            entries.append((tid, dev(w), X, y, si))
            if gm.fmt == synth.Q8_0:
                rows = np.arange(0, gm.rows, 61)          # sampled head rows
                deq = oracle.dequant_q8_0_f32(w[rows], len(rows), gm.cols)
            else:
                rows = np.arange(gm.rows)
                deq = oracle.dequant_q4_k_f32(w, gm.rows, gm.cols)
            refs.append((y, rows, oracle.matvec_f64(deq, st.x)))
    say("batch of", len(entries), "GEMVs")
    g.gguf_qmatvec_batch(g.GemvBatch(entries))
    for (y, rows, ref) in refs:
        got = host(y)[rows]
        e, ok = oracle.floored_rel_err(got, ref)
        assert ok and e <= TOL_F32, e


def test_batch_chained_steps_read_previous_outputs():
    """Step 1 computes y1 = W1 x; step 2 reads y1 as its input: y2 = W2 y1."""
    rng = synth.rng_for(15, 0, 0)
    w1 = synth.q4_k_weights(rng, 512, 2048)
    w2 = synth.q8_0_weights(rng, 300, 512)
    x = synth.activations_f32(rng, 2048)
    y1 = torch.empty(512, dtype=torch.float32, device=DEV)
    y2 = torch.empty(300, dtype=torch.float32, device=DEV)
    b = g.GemvBatch([(g.TYPE_Q4_K, dev(w1), dev(x), y1, 0), (g.TYPE_Q8_0, dev(w2), y1, y2, 1)])
    for _ in range(3):
        y1.fill_(float("nan"))
        y2.fill_(float("nan"))
        g.gguf_qmatvec_batch(b)
        r1 = oracle.matvec_f64(oracle.dequant_q4_k_f32(w1, 512, 2048), x)
        got1 = host(y1)
        e1, ok1 = oracle.floored_rel_err(got1, r1)
        r2 = oracle.matvec_f64(oracle.dequant_q8_0_f32(w2, 300, 512), got1)
        e2, ok2 = oracle.floored_rel_err(host(y2), r2)
        assert ok1 and ok2 and e1 <= TOL_F32 and e2 <= TOL_F32


def test_batch_in_hip_graph_replays_match_eager():
    rng = synth.rng_for(16, 0, 0)
    w = [synth.q4_k_weights(rng, r, c) for r, c in ((2048, 2048), (512, 2048), (11008, 2048))]
    x = dev(synth.activations_f32(rng, 2048))
    ys = [torch.empty(m.shape[0], dtype=torch.float32, device=DEV) for m in w]
    b = g.GemvBatch([(g.TYPE_Q4_K, dev(m), x, y, 0) for m, y in zip(w, ys)])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g.gguf_qmatvec_batch(b, s)
    torch.cuda.synchronize()
    eager = [host(y).copy() for y in ys]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.gguf_qmatvec_batch(b, s)
    for _ in range(3):
        for y in ys:
            y.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert np.array_equal(host(y).view(np.uint32), e.view(np.uint32))
    g.gguf_qk_stream_release(s)


# (Each token's output over a matrix is one vector of the floored metric; a
# matrix of one row would make that floor the value itself.)
@pytest.mark.parametrize("n,rows", [(512, (2048, 512, 512)), (100, (200, 129, 1000)), (64, (11008, 11008)),
                                    (129, (65,)), (512, (300, 0, 700, 128)), (512, (11008, 11008)),
                                    (300, (16384 + 77,))])
def test_matmul_multi_matches_oracle(n, rows):
    """Up to four matrices of one X in one launch (q/k/v and gate/up shapes,
    ragged row counts, a matrix of no rows): each Y against the oracle within
    the bf16 bar. The prefill gate/up launch (512 tokens, 2 x 11008 rows) and
    300 tokens over 16461 rows have enough row tiles for 256-token blocks; the
    latter's second token tile is ragged (44 tokens)."""
    rng = synth.rng_for(19, n, len(rows))
    cols = 2048
    ws = [synth.q4_k_weights(rng, r, cols) if r else np.zeros((0, cols // 256 * 144), np.uint8)
          for r in rows]
    xb = synth.activations_bf16_bits(rng, n, cols)
    say("matmul multi", n, rows)
    Ys = g.gguf_qmatmul_q4_k_multi([dev(w) for w in ws], bf16_tensor(xb), rows=list(rows))
    for w, r, Y in zip(ws, rows, Ys):
        if r == 0:
            continue
        ref = oracle.matmul_bf16_x_f64(xb, oracle.dequant_q4_k_f32(w, r, cols))
        e, ok = oracle.floored_rel_err(oracle.bf16_bits_to_f64(bf16_bits(Y)), ref)
        assert ok and e <= TOL_BF16, (r, e)


def test_matmul_multi_single_matrix_equals_matmul():
    rng = synth.rng_for(20, 0, 0)
    w = synth.q4_k_weights(rng, 777, 2048)
    xb = synth.activations_bf16_bits(rng, 300, 2048)
    W, X = dev(w), bf16_tensor(xb)
    a = bf16_bits(g.gguf_qmatmul_q4_k(W, X))
    b = bf16_bits(g.gguf_qmatmul_q4_k_multi([W], X)[0])
    assert np.array_equal(a, b)
