"""Small-batch products gguf_qmatmul_f32_{q8_0,q4_k} (fp32 X [n_tokens, K],
fp32 Y [n_tokens, rows]) against the oracle, through the C ABI.

Bar: floored relative error 1e-3 per token row (the fp32 matvec bar); bit
equality where every partial sum is an exactly representable integer; two
calls bit-identical; one token agrees with the batch-1 GEMV. Shapes cover one
and several row blocks (128 rows), one and two token blocks (32 tokens),
ragged rows and tokens, short and long K, with and without split K."""

import numpy as np
import pytest
import torch

import gguf_block_quant_dequant_amd as g
import oracle
import synth
from oracle.formats import pack_q4_k_block
from oracle.linalg import literal_rel_err_stats

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


def _weights(fmt, rng, rows, cols):
    if fmt == "q8_0":
        w = synth.q8_0_weights(rng, rows, cols)
        return w, oracle.dequant_q8_0_f32(w, rows, cols)
    w = synth.q4_k_weights(rng, rows, cols)
    return w, oracle.dequant_q4_k_f32(w, rows, cols)


def _call(fmt, W, X, rows):
    f = g.gguf_qmatmul_f32_q8_0 if fmt == "q8_0" else g.gguf_qmatmul_f32_q4_k
    return f(W, X, rows=rows)


SHAPES = [
    ("q4_k", 128, 256, 1),
    ("q4_k", 130, 512, 2),
    ("q4_k", 64, 256, 32),
    ("q4_k", 1000, 2048, 7),
    ("q4_k", 2048, 2048, 32),
    ("q4_k", 511, 768, 33),
    ("q4_k", 257, 256, 64),
    ("q4_k", 2048, 11008, 16),
    ("q4_k", 300, 2048, 20),     # two token chunks of the Q4_K kernel up to 32 tokens, the second ragged
    ("q4_k", 520, 11008, 27),    # the same with K split over blocks
    ("q4_k", 70, 20480, 5),      # K split over more than eight ranges (80 super-blocks): paired layout
    ("q4_k", 40, 20480, 20),     # the same, two token chunks of 16
    ("q4_k", 90, 20480, 64),     # the same on the 32-token tile kernel
    ("q4_k", 11008, 2048, 5),
    ("q8_0", 128, 256, 1),
    ("q8_0", 257, 512, 5),
    ("q8_0", 2048, 2048, 32),
    ("q8_0", 640, 11008, 3),
    ("q8_0", 11008, 2048, 9),
    ("q8_0", 100, 768, 64),
]


@pytest.mark.parametrize("fmt,rows,cols,n", SHAPES)
def test_small_batch_matches_oracle(fmt, rows, cols, n):
    rng = np.random.default_rng([rows, cols, n, len(fmt)])
    w, w32 = _weights(fmt, rng, rows, cols)
    X = np.stack([synth.activations_f32(rng, cols) for _ in range(n)])
    say("small batch", fmt, rows, cols, n)
    Wd, Xd = dev(w), dev(X)
    Y = host(_call(fmt, Wd, Xd, rows))
    ref = oracle.matmul_f32_x_f64(X, w32)
    e, ok = oracle.floored_rel_err(Y, ref)
    say("  floored error", e, literal_rel_err_stats(Y, ref, TOL_F32))
    assert ok and e <= TOL_F32, e
    Y2 = host(_call(fmt, Wd, Xd, rows))
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32))


def test_small_batch_q4_k_integer_case_is_exact():
    """d = 1, dmin = 1: every weight sc q - m is an integer, and so is every
    partial sum with integer activations, so the result is exact."""
    rng = np.random.default_rng(21)
    rows, cols, n = 300, 1024, 19
    blocks = []
    for _ in range(rows * cols // 256):
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        blocks.append(pack_q4_k_block(0x3C00, 0x3C00, list(sc), list(m), list(q)))
    w = np.frombuffer(b"".join(blocks), np.uint8)
    w32 = oracle.dequant_q4_k_f32(w, rows, cols)
    X = rng.integers(-8, 9, size=(n, cols)).astype(np.float32)
    Y = host(g.gguf_qmatmul_f32_q4_k(dev(w), dev(X), rows=rows))
    ref = X.astype(np.float64) @ w32.astype(np.float64).T
    assert np.array_equal(Y.astype(np.float64), ref)


def test_small_batch_q8_0_integer_case_is_exact():
    rng = np.random.default_rng(22)
    rows, cols, n = 200, 2048, 40
    blk = np.empty((rows * cols // 32, 34), np.uint8)
    blk[:, 0], blk[:, 1] = 0x00, 0x3C                      # d = 1.0
    blk[:, 2:] = rng.integers(0, 256, size=(blk.shape[0], 32), dtype=np.uint8)
    w = blk.reshape(-1)
    w32 = oracle.dequant_q8_0_f32(w, rows, cols)
    X = rng.integers(-8, 9, size=(n, cols)).astype(np.float32)
    Y = host(g.gguf_qmatmul_f32_q8_0(dev(w), dev(X), rows=rows))
    ref = X.astype(np.float64) @ w32.astype(np.float64).T
    assert np.array_equal(Y.astype(np.float64), ref)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_k"])
def test_one_token_agrees_with_gemv(fmt):
    rng = np.random.default_rng(23)
    rows, cols = 777, 2048
    w, w32 = _weights(fmt, rng, rows, cols)
    x = synth.activations_f32(rng, cols)
    Wd = dev(w)
    Y = host(_call(fmt, Wd, dev(x[None, :]), rows))[0]
    f = g.gguf_qmatvec_q8_0 if fmt == "q8_0" else g.gguf_qmatvec_q4_k
    y = host(f(Wd, dev(x), rows=rows, cols=cols))
    ref = oracle.matvec_f64(w32, x)
    for got in (Y, y):
        e, ok = oracle.floored_rel_err(got, ref)
        assert ok and e <= TOL_F32, e
    e, _ = oracle.floored_rel_err(Y, y.astype(np.float64))
    assert e <= 2 * TOL_F32, e


def test_zero_tokens_or_rows_launch_nothing():
    """n_tokens == 0 or rows == 0 returns OK and leaves Y untouched (called
    through the C entry point with real buffers)."""
    rng = np.random.default_rng(24)
    w, _ = _weights("q4_k", rng, 4, 256)
    Wd = dev(w)
    X = dev(np.stack([synth.activations_f32(rng, 256) for _ in range(3)]))
    Y = torch.full((3, 4), 7.0, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    L = g.lib()
    for fn in (L.gguf_qmatmul_f32_q4_k, L.gguf_qmatmul_f32_q8_0):
        cols = 256
        Wp = Wd.data_ptr()
        assert fn(Wp, X.data_ptr(), Y.data_ptr(), 0, 4, cols, s) == 0
        assert fn(Wp, X.data_ptr(), Y.data_ptr(), 3, 0, cols, s) == 0
    assert bool(torch.all(Y == 7.0))


# A few tokens (1 .. 8) on every row length of 256 .. 4096 weights, row
# counts that leave partial row blocks.
LK_SHAPES = [(1, 256, 8), (3, 2048, 2), (64, 1024, 4), (130, 512, 6), (33, 4096, 3),
             (257, 2048, 8), (999, 4096, 8), (2048, 2048, 5)]


@pytest.mark.parametrize("fmt", ["q4_k", "q8_0"])
@pytest.mark.parametrize("rows,cols,n", LK_SHAPES)
def test_small_batch_few_tokens(fmt, rows, cols, n):
    rng = np.random.default_rng([rows, cols, n, 7])
    w, w32 = _weights(fmt, rng, rows, cols)
    X = np.stack([synth.activations_f32(rng, cols) for _ in range(n)])
    say("small batch few tokens", fmt, rows, cols, n)
    Wd, Xd = dev(w), dev(X)
    Y = host(_call(fmt, Wd, Xd, rows))
    ref = oracle.matmul_f32_x_f64(X, w32)
    e, ok = oracle.floored_rel_err(Y, ref)
    assert ok and e <= TOL_F32, e
    Y2 = host(_call(fmt, Wd, Xd, rows))
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32))


@pytest.mark.parametrize("n,cols", [(8, 2048), (3, 4096)])
def test_small_batch_few_tokens_integer_cases_are_exact(n, cols):
    rng = np.random.default_rng([n, cols, 24])
    rows = 150
    blocks = []
    for _ in range(rows * cols // 256):
        blocks.append(pack_q4_k_block(0x3C00, 0x3C00, list(rng.integers(0, 64, 8)),
                                      list(rng.integers(0, 64, 8)), list(rng.integers(0, 16, 256))))
    w = np.frombuffer(b"".join(blocks), np.uint8)
    X = rng.integers(-8, 9, size=(n, cols)).astype(np.float32)
    Y = host(g.gguf_qmatmul_f32_q4_k(dev(w), dev(X), rows=rows))
    assert np.array_equal(Y.astype(np.float64),
                          X.astype(np.float64) @ oracle.dequant_q4_k_f64(w, rows, cols).T)
    blk = np.empty((rows * cols // 32, 34), np.uint8)
    blk[:, 0], blk[:, 1] = 0x00, 0x3C                      # d = 1.0
    blk[:, 2:] = rng.integers(0, 256, size=(blk.shape[0], 32), dtype=np.uint8)
    w8 = blk.reshape(-1)
    Y8 = host(g.gguf_qmatmul_f32_q8_0(dev(w8), dev(X), rows=rows))
    assert np.array_equal(Y8.astype(np.float64),
                          X.astype(np.float64) @ oracle.dequant_q8_0_f32(w8, rows, cols).astype(np.float64).T)


@pytest.mark.parametrize("fmt,rows,cols,n", [("q4_k", (2048, 512, 512), 2048, 8),
                                             ("q4_k", (11008, 11008), 2048, 32),
                                             ("q4_k", (300, 0, 129, 64), 1024, 5),
                                             ("q8_0", (777, 33), 2048, 3)])
def test_small_batch_multi_matches_oracle(fmt, rows, cols, n):
    """Up to four matrices of one X in one launch (q/k/v and gate/up shapes,
    ragged rows, a matrix of no rows): every Y against the oracle."""
    rng = np.random.default_rng([sum(rows), cols, n, 3])
    ws = [_weights(fmt, rng, r, cols) if r else (None, None) for r in rows]
    X = np.stack([synth.activations_f32(rng, cols) for _ in range(n)])
    say("small batch multi", fmt, rows, cols, n)
    f = g.gguf_qmatmul_f32_q8_0_multi if fmt == "q8_0" else g.gguf_qmatmul_f32_q4_k_multi
    Wd = [dev(w) if w is not None else torch.empty(0, dtype=torch.uint8, device=DEV) for w, _ in ws]
    Ys = f(Wd, dev(X), rows=list(rows))
    for (w, w32), r, Y in zip(ws, rows, Ys):
        if r == 0:
            continue
        e, ok = oracle.floored_rel_err(host(Y), oracle.matmul_f32_x_f64(X, w32))
        assert ok and e <= TOL_F32, (r, e)
