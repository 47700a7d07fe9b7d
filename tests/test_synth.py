"""The seeded input generators: determinism, ranges and workload totals."""

import numpy as np

import synth
from oracle.formats import fp16_bits_to_f64, q4_k_fields


def test_deterministic_per_seed():
    a = synth.q4_k_weights(synth.rng_for(3, 0, 0), 4, 512)
    b = synth.q4_k_weights(synth.rng_for(3, 0, 0), 4, 512)
    c = synth.q4_k_weights(synth.rng_for(3, 0, 1), 4, 512)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_q8_0_ranges():
    w = synth.q8_0_weights(synth.rng_for(1, 0, 0), 256, 512)
    assert w.shape == (256, 16 * 34)
    blk = w.reshape(-1, 34)
    d = fp16_bits_to_f64(blk[:, 0].astype(np.uint16) | (blk[:, 1].astype(np.uint16) << 8))
    assert d.min() >= np.float16(1e-3) and d.max() <= np.float16(1e-2)
    q = blk[:, 2:].view(np.int8)
    assert q.min() == -127 and q.max() == 127


def test_q4_k_field_ranges_are_uniform():
    rows, cols = 512, 2048
    w = synth.q4_k_weights(synth.rng_for(3, 0, 0), rows, cols)
    d, dmin, sc, m, q = q4_k_fields(w, rows, cols)
    for v in (d, dmin):
        assert v.min() >= np.float16(1e-4) and v.max() <= np.float16(1e-2)
    for v, n in ((sc, 64), (m, 64), (q, 16)):
        counts = np.bincount(v.ravel(), minlength=n)
        assert len(counts) == n
        expect = v.size / n
        assert np.all(np.abs(counts - expect) < 6 * np.sqrt(expect))


def test_decode_stream_total_bytes():
    assert synth.decode_stream_bytes() == 1_860_993_024
    assert synth.decode_stream_bytes(n_layers=1, head=False) == 43_941_888


def test_small_decode_stream_structure():
    st = synth.decode_stream(n_layers=1, head=False, threads=2)
    assert [tuple(g.name for g in s.gemvs) for s in st] == [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    for s in st:
        for g, w in zip(s.gemvs, s.weights):
            assert w.shape == (g.rows, synth.row_bytes(g.fmt, g.cols))
        assert s.x.shape == (s.gemvs[0].cols,) and s.x.dtype == np.float32
