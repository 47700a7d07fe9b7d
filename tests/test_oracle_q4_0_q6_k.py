"""Pins of the oracle's Q4_0 and Q6_K decoders.

The pages fix the block sizes (18 bytes per 32 weights, 210 per 256) and that
Q4_0 is Q8_0's recipe with 4-bit integers. The field maps are GGUF's layout
(the reading in oracle/formats.py): here they are pinned by single-field
probes written from the stated map (one byte or bit set by hand, the one
weight it must move checked), by the vectorised decoder agreeing with the
per-block pure-Python decoder, by pack/unpack round trips, and by exactness
closed forms. Agreement with real GGUF files stays unpinned."""

import json
import os
from fractions import Fraction

import numpy as np

from oracle.formats import (dequant_q4_0_f32, dequant_q4_0_f64, dequant_q6_k_f32, dequant_q6_k_f64,
                            fp16_bits_to_f64, pack_q4_0_block, pack_q6_k_block, q4_0_block_scalar,
                            q6_k_block_scalar, row_bytes, unpack_q4_0_block, unpack_q6_k_block)

from tests.pins import check_q4_0_byte_map, check_q6_k_bit_map, check_q6_k_signed_scales

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_block_sizes_match_the_pages_listing():
    doc = json.load(open(os.path.join(GOLDEN, "p2_bits_per_weight.json")))
    sizes = {r[0]: (r[1], r[2]) for r in doc["rows"]}
    assert row_bytes("q4_0", 32) == sizes["Q4_0"][0] and sizes["Q4_0"][1] == 32
    assert row_bytes("q6_k", 256) == sizes["Q6_K"][0] and sizes["Q6_K"][1] == 256
    assert row_bytes("q4_0", 2048) == 1152 and row_bytes("q6_k", 2048) == 1680


def test_q4_0_byte_map_by_hand():
    assert check_q4_0_byte_map(dequant_q4_0_f64)


def test_q4_0_scale_times_every_code_is_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    qb = np.array([c | (((c + 7) % 16) << 4) for c in range(16)], np.uint8)
    blk = np.empty((65536, 18), np.uint8)
    blk[:, 0] = bits & 255
    blk[:, 1] = bits >> 8
    blk[:, 2:] = qb
    w64 = dequant_q4_0_f64(blk.reshape(-1), 65536, 32)
    d = fp16_bits_to_f64(bits)
    codes = np.concatenate([qb & 15, qb >> 4]).astype(np.float64) - 8
    with np.errstate(invalid="ignore"):
        want = d[:, None] * codes[None, :]
    assert np.array_equal(np.isnan(w64), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(w64[ok], want[ok])
    w32 = dequant_q4_0_f32(blk.reshape(-1), 65536, 32)
    assert np.array_equal(w32[ok].astype(np.float64), w64[ok])     # exact in fp32


def test_q4_0_vectorised_equals_scalar_and_round_trips():
    rng = np.random.default_rng(40)
    blocks = []
    for _ in range(50):
        d_bits = int(rng.integers(0, 0x7C00))
        q = [int(v) for v in rng.integers(0, 16, 32)]
        b = pack_q4_0_block(d_bits, q)
        assert unpack_q4_0_block(b) == (d_bits, q)
        blocks.append(b)
    w = dequant_q4_0_f64(np.frombuffer(b"".join(blocks), np.uint8), 5, 320)
    for i, b in enumerate(blocks):
        r, c = divmod(i, 10)
        exact = q4_0_block_scalar(b)
        assert [Fraction(float(v)) for v in w[r, 32 * c:32 * c + 32]] == exact


def test_q6_k_bit_map_by_hand():
    assert check_q6_k_bit_map(dequant_q6_k_f64)


def test_q6_k_scales_are_signed_per_16_weights():
    assert check_q6_k_signed_scales(dequant_q6_k_f64)


def test_q6_k_vectorised_equals_scalar_and_round_trips():
    rng = np.random.default_rng(41)
    blocks = []
    for _ in range(12):
        d_bits = int(rng.integers(0, 0x7C00))
        sc = [int(v) for v in rng.integers(-128, 128, 16)]
        code = [int(v) for v in rng.integers(0, 64, 256)]
        b = pack_q6_k_block(d_bits, sc, code)
        assert unpack_q6_k_block(b) == (d_bits, sc, code)
        blocks.append(b)
    # random raw bytes are blocks too: unpack -> pack gives the same bytes back
    raw = rng.integers(0, 256, 210).astype(np.uint8).tobytes()
    assert pack_q6_k_block(*unpack_q6_k_block(raw)) == raw
    w = dequant_q6_k_f64(np.frombuffer(b"".join(blocks), np.uint8), 3, 1024)
    for i, b in enumerate(blocks):
        r, c = divmod(i, 4)
        assert [Fraction(float(v)) for v in w[r, 256 * c:256 * c + 256]] == q6_k_block_scalar(b)


def test_q6_k_fp32_is_exact():
    """Largest significands: d = 2047/1024 (fp16 0x3FFF), sc = 127, code - 32 = -31."""
    b = pack_q6_k_block(0x3FFF, [127] * 16, [1] * 256)
    w64 = dequant_q6_k_f64(np.frombuffer(b, np.uint8), 1, 256)
    w32 = dequant_q6_k_f32(np.frombuffer(b, np.uint8), 1, 256)
    assert w64[0, 0] == -(2047 / 1024) * 127 * 31
    assert np.array_equal(w32.astype(np.float64), w64)
