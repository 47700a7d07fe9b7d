"""Pins of the oracle's Q8_0 decode and quantizer."""

import csv
import os

import numpy as np
import pytest

from oracle.formats import (Q8_0_BLOCK_BYTES, Q4_K_BLOCK_BYTES, dequant_q8_0_f32,
                            dequant_q8_0_f64, q8_0_block_scalar, quantize_q8_0_row, row_bytes)
from oracle.linalg import matvec_f64
from tests.pins import GOLDEN, check_q8_0_hand_blocks, load_golden


def test_hand_packed_blocks_decode_to_hand_worked_values():
    assert check_q8_0_hand_blocks(dequant_q8_0_f64)


def test_hand_packed_blocks_scalar_path():
    doc = load_golden("q8_0_hand_blocks.json")
    for blk in doc["blocks"]:
        raw = bytes.fromhex(blk["hex"])
        if blk["name"] == "scale_plus_inf":
            continue  # Fractions are finite only
        got = q8_0_block_scalar(raw)
        for g, w in zip(got, blk["expect"]):
            assert float(g) == float(w)


def test_matvec_worked_example():
    doc = load_golden("q8_0_hand_blocks.json")["matvec_example"]
    raw = np.frombuffer(bytes.fromhex(doc["scale_hex"]) + bytes(doc["q"]), np.uint8)
    w = dequant_q8_0_f32(raw, 1, 32)
    assert matvec_f64(w, np.ones(32, np.float32))[0] == doc["y"]


def _tensor_table():
    rows = []
    with open(os.path.join(GOLDEN, "p1_tensor_table.tsv")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            name, cols, nrows, typ, off = line.rstrip("\n").split("\t")
            rows.append((name, int(cols), int(nrows), typ, int(off)))
    return rows


def test_tensor_table_offsets_pin_block_size_and_no_row_padding():
    """Every tensor of the printed SmolLM3 Q8_0 file starts where the previous
    one ends, with Q8_0 tensors taking rows x (cols/32) x 34 bytes and F32
    tensors rows x cols x 4 bytes."""
    t = sorted(_tensor_table(), key=lambda r: r[4])
    assert len(t) == 326
    for (n0, c0, r0, ty0, o0), (n1, c1, r1, ty1, o1) in zip(t, t[1:]):
        size = r0 * row_bytes("q8_0", c0) if ty0 == "Q8_0" else r0 * c0 * 4
        assert o1 - o0 == size, (n0, n1)


def test_tensor_table_shapes_match_decode_workload():
    t = {r[0]: r for r in _tensor_table()}
    assert t["blk.0.attn_q.weight"][1:3] == (2048, 2048)
    assert t["blk.0.attn_k.weight"][1:3] == (2048, 512)
    assert t["blk.0.attn_v.weight"][1:3] == (2048, 512)
    assert t["blk.0.attn_output.weight"][1:3] == (2048, 2048)
    assert t["blk.0.ffn_gate.weight"][1:3] == (2048, 11008)
    assert t["blk.0.ffn_up.weight"][1:3] == (2048, 11008)
    assert t["blk.0.ffn_down.weight"][1:3] == (11008, 2048)
    assert t["token_embd.weight"][1:3] == (2048, 128256)


def test_bits_per_weight_table():
    doc = load_golden("p2_bits_per_weight.json")
    sizes = {"Q8_0": (Q8_0_BLOCK_BYTES, 32), "Q4_K": (Q4_K_BLOCK_BYTES, 256)}
    for name, nbytes, nweights, printed in doc["rows"]:
        assert f"{nbytes * 8 / nweights:.4g}" == printed
        if name in sizes:
            assert sizes[name] == (nbytes, nweights)
    assert row_bytes("q8_0", 32) == 34 and row_bytes("q4_k", 256) == 144


def test_round_trip_reproduces_printed_mean_error():
    doc = load_golden("p2_q8_0_roundtrip.json")
    rng = np.random.default_rng(doc["seed"])
    w = rng.normal(0, doc["sigma"], size=doc["n_weights"]).astype(np.float32)
    packed = quantize_q8_0_row(w)
    assert len(packed) // (doc["n_weights"] // doc["block_weights"]) == doc["printed_bytes_per_block"]
    assert len(packed) * 8 / doc["n_weights"] == doc["printed_bits_per_weight"]
    back = dequant_q8_0_f32(np.frombuffer(packed, np.uint8), 1, doc["n_weights"])[0]
    err = float(np.abs(back - w).mean())
    assert f"{err:.{doc['printed_decimals']}f}" == doc["printed_mean_abs_error"]
    assert w.nbytes == doc["printed_fp32_bytes"] and w.astype(np.float16).nbytes == doc["printed_fp16_bytes"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_trip_error_within_half_step(seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(32 * 64) * rng.uniform(1e-3, 10, size=32 * 64)).astype(np.float32)
    w[:32] = 0.0  # an all-zero block
    packed = np.frombuffer(quantize_q8_0_row(w), np.uint8).reshape(64, 34)
    back = dequant_q8_0_f32(packed.reshape(-1), 1, w.size)[0]
    d = packed[:, 0:2].copy().view("<f2").astype(np.float64).reshape(-1)
    step = np.repeat(d, 32)
    assert np.all(np.abs(back.astype(np.float64) - w) <= step / 2 * (1 + 1e-6) + 1e-30)
    assert np.all(back[:32] == 0)


def test_vectorised_decode_matches_scalar_on_random_bytes():
    rng = np.random.default_rng(7)
    rows, cols = 3, 128
    raw = rng.integers(0, 256, size=rows * row_bytes("q8_0", cols), dtype=np.uint8)
    # keep scales finite for the Fraction path
    blk = raw.reshape(-1, 34)
    blk[:, 1] &= 0x7B
    w = dequant_q8_0_f64(raw, rows, cols).reshape(-1, 32)
    for b in range(blk.shape[0]):
        ref = q8_0_block_scalar(bytes(blk[b]))
        assert all(float(r) == g for r, g in zip(ref, w[b]))


def test_decoder_accepts_minus_128():
    raw = np.frombuffer(bytes.fromhex("003C") + bytes([0x80] * 32), np.uint8)
    assert np.all(dequant_q8_0_f64(raw, 1, 32) == -128.0)
