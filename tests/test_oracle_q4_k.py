"""Pins of the oracle's Q4_K decode and quantizer."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.formats import (dequant_q4_k_bf16_bits, dequant_q4_k_f32, dequant_q4_k_f64,
                            f32_to_bf16_bits, fp16_bits_to_fraction, pack_q4_k_block,
                            q4_k_block_scalar, q4_k_fields, quantize_q4_k_row, row_bytes,
                            unpack_q4_k_block)
from tests.pins import (check_q4_k_hand_sums, check_q4_k_hand_superblock, q4_k_hand_bytes,
                        q4_k_hand_expected)


def test_hand_superblock_spot_values_and_all_256():
    assert check_q4_k_hand_superblock(dequant_q4_k_f64)


def test_hand_superblock_weighted_sums():
    assert check_q4_k_hand_sums(dequant_q4_k_f64)


def test_hand_superblock_scalar_path():
    assert q4_k_block_scalar(q4_k_hand_bytes()) == q4_k_hand_expected()


def test_hand_superblock_fields():
    d_bits, dmin_bits, sc, m, q = unpack_q4_k_block(q4_k_hand_bytes())
    assert (d_bits, dmin_bits) == (0x3C00, 0x3800)
    assert sc == [63, 1, 32, 17, 48, 33, 16, 62]
    assert m == [0, 63, 21, 42, 15, 47, 32, 1]
    assert q == [(i + i // 32) % 16 for i in range(256)]


@pytest.mark.parametrize("seed", range(5))
def test_pack_unpack_are_inverse_bijections(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        raw = bytes(rng.integers(0, 256, 144, dtype=np.uint8))
        assert pack_q4_k_block(*unpack_q4_k_block(raw)) == raw
        d, dm = (int(v) for v in rng.integers(0, 65536, 2))
        sc = [int(v) for v in rng.integers(0, 64, 8)]
        m = [int(v) for v in rng.integers(0, 64, 8)]
        q = [int(v) for v in rng.integers(0, 16, 256)]
        assert unpack_q4_k_block(pack_q4_k_block(d, dm, sc, m, q)) == (d, dm, sc, m, q)


def test_every_scale_bit_lands_in_exactly_one_field():
    """Flip each of the 96 scale bits alone: exactly one of the 16 fields changes, by a power of two."""
    base = bytes(144)
    seen = set()
    for byte in range(4, 16):
        for bit in range(8):
            raw = bytearray(base)
            raw[byte] ^= 1 << bit
            _, _, sc, m, _ = unpack_q4_k_block(bytes(raw))
            fields = sc + m
            nz = [i for i, v in enumerate(fields) if v]
            assert len(nz) == 1 and bin(fields[nz[0]]).count("1") == 1
            seen.add((nz[0], fields[nz[0]]))
    assert len(seen) == 96   # all 16 fields x 6 bits reached


def test_vectorised_fields_match_scalar():
    rng = np.random.default_rng(11)
    rows, cols = 3, 768
    raw = rng.integers(0, 256, size=rows * row_bytes("q4_k", cols), dtype=np.uint8)
    d, dmin, sc, m, q = q4_k_fields(raw, rows, cols)
    blocks = raw.reshape(rows, cols // 256, 144)
    for r in range(rows):
        for s in range(cols // 256):
            db, dmb, sc_s, m_s, q_s = unpack_q4_k_block(bytes(blocks[r, s]))
            assert list(sc[r, s]) == sc_s and list(m[r, s]) == m_s and list(q[r, s]) == q_s


def test_vectorised_values_match_exact_fractions():
    rng = np.random.default_rng(12)
    rows, cols = 2, 512
    raw = rng.integers(0, 256, size=rows * row_bytes("q4_k", cols), dtype=np.uint8)
    blk = raw.reshape(-1, 144)
    blk[:, 1] &= 0x7B   # finite d
    blk[:, 3] &= 0x7B   # finite dmin
    w = dequant_q4_k_f64(raw, rows, cols).reshape(-1, 256)
    for b in range(blk.shape[0]):
        exact = q4_k_block_scalar(bytes(blk[b]))
        assert all(Fraction(float(g)) == e for g, e in zip(w[b], exact))   # fp64 is exact


def test_fp32_dequant_is_single_rounding_of_exact_value():
    rng = np.random.default_rng(13)
    raw = rng.integers(0, 256, size=row_bytes("q4_k", 2048), dtype=np.uint8)
    blk = raw.reshape(-1, 144)
    blk[:, 1] &= 0x7B
    blk[:, 3] &= 0x7B
    w32 = dequant_q4_k_f32(raw, 1, 2048).reshape(-1, 256)
    for b in range(blk.shape[0]):
        exact = q4_k_block_scalar(bytes(blk[b]))
        for g, e in zip(w32[b], exact):
            # g must be the fp32 nearest to e (ties to even): check neighbours are not closer
            g = np.float32(g)
            lo = np.nextafter(g, np.float32(-np.inf))
            hi = np.nextafter(g, np.float32(np.inf))
            dg = abs(Fraction(float(g)) - e)
            assert dg <= abs(Fraction(float(lo)) - e) and dg <= abs(Fraction(float(hi)) - e)


def test_extreme_fields_are_exact():
    # largest d, sc, q and smallest nonzero dmin, m: t - u still exact in fp64
    raw = pack_q4_k_block(0x7BFF, 0x0001, [63] * 8, [1] * 8, [15] * 256)
    w = dequant_q4_k_f64(np.frombuffer(raw, np.uint8), 1, 256)[0]
    assert Fraction(float(w[0])) == Fraction(65504 * 63 * 15) - Fraction(1, 1 << 24)


def test_integer_special_case():
    q = [(3 * i) % 16 for i in range(256)]
    raw = pack_q4_k_block(0x3C00, 0x0000, [1] * 8, [5] * 8, q)
    w = dequant_q4_k_f64(np.frombuffer(raw, np.uint8), 1, 256)[0]
    assert list(w) == [float(v) for v in q]


def test_non_finite_scales_follow_ieee():
    q = [0] * 255 + [1]
    raw = pack_q4_k_block(0x7C00, 0x0000, [1] * 8, [0] * 8, q)   # d = +inf
    w = dequant_q4_k_f64(np.frombuffer(raw, np.uint8), 1, 256)[0]
    assert np.all(np.isnan(w[:255])) and w[255] == np.inf


def test_bf16_tile_values_are_rounded_fp32_dequant():
    rng = np.random.default_rng(14)
    raw = rng.integers(0, 256, size=4 * row_bytes("q4_k", 512), dtype=np.uint8)
    got = dequant_q4_k_bf16_bits(raw, 4, 512)
    assert np.array_equal(got, f32_to_bf16_bits(dequant_q4_k_f32(raw, 4, 512)))


@pytest.mark.parametrize("seed", range(3))
def test_quantizer_round_trip_picks_nearest_grid_point(seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(256 * 8) * 0.05 + rng.uniform(-0.02, 0.02)).astype(np.float32)
    raw = quantize_q4_k_row(w)
    back = dequant_q4_k_f64(np.frombuffer(raw, np.uint8), 1, w.size)[0]
    for s in range(w.size // 256):
        d_bits, dmin_bits, sc, m, _ = unpack_q4_k_block(raw[s * 144:(s + 1) * 144])
        d = float(fp16_bits_to_fraction(d_bits))
        dmin = float(fp16_bits_to_fraction(dmin_bits))
        for i in range(256):
            j = i // 32
            grid = d * sc[j] * np.arange(16) - dmin * m[j]
            k = s * 256 + i
            best = np.min(np.abs(grid - float(w[k])))
            assert abs(back[k] - float(w[k])) <= best + 1e-12
