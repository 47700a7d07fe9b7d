"""Planted mistakes, on the CPU only: each test builds a broken copy of one
oracle step (a plausible slip: a dropped term, a wrong sign, a swapped index,
a transposed operand) and shows that at least one pin rejects it. The real
oracle passing the same pins is checked in the other test files."""

import numpy as np

from oracle.formats import (_le_u16, _twos_complement_i8, dequant_q4_k_f64, dequant_q8_0_f64,
                            fp16_bits_to_f64, pack_q4_k_block, q4_k_fields)
from oracle.linalg import matvec_f64
from tests.pins import (check_integer_matvec, check_one_hot_columns, check_q4_0_byte_map,
                        check_q4_k_hand_sums, check_q4_k_hand_superblock, check_q6_k_bit_map,
                        check_q6_k_signed_scales, check_q8_0_hand_blocks)


def _q4k_from_fields(fields_fn, combine):
    def dq(raw, rows, cols):
        d, dmin, sc, m, q = fields_fn(raw, rows, cols)
        j = np.arange(256) // 32
        t = d[..., None] * sc[..., j] * q
        u = dmin[..., None] * m[..., j]
        return combine(t, u).reshape(rows, cols)
    return dq


def _swap_quant_nibbles(raw):
    b = np.array(raw, np.uint8).reshape(-1, 144).copy()
    b[:, 16:] = ((b[:, 16:] & 15) << 4) | (b[:, 16:] >> 4)
    return b.reshape(-1)


def test_swapped_nibble_order_is_caught():
    bad = lambda raw, r, c: dequant_q4_k_f64(_swap_quant_nibbles(raw), r, c)
    assert not check_q4_k_hand_superblock(bad)


def test_even_odd_nibble_interleave_is_caught():
    def fields(raw, rows, cols):
        d, dmin, sc, m, _ = q4_k_fields(raw, rows, cols)
        qb = np.asarray(raw, np.uint8).reshape(rows, cols // 256, 144)[..., 16:].astype(np.int64)
        q = np.empty(qb.shape[:2] + (256,), np.int64)
        q[..., 0::2] = qb & 15
        q[..., 1::2] = qb >> 4
        return d, dmin, sc, m, q
    assert not check_q4_k_hand_superblock(_q4k_from_fields(fields, lambda t, u: t - u))


def test_min_added_instead_of_subtracted_is_caught():
    assert not check_q4_k_hand_superblock(_q4k_from_fields(q4_k_fields, lambda t, u: t + u))


def test_dropped_min_term_is_caught():
    assert not check_q4_k_hand_superblock(_q4k_from_fields(q4_k_fields, lambda t, u: t))


def test_wrong_high_bits_of_upper_scales_is_caught():
    def fields(raw, rows, cols):
        d, dmin, sc, m, q = q4_k_fields(raw, rows, cols)
        S = np.asarray(raw, np.uint8).reshape(rows, cols // 256, 144)[..., 4:16].astype(np.int64)
        sc = sc.copy()
        for j in range(4, 8):
            sc[..., j] = (S[..., j + 4] & 15) | ((S[..., j] >> 6) << 4)   # S[j] instead of S[j-4]
        return d, dmin, sc, m, q
    bad = _q4k_from_fields(fields, lambda t, u: t - u)
    assert not (check_q4_k_hand_superblock(bad) and check_q4_k_hand_sums(bad))


def test_scales_and_mins_swapped_is_caught():
    def fields(raw, rows, cols):
        d, dmin, sc, m, q = q4_k_fields(raw, rows, cols)
        return d, dmin, m, sc, q
    assert not check_q4_k_hand_superblock(_q4k_from_fields(fields, lambda t, u: t - u))


def test_q8_0_unsigned_quants_are_caught():
    def bad(raw, rows, cols):
        blk = np.asarray(raw, np.uint8).reshape(rows, cols // 32, 34)
        d = fp16_bits_to_f64(_le_u16(blk[..., 0], blk[..., 1]))
        return (blk[..., 2:].astype(np.float64) * d[..., None]).reshape(rows, cols)
    assert not check_q8_0_hand_blocks(bad)


def test_q8_0_big_endian_scale_is_caught():
    def bad(raw, rows, cols):
        b = np.array(raw, np.uint8).reshape(-1, 34).copy()
        b[:, [0, 1]] = b[:, [1, 0]]
        return dequant_q8_0_f64(b.reshape(-1), rows, cols)
    assert not check_q8_0_hand_blocks(bad)


def test_fp16_exponent_bias_off_by_one_is_caught():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    good = fp16_bits_to_f64(bits)
    lib = bits.view(np.float16).astype(np.float64)
    bad = np.where(np.isfinite(good), good * 2.0, good)    # bias 14 instead of 15
    finite = np.isfinite(lib)
    assert np.array_equal(good[finite], lib[finite])
    assert not np.array_equal(bad[finite], lib[finite])


def test_transposed_matvec_is_caught():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((6, 6)).astype(np.float32)
    assert check_one_hot_columns(matvec_f64, w)
    assert not check_one_hot_columns(lambda a, x: np.asarray(x, np.float64) @ np.asarray(a, np.float64), w)


def test_integer_matvec_catches_dropped_scale():
    def bad_dq(raw, rows, cols):
        return _q4k_from_fields(q4_k_fields, lambda t, u: t - u)(raw, rows, cols) * 0.5
    assert check_integer_matvec(matvec_f64, dequant_q4_k_f64, pack_q4_k_block)
    assert not check_integer_matvec(matvec_f64, bad_dq, pack_q4_k_block)


# ------------------------------------------------------------ Q4_0 and Q6_K

def _q4_0_variant(codes_of, offset):
    def dq(raw, rows, cols):
        blk = np.asarray(raw, np.uint8).reshape(rows, cols // 32, 18)
        d = fp16_bits_to_f64(_le_u16(blk[..., 0], blk[..., 1]))
        qb = blk[..., 2:].astype(np.int64)
        return ((codes_of(qb) - offset).astype(np.float64) * d[..., None]).reshape(rows, cols)
    return dq


def test_q4_0_unsigned_codes_are_caught():
    codes = lambda qb: np.concatenate([qb & 15, qb >> 4], axis=-1)
    assert not check_q4_0_byte_map(_q4_0_variant(codes, 0))


def test_q4_0_interleaved_nibbles_are_caught():
    def codes(qb):
        c = np.empty(qb.shape[:-1] + (32,), np.int64)
        c[..., 0::2] = qb & 15
        c[..., 1::2] = qb >> 4
        return c
    assert not check_q4_0_byte_map(_q4_0_variant(codes, 8))


def _q6_k_variant(high_shift, scale_group, signed=True):
    def dq(raw, rows, cols):
        nsb = cols // 256
        blk = np.asarray(raw, np.uint8).reshape(rows, nsb, 210).astype(np.int64)
        ql, qh = blk[..., 0:128], blk[..., 128:192]
        scb = blk[..., 192:208].astype(np.uint8)
        sc = (_twos_complement_i8(scb) if signed else scb).astype(np.float64)
        d = fp16_bits_to_f64(_le_u16(blk[..., 208], blk[..., 209]))
        code = np.empty(blk.shape[:2] + (256,), np.int64)
        for n in range(2):
            L, H = ql[..., 64 * n:64 * n + 64], qh[..., 32 * n:32 * n + 32]
            b = 128 * n
            code[..., b:b + 32] = (L[..., 0:32] & 15) | (((H >> high_shift[0]) & 3) << 4)
            code[..., b + 32:b + 64] = (L[..., 32:64] & 15) | (((H >> high_shift[1]) & 3) << 4)
            code[..., b + 64:b + 96] = (L[..., 0:32] >> 4) | (((H >> high_shift[2]) & 3) << 4)
            code[..., b + 96:b + 128] = (L[..., 32:64] >> 4) | (((H >> high_shift[3]) & 3) << 4)
        j = np.arange(256) // scale_group
        return (d[..., None] * sc[..., j] * (code - 32)).reshape(rows, cols)
    return dq


def test_q6_k_reference_variant_passes():
    # the variant builder with the stated map passes, so the failures below are the slips
    good = _q6_k_variant((0, 2, 4, 6), 16)
    assert check_q6_k_bit_map(good) and check_q6_k_signed_scales(good)


def test_q6_k_high_bit_pairs_swapped_are_caught():
    assert not check_q6_k_bit_map(_q6_k_variant((0, 4, 2, 6), 16))


def test_q6_k_scale_per_32_weights_is_caught():
    assert not check_q6_k_signed_scales(_q6_k_variant((0, 2, 4, 6), 32))


def test_q6_k_unsigned_scales_are_caught():
    assert not check_q6_k_signed_scales(_q6_k_variant((0, 2, 4, 6), 16, signed=False))
