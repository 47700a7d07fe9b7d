"""Pins of the oracle's fp16 and bf16 conversions against independent library routines."""

import numpy as np
import pytest
import torch

from oracle.formats import (bf16_bits_to_f64, f32_to_bf16_bits, fp16_bits_to_f64,
                            fp16_bits_to_fraction)


def _same_f64(a, b):
    """Bitwise equality of fp64 arrays with every NaN treated as equal."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (a.view(np.uint64) == b.view(np.uint64))))


def test_fp16_all_65536_patterns_match_numpy_half():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = fp16_bits_to_f64(bits)
    lib = bits.view(np.float16).astype(np.float64)
    assert _same_f64(ours, lib)


def test_fp16_special_patterns():
    v = fp16_bits_to_f64(np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF,
                                   0x7C00, 0xFC00, 0x7E00], np.uint16))
    assert v[0] == 0 and not np.signbit(v[0])
    assert v[1] == 0 and np.signbit(v[1])
    assert v[2] == 2.0 ** -24
    assert v[3] == 1023 * 2.0 ** -24
    assert v[4] == 2.0 ** -14
    assert v[5] == 1.0
    assert v[6] == 65504.0
    assert v[7] == np.inf and v[8] == -np.inf and np.isnan(v[9])


def test_fp16_fraction_agrees_on_all_finite():
    for b in range(0, 65536, 7):
        if ((b >> 10) & 0x1F) == 31:
            continue
        f = fp16_bits_to_fraction(b)
        x = float(fp16_bits_to_f64(np.array([b], np.uint16))[0])
        assert f == x or (f == 0 and x == 0)


def test_bf16_rounding_matches_torch_on_random_and_special():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-40).astype(np.float32),   # fp32 subnormals
        rng.integers(0, 2**32, 100_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4028235e38, -3.4028235e38,
                  1.00390625, 1.01171875, 1.0078125], np.float32),  # ties to even
    ])
    ours = f32_to_bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    a = bf16_bits_to_f64(ours)
    b = bf16_bits_to_f64(lib)
    assert _same_f64(a, b)


def test_bf16_ties_round_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: even mantissa wins (1.0)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even wins (1 + 2^-6)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)
    out = bf16_bits_to_f64(f32_to_bf16_bits(x))
    assert out[0] == 1.0
    assert out[1] == 1.0 + 2.0 ** -6


@pytest.mark.parametrize("bits", [0x0000, 0x8000, 0x3F80, 0x7F80, 0xFF80, 0x0001, 0x7F7F])
def test_bf16_decode_is_upper_half_of_f32(bits):
    v = bf16_bits_to_f64(np.array([bits], np.uint16))[0]
    f = np.array([bits << 16], np.uint32).view(np.float32)[0]
    assert _same_f64([v], [np.float64(f)])
