"""Pin checks for the oracle, written as functions of the decode/product routine
they check, so that tests/test_oracle_mutations.py can run the same checks on
deliberately broken copies of the oracle and show that each plausible mistake
is caught."""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _eq_value(got: float, want: str) -> bool:
    w = float(want)
    if math.isnan(w):
        return math.isnan(got)
    if got != w:
        return False
    return math.copysign(1.0, got) == math.copysign(1.0, w)


def check_q8_0_hand_blocks(dequant_f64) -> bool:
    """dequant_f64(bytes_u8, rows, cols) -> [rows, cols]; every hand-packed
    block must decode to its hand-worked values (sign of zero and NaN included)."""
    doc = load_golden("q8_0_hand_blocks.json")
    for blk in doc["blocks"]:
        raw = np.frombuffer(bytes.fromhex(blk["hex"]), dtype=np.uint8)
        got = np.asarray(dequant_f64(raw, 1, 32), dtype=np.float64).reshape(-1)
        for g, w in zip(got, blk["expect"]):
            if not _eq_value(float(g), w):
                return False
    return True


def q4_k_hand_bytes() -> bytes:
    doc = load_golden("q4_k_hand_superblock.json")
    return bytes.fromhex(doc["d_hex_le"] + doc["dmin_hex_le"] + doc["scales_hex"] + doc["quants_hex"])


def q4_k_hand_expected() -> list:
    """All 256 weights of the hand super-block, from its logical fields (not
    from its bytes), exactly."""
    doc = load_golden("q4_k_hand_superblock.json")
    d = Fraction(doc["d"])
    dmin = Fraction(doc["dmin"])
    q = [(i + i // 32) % 16 for i in range(256)]
    return [d * doc["sc"][i // 32] * q[i] - dmin * doc["m"][i // 32] for i in range(256)]


def check_q4_k_hand_superblock(dequant_f64) -> bool:
    doc = load_golden("q4_k_hand_superblock.json")
    raw = np.frombuffer(q4_k_hand_bytes(), dtype=np.uint8)
    got = np.asarray(dequant_f64(raw, 1, 256), dtype=np.float64).reshape(-1)
    for i, w in doc["expect"].items():
        if got[int(i)] != w:
            return False
    exp = q4_k_hand_expected()
    return all(Fraction(float(g)) == e for g, e in zip(got, exp))


def check_q4_k_hand_sums(dequant_f64) -> bool:
    """Two weighted sums over the whole hand super-block, against the exact
    values computed from the logical fields."""
    raw = np.frombuffer(q4_k_hand_bytes(), dtype=np.uint8)
    got = np.asarray(dequant_f64(raw, 1, 256), dtype=np.float64).reshape(-1)
    exp = q4_k_hand_expected()
    s_got = sum(Fraction(float(v)) for v in got)
    s_exp = sum(exp)
    t_got = sum(Fraction(float(v)) * ((k % 5) - 2) for k, v in enumerate(got))
    t_exp = sum(e * ((k % 5) - 2) for k, e in enumerate(exp))
    return s_got == s_exp and t_got == t_exp


def check_integer_matvec(matvec_f64, dequant_q4_k_f64, pack_block, seed=0) -> bool:
    """d = 1, dmin = 0, every sc = 1: W is the integer matrix of the quants,
    so W x for integer x is an integer matvec (numpy int64 matmul)."""
    rng = np.random.default_rng(seed)
    rows, cols = 5, 512
    q = rng.integers(0, 16, size=(rows, cols))
    m = rng.integers(0, 64, size=(rows, cols // 256, 8))
    raw = bytearray()
    for r in range(rows):
        for s in range(cols // 256):
            raw += pack_block(0x3C00, 0x0000, [1] * 8, list(m[r, s]), list(q[r, s * 256:(s + 1) * 256]))
    w = dequant_q4_k_f64(np.frombuffer(bytes(raw), np.uint8), rows, cols)
    x = rng.integers(-50, 51, size=cols)
    y = matvec_f64(w.astype(np.float32), x.astype(np.float32))
    return bool(np.array_equal(y, (q @ x).astype(np.float64)))


def check_one_hot_columns(matvec_f64, w32) -> bool:
    rows, cols = w32.shape
    for k in (0, 1, cols // 2, cols - 1):
        e = np.zeros(cols, np.float32)
        e[k] = 1.0
        if not np.array_equal(np.asarray(matvec_f64(w32, e)), w32[:, k].astype(np.float64)):
            return False
    return True


# ------------------------------------------------------------ Q4_0 and Q6_K

def _q4_0_bytes(d_bits, qbytes):
    return np.frombuffer(bytes([d_bits & 255, d_bits >> 8] + list(qbytes)), np.uint8)


def check_q4_0_byte_map(dequant_f64) -> bool:
    """d = 1: byte j's low nibble is weight j, its high nibble weight j + 16,
    and a code c stands for c - 8 (one byte set by hand per probe)."""
    for j in (0, 5, 15):
        for lo, hi in ((3, 0), (0, 12), (15, 9)):
            qb = [0x88] * 16
            qb[j] = lo | (hi << 4)
            w = dequant_f64(_q4_0_bytes(0x3C00, qb), 1, 32)[0]
            want = np.zeros(32)
            want[j] = lo - 8
            want[j + 16] = hi - 8
            if not np.array_equal(w, want):
                return False
    return True


def _q6_k_bytes(ql, qh, sc, d_bits):
    return np.frombuffer(bytes(list(ql) + list(qh) + [v & 255 for v in sc] +
                               [d_bits & 255, d_bits >> 8]), np.uint8)


def check_q6_k_bit_map(dequant_f64) -> bool:
    """d = 1, every scale 1, so w = code - 32. One low nibble or one high 2-bit
    field set by hand must move exactly the weight the stated map names."""
    probes = []
    for n in (0, 1):
        for l in (0, 7, 31):
            probes.append(("ql", 64 * n + l, 0x05, 128 * n + l, 5))
            probes.append(("ql", 64 * n + l, 0x90, 128 * n + l + 64, 9))
            probes.append(("ql", 64 * n + l + 32, 0x0B, 128 * n + l + 32, 11))
            probes.append(("ql", 64 * n + l + 32, 0xE0, 128 * n + l + 96, 14))
            for k in range(4):
                probes.append(("qh", 32 * n + l, 3 << (2 * k), 128 * n + l + 32 * k, 48))
    base = dequant_f64(_q6_k_bytes([0] * 128, [0] * 64, [1] * 16, 0x3C00), 1, 256)[0]
    if not np.array_equal(base, np.full(256, -32.0)):
        return False
    for field, pos, byte, weight, code in probes:
        ql, qh = [0] * 128, [0] * 64
        (ql if field == "ql" else qh)[pos] = byte
        w = dequant_f64(_q6_k_bytes(ql, qh, [1] * 16, 0x3C00), 1, 256)[0]
        want = np.full(256, -32.0)
        want[weight] = code - 32
        if not np.array_equal(w, want):
            return False
    return True


def check_q6_k_signed_scales(dequant_f64) -> bool:
    """d = 0.5, every code 33 (value 1): the weights are 0.5 x the signed scale
    of their 16-weight sub-block (scale bytes set by hand)."""
    sc = [1, -1, 2, -2, 127, -128, 0, 5, -7, 64, -64, 3, 9, -9, 100, -100]
    ql = [0x11] * 128                       # low nibbles 1
    qh = [0xAA] * 64                        # high bits 2 -> code 33
    w = dequant_f64(_q6_k_bytes(ql, qh, sc, 0x3800), 1, 256)[0]
    return bool(np.array_equal(w, np.repeat(0.5 * np.array(sc, dtype=np.float64), 16)))
