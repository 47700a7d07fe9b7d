"""Block formats decoded per their definitions (oracle; test infrastructure only).

Plain and slow on purpose: vectorised numpy where a whole matrix is decoded,
pure-Python per-block versions beside them for tiny cases. Every floating-point
value is produced exactly in fp64 first and rounded once to fp32 (numpy's
round-to-nearest-even cast) where an fp32 result is asked for.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

# Block sizes: "GGUF: The File Format...", gguf_demo.py bits-per-weight table
# (Q8_0 34 bytes per 32 weights, Q4_K 144 bytes per 256 weights).
Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32
Q4_K_BLOCK_BYTES = 144
Q4_K_BLOCK_WEIGHTS = 256
Q4_K_SUBBLOCKS = 8
Q4_K_SUBBLOCK_WEIGHTS = 32
# Same table: Q4_0 18 bytes per 32 weights, Q6_K 210 bytes per 256 weights.
Q4_0_BLOCK_BYTES = 18
Q4_0_BLOCK_WEIGHTS = 32
Q6_K_BLOCK_BYTES = 210
Q6_K_BLOCK_WEIGHTS = 256


def row_bytes(fmt: str, cols: int) -> int:
    """Bytes of one row: rows are runs of whole blocks with no padding
    ("GGUF Inferencer in R", section 2.1: a Q8_0 row of 2048 values is 64
    chunks; the tensor offsets in the same section's table step by exactly
    rows x chunks x 34)."""
    if fmt == "q8_0":
        if cols % Q8_0_BLOCK_WEIGHTS:
            raise ValueError("Q8_0 needs cols % 32 == 0")
        return cols // Q8_0_BLOCK_WEIGHTS * Q8_0_BLOCK_BYTES
    if fmt == "q4_k":
        if cols % Q4_K_BLOCK_WEIGHTS:
            raise ValueError("Q4_K needs cols % 256 == 0")
        return cols // Q4_K_BLOCK_WEIGHTS * Q4_K_BLOCK_BYTES
    if fmt == "q4_0":
        if cols % Q4_0_BLOCK_WEIGHTS:
            raise ValueError("Q4_0 needs cols % 32 == 0")
        return cols // Q4_0_BLOCK_WEIGHTS * Q4_0_BLOCK_BYTES
    if fmt == "q6_k":
        if cols % Q6_K_BLOCK_WEIGHTS:
            raise ValueError("Q6_K needs cols % 256 == 0")
        return cols // Q6_K_BLOCK_WEIGHTS * Q6_K_BLOCK_BYTES
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# fp16 and bf16
# ---------------------------------------------------------------------------

def fp16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact fp64 values.

    Half precision is 1 sign, 5 exponent and 10 fraction bits (culpeo.ws, the
    throughput-estimate post, BF16 paragraph). Exponent bias 15; exponent 0 is
    subnormal f * 2^-24; exponent 31 is infinity (f = 0) or NaN.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = (b >> 15) & 1
    e = (b >> 10) & 0x1F
    f = b & 0x3FF
    normal = np.ldexp((1024 + f).astype(np.float64), e - 25)   # (1 + f/1024) 2^(e-15)
    sub = np.ldexp(f.astype(np.float64), -24)
    mag = np.where(e == 0, sub, normal)
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(sign == 1, -mag, mag)


def fp16_bits_to_fraction(bits: int) -> Fraction:
    """Exact value of a finite fp16 bit pattern as a Fraction (pure Python)."""
    sign = -1 if (bits >> 15) & 1 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 31:
        raise ValueError("not finite")
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * Fraction(1024 + f) * (Fraction(2) ** (e - 25))


def f32_to_bf16_bits(x32) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    bf16 keeps fp32's sign and 8 exponent bits and the top 7 fraction bits
    (culpeo.ws, BF16 paragraph), i.e. the upper half of the fp32 word. NaN maps
    to a quiet NaN with the same sign.
    """
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (b & 0x7FFFFFFF) > 0x7F800000
    keep_lsb = (b >> 16) & 1
    rounded = (b + 0x7FFF + keep_lsb) >> 16
    quiet = (b >> 16) | 0x40
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 (the pattern is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _le_u16(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """Little-endian 16-bit word from its two bytes (all GGUF numbers are
    little-endian: "GGUF: The File Format...", "What is stored inside")."""
    return lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)


def _twos_complement_i8(u8: np.ndarray) -> np.ndarray:
    v = u8.astype(np.int16)
    return np.where(v >= 128, v - 256, v)


# ---------------------------------------------------------------------------
# Q8_0
# ---------------------------------------------------------------------------

def dequant_q8_0_f64(w_bytes, rows: int, cols: int) -> np.ndarray:
    """Q8_0 matrix -> exact weights [rows, cols] in fp64.

    Each 34-byte block covers 32 consecutive weights of one row: a fp16
    multiplier, then 32 int8 values; weight = int8 value x multiplier
    ("GGUF Inferencer in R", section 2.1 byte blueprint; "GGUF: The File
    Format...", "How a Q8_0 block is stored", and the practice script's unpack
    step). The product has at most 8 + 11 significant bits, so it is exact in
    fp64 and in fp32.
    """
    nb = cols // Q8_0_BLOCK_WEIGHTS
    blk = np.asarray(w_bytes, dtype=np.uint8).reshape(rows, nb, Q8_0_BLOCK_BYTES)
    d = fp16_bits_to_f64(_le_u16(blk[..., 0], blk[..., 1]))
    q = _twos_complement_i8(blk[..., 2:34]).astype(np.float64)
    with np.errstate(invalid="ignore"):          # inf * 0 = NaN, as IEEE says
        return (q * d[..., None]).reshape(rows, cols)


def dequant_q8_0_f32(w_bytes, rows: int, cols: int) -> np.ndarray:
    """fp32 dequant: the exact value rounded once (it is already exact)."""
    return dequant_q8_0_f64(w_bytes, rows, cols).astype(np.float32)


def q8_0_block_scalar(block: bytes) -> list:
    """One Q8_0 block in pure Python: 32 weights as Fractions (finite scales)."""
    assert len(block) == Q8_0_BLOCK_BYTES
    d = fp16_bits_to_fraction(block[0] | (block[1] << 8))
    out = []
    for i in range(32):
        v = block[2 + i]
        q = v - 256 if v >= 128 else v
        out.append(q * d)
    return out


def quantize_q8_0_row(w32: np.ndarray) -> bytes:
    """Q8_0 quantizer (test helper for the round trip), steps from "GGUF: The
    File Format...", "How a Q8_0 block is stored": per block of 32 weights the
    scale is max|w| / 127 (here computed in fp32, then stored as fp16 rounded to
    nearest even), each weight is stored as round(w / scale) (ties to even, in
    fp32) clipped to [-127, 127] as int8. An all-zero block stores scale 0 and
    zeros (the pages leave 0/0 open)."""
    w32 = np.asarray(w32, dtype=np.float32)
    assert w32.size % Q8_0_BLOCK_WEIGHTS == 0
    out = bytearray()
    for b in range(w32.size // Q8_0_BLOCK_WEIGHTS):
        blk = w32[b * 32:(b + 1) * 32]
        amax = np.float32(np.max(np.abs(blk)))
        d16 = np.float16(amax / np.float32(127))
        d32 = np.float32(d16)
        if d32 == 0:
            q = np.zeros(32, dtype=np.int8)
        else:
            q = np.clip(np.rint(blk / d32), -127, 127).astype(np.int8)
        out += np.array([d16], dtype="<f2").tobytes() + q.tobytes()
    return bytes(out)


# ---------------------------------------------------------------------------
# Q4_K
#
# Structure ("GGUF: The File Format...", k-quant paragraph): super-blocks of 256
# weights split into sub-blocks, each sub-block with its own scale and minimum
# quantized to 6 bits, 144 bytes per 256 weights. Reading of what the page
# leaves open (byte arithmetic fixes the counts: 144 = 128 bytes of 4-bit
# quants + 12 bytes of sixteen 6-bit fields + 4 bytes = two fp16):
#
#   bytes [0:2]    d     fp16 super-scale for the sub-block scales
#   bytes [2:4]    dmin  fp16 super-scale for the sub-block mins
#   bytes [4:16]   S[0..11]: eight 6-bit scales sc[j] and eight 6-bit mins m[j]
#       j < 4 : sc[j] = S[j] & 63            m[j] = S[j+4] & 63
#       j >= 4: sc[j] = (S[j+4] & 15) | ((S[j-4] >> 6) << 4)
#               m[j]  = (S[j+4] >> 4) | ((S[j]   >> 6) << 4)
#   bytes [16:144] Qb[0..127]: for g in 0..3 and l in 0..31,
#       q[64g + l]      = Qb[32g + l] & 15    (sub-block 2g)
#       q[64g + 32 + l] = Qb[32g + l] >> 4    (sub-block 2g + 1)
#
#   weight i (sub-block j = i // 32):  w_i = d * sc[j] * q_i - dmin * m[j]
#
# The field placement is the layout GGUF files use on disk; the pages do not
# print it, so agreement with real files is unpinned here.
# ---------------------------------------------------------------------------

def unpack_q4_k_block(block: bytes):
    """Logical fields of one 144-byte super-block, in pure Python:
    (d_bits, dmin_bits, sc[8], m[8], q[256])."""
    assert len(block) == Q4_K_BLOCK_BYTES
    d_bits = block[0] | (block[1] << 8)
    dmin_bits = block[2] | (block[3] << 8)
    S = block[4:16]
    sc = [0] * 8
    m = [0] * 8
    for j in range(4):
        sc[j] = S[j] & 63
        m[j] = S[j + 4] & 63
    for j in range(4, 8):
        sc[j] = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4)
        m[j] = (S[j + 4] >> 4) | ((S[j] >> 6) << 4)
    Qb = block[16:144]
    q = [0] * 256
    for g in range(4):
        for l in range(32):
            q[64 * g + l] = Qb[32 * g + l] & 15
            q[64 * g + 32 + l] = Qb[32 * g + l] >> 4
    return d_bits, dmin_bits, sc, m, q


def pack_q4_k_block(d_bits: int, dmin_bits: int, sc, m, q) -> bytes:
    """Inverse of unpack_q4_k_block (fields must be in range)."""
    assert all(0 <= v < 64 for v in sc) and all(0 <= v < 64 for v in m)
    assert all(0 <= v < 16 for v in q) and len(q) == 256
    S = [0] * 12
    for j in range(4):
        S[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        S[j + 4] = m[j] | ((m[j + 4] >> 4) << 6)
        S[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    Qb = [0] * 128
    for g in range(4):
        for l in range(32):
            Qb[32 * g + l] = q[64 * g + l] | (q[64 * g + 32 + l] << 4)
    return bytes([d_bits & 255, d_bits >> 8, dmin_bits & 255, dmin_bits >> 8] + S + Qb)


def q4_k_block_scalar(block: bytes) -> list:
    """One super-block in pure Python: 256 exact weights as Fractions."""
    d_bits, dmin_bits, sc, m, q = unpack_q4_k_block(block)
    d = fp16_bits_to_fraction(d_bits)
    dmin = fp16_bits_to_fraction(dmin_bits)
    return [d * sc[i // 32] * q[i] - dmin * m[i // 32] for i in range(256)]


def q4_k_fields(w_bytes, rows: int, cols: int):
    """Vectorised field unpacking of a Q4_K matrix (same map as
    unpack_q4_k_block). Returns d, dmin [rows, nsb] fp64 and sc, m [rows, nsb,
    8], q [rows, nsb, 256] as int64."""
    nsb = cols // Q4_K_BLOCK_WEIGHTS
    blk = np.asarray(w_bytes, dtype=np.uint8).reshape(rows, nsb, Q4_K_BLOCK_BYTES).astype(np.int64)
    d = fp16_bits_to_f64(_le_u16(blk[..., 0], blk[..., 1]))
    dmin = fp16_bits_to_f64(_le_u16(blk[..., 2], blk[..., 3]))
    S = blk[..., 4:16]
    sc = np.empty(blk.shape[:2] + (8,), dtype=np.int64)
    m = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = S[..., j] & 63
        m[..., j] = S[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (S[..., j + 4] & 15) | ((S[..., j - 4] >> 6) << 4)
        m[..., j] = (S[..., j + 4] >> 4) | ((S[..., j] >> 6) << 4)
    Qb = blk[..., 16:144]
    q = np.empty(blk.shape[:2] + (256,), dtype=np.int64)
    for g in range(4):
        q[..., 64 * g:64 * g + 32] = Qb[..., 32 * g:32 * g + 32] & 15
        q[..., 64 * g + 32:64 * g + 64] = Qb[..., 32 * g:32 * g + 32] >> 4
    return d, dmin, sc, m, q


def dequant_q4_k_f64(w_bytes, rows: int, cols: int) -> np.ndarray:
    """Q4_K matrix -> exact weights [rows, cols] in fp64.

    w = d*sc[j]*q - dmin*m[j]. Both products have at most 21 significant bits
    and every value is an integer multiple of 2^-24 below 2^27 in magnitude, so
    the difference is exact in fp64 (non-finite d/dmin follow IEEE rules)."""
    d, dmin, sc, m, q = q4_k_fields(w_bytes, rows, cols)
    nsb = cols // Q4_K_BLOCK_WEIGHTS
    j_of_i = np.arange(256) // Q4_K_SUBBLOCK_WEIGHTS
    with np.errstate(invalid="ignore"):
        t = d[..., None] * sc[..., j_of_i].astype(np.float64) * q.astype(np.float64)
        u = dmin[..., None] * m[..., j_of_i].astype(np.float64)
        w = t - u
    return w.reshape(rows, nsb * 256)


def dequant_q4_k_f32(w_bytes, rows: int, cols: int) -> np.ndarray:
    """fp32 dequant: the exact value rounded once to nearest even."""
    return dequant_q4_k_f64(w_bytes, rows, cols).astype(np.float32)


def dequant_q4_k_bf16_bits(w_bytes, rows: int, cols: int) -> np.ndarray:
    """bf16 tile values: the fp32 dequant rounded to nearest-even bf16."""
    return f32_to_bf16_bits(dequant_q4_k_f32(w_bytes, rows, cols))


def quantize_q4_k_row(w32: np.ndarray) -> bytes:
    """A simple Q4_K quantizer (test helper only; the pages give no rule).

    Per 32-weight sub-block: lo = min(0, min w), hi = max w, scale = (hi-lo)/15,
    min = -lo. d = fp16(max scale / 63), dmin = fp16(max min / 63); each 6-bit
    field is its value divided by the super-scale, rounded and clipped to
    [0, 63]. Each quant is the nearest grid index: clip(round((w + dmin*m) /
    (d*sc)), 0, 15), 0 where d*sc = 0."""
    w = np.asarray(w32, dtype=np.float32).astype(np.float64)
    assert w.size % 256 == 0
    out = bytearray()
    for s in range(w.size // 256):
        sub = w[s * 256:(s + 1) * 256].reshape(8, 32)
        lo = np.minimum(0.0, sub.min(axis=1))
        hi = sub.max(axis=1)
        scale = (hi - lo) / 15.0
        mins = -lo
        d16 = np.float16(scale.max() / 63.0)
        dmin16 = np.float16(mins.max() / 63.0)
        d = float(d16)
        dmin = float(dmin16)
        sc = np.clip(np.rint(scale / d), 0, 63).astype(np.int64) if d > 0 else np.zeros(8, np.int64)
        m = np.clip(np.rint(mins / dmin), 0, 63).astype(np.int64) if dmin > 0 else np.zeros(8, np.int64)
        q = np.zeros(256, dtype=np.int64)
        for j in range(8):
            t = d * sc[j]
            u = dmin * m[j]
            if t > 0:
                q[j * 32:(j + 1) * 32] = np.clip(np.rint((sub[j] + u) / t), 0, 15)
        d_bits = int(np.array([d16], dtype="<f2").view("<u2")[0])
        dmin_bits = int(np.array([dmin16], dtype="<f2").view("<u2")[0])
        out += pack_q4_k_block(d_bits, dmin_bits, list(sc), list(m), list(q))
    return bytes(out)


# ---------------------------------------------------------------------------
# Q4_0: 18-byte block of 32 weights. "GGUF: The File Format...", "How a Q8_0
# block is stored", step 4: the Q8_0 recipe with 4-bit integers, a 2-byte
# fp16 scale d and 16 bytes of 4-bit values. Reading (GGUF's on-disk layout;
# the pages print neither the nibble order nor the offset of the 4-bit code):
#   byte j of the 16 (j = 0..15): low nibble = code of weight j,
#                                 high nibble = code of weight j + 16
#   w = (code - 8) * d          (codes 0..15 stand for -8..7)
# (code - 8) * d has at most 4 + 11 significant bits: exact in fp32.
# Agreement with real files is unpinned.
# ---------------------------------------------------------------------------

def unpack_q4_0_block(block: bytes):
    """(d_bits, codes[32]) of one 18-byte block, in pure Python."""
    assert len(block) == Q4_0_BLOCK_BYTES
    d_bits = block[0] | (block[1] << 8)
    q = [0] * 32
    for j in range(16):
        q[j] = block[2 + j] & 15
        q[j + 16] = block[2 + j] >> 4
    return d_bits, q


def pack_q4_0_block(d_bits: int, q) -> bytes:
    """Inverse of unpack_q4_0_block."""
    assert len(q) == 32 and all(0 <= v < 16 for v in q)
    return bytes([d_bits & 255, d_bits >> 8] + [q[j] | (q[j + 16] << 4) for j in range(16)])


def q4_0_block_scalar(block: bytes) -> list:
    """One Q4_0 block in pure Python: 32 exact weights as Fractions."""
    d_bits, q = unpack_q4_0_block(block)
    d = fp16_bits_to_fraction(d_bits)
    return [(v - 8) * d for v in q]


def dequant_q4_0_f64(w_bytes, rows: int, cols: int) -> np.ndarray:
    """Q4_0 matrix -> exact weights [rows, cols] in fp64."""
    nb = cols // Q4_0_BLOCK_WEIGHTS
    blk = np.asarray(w_bytes, dtype=np.uint8).reshape(rows, nb, Q4_0_BLOCK_BYTES)
    d = fp16_bits_to_f64(_le_u16(blk[..., 0], blk[..., 1]))
    qb = blk[..., 2:18].astype(np.int64)
    code = np.concatenate([qb & 15, qb >> 4], axis=-1)        # weights 0..15, then 16..31
    with np.errstate(invalid="ignore"):
        return ((code - 8).astype(np.float64) * d[..., None]).reshape(rows, cols)


def dequant_q4_0_f32(w_bytes, rows: int, cols: int) -> np.ndarray:
    """fp32 dequant (the exact value; no rounding is needed)."""
    return dequant_q4_0_f64(w_bytes, rows, cols).astype(np.float32)


# ---------------------------------------------------------------------------
# Q6_K: 210-byte super-block of 256 weights (size: "GGUF: The File Format...",
# bits-per-weight listing; a k-quant, so sub-blocks with their own scales under
# one fp16 super-scale, k-quant paragraph). Reading (GGUF's on-disk layout, not
# printed on the pages): 16 sub-blocks of 16 weights, each with a signed 8-bit
# scale; 6-bit codes split into a low nibble and a high 2-bit part:
#   bytes   0..127  ql   low 4 bits of the codes
#   bytes 128..191  qh   high 2 bits of the codes
#   bytes 192..207  sc   16 int8 sub-block scales
#   bytes 208..209  d    fp16 super-scale
# For half n = 0, 1 and l = 0..31, with L = ql[64 n:] and H = qh[32 n:]:
#   code[128 n + l]      = (L[l] & 15)      | ((H[l] >> 0) & 3) << 4
#   code[128 n + l + 32] = (L[l + 32] & 15) | ((H[l] >> 2) & 3) << 4
#   code[128 n + l + 64] = (L[l] >> 4)      | ((H[l] >> 4) & 3) << 4
#   code[128 n + l + 96] = (L[l + 32] >> 4) | ((H[l] >> 6) & 3) << 4
#   weight i:  w_i = d * sc[i // 16] * (code_i - 32)
# The product is exact in fp32: d has 11 significant bits, abs(sc) <= 128 at
# most 7 (128 is a power of two) and abs(code - 32) <= 32 at most 5, so at most
# 23. Agreement with real files is unpinned.
# ---------------------------------------------------------------------------

def unpack_q6_k_block(block: bytes):
    """(d_bits, sc[16] as signed ints, codes[256]) of one 210-byte super-block."""
    assert len(block) == Q6_K_BLOCK_BYTES
    ql, qh = block[0:128], block[128:192]
    sc = [v - 256 if v >= 128 else v for v in block[192:208]]
    d_bits = block[208] | (block[209] << 8)
    code = [0] * 256
    for n in range(2):
        L, H = ql[64 * n:64 * n + 64], qh[32 * n:32 * n + 32]
        for l in range(32):
            code[128 * n + l] = (L[l] & 15) | (((H[l] >> 0) & 3) << 4)
            code[128 * n + l + 32] = (L[l + 32] & 15) | (((H[l] >> 2) & 3) << 4)
            code[128 * n + l + 64] = (L[l] >> 4) | (((H[l] >> 4) & 3) << 4)
            code[128 * n + l + 96] = (L[l + 32] >> 4) | (((H[l] >> 6) & 3) << 4)
    return d_bits, sc, code


def pack_q6_k_block(d_bits: int, sc, code) -> bytes:
    """Inverse of unpack_q6_k_block (sc in -128..127, codes in 0..63)."""
    assert len(sc) == 16 and all(-128 <= v < 128 for v in sc)
    assert len(code) == 256 and all(0 <= v < 64 for v in code)
    ql, qh = [0] * 128, [0] * 64
    for n in range(2):
        for l in range(32):
            c0, c1, c2, c3 = (code[128 * n + l + 32 * k] for k in range(4))
            ql[64 * n + l] = (c0 & 15) | ((c2 & 15) << 4)
            ql[64 * n + l + 32] = (c1 & 15) | ((c3 & 15) << 4)
            qh[32 * n + l] = (c0 >> 4) | ((c1 >> 4) << 2) | ((c2 >> 4) << 4) | ((c3 >> 4) << 6)
    return bytes(ql + qh + [v & 255 for v in sc] + [d_bits & 255, d_bits >> 8])


def q6_k_block_scalar(block: bytes) -> list:
    """One super-block in pure Python: 256 exact weights as Fractions."""
    d_bits, sc, code = unpack_q6_k_block(block)
    d = fp16_bits_to_fraction(d_bits)
    return [d * sc[i // 16] * (code[i] - 32) for i in range(256)]


def dequant_q6_k_f64(w_bytes, rows: int, cols: int) -> np.ndarray:
    """Q6_K matrix -> exact weights [rows, cols] in fp64 (same map as
    unpack_q6_k_block, vectorised)."""
    nsb = cols // Q6_K_BLOCK_WEIGHTS
    blk = np.asarray(w_bytes, dtype=np.uint8).reshape(rows, nsb, Q6_K_BLOCK_BYTES).astype(np.int64)
    ql, qh = blk[..., 0:128], blk[..., 128:192]
    sc = _twos_complement_i8(blk[..., 192:208].astype(np.uint8)).astype(np.float64)
    d = fp16_bits_to_f64(_le_u16(blk[..., 208], blk[..., 209]))
    code = np.empty(blk.shape[:2] + (256,), dtype=np.int64)
    for n in range(2):
        L, H = ql[..., 64 * n:64 * n + 64], qh[..., 32 * n:32 * n + 32]
        b = 128 * n
        code[..., b:b + 32] = (L[..., 0:32] & 15) | (((H >> 0) & 3) << 4)
        code[..., b + 32:b + 64] = (L[..., 32:64] & 15) | (((H >> 2) & 3) << 4)
        code[..., b + 64:b + 96] = (L[..., 0:32] >> 4) | (((H >> 4) & 3) << 4)
        code[..., b + 96:b + 128] = (L[..., 32:64] >> 4) | (((H >> 6) & 3) << 4)
    j_of_i = np.arange(256) // 16
    with np.errstate(invalid="ignore"):
        w = d[..., None] * sc[..., j_of_i] * (code - 32).astype(np.float64)
    return w.reshape(rows, nsb * 256)


def dequant_q6_k_f32(w_bytes, rows: int, cols: int) -> np.ndarray:
    """fp32 dequant (the exact value; no rounding is needed)."""
    return dequant_q6_k_f64(w_bytes, rows, cols).astype(np.float32)
