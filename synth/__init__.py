"""Seeded synthetic inputs shared by the oracle tests, the GPU tests, the bench and smoke().

This module draws random numbers and places them at the byte offsets a block
format defines. It holds none of the method's arithmetic: nothing here decodes
a block, applies a scale or multiplies anything. Both sides of every parity
check (the CPU oracle and the HIP library) consume exactly these bytes.

Block byte layouts used to place the draws:

* Q8_0, 34 bytes per 32 consecutive weights of one row: a little-endian fp16
  scale, then 32 int8 values ("GGUF Inferencer in R", section 2.1 byte
  blueprint; "GGUF: The File Format...", "How a Q8_0 block is stored").
* Q4_K, 144 bytes per 256 weights ("GGUF: The File Format...", k-quant
  paragraph and bits-per-weight table): fp16 d, fp16 dmin, then 12 bytes of
  packed 6-bit sub-block scales/mins and 128 bytes of 4-bit quants.

Why the Q4_K generator draws raw bytes for the last 140 bytes: the 12 scale
bytes hold sixteen 6-bit fields (8 scales + 8 mins) with every bit of the 96
belonging to exactly one field, and the 128 quant bytes hold 256 nibbles with
every bit belonging to exactly one nibble. Both packings are bijections between
bit strings, so independent uniform bytes are the same distribution as
independent uniform 6-bit fields in [0, 63] and uniform nibbles in [0, 15].
No knowledge of where each field sits is needed to draw them.

Rows are stored back to back with no padding, K (the column count) fastest.
"""

from __future__ import annotations

import concurrent.futures as _cf
from dataclasses import dataclass

import numpy as np

Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32
Q4_K_BLOCK_BYTES = 144
Q4_K_BLOCK_WEIGHTS = 256

ROOT_SEED = 0


def rng_for(cfg_id: int, layer: int, tensor_id: int) -> np.random.Generator:
    """One independent PCG64 stream per (workload, layer, tensor)."""
    return np.random.default_rng([ROOT_SEED, cfg_id, layer, tensor_id])


def _fp16_uniform(rng: np.random.Generator, lo: float, hi: float, n: int) -> np.ndarray:
    """n fp16 values: uniform draws in fp64, rounded to nearest-even fp16."""
    return rng.uniform(lo, hi, size=n).astype(np.float16)


def q8_0_weights(rng: np.random.Generator, rows: int, cols: int,
                 scale_lo: float = 1e-3, scale_hi: float = 1e-2) -> np.ndarray:
    """Q8_0 matrix bytes, shape [rows, cols/32*34] uint8.

    Scale fp16 ~ U[scale_lo, scale_hi]; quants int8 ~ U{-127..127}.
    """
    if cols % Q8_0_BLOCK_WEIGHTS:
        raise ValueError("cols must be a multiple of 32")
    nb = rows * (cols // Q8_0_BLOCK_WEIGHTS)
    out = np.empty((nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = _fp16_uniform(rng, scale_lo, scale_hi, nb).view(np.uint8).reshape(nb, 2)
    out[:, 2:34] = rng.integers(-127, 128, size=(nb, 32), dtype=np.int8).view(np.uint8)
    return out.reshape(rows, -1)


def q4_k_weights(rng: np.random.Generator, rows: int, cols: int,
                 d_lo: float = 1e-4, d_hi: float = 1e-2) -> np.ndarray:
    """Q4_K matrix bytes, shape [rows, cols/256*144] uint8.

    d, dmin fp16 ~ U[d_lo, d_hi]; 6-bit scales/mins ~ U{0..63}; quants ~ U{0..15}
    (drawn as uniform bytes, see the module docstring).
    """
    if cols % Q4_K_BLOCK_WEIGHTS:
        raise ValueError("cols must be a multiple of 256")
    nb = rows * (cols // Q4_K_BLOCK_WEIGHTS)
    out = np.empty((nb, Q4_K_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = _fp16_uniform(rng, d_lo, d_hi, nb).view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = _fp16_uniform(rng, d_lo, d_hi, nb).view(np.uint8).reshape(nb, 2)
    out[:, 4:] = rng.integers(0, 256, size=(nb, Q4_K_BLOCK_BYTES - 4), dtype=np.uint8)
    return out.reshape(rows, -1)


def q4_0_weights(rng: np.random.Generator, rows: int, cols: int,
                 scale_lo: float = 1e-3, scale_hi: float = 1e-2) -> np.ndarray:
    """Q4_0 matrix bytes, shape [rows, cols/32*18] uint8: fp16 scale ~
    U[scale_lo, scale_hi] in bytes 0-1, then 16 uniform bytes (every 4-bit code
    uniform on 0..15 whatever the nibble order)."""
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    nb = rows * (cols // 32)
    out = np.empty((nb, 18), dtype=np.uint8)
    out[:, 0:2] = _fp16_uniform(rng, scale_lo, scale_hi, nb).view(np.uint8).reshape(nb, 2)
    out[:, 2:] = rng.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    return out.reshape(rows, -1)


def q6_k_weights(rng: np.random.Generator, rows: int, cols: int,
                 d_lo: float = 1e-4, d_hi: float = 1e-3) -> np.ndarray:
    """Q6_K matrix bytes, shape [rows, cols/256*210] uint8: 208 uniform bytes
    (the 6-bit codes and the 16 int8 scales uniform whatever the bit map), then
    the fp16 super-scale ~ U[d_lo, d_hi] in bytes 208-209."""
    if cols % 256:
        raise ValueError("cols must be a multiple of 256")
    nb = rows * (cols // 256)
    out = np.empty((nb, 210), dtype=np.uint8)
    out[:, :208] = rng.integers(0, 256, size=(nb, 208), dtype=np.uint8)
    out[:, 208:210] = _fp16_uniform(rng, d_lo, d_hi, nb).view(np.uint8).reshape(nb, 2)
    return out.reshape(rows, -1)


def activations_f32(rng: np.random.Generator, n: int) -> np.ndarray:
    """fp32 vector ~ N(0, 1) (drawn in fp64, rounded to fp32)."""
    return rng.standard_normal(n).astype(np.float32)


def activations_bf16_bits(rng: np.random.Generator, n_tokens: int, cols: int) -> np.ndarray:
    """bf16 matrix [n_tokens, cols] ~ N(0, 1), returned as its uint16 bit patterns.

    Rounding fp64 -> fp32 -> bf16 uses numpy and torch's CPU conversions.
    """
    import torch

    x32 = rng.standard_normal((n_tokens, cols)).astype(np.float32)
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# Workload shapes. The decode-layer shapes follow the SmolLM3-3B tensor table
# ("GGUF Inferencer in R", section 2.1 tensor listing): per layer q 2048x2048,
# k/v 512x2048, o 2048x2048, gate/up 11008x2048, down 2048x11008, 36 layers,
# and the tied 128256x2048 token embedding used as the output head.
# ---------------------------------------------------------------------------

N_LAYERS = 36
HIDDEN = 2048
FFN = 11008
KV = 512
VOCAB = 128256

Q8_0 = "q8_0"
Q4_K = "q4_k"


@dataclass(frozen=True)
class Gemv:
    name: str
    fmt: str
    rows: int
    cols: int


# Per-layer tensors in execution order, grouped into stages: tensors of one
# stage read the same input vector (q/k/v read the normed residual; gate/up
# read the normed residual), and each stage's input depends on the previous
# stage's output in a real decode step.
LAYER_STAGES: tuple[tuple[Gemv, ...], ...] = (
    (Gemv("q", Q4_K, HIDDEN, HIDDEN), Gemv("k", Q4_K, KV, HIDDEN), Gemv("v", Q4_K, KV, HIDDEN)),
    (Gemv("o", Q4_K, HIDDEN, HIDDEN),),
    (Gemv("gate", Q4_K, FFN, HIDDEN), Gemv("up", Q4_K, FFN, HIDDEN)),
    (Gemv("down", Q4_K, HIDDEN, FFN),),
)
HEAD = Gemv("head", Q8_0, VOCAB, HIDDEN)

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "head": 7}


def row_bytes(fmt: str, cols: int) -> int:
    if fmt == Q8_0:
        return cols // Q8_0_BLOCK_WEIGHTS * Q8_0_BLOCK_BYTES
    if fmt == Q4_K:
        return cols // Q4_K_BLOCK_WEIGHTS * Q4_K_BLOCK_BYTES
    raise ValueError(fmt)


def gemv_weights(rng: np.random.Generator, g: Gemv) -> np.ndarray:
    if g.fmt == Q8_0:
        return q8_0_weights(rng, g.rows, g.cols)
    return q4_k_weights(rng, g.rows, g.cols)


@dataclass
class DecodeStage:
    """One stage of the decode stream: GEMVs sharing one input vector."""
    layer: int               # -1 for the head
    gemvs: tuple[Gemv, ...]
    weights: list            # per GEMV: uint8 [rows, row_bytes]
    x: np.ndarray            # fp32 [cols]


DECODE_CFG_ID = 4
PREFILL_CFG_ID = 5


def decode_stream(n_layers: int = N_LAYERS, head: bool = True, threads: int = 8,
                  cfg_id: int = DECODE_CFG_ID) -> list[DecodeStage]:
    """The full decode-step weight stream: n_layers x {qkv, o, gate+up, down}
    Q4_K stages, then the Q8_0 head. One seeded stream per tensor
    (rng_for(cfg_id, layer, tensor_id)); the input of each stage is drawn from
    rng_for(cfg_id, layer, 100 + stage index)."""
    jobs = []
    for layer in range(n_layers):
        for st in LAYER_STAGES:
            for g in st:
                jobs.append((layer, g))
    if head:
        jobs.append((-1, HEAD))

    def make(job):
        layer, g = job
        return gemv_weights(rng_for(cfg_id, layer if layer >= 0 else 1000, TENSOR_IDS[g.name]), g)

    with _cf.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        mats = list(ex.map(make, jobs))

    stages: list[DecodeStage] = []
    it = iter(mats)
    for layer in range(n_layers):
        for si, st in enumerate(LAYER_STAGES):
            ws = [next(it) for _ in st]
            x = activations_f32(rng_for(cfg_id, layer, 100 + si), st[0].cols)
            stages.append(DecodeStage(layer, st, ws, x))
    if head:
        ws = [next(it)]
        x = activations_f32(rng_for(cfg_id, 1000, 100), HEAD.cols)
        stages.append(DecodeStage(-1, (HEAD,), ws, x))
    return stages


def decode_stream_bytes(n_layers: int = N_LAYERS, head: bool = True) -> int:
    total = 0
    for st in LAYER_STAGES:
        for g in st:
            total += g.rows * row_bytes(g.fmt, g.cols)
    total *= n_layers
    if head:
        total += HEAD.rows * row_bytes(HEAD.fmt, HEAD.cols)
    return total


# ---------------------------------------------------------------------------
# Single-matrix configurations: the 256x512 Q8_0 GEMV (seed stream cfg 1), the
# Q8_0 GEMVs at decode shapes (cfg 2) and the Q4_K ffn_up-like and
# ffn_down-like GEMVs (cfg 3), batch 1. Weights from rng_for(cfg, 0, tensor),
# the input vector from rng_for(cfg, 0, 100 + tensor).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class SingleMatrix:
    label: str
    fmt: str
    rows: int
    cols: int
    cfg: int
    tensor: int


SINGLE_MATRICES: tuple[SingleMatrix, ...] = (
    SingleMatrix("cfg1 Q8_0 256x512", Q8_0, 256, 512, 1, 0),
    SingleMatrix("cfg2 Q8_0 2048x2048", Q8_0, 2048, 2048, 2, 0),
    SingleMatrix("cfg2 Q8_0 11008x2048", Q8_0, 11008, 2048, 2, 1),
    SingleMatrix("cfg3 Q4_K 11008x2048 (ffn_up-like)", Q4_K, 11008, 2048, 3, 0),
    SingleMatrix("cfg3 Q4_K 2048x11008 (ffn_down-like)", Q4_K, 2048, 11008, 3, 1),
)


def single_matrix(m: SingleMatrix) -> tuple[np.ndarray, np.ndarray]:
    """(weights uint8 [rows, row_bytes], x fp32 [cols]) of a single-matrix case."""
    w = gemv_weights(rng_for(m.cfg, 0, m.tensor), Gemv(m.label, m.fmt, m.rows, m.cols))
    x = activations_f32(rng_for(m.cfg, 0, 100 + m.tensor), m.cols)
    return w, x
