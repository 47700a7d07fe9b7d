"""CPU oracle for GGUF Q8_0 / Q4_K dequantization and dequant-times-activation products.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check in __graft_entry__ and
the bench's CPU-baseline leg may import this package. The HIP library never
calls into it, shares no code, tables or helpers with it, and must fail loudly
(not fall back here) when its native extension is missing.

What it computes, and from which passage:

* fp16 decode from bits: IEEE binary16, 1 sign / 5 exponent / 10 fraction bits
  (culpeo.ws blog, the throughput-estimate post, paragraph on BF16 vs half
  precision; "GGUF: The File Format...", practice script, little-endian "<e").
* Q8_0: 34-byte block = fp16 scale + 32 int8, weight = int8 x scale
  ("GGUF Inferencer in R", section 2.1 byte blueprint; "GGUF: The File
  Format...", "How a Q8_0 block is stored" and the practice unpack step).
* Q4_K: 144-byte super-block of 256 weights in 8 sub-blocks of 32, each with a
  6-bit scale and 6-bit min, two fp16 super-scales ("GGUF: The File Format...",
  k-quant paragraph and bits-per-weight table). The bit placement of the
  6-bit fields and nibbles is not on the pages; the reading taken is GGUF's
  on-disk layout, stated in formats.py. PARITY UNPINNED against real GGUF
  files (none available); pinned for self-consistency by hand-packed bytes.
* Q4_0: 18-byte block = fp16 scale + 16 bytes of 4-bit codes, the Q8_0
  recipe with 4-bit integers ("GGUF: The File Format...", "How a Q8_0 block
  is stored", step 4). Nibble order and code offset: GGUF's layout (not on
  the pages). PARITY UNPINNED against real files.
* Q6_K: 210-byte super-block of 256 weights ("GGUF: The File Format...",
  bits-per-weight listing). Field map: GGUF's layout (not on the pages).
  PARITY UNPINNED against real files; pinned for self-consistency.
* matvec y = W x ("culpeo.ws", naive-implementation post, the matvec op), in
  fp64 from the fp32 dequantized weights.
* small batch Y = X W^T with fp32 X (the matvec of each token row), in fp64.
* the steps either side of the GEMVs ("GGUF Inferencer in R", section 5.2):
  RMSN(v) = norm * v / sqrt(mean(v^2) + eps), SiLU(x) = x / (1 + exp(-x)),
  the gated activation SiLU(G) * U, in fp64.
* prefill Y = X W^T with bf16 X ("GGUF Inferencer in R", section 1 and section
  4: prefill is the same math on the whole prompt as one matrix), in fp64.
"""

from .formats import (  # noqa: F401
    Q4_0_BLOCK_BYTES,
    Q4_0_BLOCK_WEIGHTS,
    Q4_K_BLOCK_BYTES,
    Q4_K_BLOCK_WEIGHTS,
    Q8_0_BLOCK_BYTES,
    Q6_K_BLOCK_BYTES,
    Q6_K_BLOCK_WEIGHTS,
    Q8_0_BLOCK_WEIGHTS,
    bf16_bits_to_f64,
    dequant_q4_0_f32,
    dequant_q4_0_f64,
    dequant_q4_k_bf16_bits,
    dequant_q4_k_f32,
    dequant_q4_k_f64,
    dequant_q6_k_f32,
    dequant_q6_k_f64,
    dequant_q8_0_f32,
    dequant_q8_0_f64,
    f32_to_bf16_bits,
    fp16_bits_to_f64,
    pack_q4_0_block,
    pack_q4_k_block,
    pack_q6_k_block,
    q4_0_block_scalar,
    q4_k_block_scalar,
    q6_k_block_scalar,
    q8_0_block_scalar,
    quantize_q4_k_row,
    quantize_q8_0_row,
    row_bytes,
    unpack_q4_0_block,
    unpack_q4_k_block,
    unpack_q6_k_block,
)
from .layer import rmsnorm_f64, silu_f64, swiglu_f64  # noqa: F401
from .linalg import (  # noqa: F401
    floored_rel_err,
    matmul_bf16_x_f64,
    matmul_f32_x_f64,
    matvec_exact,
    matvec_f64,
)
