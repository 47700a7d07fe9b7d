"""Python binding of libgguf_qk (include/gguf_qk.h): GGUF Q8_0 / Q4_K dequant and
fused dequant x activation products on an MI355X (gfx950).

Argument marshalling only: each function takes torch device tensors, passes
their raw pointers, sizes and the current HIP stream to the C entry point of
the same name, and raises on a negative status. Every arithmetic step runs in
the library's kernels; there is no CPU path. If the library has not been built
the first call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

TYPE_Q8_0 = 8
TYPE_Q4_K = 12

OK = 0
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ALIAS, ERR_DEVICE, ERR_LAUNCH, ERR_LIMIT = -1, -2, -3, -4, -5, -6, -7

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "gguf_qk_abi_version": (ctypes.c_int, []),
    "gguf_qk_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "gguf_row_bytes": (_I64, [ctypes.c_int, _I64]),
    "dequant_q8_0": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "dequant_q4_k": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "dequant_q4_k_bf16": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "gguf_qmatvec_q8_0": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "gguf_qmatvec_q4_k": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "gguf_qmatmul_q4_k": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "gguf_qmatmul_f32_q8_0": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "gguf_qmatmul_f32_q4_k": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "gguf_qk_probe_read": (ctypes.c_int, [_P, _I64, _P, _P]),
    "gguf_qmatvec_batch": (ctypes.c_int, [_P, ctypes.c_int32, _P]),
}


class GemvEntry(ctypes.Structure):
    """struct gguf_qk_gemv of the C ABI."""
    _fields_ = [("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("type", ctypes.c_int32),
                ("stage", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


def lib() -> ctypes.CDLL:
    """The loaded libgguf_qk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gguf_block_quant_dequant_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class GgufQkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gguf_qk_strerror(status)} (status {status})")


class GgufQkArgumentError(GgufQkError, ValueError):
    pass


def _check(status: int, where: str) -> None:
    if status == OK:
        return
    if status in (ERR_DEVICE, ERR_LAUNCH):
        raise GgufQkError(status, where)
    raise GgufQkArgumentError(status, where)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _rows_cols(W: torch.Tensor, fmt: int, rows, cols):
    if rows is None or cols is None:
        if W.dim() != 2:
            raise ValueError("pass rows and cols, or W as a [rows, row_bytes] uint8 tensor")
        r = W.shape[0]
        rb = W.shape[1]
        blk_b, blk_w = (34, 32) if fmt == TYPE_Q8_0 else (144, 256)
        if rb % blk_b:
            raise ValueError("W row bytes are not a whole number of blocks")
        rows = r if rows is None else rows
        cols = rb // blk_b * blk_w if cols is None else cols
    need = gguf_row_bytes(fmt, cols)
    if need < 0:
        raise GgufQkArgumentError(need, "row bytes")
    if W.numel() * W.element_size() < rows * need:
        raise ValueError("W is smaller than rows x row bytes")
    return int(rows), int(cols)


def gguf_qk_abi_version() -> int:
    return lib().gguf_qk_abi_version()


def gguf_qk_strerror(status: int) -> str:
    return lib().gguf_qk_strerror(status).decode()


def gguf_row_bytes(type_id: int, cols: int) -> int:
    return lib().gguf_row_bytes(type_id, cols)


def _dequant(name, fmt, W, out, rows, cols, out_dtype, stream):
    rows, cols = _rows_cols(W, fmt, rows, cols)
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=W.device)
    if out.numel() < rows * cols:
        raise ValueError("out is too small")
    _check(getattr(lib(), name)(_dev(W, "W", torch.uint8), _dev(out, "out", out_dtype), rows, cols,
                                _stream(stream)), name)
    return out


def dequant_q8_0(W, out=None, rows=None, cols=None, stream=None):
    """fp32 [rows, cols] dequant of a Q8_0 matrix (bit-exact)."""
    return _dequant("dequant_q8_0", TYPE_Q8_0, W, out, rows, cols, torch.float32, stream)


def dequant_q4_k(W, out=None, rows=None, cols=None, stream=None):
    """fp32 [rows, cols] dequant of a Q4_K matrix (bit-exact)."""
    return _dequant("dequant_q4_k", TYPE_Q4_K, W, out, rows, cols, torch.float32, stream)


def dequant_q4_k_bf16(W, out=None, rows=None, cols=None, stream=None):
    """bf16 [rows, cols]: the fp32 dequant rounded to nearest-even."""
    return _dequant("dequant_q4_k_bf16", TYPE_Q4_K, W, out, rows, cols, torch.bfloat16, stream)


def _matvec(name, fmt, W, x, y, rows, cols, stream):
    rows, cols = _rows_cols(W, fmt, rows, x.numel() if cols is None else cols)
    if x.numel() != cols:
        raise ValueError(f"x has {x.numel()} elements, expected {cols}")
    if y is None:
        y = torch.empty(rows, dtype=torch.float32, device=W.device)
    if y.numel() != rows:
        raise ValueError(f"y has {y.numel()} elements, expected {rows}")
    _check(getattr(lib(), name)(_dev(W, "W", torch.uint8), _dev(x, "x", torch.float32),
                                _dev(y, "y", torch.float32), rows, cols, _stream(stream)), name)
    return y


def gguf_qmatvec_q8_0(W, x, y=None, rows=None, cols=None, stream=None):
    """y = dequant(W) @ x for a Q8_0 W (fp32 x and y)."""
    return _matvec("gguf_qmatvec_q8_0", TYPE_Q8_0, W, x, y, rows, cols, stream)


def gguf_qmatvec_q4_k(W, x, y=None, rows=None, cols=None, stream=None):
    """y = dequant(W) @ x for a Q4_K W (fp32 x and y)."""
    return _matvec("gguf_qmatvec_q4_k", TYPE_Q4_K, W, x, y, rows, cols, stream)


def gguf_qmatmul_q4_k(W, X, Y=None, rows=None, stream=None):
    """Y = X @ dequant(W)^T for a Q4_K W, X bf16 [n_tokens, cols], Y bf16 [n_tokens, rows]."""
    if X.dim() != 2:
        raise ValueError("X must be [n_tokens, cols]")
    n, cols = X.shape
    rows, cols = _rows_cols(W, TYPE_Q4_K, rows, cols)
    if Y is None:
        Y = torch.empty((n, rows), dtype=torch.bfloat16, device=W.device)
    if Y.numel() != n * rows:
        raise ValueError("Y must have n_tokens x rows elements")
    _check(lib().gguf_qmatmul_q4_k(_dev(W, "W", torch.uint8), _dev(X, "X", torch.bfloat16),
                                   _dev(Y, "Y", torch.bfloat16), n, rows, cols, _stream(stream)),
           "gguf_qmatmul_q4_k")
    return Y


def _matmul_f32(name, fmt, W, X, Y, rows, stream):
    if X.dim() != 2:
        raise ValueError("X must be [n_tokens, cols]")
    n, cols = X.shape
    rows, cols = _rows_cols(W, fmt, rows, cols)
    if Y is None:
        Y = torch.empty((n, rows), dtype=torch.float32, device=W.device)
    if Y.numel() != n * rows:
        raise ValueError("Y must have n_tokens x rows elements")
    _check(getattr(lib(), name)(_dev(W, "W", torch.uint8), _dev(X, "X", torch.float32),
                                _dev(Y, "Y", torch.float32), n, rows, cols, _stream(stream)), name)
    return Y


def gguf_qmatmul_f32_q8_0(W, X, Y=None, rows=None, stream=None):
    """Y = X @ dequant(W)^T for a Q8_0 W, X fp32 [n_tokens, cols], Y fp32 [n_tokens, rows]."""
    return _matmul_f32("gguf_qmatmul_f32_q8_0", TYPE_Q8_0, W, X, Y, rows, stream)


def gguf_qmatmul_f32_q4_k(W, X, Y=None, rows=None, stream=None):
    """Y = X @ dequant(W)^T for a Q4_K W, X fp32 [n_tokens, cols], Y fp32 [n_tokens, rows]."""
    return _matmul_f32("gguf_qmatmul_f32_q4_k", TYPE_Q4_K, W, X, Y, rows, stream)


def gguf_qk_probe_read(buf, sink=None, stream=None):
    """Enqueue one streaming read of the whole device tensor `buf` (its byte size
    must be a multiple of 16). Returns the 16-byte-aligned sink tensor."""
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=buf.device)
    _check(lib().gguf_qk_probe_read(_dev(buf, "buf"), nbytes, _dev(sink, "sink", torch.int32),
                                    _stream(stream)), "gguf_qk_probe_read")
    return sink


class GemvBatch:
    """A prepared gguf_qmatvec_batch list: entries (type, W, x, y, stage) with
    device tensors; keeps the tensors alive and the C array built once."""

    def __init__(self, entries):
        self._keep = []
        arr = (GemvEntry * len(entries))()
        for i, (type_id, W, x, y, stage) in enumerate(entries):
            rows, cols = y.numel(), x.numel()
            _rows_cols(W, type_id, rows, cols)
            arr[i] = GemvEntry(_dev(W, "W", torch.uint8), _dev(x, "x", torch.float32),
                               _dev(y, "y", torch.float32), rows, cols, type_id, stage, (0, 0))
            self._keep.append((W, x, y))
        self.array = arr
        self.n = len(entries)


def gguf_qmatvec_batch(batch: GemvBatch, stream=None):
    """Run a prepared GemvBatch (steps in order on the stream)."""
    _check(lib().gguf_qmatvec_batch(ctypes.cast(batch.array, ctypes.c_void_p), batch.n,
                                    _stream(stream)), "gguf_qmatvec_batch")
