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
import struct

import torch

from .build import LIB_PATH, TIMELINE_LIB_PATH

TYPE_Q8_0 = 8
TYPE_Q4_K = 12
TYPE_Q4_0 = 2
TYPE_Q6_K = 14

OK = 0
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ALIAS, ERR_DEVICE, ERR_LAUNCH, ERR_LIMIT = -1, -2, -3, -4, -5, -6, -7
ERR_FORMAT, ERR_IO, ERR_NOT_FOUND = -8, -9, -10

# GGUF tensor and metadata value type ids (include/gguf_file.h)
TENSOR_F32, TENSOR_F16, TENSOR_Q4_0, TENSOR_Q8_0, TENSOR_Q4_K, TENSOR_Q6_K, TENSOR_BF16 = 0, 1, 2, 8, 12, 14, 30
(VALUE_U8, VALUE_I8, VALUE_U16, VALUE_I16, VALUE_U32, VALUE_I32, VALUE_F32, VALUE_BOOL, VALUE_STRING,
 VALUE_ARRAY, VALUE_U64, VALUE_I64, VALUE_F64) = range(13)
_SCALAR_FMT = {VALUE_U8: "<B", VALUE_I8: "<b", VALUE_U16: "<H", VALUE_I16: "<h", VALUE_U32: "<I",
               VALUE_I32: "<i", VALUE_F32: "<f", VALUE_BOOL: "<?", VALUE_U64: "<Q", VALUE_I64: "<q",
               VALUE_F64: "<d"}

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
    "dequant_q4_0": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "dequant_q6_k": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "gguf_qmatvec_q4_0": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "gguf_qmatvec_q6_k": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "gguf_qmatmul_q4_k": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "gguf_qmatmul_q4_k_multi": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _I64, _I64, _P]),
    "gguf_qmatmul_f32_q8_0": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "gguf_qmatmul_f32_q4_k": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "gguf_qmatmul_f32_q8_0_multi": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _I64, _I64, _P]),
    "gguf_qmatmul_f32_q4_k_multi": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _I64, _I64, _P]),
    "gguf_qk_probe_read": (ctypes.c_int, [_P, _I64, _P, _P]),
    "gguf_qk_probe_latency": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "gguf_qk_stream_release": (ctypes.c_int, [_P]),
    "gguf_qk_last_launch": (ctypes.c_int, []),
    "gguf_qk_timeline_setup": (ctypes.c_int, [ctypes.c_uint64]),
    "gguf_qk_timeline_fetch": (ctypes.c_int, [_P, _I64]),
    "gguf_qmatvec_batch": (ctypes.c_int, [_P, ctypes.c_int32, _P]),
    "gguf_qmatvec_batch_ep": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P]),
    "gguf_rmsnorm_prep_f32": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P]),
    "gguf_rmsnorm_f32": (ctypes.c_int, [_P, _P, ctypes.c_float, _P, _I64, _P]),
    "gguf_swiglu_f32": (ctypes.c_int, [_P, _P, _P, _I64, _P]),
    "gguf_add_f32": (ctypes.c_int, [_P, _P, _P, _I64, _P]),
    "gguf_tensor_nbytes": (_I64, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]),
    "gguf_file_open": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_void_p)]),
    "gguf_file_close": (None, [_P]),
    "gguf_file_version": (ctypes.c_int32, [_P]),
    "gguf_file_tensor_count": (_I64, [_P]),
    "gguf_file_kv_count": (_I64, [_P]),
    "gguf_file_alignment": (_I64, [_P]),
    "gguf_file_data_offset": (_I64, [_P]),
    "gguf_file_size": (_I64, [_P]),
    "gguf_file_tensor": (ctypes.c_int, [_P, _I64, _P]),
    "gguf_file_kv": (ctypes.c_int, [_P, _I64, _P]),
    "gguf_file_find_tensor": (_I64, [_P, ctypes.c_char_p]),
    "gguf_file_find_kv": (_I64, [_P, ctypes.c_char_p]),
    "gguf_file_kv_array_string": (ctypes.c_int, [_P, _I64, _I64, ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.POINTER(ctypes.c_int64)]),
    "gguf_file_upload_tensor": (ctypes.c_int, [_P, _I64, _P, _P]),
}


class GgufTensorInfo(ctypes.Structure):
    """struct gguf_tensor_info of the C ABI."""
    _fields_ = [("name", ctypes.c_char_p), ("type", ctypes.c_int32), ("n_dims", ctypes.c_int32),
                ("dims", ctypes.c_int64 * 4), ("offset", ctypes.c_int64), ("nbytes", ctypes.c_int64),
                ("data", ctypes.c_void_p)]


class GgufKvInfo(ctypes.Structure):
    """struct gguf_kv_info of the C ABI."""
    _fields_ = [("key", ctypes.c_char_p), ("type", ctypes.c_int32), ("elem_type", ctypes.c_int32),
                ("count", ctypes.c_int64), ("data", ctypes.c_void_p), ("nbytes", ctypes.c_int64)]


class GemvEntry(ctypes.Structure):
    """struct gguf_qk_gemv of the C ABI."""
    _fields_ = [("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("type", ctypes.c_int32),
                ("stage", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


def library_path() -> str:
    """The build of libgguf_qk.so that lib() loads: GGUF_QK_LIBRARY=<path> (another
    build of the same library: the sanitized host build, measurement of build
    variants), else with GGUF_QK_TIMELINE=1 the instrumented build (stage
    timelines), else the default build."""
    path = TIMELINE_LIB_PATH if os.environ.get("GGUF_QK_TIMELINE") == "1" else LIB_PATH
    return os.environ.get("GGUF_QK_LIBRARY", path)


def lib() -> ctypes.CDLL:
    """The loaded libgguf_qk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m gguf_block_quant_dequant_amd.build`")
        L = ctypes.CDLL(path)
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
        blk_b, blk_w = {TYPE_Q8_0: (34, 32), TYPE_Q4_K: (144, 256), TYPE_Q4_0: (18, 32),
                        TYPE_Q6_K: (210, 256)}[fmt]
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


def dequant_q4_0(W, out=None, rows=None, cols=None, stream=None):
    """fp32 [rows, cols] dequant of a Q4_0 matrix (bit-exact)."""
    return _dequant("dequant_q4_0", TYPE_Q4_0, W, out, rows, cols, torch.float32, stream)


def dequant_q6_k(W, out=None, rows=None, cols=None, stream=None):
    """fp32 [rows, cols] dequant of a Q6_K matrix (bit-exact)."""
    return _dequant("dequant_q6_k", TYPE_Q6_K, W, out, rows, cols, torch.float32, stream)


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


def gguf_qmatvec_q4_0(W, x, y=None, rows=None, cols=None, stream=None):
    """y = dequant(W) @ x for a Q4_0 W (fp32 x and y)."""
    return _matvec("gguf_qmatvec_q4_0", TYPE_Q4_0, W, x, y, rows, cols, stream)


def gguf_qmatvec_q6_k(W, x, y=None, rows=None, cols=None, stream=None):
    """y = dequant(W) @ x for a Q6_K W (fp32 x and y)."""
    return _matvec("gguf_qmatvec_q6_k", TYPE_Q6_K, W, x, y, rows, cols, stream)


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


def gguf_qmatmul_q4_k_multi(Ws, X, Ys=None, rows=None, stream=None):
    """Y[m] = X @ dequant(Ws[m])^T for up to four Q4_K matrices of one X (same
    cols), one launch; returns the list of Y (bf16 [n_tokens, rows[m]])."""
    if X.dim() != 2:
        raise ValueError("X must be [n_tokens, cols]")
    if not 1 <= len(Ws) <= 4:
        raise ValueError("one to four matrices")
    n, cols = X.shape
    rows = list(rows) if rows is not None else [None] * len(Ws)
    if len(rows) != len(Ws):
        raise ValueError("one row count per matrix")
    rows = [_rows_cols(W, TYPE_Q4_K, r, cols)[0] for W, r in zip(Ws, rows)]
    if Ys is None:
        Ys = [torch.empty((n, r), dtype=torch.bfloat16, device=X.device) for r in rows]
    if len(Ys) != len(Ws) or any(Y.numel() != n * r for Y, r in zip(Ys, rows)):
        raise ValueError("one Y of n_tokens x rows[m] elements per matrix")
    k = len(Ws)
    warr = (ctypes.c_void_p * k)(*[_dev(W, "W", torch.uint8) for W in Ws])
    yarr = (ctypes.c_void_p * k)(*[_dev(Y, "Y", torch.bfloat16) for Y in Ys])
    rarr = (ctypes.c_int64 * k)(*rows)
    _check(lib().gguf_qmatmul_q4_k_multi(warr, yarr, rarr, k, _dev(X, "X", torch.bfloat16), n, cols,
                                         _stream(stream)),
           "gguf_qmatmul_q4_k_multi")
    return Ys


def _matmul_f32_multi(name, fmt, Ws, X, Ys, rows, stream):
    if X.dim() != 2:
        raise ValueError("X must be [n_tokens, cols]")
    if not 1 <= len(Ws) <= 4:
        raise ValueError("one to four matrices")
    n, cols = X.shape
    rows = list(rows) if rows is not None else [None] * len(Ws)
    if len(rows) != len(Ws):
        raise ValueError("one row count per matrix")
    rows = [_rows_cols(W, fmt, r, cols)[0] for W, r in zip(Ws, rows)]
    if Ys is None:
        Ys = [torch.empty((n, r), dtype=torch.float32, device=X.device) for r in rows]
    if len(Ys) != len(Ws) or any(Y.numel() != n * r for Y, r in zip(Ys, rows)):
        raise ValueError("one Y of n_tokens x rows[m] elements per matrix")
    k = len(Ws)
    warr = (ctypes.c_void_p * k)(*[_dev(W, "W", torch.uint8) for W in Ws])
    yarr = (ctypes.c_void_p * k)(*[_dev(Y, "Y", torch.float32) for Y in Ys])
    rarr = (ctypes.c_int64 * k)(*rows)
    _check(getattr(lib(), name)(warr, yarr, rarr, k, _dev(X, "X", torch.float32), n, cols, _stream(stream)),
           name)
    return Ys


def gguf_qmatmul_f32_q8_0_multi(Ws, X, Ys=None, rows=None, stream=None):
    """Y[m] = X @ dequant(Ws[m])^T for up to four Q8_0 matrices of one fp32 X, one launch."""
    return _matmul_f32_multi("gguf_qmatmul_f32_q8_0_multi", TYPE_Q8_0, Ws, X, Ys, rows, stream)


def gguf_qmatmul_f32_q4_k_multi(Ws, X, Ys=None, rows=None, stream=None):
    """Y[m] = X @ dequant(Ws[m])^T for up to four Q4_K matrices of one fp32 X, one launch."""
    return _matmul_f32_multi("gguf_qmatmul_f32_q4_k_multi", TYPE_Q4_K, Ws, X, Ys, rows, stream)


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


def gguf_qk_probe_latency(next_idx, steps, out=None, stream=None):
    """Enqueue the dependent-load chase over the int32 device tensor `next_idx`
    (a power-of-two number of entries); returns the int64 tensor out whose
    element 0 becomes the elapsed 100 MHz ticks of `steps` dependent loads."""
    if next_idx.dtype != torch.int32:
        raise TypeError("next_idx must be int32")
    if out is None:
        out = torch.zeros(2, dtype=torch.int64, device=next_idx.device)
    _check(lib().gguf_qk_probe_latency(_dev(next_idx, "next_idx", torch.int32), next_idx.numel(), int(steps),
                                       _dev(out, "out", torch.int64), _stream(stream)), "gguf_qk_probe_latency")
    return out


STREAM_SLOTS = 8   # GGUF_QK_STREAM_SLOTS: scratch slots per device
# GGUF_QK_LAUNCH_*: kernel families reported by gguf_qk_last_launch
(LAUNCH_NONE, LAUNCH_LK_SINGLE, LAUNCH_LK_TWO, LAUNCH_LK_THREE, LAUNCH_LK_GROUP, LAUNCH_LK_LONG, LAUNCH_LKS,
 LAUNCH_SPLIT_K, LAUNCH_OTHER, LAUNCH_ROWWISE) = range(10)


def gguf_qk_last_launch() -> int:
    """Kernel family (LAUNCH_*) of this thread's most recent GEMV launch."""
    return lib().gguf_qk_last_launch()


def gguf_qk_stream_release(stream=None):
    """Give back the scratch slot `stream` holds (synchronize the stream first)."""
    _check(lib().gguf_qk_stream_release(_stream(stream)), "gguf_qk_stream_release")


TIMELINE_SLOTS, TIMELINE_WAVES, TIMELINE_REC_BYTES = 4096, 2048, 32


def timeline_slot(key: int, mult: int) -> int:
    """Record slot of a launch key (its first weight pointer) under `mult`."""
    return ((key * mult) & ((1 << 64) - 1)) >> 52


def gguf_qk_timeline_setup(keys, seed=1):
    """Arm the instrumented build's per-wave stage records; picks an odd
    multiplier under which the launch keys `keys` take distinct slots and
    returns {key: slot}."""
    import random
    ks = sorted(set(int(k) for k in keys))
    rnd = random.Random(seed)
    for _ in range(100000):
        mult = rnd.getrandbits(64) | 1
        slots = [timeline_slot(k, mult) for k in ks]
        if len(set(slots)) == len(slots):
            _check(lib().gguf_qk_timeline_setup(mult), "gguf_qk_timeline_setup")
            return dict(zip(ks, slots))
    raise GgufQkError(ERR_LIMIT, "gguf_qk_timeline_setup: no multiplier separates the keys")


def gguf_qk_timeline_fetch():
    """The record array as a numpy uint32 array [4096, 2048, 8] (six time stamps,
    HW_ID, XCD id per wave)."""
    import numpy as np
    out = np.zeros((TIMELINE_SLOTS, TIMELINE_WAVES, TIMELINE_REC_BYTES // 4), dtype=np.uint32)
    _check(lib().gguf_qk_timeline_fetch(out.ctypes.data, out.nbytes), "gguf_qk_timeline_fetch")
    return out


class GemvEpEntry(ctypes.Structure):
    """struct gguf_qk_gemv_ep of the C ABI."""
    _fields_ = [("scale_ss", ctypes.c_void_p), ("scale_n", ctypes.c_int64), ("eps", ctypes.c_float),
                ("pair", ctypes.c_int32), ("residual", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("norm_out", ctypes.c_void_p), ("ss_out", ctypes.c_void_p), ("act", ctypes.c_void_p),
                ("scale_v", ctypes.c_void_p)]


def _opt(t, name):
    return None if t is None else _dev(t, name, torch.float32)


class GemvBatch:
    """A prepared gguf_qmatvec_batch list: entries (type, W, x, y, stage) with
    device tensors; keeps the tensors alive and the C array built once.

    `epilogues` (optional, one per entry, None for none) are dicts with the
    gguf_qk_gemv_ep fields as keys (scale_ss, eps, pair, residual, norm_w,
    norm_out, ss_out, act, scale_v; tensors for the vectors); the batch then
    runs through gguf_qmatvec_batch_ep."""

    # floats each epilogue vector holds at least, for an entry of `rows` rows
    # (the C ABI takes these pointers without lengths)
    _EP_SIZES = {"residual": lambda r: r, "norm_w": lambda r: r, "norm_out": lambda r: r,
                 "act": lambda r: r, "ss_out": lambda r: (r + 63) // 64}

    def __init__(self, entries, epilogues=None):
        if epilogues is not None:
            if len(epilogues) != len(entries):
                raise ValueError("one epilogue (or None) per entry")
            for (_, _, x, y, _), e in zip(entries, epilogues):
                for key, need in self._EP_SIZES.items():
                    t = (e or {}).get(key)
                    if t is not None and t.numel() < need(y.numel()):
                        raise ValueError(f"epilogue {key} holds {t.numel()} floats, the entry needs "
                                         f"{need(y.numel())}")
                v = (e or {}).get("scale_v")
                if v is not None and v.numel() < x.numel():
                    raise ValueError(f"epilogue scale_v holds {v.numel()} floats, the entry needs {x.numel()}")
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
        self.ep = None
        if epilogues is not None:
            ep = (GemvEpEntry * len(entries))()
            for i, e in enumerate(epilogues):
                if not e:
                    continue
                ss = e.get("scale_ss")
                ep[i] = GemvEpEntry(_opt(ss, "scale_ss"), 0 if ss is None else ss.numel(),
                                    float(e.get("eps", 0.0)), int(e.get("pair", 0)),
                                    _opt(e.get("residual"), "residual"), _opt(e.get("norm_w"), "norm_w"),
                                    _opt(e.get("norm_out"), "norm_out"), _opt(e.get("ss_out"), "ss_out"),
                                    _opt(e.get("act"), "act"), _opt(e.get("scale_v"), "scale_v"))
                self._keep.append(tuple(v for v in e.values() if isinstance(v, torch.Tensor)))
            self.ep = ep


def gguf_qmatvec_batch(batch: GemvBatch, stream=None):
    """Run a prepared GemvBatch (steps in order on the stream)."""
    if batch.ep is not None:
        return gguf_qmatvec_batch_ep(batch, stream)
    _check(lib().gguf_qmatvec_batch(ctypes.cast(batch.array, ctypes.c_void_p), batch.n,
                                    _stream(stream)), "gguf_qmatvec_batch")


def gguf_qmatvec_batch_ep(batch: GemvBatch, stream=None):
    """Run a prepared GemvBatch with its per-entry epilogues."""
    ep = ctypes.cast(batch.ep, ctypes.c_void_p) if batch.ep is not None else None
    _check(lib().gguf_qmatvec_batch_ep(ctypes.cast(batch.array, ctypes.c_void_p), ep, batch.n,
                                       _stream(stream)), "gguf_qmatvec_batch_ep")


def _vec(t, name, n=None):
    p = _dev(t, name, torch.float32)
    if n is not None and t.numel() < n:
        raise ValueError(f"{name} is too small")
    return p


def gguf_rmsnorm_prep_f32(v, norm_w, vw=None, ss=None, stream=None):
    """vw = v * norm_w and ss[j] = sum of v^2 over elements 64 j .. 64 j + 63."""
    n = v.numel()
    vw = torch.empty_like(v) if vw is None else vw
    ss = torch.empty((n + 63) // 64, dtype=torch.float32, device=v.device) if ss is None else ss
    _check(lib().gguf_rmsnorm_prep_f32(_vec(v, "v"), _vec(norm_w, "norm_w", n), _vec(vw, "vw", n),
                                       _vec(ss, "ss", (n + 63) // 64), n, _stream(stream)),
           "gguf_rmsnorm_prep_f32")
    return vw, ss


def gguf_rmsnorm_f32(v, norm_w, eps, out=None, stream=None):
    """out = norm_w * v / sqrt(mean(v^2) + eps)."""
    n = v.numel()
    out = torch.empty_like(v) if out is None else out
    _check(lib().gguf_rmsnorm_f32(_vec(v, "v"), _vec(norm_w, "norm_w", n), float(eps),
                                  _vec(out, "out", n), n, _stream(stream)), "gguf_rmsnorm_f32")
    return out


def gguf_swiglu_f32(g, u, out=None, stream=None):
    """out = SiLU(g) * u."""
    n = g.numel()
    out = torch.empty_like(g) if out is None else out
    _check(lib().gguf_swiglu_f32(_vec(g, "g"), _vec(u, "u", n), _vec(out, "out", n), n,
                                 _stream(stream)), "gguf_swiglu_f32")
    return out


def gguf_add_f32(a, b, out=None, stream=None):
    """out = a + b."""
    n = a.numel()
    out = torch.empty_like(a) if out is None else out
    _check(lib().gguf_add_f32(_vec(a, "a"), _vec(b, "b", n), _vec(out, "out", n), n, _stream(stream)),
           "gguf_add_f32")
    return out


# ------------------------------------------------------------------ GGUF files

def gguf_tensor_nbytes(type_id: int, dims) -> int:
    """Bytes of a tensor of this type and dims (fastest first), or a negative status."""
    d = (ctypes.c_int64 * 4)(*([int(v) for v in dims] + [1] * (4 - len(dims))))
    return lib().gguf_tensor_nbytes(type_id, len(dims), d)


def gguf_file_open(path):
    """Maps and parses a GGUF file; returns the library handle (ctypes.c_void_p)."""
    h = ctypes.c_void_p()
    _check(lib().gguf_file_open(os.fsencode(os.fspath(path)), ctypes.byref(h)), "gguf_file_open")
    return h


def gguf_file_close(h) -> None:
    lib().gguf_file_close(h)


def gguf_file_version(h) -> int:
    return lib().gguf_file_version(h)


def gguf_file_tensor_count(h) -> int:
    return lib().gguf_file_tensor_count(h)


def gguf_file_kv_count(h) -> int:
    return lib().gguf_file_kv_count(h)


def gguf_file_alignment(h) -> int:
    return lib().gguf_file_alignment(h)


def gguf_file_data_offset(h) -> int:
    return lib().gguf_file_data_offset(h)


def gguf_file_size(h) -> int:
    return lib().gguf_file_size(h)


def gguf_file_tensor(h, i: int) -> GgufTensorInfo:
    info = GgufTensorInfo()
    _check(lib().gguf_file_tensor(h, i, ctypes.byref(info)), "gguf_file_tensor")
    return info


def gguf_file_kv(h, i: int) -> GgufKvInfo:
    info = GgufKvInfo()
    _check(lib().gguf_file_kv(h, i, ctypes.byref(info)), "gguf_file_kv")
    return info


def gguf_file_find_tensor(h, name: str) -> int:
    """Index of the tensor, or ERR_NOT_FOUND."""
    return lib().gguf_file_find_tensor(h, name.encode())


def gguf_file_find_kv(h, key: str) -> int:
    """Index of the metadata entry, or ERR_NOT_FOUND."""
    return lib().gguf_file_find_kv(h, key.encode())


def gguf_file_kv_array_string(h, i: int, j: int) -> bytes:
    p, n = ctypes.c_void_p(), ctypes.c_int64()
    _check(lib().gguf_file_kv_array_string(h, i, j, ctypes.byref(p), ctypes.byref(n)),
           "gguf_file_kv_array_string")
    return ctypes.string_at(p, n.value) if n.value else b""


def gguf_file_upload_tensor(h, i: int, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """Copies tensor i's raw bytes into the uint8 device tensor dst."""
    _check(lib().gguf_file_upload_tensor(h, i, _dev(dst, "dst", torch.uint8), _stream(stream)),
           "gguf_file_upload_tensor")
    return dst


class GgufFile:
    """A GGUF file mapped and parsed by the library (include/gguf_file.h).

    `tensors` lists the tensor records (name, type, dims fastest first, absolute
    offset, nbytes); `metadata` decodes every entry (scalars, strings, arrays of
    scalars or strings; nested arrays are returned as their raw payload bytes);
    `upload` copies a tensor's raw bytes to a new device tensor through the
    library. Use as a context manager or call close()."""

    def __init__(self, path):
        self._h = gguf_file_open(path)

    def close(self):
        if getattr(self, "_h", None):
            gguf_file_close(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        self.close()

    def _handle(self):
        if not self._h:
            raise ValueError("the file is closed")
        return self._h

    @property
    def version(self) -> int:
        return gguf_file_version(self._handle())

    @property
    def alignment(self) -> int:
        return gguf_file_alignment(self._handle())

    @property
    def data_offset(self) -> int:
        return gguf_file_data_offset(self._handle())

    @property
    def size(self) -> int:
        return gguf_file_size(self._handle())

    def _index(self, name_or_index) -> int:
        if isinstance(name_or_index, int):
            return name_or_index
        i = gguf_file_find_tensor(self._handle(), name_or_index)
        if i < 0:
            raise KeyError(name_or_index)
        return i

    def tensor(self, name_or_index) -> dict:
        info = gguf_file_tensor(self._handle(), self._index(name_or_index))
        return {"name": info.name.decode("utf-8", "replace"), "type": info.type,
                "dims": tuple(info.dims[: info.n_dims]), "offset": info.offset,
                "nbytes": info.nbytes, "host_ptr": info.data}

    @property
    def tensors(self) -> list:
        return [self.tensor(i) for i in range(gguf_file_tensor_count(self._handle()))]

    def _kv_value(self, i: int, info: GgufKvInfo):
        raw = ctypes.string_at(info.data, info.nbytes) if info.nbytes else b""
        if info.type in _SCALAR_FMT:
            return struct.unpack(_SCALAR_FMT[info.type], raw)[0]
        if info.type == VALUE_STRING:
            return raw.decode("utf-8", "replace")
        if info.type == VALUE_ARRAY:
            if info.elem_type in _SCALAR_FMT:
                fmt = _SCALAR_FMT[info.elem_type]
                return list(struct.unpack("<%d%s" % (info.count, fmt[1]), raw))
            if info.elem_type == VALUE_STRING:
                return [gguf_file_kv_array_string(self._handle(), i, j).decode("utf-8", "replace")
                        for j in range(info.count)]
            return raw
        raise GgufQkArgumentError(ERR_FORMAT, "metadata value")

    @property
    def metadata(self) -> dict:
        out = {}
        for i in range(gguf_file_kv_count(self._handle())):
            info = gguf_file_kv(self._handle(), i)
            out[info.key.decode("utf-8", "replace")] = self._kv_value(i, info)
        return out

    def kv_type(self, key: str):
        """(value type, element type) of a metadata entry."""
        i = gguf_file_find_kv(self._handle(), key)
        if i < 0:
            raise KeyError(key)
        info = gguf_file_kv(self._handle(), i)
        return info.type, info.elem_type

    def upload(self, name_or_index, device="cuda:0", stream=None):
        """A new uint8 device tensor [nbytes] holding the tensor's raw bytes."""
        i = self._index(name_or_index)
        t = self.tensor(i)
        if t["nbytes"] < 0:
            raise GgufQkArgumentError(ERR_FORMAT, f"tensor {t['name']} has a type of unknown size")
        out = torch.empty(max(t["nbytes"], 16), dtype=torch.uint8, device=device)
        gguf_file_upload_tensor(self._handle(), i, out, stream)
        return out[: t["nbytes"]]
