"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments before any HIP call. No compute call is made: every
call here fails validation (or, with no device present, the device check)."""

import ctypes
import os
import re

import pytest

import gguf_block_quant_dequant_amd as g
from gguf_block_quant_dequant_amd.build import LIB_PATH

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = [os.path.join(INCLUDE, h) for h in sorted(os.listdir(INCLUDE)) if h.endswith(".h")]

def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0   # (counting does not initialize a device)


# Well-formed calls here carry made-up addresses and rely on the missing
# device to stop them: where a GPU is visible they would launch, so the module
# runs only where none is.
pytestmark = [pytest.mark.skipif(not os.path.exists(LIB_PATH),
                                 reason="libgguf_qk.so not built (run the build step first)"),
              pytest.mark.skipif(_gpu_visible(), reason="made-up device addresses: only where no GPU is visible")]


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        body = text.split('extern "C" {', 1)[1]
        names |= set(re.findall(
            r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
            body, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ["gguf_qmatvec_q8_0", "gguf_qmatvec_q4_k", "gguf_qmatmul_q4_k", "dequant_q8_0",
              "dequant_q4_k", "dequant_q4_k_bf16", "gguf_row_bytes", "gguf_qk_strerror",
              "gguf_qk_abi_version", "gguf_qmatvec_batch", "gguf_qmatmul_f32_q8_0",
              "gguf_qmatmul_f32_q4_k", "gguf_file_open", "gguf_file_close", "gguf_tensor_nbytes",
              "gguf_file_tensor", "gguf_file_kv", "gguf_file_upload_tensor"]:
        assert n in names


def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(g.library_path())
    missing = [n for n in _declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_binding_names_match_header():
    for n in _declared_functions():
        assert hasattr(g, n), n


def test_version_and_strerror():
    assert g.gguf_qk_abi_version() == 2
    for s in range(-10, 1):
        assert g.gguf_qk_strerror(s)
    assert g.gguf_qk_strerror(-99) == "unknown status"


def test_row_bytes_other_types():
    assert g.gguf_row_bytes(g.TYPE_Q4_0, 2048) == 1152
    assert g.gguf_row_bytes(g.TYPE_Q4_0, 96) == 54
    assert g.gguf_row_bytes(g.TYPE_Q6_K, 11008) == 9030
    assert g.gguf_row_bytes(g.TYPE_Q4_0, 48) == g.ERR_SHAPE
    assert g.gguf_row_bytes(g.TYPE_Q6_K, 128) == g.ERR_SHAPE


def test_batch_type_checks():
    e = g.GemvEntry(0x10000, 0x20000, 0x30000, 4, 256, g.TYPE_Q6_K, 0)
    assert g.lib().gguf_qmatvec_batch(ctypes.byref(e), 1, None) == g.ERR_DEVICE   # accepted
    e = g.GemvEntry(0x10000, 0x20000, 0x30000, 4, 256, 99, 0)
    assert g.lib().gguf_qmatvec_batch(ctypes.byref(e), 1, None) == g.ERR_SHAPE
    # no fused epilogue for Q4_0 / Q6_K
    arr = (g.GemvEntry * 1)(g.GemvEntry(0x1000000, 0x5000000, 0x6000000, 64, 2048, g.TYPE_Q6_K, 0, (0, 0)))
    assert _run_ep(arr, [_ep(residual=0xC000000)]) == g.ERR_SHAPE


def test_row_bytes():
    assert g.gguf_row_bytes(g.TYPE_Q8_0, 2048) == 2176
    assert g.gguf_row_bytes(g.TYPE_Q8_0, 512) == 544
    assert g.gguf_row_bytes(g.TYPE_Q4_K, 2048) == 1152
    assert g.gguf_row_bytes(g.TYPE_Q4_K, 11008) == 6192
    assert g.gguf_row_bytes(g.TYPE_Q4_K, 100) == g.ERR_SHAPE
    assert g.gguf_row_bytes(g.TYPE_Q8_0, 33) == g.ERR_SHAPE
    assert g.gguf_row_bytes(g.TYPE_Q8_0, 0) == g.ERR_SHAPE
    assert g.gguf_row_bytes(99, 256) == g.ERR_SHAPE


# Fake, never-dereferenced addresses: every call below fails validation first.
A = 0x10000
B = 0x20000
C = 0x30000


def _mv(name, W, x, y, rows, cols):
    return getattr(g.lib(), name)(W, x, y, rows, cols, None)


@pytest.mark.parametrize("name", ["gguf_qmatvec_q8_0", "gguf_qmatvec_q4_k", "gguf_qmatvec_q4_0",
                                  "gguf_qmatvec_q6_k"])
def test_matvec_validation(name):
    assert _mv(name, None, B, C, 4, 256) == g.ERR_NULL
    assert _mv(name, A, None, C, 4, 256) == g.ERR_NULL
    assert _mv(name, A, B, None, 4, 256) == g.ERR_NULL
    assert _mv(name, A, B, C, -1, 256) == g.ERR_SHAPE
    assert _mv(name, A, B, C, 4, 0) == g.ERR_SHAPE
    assert _mv(name, A, B, C, 4, -256) == g.ERR_SHAPE
    assert _mv(name, A, B, C, 4, 255) == g.ERR_SHAPE
    assert _mv(name, A, B, C, 1 << 62, 1 << 40) == g.ERR_SHAPE      # byte size overflows
    assert _mv(name, A + 2, B, C, 4, 256) == g.ERR_ALIGN
    assert _mv(name, A, B + 4, C, 4, 256) == g.ERR_ALIGN
    assert _mv(name, A, B, C + 8, 4, 256) == g.ERR_ALIGN
    assert _mv(name, A, B, A + 16, 4, 256) == g.ERR_ALIAS           # y inside W
    assert _mv(name, A, B, B, 4, 256) == g.ERR_ALIAS                # y == x
    assert _mv(name, A, B, C, 0, 256) == g.OK                       # nothing to do


def test_q4_k_matvec_rejects_q8_0_only_widths():
    assert _mv("gguf_qmatvec_q4_k", A, B, C, 4, 32) == g.ERR_SHAPE
    assert _mv("gguf_qmatvec_q8_0", A, B, C, 0, 32) == g.OK


@pytest.mark.parametrize("name,cols", [("dequant_q8_0", 64), ("dequant_q4_k", 256),
                                       ("dequant_q4_k_bf16", 256), ("dequant_q4_0", 64),
                                       ("dequant_q6_k", 256)])
def test_dequant_validation(name, cols):
    f = getattr(g.lib(), name)
    assert f(None, B, 4, cols, None) == g.ERR_NULL
    assert f(A, None, 4, cols, None) == g.ERR_NULL
    assert f(A, B, -1, cols, None) == g.ERR_SHAPE
    assert f(A, B, 4, cols + 1, None) == g.ERR_SHAPE
    assert f(A + 1, B, 4, cols, None) == g.ERR_ALIGN
    assert f(A, B + 2, 4, cols, None) == g.ERR_ALIGN
    assert f(A, A + 16, 4, cols, None) == g.ERR_ALIAS
    assert f(A, B, 0, cols, None) == g.OK


def test_matmul_validation():
    f = g.lib().gguf_qmatmul_q4_k
    assert f(None, B, C, 8, 4, 256, None) == g.ERR_NULL
    assert f(A, None, C, 8, 4, 256, None) == g.ERR_NULL
    assert f(A, B, None, 8, 4, 256, None) == g.ERR_NULL
    assert f(A, B, C, -1, 4, 256, None) == g.ERR_SHAPE
    assert f(A, B, C, 8, -4, 256, None) == g.ERR_SHAPE
    assert f(A, B, C, 8, 4, 128, None) == g.ERR_SHAPE
    assert f(A, B + 2, C, 8, 4, 256, None) == g.ERR_ALIGN
    assert f(A, B, B + 16, 8, 4, 256, None) == g.ERR_ALIAS          # Y overlaps X
    assert f(A, B, C, 0, 4, 256, None) == g.OK
    assert f(A, B, C, 8, 0, 256, None) == g.OK


def test_matmul_multi_validation():
    f = g.lib().gguf_qmatmul_q4_k_multi
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    W2, Y2, R2 = (P * 2)(A, A + 4096), (P * 2)(C, C + (1 << 20)), (I64 * 2)(4, 8)
    assert f(None, Y2, R2, 2, B, 8, 256, None) == g.ERR_NULL
    assert f(W2, None, R2, 2, B, 8, 256, None) == g.ERR_NULL
    assert f(W2, Y2, None, 2, B, 8, 256, None) == g.ERR_NULL
    assert f(W2, Y2, R2, 0, B, 8, 256, None) == g.ERR_SHAPE           # 1 .. 4 matrices
    assert f(W2, Y2, R2, 5, B, 8, 256, None) == g.ERR_SHAPE
    assert f(W2, Y2, R2, 2, None, 8, 256, None) == g.ERR_NULL
    assert f(W2, Y2, (I64 * 2)(4, -1), 2, B, 8, 256, None) == g.ERR_SHAPE
    assert f(W2, Y2, R2, 2, B, 8, 128, None) == g.ERR_SHAPE          # K % 256
    assert f(W2, (P * 2)(C, None), R2, 2, B, 8, 256, None) == g.ERR_NULL
    assert f((P * 2)(A, None), (P * 2)(C, None), (I64 * 2)(4, 0), 2, B, 0, 256, None) == g.OK
    assert f(W2, (P * 2)(C, C + 2), R2, 2, B, 8, 256, None) == g.ERR_ALIGN
    assert f(W2, (P * 2)(C, C + 16), R2, 2, B, 8, 256, None) == g.ERR_ALIAS   # Y1 overlaps Y0
    assert f(W2, (P * 2)(C, A), R2, 2, B, 8, 256, None) == g.ERR_ALIAS        # Y1 overlaps W0
    assert f(W2, Y2, R2, 2, B, 0, 256, None) == g.OK                 # no tokens: nothing to do
    assert f(W2, Y2, (I64 * 2)(0, 0), 2, B, 8, 256, None) == g.OK    # no rows: nothing to do


@pytest.mark.parametrize("name", ["gguf_qmatmul_f32_q8_0_multi", "gguf_qmatmul_f32_q4_k_multi"])
def test_small_batch_multi_validation(name):
    f = getattr(g.lib(), name)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    W2, Y2, R2 = (P * 2)(A, A + 8192), (P * 2)(C, C + (1 << 20)), (I64 * 2)(4, 8)
    assert f(None, Y2, R2, 2, B, 8, 256, None) == g.ERR_NULL
    assert f(W2, Y2, R2, 0, B, 8, 256, None) == g.ERR_SHAPE
    assert f(W2, Y2, R2, 5, B, 8, 256, None) == g.ERR_SHAPE
    assert f(W2, Y2, R2, 2, B, 8, 288, None) == g.ERR_SHAPE          # K % 256
    assert f(W2, (P * 2)(C, C + 16), R2, 2, B, 8, 256, None) == g.ERR_ALIAS   # Y1 overlaps Y0
    assert f(W2, Y2, R2, 2, B, 0, 256, None) == g.OK
    assert f((P * 2)(A, None), (P * 2)(C, None), (I64 * 2)(4, 0), 2, B, 0, 256, None) == g.OK


@pytest.mark.parametrize("name", ["gguf_qmatmul_f32_q8_0", "gguf_qmatmul_f32_q4_k"])
def test_small_batch_validation(name):
    f = getattr(g.lib(), name)
    assert f(None, B, C, 8, 4, 256, None) == g.ERR_NULL
    assert f(A, None, C, 8, 4, 256, None) == g.ERR_NULL
    assert f(A, B, None, 8, 4, 256, None) == g.ERR_NULL
    assert f(A, B, C, -1, 4, 256, None) == g.ERR_SHAPE
    assert f(A, B, C, 8, -4, 256, None) == g.ERR_SHAPE
    assert f(A, B, C, 8, 4, 0, None) == g.ERR_SHAPE
    assert f(A, B, C, 8, 4, 224, None) == g.ERR_SHAPE              # K steps are 256 wide
    assert f(A, B, C, 1 << 40, 4, 1 << 30, None) == g.ERR_SHAPE    # X bytes overflow
    assert f(A + 8, B, C, 8, 4, 256, None) == g.ERR_ALIGN
    assert f(A, B + 4, C, 8, 4, 256, None) == g.ERR_ALIGN
    assert f(A, B, C + 4, 8, 4, 256, None) == g.ERR_ALIGN
    assert f(A, B, B + 16, 8, 4, 256, None) == g.ERR_ALIAS          # Y overlaps X
    assert f(A, B, A + 16, 8, 4, 256, None) == g.ERR_ALIAS          # Y overlaps W
    assert f(A, B, C, 0, 4, 256, None) == g.OK
    assert f(A, B, C, 8, 0, 256, None) == g.OK


def _no_gpu_visible():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu_visible(), reason="only meaningful where no GPU is visible")
def test_valid_arguments_without_a_device_report_no_device():
    # Arguments pass validation; with no device the call stops at the device
    # check and never launches.
    assert _mv("gguf_qmatvec_q4_k", A, B, C, 4, 256) == g.ERR_DEVICE
    assert g.lib().dequant_q8_0(A, B, 4, 64, None) == g.ERR_DEVICE
    assert g.lib().gguf_qmatmul_q4_k(A, B, C, 8, 4, 256, None) == g.ERR_DEVICE


def test_binding_rejects_host_tensors():
    import torch
    W = torch.zeros((4, 144), dtype=torch.uint8)
    x = torch.zeros(256, dtype=torch.float32)
    with pytest.raises(ValueError):
        g.gguf_qmatvec_q4_k(W, x)


def _entry(W, x, y, rows, cols, typ, stage):
    return g.GemvEntry(W, x, y, rows, cols, typ, stage, (0, 0))


def test_batch_validation():
    f = g.lib().gguf_qmatvec_batch
    arr = (g.GemvEntry * 2)(_entry(A, B, C, 4, 256, g.TYPE_Q4_K, 0),
                            _entry(A, B, C + 4096, 4, 256, g.TYPE_Q4_K, 0))
    p = ctypes.cast(arr, ctypes.c_void_p)
    assert f(None, 1, None) == g.ERR_NULL
    assert f(p, -1, None) == g.ERR_SHAPE
    assert f(p, 0, None) == g.OK
    bad = (g.GemvEntry * 1)(_entry(A, B, C, 4, 256, 3, 0))
    assert f(ctypes.cast(bad, ctypes.c_void_p), 1, None) == g.ERR_SHAPE
    bad = (g.GemvEntry * 1)(_entry(A, B, C, 4, 100, g.TYPE_Q4_K, 0))
    assert f(ctypes.cast(bad, ctypes.c_void_p), 1, None) == g.ERR_SHAPE
    bad = (g.GemvEntry * 1)(_entry(A, B + 4, C, 4, 256, g.TYPE_Q4_K, 0))
    assert f(ctypes.cast(bad, ctypes.c_void_p), 1, None) == g.ERR_ALIGN
    # same step: second y overlaps the first entry's x -> alias
    bad = (g.GemvEntry * 2)(_entry(A, B, C, 4, 256, g.TYPE_Q4_K, 0),
                            _entry(A, B, B, 4, 256, g.TYPE_Q4_K, 0))
    assert f(ctypes.cast(bad, ctypes.c_void_p), 2, None) == g.ERR_ALIAS
    # same step: two entries write the same y -> alias
    bad = (g.GemvEntry * 2)(_entry(A, B, C, 4, 256, g.TYPE_Q4_K, 0),
                            _entry(A + 4096, B, C, 4, 256, g.TYPE_Q4_K, 0))
    assert f(ctypes.cast(bad, ctypes.c_void_p), 2, None) == g.ERR_ALIAS


# ---------------------------------------------------- fused epilogues (batch_ep)

def _pair_entries(type_id=None, cols=2048, rows=64):
    """gate/up entries at fake, non-overlapping addresses."""
    t = g.TYPE_Q4_K if type_id is None else type_id
    arr = (g.GemvEntry * 2)()
    arr[0] = g.GemvEntry(0x1000000, 0x5000000, 0x6000000, rows, cols, t, 0, (0, 0))
    arr[1] = g.GemvEntry(0x2000000, 0x5000000, 0x7000000, rows, cols, t, 0, (0, 0))
    return arr


def _ep(**kw):
    e = g.GemvEpEntry()
    for k, v in kw.items():
        setattr(e, k, v)
    return e


def _run_ep(arr, eps):
    ep = (g.GemvEpEntry * len(eps))(*eps)
    return g.lib().gguf_qmatvec_batch_ep(ctypes.cast(arr, ctypes.c_void_p), ctypes.cast(ep, ctypes.c_void_p),
                                         len(eps), None)


def test_batch_ep_validation():
    ACT = 0x8000000
    ok = [_ep(pair=1, act=ACT), _ep(pair=2, act=ACT)]
    assert _run_ep(_pair_entries(), ok) == g.ERR_DEVICE          # valid: fails only at the device check
    assert _run_ep(_pair_entries(), [_ep(pair=1, act=ACT), _ep()]) == g.ERR_SHAPE       # partner missing
    assert _run_ep(_pair_entries(), [_ep(pair=1, act=ACT), _ep(pair=2, act=ACT + 64)]) == g.ERR_SHAPE
    assert _run_ep(_pair_entries(), [_ep(pair=3, act=ACT), _ep()]) == g.ERR_SHAPE
    assert _run_ep(_pair_entries(), [_ep(pair=1), _ep(pair=2)]) == g.ERR_NULL          # no act
    assert _run_ep(_pair_entries(), [_ep(pair=1, act=ACT + 2), _ep(pair=2, act=ACT + 2)]) == g.ERR_ALIGN
    assert _run_ep(_pair_entries(), [_ep(pair=1, act=0x6000000), _ep(pair=2, act=0x6000000)]) == g.ERR_ALIAS
    assert _run_ep(_pair_entries(), [_ep(norm_w=0x9000000), _ep()]) == g.ERR_NULL
    assert _run_ep(_pair_entries(), [_ep(norm_w=0x9000000, norm_out=0x7000000, ss_out=0xA000000),
                                     _ep()]) == g.ERR_ALIAS                              # over the other y
    assert _run_ep(_pair_entries(), [_ep(scale_ss=0xB000000, scale_n=0), _ep()]) == g.ERR_SHAPE
    # the input RMSN from the vector itself: alone, 16-byte aligned, not over an output of the step
    assert _run_ep(_pair_entries(), [_ep(scale_v=0xB000000), _ep()]) == g.ERR_DEVICE
    assert _run_ep(_pair_entries(), [_ep(scale_v=0xB000000, scale_ss=0xB100000, scale_n=4), _ep()]) == g.ERR_SHAPE
    assert _run_ep(_pair_entries(), [_ep(scale_v=0xB000004), _ep()]) == g.ERR_ALIGN
    assert _run_ep(_pair_entries(), [_ep(scale_v=0x7000000), _ep()]) == g.ERR_ALIAS    # the other entry's y
    assert _run_ep(_pair_entries(), [_ep(scale_v=0xB000000, eps=-1.0), _ep()]) == g.ERR_SHAPE
    # norm_out without the partial sums is complete; ss_out alone is not
    assert _run_ep(_pair_entries(), [_ep(norm_w=0x9000000, norm_out=0xA000000), _ep()]) == g.ERR_DEVICE
    assert _run_ep(_pair_entries(), [_ep(ss_out=0xA000000), _ep()]) == g.ERR_NULL
    assert _run_ep(_pair_entries(), [_ep(scale_ss=0xB000000, scale_n=4, eps=-1.0), _ep()]) == g.ERR_SHAPE
    assert _run_ep(_pair_entries(), [_ep(scale_ss=0xB000000, scale_n=4, eps=float("nan")), _ep()]) == g.ERR_SHAPE
    assert _run_ep(_pair_entries(), [_ep(residual=0xC000001), _ep()]) == g.ERR_ALIGN
    assert _run_ep(_pair_entries(), [_ep(residual=0x6000000 + 4), _ep()]) == g.ERR_ALIAS   # partial overlap with y
    assert _run_ep(_pair_entries(), [_ep(residual=0x6000000), _ep()]) == g.ERR_DEVICE      # y itself: in place
    # Q8_0 rows that are not whole 256-weight chunks take the row-wise kernel, which has no epilogue
    assert _run_ep(_pair_entries(g.TYPE_Q8_0, cols=96), [_ep(residual=0xC000000), _ep()]) == g.ERR_SHAPE
    assert _run_ep(_pair_entries(g.TYPE_Q8_0, cols=96), [_ep(), _ep()]) == g.ERR_DEVICE


def test_layer_ops_validation():
    L = g.lib()
    assert L.gguf_rmsnorm_prep_f32(None, B, C, 0x40000, 64, None) == g.ERR_NULL
    assert L.gguf_rmsnorm_prep_f32(A, B, C + 4, 0x40000, 64, None) == g.ERR_ALIGN
    assert L.gguf_rmsnorm_prep_f32(A, B, A, 0x40000, 64, None) == g.ERR_ALIAS
    assert L.gguf_rmsnorm_prep_f32(A, B, C, 0x40000, 0, None) == g.OK
    assert L.gguf_rmsnorm_prep_f32(A, B, C, 0x40000, 64, None) == g.ERR_DEVICE
    assert L.gguf_rmsnorm_f32(A, B, ctypes.c_float(-1.0), C, 64, None) == g.ERR_SHAPE
    assert L.gguf_rmsnorm_f32(A, B, ctypes.c_float(1e-6), A + 16, 64, None) == g.ERR_ALIAS
    assert L.gguf_rmsnorm_f32(A, B, ctypes.c_float(1e-6), C, 64, None) == g.ERR_DEVICE
    for f in (L.gguf_swiglu_f32, L.gguf_add_f32):
        assert f(A, B, None, 64, None) == g.ERR_NULL
        assert f(A, B, A + 16, 64, None) == g.ERR_ALIAS       # partial overlap
        assert f(A, B, A, 64, None) == g.ERR_DEVICE           # in place is allowed
        assert f(A, B, C, -1, None) == g.ERR_SHAPE
        assert f(A, B, C, 0, None) == g.OK


def test_batch_binding_rejects_short_epilogue_vectors():
    """The C ABI takes the epilogue vectors without lengths: the binding checks
    each against the entry's rows (ss_out: one float per 64 rows) before
    anything is built or launched."""
    import torch
    rows, cols = 130, 256
    W = torch.zeros((rows, 144), dtype=torch.uint8)
    x, y = torch.zeros(cols), torch.zeros(rows)
    entries = [(g.TYPE_Q4_K, W, x, y, 0)]
    for key, short in (("residual", rows - 1), ("norm_w", rows - 1), ("norm_out", 1), ("act", rows - 1),
                       ("ss_out", 2)):
        with pytest.raises(ValueError, match=key):
            g.GemvBatch(entries, [{key: torch.zeros(short)}])
    with pytest.raises(ValueError, match="one epilogue"):
        g.GemvBatch(entries, [None, None])
    # sizes that fit pass this check (host tensors are then refused as such)
    with pytest.raises(ValueError, match="device tensor"):
        g.GemvBatch(entries, [{"residual": torch.zeros(rows), "ss_out": torch.zeros(3)}])


def test_probe_validation():
    """The probes check their arguments before any HIP call: the latency
    probe's chain length must be a power of two (its indices are masked with
    n - 1, which then keeps every load inside the buffer) and at least one
    wave's worth of start entries."""
    L = g.lib()
    assert L.gguf_qk_probe_read(None, 64, C, None) == g.ERR_NULL
    assert L.gguf_qk_probe_read(A, 63, C, None) == g.ERR_SHAPE
    assert L.gguf_qk_probe_read(A, 64, A + 16, None) == g.ERR_ALIAS
    assert L.gguf_qk_probe_read(A, 64, C, None) == g.ERR_DEVICE
    assert L.gguf_qk_probe_latency(None, 64, 1, C, None) == g.ERR_NULL
    assert L.gguf_qk_probe_latency(A, 64, 1, None, None) == g.ERR_NULL
    for n in (0, 32, 63, 96, 1000, (1 << 31) + 1, 1 << 32):
        assert L.gguf_qk_probe_latency(A, n, 1, C, None) == g.ERR_SHAPE, n
    assert L.gguf_qk_probe_latency(A, 64, 0, C, None) == g.ERR_SHAPE
    assert L.gguf_qk_probe_latency(A + 4, 64, 1, C, None) == g.ERR_ALIGN
    assert L.gguf_qk_probe_latency(A, 64, 1, A + 16, None) == g.ERR_ALIAS
    assert L.gguf_qk_probe_latency(A, 64, 1, C, None) == g.ERR_DEVICE
    assert L.gguf_qk_probe_latency(C, 1 << 31, 1, A, None) == g.ERR_DEVICE   # out below the 8 GiB chain
