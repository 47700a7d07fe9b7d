"""A GGUF file written by the tests' own writer, mapped by the library's reader,
uploaded through its C ABI and multiplied: the uploaded bytes equal the
written ones, and the products on them match the oracle computed from the
written bytes (not from anything the reader returned)."""

import numpy as np
import pytest
import torch

import gguf_block_quant_dequant_amd as g
import oracle
import synth
from tests.gguf_writer import ARRAY, STRING, gguf_bytes

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_F32 = 1e-3


def test_file_to_products(tmp_path):
    rng = np.random.default_rng(77)
    q4 = synth.q4_k_weights(rng, 384, 2048)
    q8 = synth.q8_0_weights(rng, 300, 512)
    norm = rng.standard_normal(2048).astype(np.float32)
    tensors = [("blk.0.attn_norm.weight", [2048], g.TENSOR_F32, norm.tobytes()),
               ("blk.0.ffn_gate.weight", [2048, 384], g.TENSOR_Q4_K, q4.tobytes()),
               ("blk.0.attn_k.weight", [512, 300], g.TENSOR_Q8_0, q8.tobytes())]
    kvs = [("general.architecture", STRING, "smollm3"), ("smollm3.block_count", 5, 1),
           ("general.languages", ARRAY, (STRING, ["en", "fr"]))]
    blob, start, offs = gguf_bytes(kvs, tensors)
    path = tmp_path / "m.gguf"
    path.write_bytes(blob)
    print("gguf file", len(blob), "bytes, data at", start, flush=True)
    with g.GgufFile(path) as f:
        assert f.metadata["general.languages"] == ["en", "fr"]
        Wq4 = f.upload("blk.0.ffn_gate.weight")
        Wq8 = f.upload("blk.0.attn_k.weight")
        Wn = f.upload("blk.0.attn_norm.weight")
        torch.cuda.synchronize()
        assert np.array_equal(Wq4.cpu().numpy(), q4.reshape(-1))
        assert np.array_equal(Wq8.cpu().numpy(), q8.reshape(-1))
        assert np.array_equal(Wn.cpu().numpy().view(np.float32), norm)
        x = synth.activations_f32(rng, 2048)
        y = g.gguf_qmatvec_q4_k(Wq4, torch.from_numpy(x).to(DEV), rows=384, cols=2048)
        ref = oracle.matvec_f64(oracle.dequant_q4_k_f32(q4, 384, 2048), x)
        e, ok = oracle.floored_rel_err(y.cpu().numpy(), ref)
        assert ok and e <= TOL_F32, e
        X = np.stack([synth.activations_f32(rng, 512) for _ in range(5)])
        Y = g.gguf_qmatmul_f32_q8_0(Wq8, torch.from_numpy(X).to(DEV), rows=300)
        ref = oracle.matmul_f32_x_f64(X, oracle.dequant_q8_0_f32(q8, 300, 512))
        e, ok = oracle.floored_rel_err(Y.cpu().numpy(), ref)
        assert ok and e <= TOL_F32, e


def test_close_right_after_upload_keeps_the_bytes(tmp_path):
    """upload returns once its copy has completed, so closing the file (which
    unmaps it) right after, with no synchronization of our own, cannot cut a
    copy short: a 64 MiB tensor arrives whole."""
    rng = np.random.default_rng(78)
    big = rng.integers(0, 256, size=64 << 20, dtype=np.uint8)
    tensors = [("big.weight", [big.size // 4], g.TENSOR_F32, big.tobytes())]
    blob, _, _ = gguf_bytes([("general.architecture", STRING, "test")], tensors)
    path = tmp_path / "big.gguf"
    path.write_bytes(blob)
    del blob
    print("upload then close", flush=True)
    with g.GgufFile(path) as f:
        W = f.upload("big.weight")
    torch.cuda.synchronize()
    assert np.array_equal(W.cpu().numpy(), big)
