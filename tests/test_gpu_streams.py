"""GPU: calls on different streams that overlap in time, each with kernels
that keep split-K partial sums and counters in scratch (the bf16 prefill GEMM,
the fp32 small-batch multiply, the Q8_0 lane-per-row GEMV for rows longer than
4096 weights), all against the oracle; and the per-device limit on streams
that hold scratch at one time.
"""

import numpy as np
import pytest
import torch

import gguf_block_quant_dequant_amd as g
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_F32 = 1e-3
TOL_BF16 = 2e-2


def say(*a):
    print(*a, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_tensor(bits):
    return dev(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def test_split_k_calls_on_three_streams_at_once_match_oracle():
    rng = synth.rng_for(41, 0, 0)
    # prefill: 300 rows x 43 super-blocks, 129 tokens (split K over blocks)
    wp = synth.q4_k_weights(rng, 300, 11008)
    xp = synth.activations_bf16_bits(rng, 129, 11008)
    # small batch: 520 rows x 43 super-blocks, 16 tokens (split K over blocks)
    ws = synth.q4_k_weights(rng, 520, 11008)
    xs = rng.standard_normal((16, 11008)).astype(np.float32)
    # Q8_0 GEMV with 11008-weight rows: split-K partials and row-group counters
    wq = synth.q8_0_weights(rng, 1000, 11008)
    xq = rng.standard_normal(11008).astype(np.float32)
    Wp, Xp, Ws, Xs, Wq, Xq = dev(wp), bf16_tensor(xp), dev(ws), dev(xs), dev(wq), dev(xq)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    outs = []
    say("three streams, 4 rounds each, no synchronization in between")
    for _ in range(4):
        with torch.cuda.stream(streams[0]):
            yp = torch.empty((129, 300), dtype=torch.bfloat16, device=DEV)
            g.gguf_qmatmul_q4_k(Wp, Xp, yp, rows=300, stream=streams[0])
        with torch.cuda.stream(streams[1]):
            ys = torch.empty((16, 520), dtype=torch.float32, device=DEV)
            g.gguf_qmatmul_f32_q4_k(Ws, Xs, ys, rows=520, stream=streams[1])
        with torch.cuda.stream(streams[2]):
            yq = torch.empty(1000, dtype=torch.float32, device=DEV)
            g.gguf_qmatvec_q8_0(Wq, Xq, yq, rows=1000, cols=11008, stream=streams[2])
        outs.append((yp, ys, yq))
    torch.cuda.synchronize()
    for s in streams:
        g.gguf_qk_stream_release(s)
    ref_p = oracle.matmul_bf16_x_f64(xp, oracle.dequant_q4_k_f32(wp, 300, 11008))
    ref_s = xs.astype(np.float64) @ oracle.dequant_q4_k_f32(ws, 520, 11008).astype(np.float64).T
    ref_q = oracle.matvec_f64(oracle.dequant_q8_0_f32(wq, 1000, 11008), xq)
    first = None
    for yp, ys, yq in outs:
        got = (yp.view(torch.int16).cpu().numpy().view(np.uint16), ys.cpu().numpy(), yq.cpu().numpy())
        e_p, ok_p = oracle.floored_rel_err(oracle.bf16_bits_to_f64(got[0]), ref_p)
        e_s, ok_s = oracle.floored_rel_err(got[1], ref_s)
        e_q, ok_q = oracle.floored_rel_err(got[2], ref_q)
        say("errors", e_p, e_s, e_q)
        assert ok_p and e_p <= TOL_BF16
        assert ok_s and e_s <= TOL_F32
        assert ok_q and e_q <= TOL_F32
        if first is None:
            first = got
        else:   # the split-K sums are ordered: every round gives the same bits
            for a, b in zip(first, got):
                assert np.array_equal(a, b)


def test_scratch_slots_are_limited_and_released():
    """Streams take scratch slots up to GGUF_QK_STREAM_SLOTS per device; a call
    on one more stream fails with GGUF_QK_ERR_LIMIT and enqueues nothing, and
    succeeds once the other streams release their slots."""
    # rows of 9 super-blocks: the small-batch multiply splits K over blocks
    # (partial tiles in the stream's scratch slot)
    rng = synth.rng_for(42, 0, 0)
    w = dev(synth.q4_k_weights(rng, 64, 2304))
    x = dev(rng.standard_normal((2, 2304)).astype(np.float32))
    torch.cuda.synchronize()
    held, refused = [], None
    for _ in range(g.STREAM_SLOTS + 1):
        s = torch.cuda.Stream()
        if any(s.cuda_stream == h.cuda_stream for h in held):
            continue   # the pool handed out a stream already holding a slot
        try:
            g.gguf_qmatmul_f32_q4_k(w, x, rows=64, stream=s)
        except g.GgufQkError as err:
            assert err.status == g.ERR_LIMIT
            refused = s
            break
        held.append(s)
    torch.cuda.synchronize()
    if refused is None:
        for s in held:
            g.gguf_qk_stream_release(s)
        pytest.skip("the stream pool handed out fewer distinct streams than slots")
    y_before = torch.full((2, 64), 7.0, device=DEV)
    with pytest.raises(g.GgufQkError) as err:
        g.gguf_qmatmul_f32_q4_k(w, x, y_before, rows=64, stream=refused)
    assert err.value.status == g.ERR_LIMIT
    torch.cuda.synchronize()
    assert torch.all(y_before == 7.0)   # nothing was enqueued
    for s in held:
        g.gguf_qk_stream_release(s)
    y = g.gguf_qmatmul_f32_q4_k(w, x, rows=64, stream=refused)
    torch.cuda.synchronize()
    g.gguf_qk_stream_release(refused)
    assert torch.isfinite(y).all()
