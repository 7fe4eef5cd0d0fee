"""Every entry point enqueues on the stream it is given (the caller's current
stream through the binding).  On a side stream, a long spin kernel is queued
first and the inputs are overwritten after it; a call that ran anywhere but
behind them would read the old inputs, so its outputs would differ from the
same call made afterwards on the default stream with the new inputs."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_03_amd as fp8
from fp8_block_scaled_03_amd import inputs
from helpers import to_dev_bf16

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 50_000_000        # a few tens of ms of device time


def _bits(t):
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def _same(a, b):
    return torch.equal(_bits(a.contiguous()), _bits(b.contiguous()))


def test_quantizers_run_on_the_callers_stream():
    M, C = 256, 512
    old = to_dev_bf16(inputs.normal((40,), (M, C)))
    new = to_dev_bf16(inputs.student_t((41,), (M, C), 3.0, 0.5))
    old_dh = to_dev_bf16(inputs.normal((45,), (M, C // 2)))
    new_dh = to_dev_bf16(inputs.normal((46,), (M, C // 2), 0.5))
    gamma = to_dev_bf16(inputs.normal((47,), (C,), 0.5))
    x, dh = old.clone(), old_dh.clone()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("quantizers and quantize-on-produce calls on a side stream", flush=True)

    def calls(x, dh):
        return (fp8.fp8_quantize_rowtile(x), fp8.fp8_quantize_dual(x),
                fp8.fp8_quantize_transposed(x), fp8.fp8_quantize_block(x),
                fp8.fp8_quantize_block_many([x, dh])[1],
                fp8.fp8_rmsnorm_quantize_dual(x, gamma, 1e-6, with_y=True),
                fp8.fp8_swiglu_quantize_dual(x, with_h=True),
                fp8.fp8_swiglu_backward_quantize_dual(dh, x, with_bf16=True))

    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN_CYCLES)
        x.copy_(new)
        dh.copy_(new_dh)
        got = calls(x, dh)
    side.synchronize()
    want = calls(new, new_dh)
    torch.cuda.synchronize()
    for g, w in zip(got, want):
        for a, b in zip(g, w):
            assert (a is None and b is None) or _same(a, b)


def test_gemms_run_on_the_callers_stream():
    M, N, K = 512, 384, 640
    xb = inputs.normal((42,), (M, K))
    wb = inputs.normal((43,), (N, K), 0.02)
    dyb = inputs.student_t((44,), (M, N), 3.0, 1e-3)
    x, w, dy = to_dev_bf16(xb), to_dev_bf16(wb), to_dev_bf16(dyb)
    xq, xs, xtq, xts = fp8.fp8_quantize_dual(x)
    wq, wqt, ws = fp8.fp8_quantize_block(w)
    dyq, dys, dytq, dyts = fp8.fp8_quantize_dual(dy)
    srcs = [xq, xs, xtq, xts, wq, wqt, ws, dyq, dys, dytq, dyts, x, w]
    live = [torch.zeros_like(t) for t in srcs]      # what the calls read: zeros until the copy
    lxq, lxs, lxtq, lxts, lwq, lwqt, lws, ldyq, ldys, ldytq, ldyts, lx, lw = live
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("GEMMs on a side stream", flush=True)
    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN_CYCLES)
        for dst, src in zip(live, srcs):
            dst.copy_(src)
        got = (fp8.fp8_gemm_fprop(lxq, lxs, lwq, lws),
               fp8.fp8_gemm_dgrad(ldyq, ldys, lwqt, lws),
               fp8.fp8_gemm_wgrad(ldytq, ldyts, lxtq, lxts, workspace="auto"),
               fp8.fp8_gemm_dgrad_quantized(ldyq, ldys, lwqt, lws),
               fp8.bf16_gemm_tn(lx, lw))
    side.synchronize()
    want = (fp8.fp8_gemm_fprop(xq, xs, wq, ws),
            fp8.fp8_gemm_dgrad(dyq, dys, wqt, ws),
            fp8.fp8_gemm_wgrad(dytq, dyts, xtq, xts, workspace="auto"),
            fp8.fp8_gemm_dgrad_quantized(dyq, dys, wqt, ws),
            fp8.bf16_gemm_tn(x, w))
    torch.cuda.synchronize()
    for g, w_ in zip(got, want):
        g = g if isinstance(g, tuple) else (g,)
        w_ = w_ if isinstance(w_, tuple) else (w_,)
        for a, b in zip(g, w_):
            assert _same(a, b)
    assert np.isfinite(got[0].float().cpu().numpy()).all()


def test_temporaries_of_a_stream_argument_live_on_that_stream():
    """A call given stream= (not the current stream) allocates its output and
    its "auto" workspace on that stream, so torch does not hand the freed
    workspace to other work while the split-K kernels still use it: the
    allocator's segments holding them are tagged with the launch stream, and
    an immediate same-size allocation on the current stream, written at
    once, leaves the result unchanged."""
    M, N, K = 4096, 1024, 1024
    dytq = torch.randint(0, 0x7E, (N, M), dtype=torch.uint8, device="cuda")
    xtq = torch.randint(0, 0x7E, (K, M), dtype=torch.uint8, device="cuda")
    dyts = torch.rand(N, M // 128, device="cuda") + 0.5
    xts = torch.rand(K, M // 128, device="cuda") + 0.5
    nbytes = fp8.fp8_gemm_wgrad_workspace_bytes(M, N, K)
    assert nbytes > 0, "the shape must split for this test"
    want = fp8.fp8_gemm_wgrad(dytq, dyts, xtq, xts, workspace="auto")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("wgrad with stream= a side stream behind a spin", flush=True)
    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN_CYCLES)
    got = fp8.fp8_gemm_wgrad(dytq, dyts, xtq, xts, workspace="auto", stream=side)
    junk = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")   # current stream
    segs = torch.cuda.memory_snapshot()
    side.synchronize()
    torch.cuda.synchronize()
    assert _same(got, want)
    side_blocks = [b["size"] for s in segs if s["stream"] == side.cuda_stream for b in s["blocks"]]
    assert any(sz >= nbytes for sz in side_blocks), side_blocks
    assert any(sz >= N * K * 4 for sz in side_blocks), side_blocks
    del junk
