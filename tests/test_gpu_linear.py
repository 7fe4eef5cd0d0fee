"""Fp8Linear (forward and backward through the C ABI) against the oracle's
quantizers and GEMMs applied to the same BF16 tensors: Y and dX within the
BF16 gate, dW (FP32) within the FP32 gate."""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8
from fp8_block_scaled_03_amd import inputs
from helpers import check_bf16, check_f32, to_dev_bf16, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _oracle_layer(xb, wb, dyb):
    xq, xs = oracle.quantize_rowtile(xb)
    xtq, xts = oracle.quantize_transposed(xb)
    wq, wqt, ws = oracle.quantize_block(wb)
    dyq, dys = oracle.quantize_rowtile(dyb)
    dytq, dyts = oracle.quantize_transposed(dyb)
    y = oracle.gemm_fprop(xq, xs, wq, ws)
    dx = oracle.gemm_dgrad(dyq, dys, wqt, ws)
    dw = oracle.gemm_wgrad(dytq, dyts, xtq, xts)
    deq = dict(x=oracle.dequantize_rows(xq, xs), w=oracle.dequantize_block(wq, ws),
               dy=oracle.dequantize_rows(dyq, dys), dyt=oracle.dequantize_rows(dytq, dyts),
               xt=oracle.dequantize_rows(xtq, xts))
    return y, dx, dw, deq


@pytest.mark.parametrize("T,d_in,d_out", [(256, 512, 384), (384, 256, 640)])
def test_fp8_linear_forward_backward(T, d_in, d_out):
    _say(f"Fp8Linear T={T} in={d_in} out={d_out}")
    xb = inputs.random_bits((40, T, d_in), (T, d_in), "normal")
    wb = inputs.normal((41, d_out, d_in), (d_out, d_in), 0.02)
    dyb = inputs.student_t((42, T, d_out), (T, d_out), 3.0, 1e-3)
    lin = fp8.Fp8Linear(d_in, d_out, device="cuda")
    with torch.no_grad():
        lin.weight.copy_(to_dev_bf16(wb))
    x = to_dev_bf16(xb).requires_grad_(True)
    y = lin(x)
    y.backward(to_dev_bf16(dyb))
    torch.cuda.synchronize()
    ry, rdx, rdw, deq = _oracle_layer(xb, wb, dyb)
    check_bf16(to_np(y), ry, deq["x"], deq["w"], "Fp8Linear Y")
    check_bf16(to_np(x.grad), rdx, deq["dy"], deq["w"].T, "Fp8Linear dX")
    # weight.grad is dW (FP32) cast to the parameter's BF16 by autograd
    assert lin.weight.grad.dtype == torch.bfloat16
    check_bf16(to_np(lin.weight.grad), rdw, deq["dyt"], deq["xt"], "Fp8Linear dW (bf16)")


def test_fp8_linear_main_grad_accumulates_fp32():
    T, d_in, d_out = 256, 256, 256
    xb = inputs.random_bits((43, T, d_in), (T, d_in), "wide")
    wb = inputs.normal((44, d_out, d_in), (d_out, d_in), 0.02)
    dyb = inputs.student_t((45, T, d_out), (T, d_out), 3.0, 1e-3)
    lin = fp8.Fp8Linear(d_in, d_out, device="cuda")
    with torch.no_grad():
        lin.weight.copy_(to_dev_bf16(wb))
    lin.weight.main_grad = torch.zeros(d_out, d_in, dtype=torch.float32, device="cuda")
    for _ in range(2):
        x = to_dev_bf16(xb).requires_grad_(True)
        lin(x).backward(to_dev_bf16(dyb))
    torch.cuda.synchronize()
    assert lin.weight.grad is None
    _, _, rdw, deq = _oracle_layer(xb, wb, dyb)
    got = to_np(lin.weight.main_grad)
    check_f32(got / 2, rdw, deq["dyt"], deq["xt"], "main_grad / 2")
    # x + x is exact in FP32, so two identical backward passes give exactly 2 dW
    one = got / 2
    assert np.array_equal(one * 2, got)


def test_fp8_linear_batched_shape_and_errors():
    lin = fp8.Fp8Linear(256, 128, device="cuda")
    x = torch.randn(2, 64, 256, device="cuda").bfloat16()
    y = lin(x)
    assert y.shape == (2, 64, 128) and y.dtype == torch.bfloat16
    y2 = lin(x.reshape(128, 256)).reshape(2, 64, 128)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    with pytest.raises(ValueError):
        lin(torch.randn(100, 256, device="cuda").bfloat16())
    with pytest.raises(ValueError):
        lin(torch.randn(128, 256, device="cuda"))         # float32 input


def test_fp8_linear_close_to_bf16_matmul():
    """Property, not parity: the FP8 layer tracks the unquantized product
    within the error of 3-bit-mantissa operands."""
    torch.manual_seed(0)
    lin = fp8.Fp8Linear(1024, 512, device="cuda")
    x = torch.randn(512, 1024, device="cuda").bfloat16()
    y = lin(x).float()
    ref = x.float() @ lin.weight.float().T
    rel = (torch.linalg.norm(y - ref) / torch.linalg.norm(ref)).item()
    assert 5e-3 < rel < 6e-2, rel


def test_fp8_linear_mfma8_runs_the_mfma8_gemms():
    """Fp8Linear(mfma8=True): Y, dX and dW equal, bit for bit, the
    fp8_gemm_*_mfma8 calls on the layer's own quantizations, and meet those
    calls' accumulation bound against the oracle."""
    from test_gpu_mfma8 import check_mfma8
    T, d_in, d_out = 384, 256, 640
    xb = inputs.random_bits((46, T, d_in), (T, d_in), "normal")
    wb = inputs.normal((47, d_out, d_in), (d_out, d_in), 0.02)
    dyb = inputs.student_t((48, T, d_out), (T, d_out), 3.0, 1e-3)
    lin = fp8.Fp8Linear(d_in, d_out, device="cuda", mfma8=True)
    with torch.no_grad():
        lin.weight.copy_(to_dev_bf16(wb))
    lin.weight.main_grad = torch.zeros(d_out, d_in, dtype=torch.float32, device="cuda")
    x = to_dev_bf16(xb).requires_grad_(True)
    y = lin(x)
    y.backward(to_dev_bf16(dyb))
    xq, xs, xtq, xts = fp8.fp8_quantize_dual(to_dev_bf16(xb))
    wq, wqt, ws = fp8.fp8_quantize_block(to_dev_bf16(wb))
    dyq, dys, dytq, dyts = fp8.fp8_quantize_dual(to_dev_bf16(dyb))
    y8 = fp8.fp8_gemm_fprop_mfma8(xq, xs, wq, ws)
    dx8 = fp8.fp8_gemm_dgrad_mfma8(dyq, dys, wqt, ws)
    dw8 = fp8.fp8_gemm_wgrad_mfma8(dytq, dyts, xtq, xts, workspace="auto")
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y), to_np(y8))
    assert np.array_equal(to_np(x.grad), to_np(dx8))
    assert np.array_equal(to_np(lin.weight.main_grad).view(np.uint32), to_np(dw8).view(np.uint32))
    ry, rdx, rdw, deq = _oracle_layer(xb, wb, dyb)
    check_mfma8(to_np(lin.weight.main_grad), rdw, deq["dyt"], deq["xt"], "Fp8Linear(mfma8) dW")
    check_mfma8(to_np(y), ry, deq["x"], deq["w"], "Fp8Linear(mfma8) Y", bf16=True)


def test_fp8_linear_small_workspace_is_replaced():
    """A workspace smaller than the wgrad's query (16 bytes, where the
    4096-token contraction of a 384 x 256 weight is split) is replaced by one
    allocated for the call, on the exact path with and without main_grad:
    the gradients equal those of a layer given no workspace, bit for bit."""
    T, d_in, d_out = 4096, 256, 384
    assert fp8.fp8_gemm_wgrad_workspace_bytes(T, d_out, d_in) > 16
    xb = inputs.normal((46, T, d_in), (T, d_in), 1.0)
    wb = inputs.normal((47, d_out, d_in), (d_out, d_in), 0.02)
    dyb = inputs.student_t((48, T, d_out), (T, d_out), 3.0, 1e-3)
    for with_main in (False, True):
        grads = []
        for ws in (None, torch.empty(16, dtype=torch.uint8, device="cuda")):
            lin = fp8.Fp8Linear(d_in, d_out, device="cuda", workspace=ws)
            with torch.no_grad():
                lin.weight.copy_(to_dev_bf16(wb))
            if with_main:
                lin.weight.main_grad = torch.zeros(d_out, d_in, dtype=torch.float32, device="cuda")
            x = to_dev_bf16(xb).requires_grad_(True)
            lin(x).backward(to_dev_bf16(dyb))
            torch.cuda.synchronize()
            dw = lin.weight.main_grad if with_main else lin.weight.grad
            grads.append((dw.clone(), x.grad.clone()))
        _say(f"Fp8Linear small workspace main_grad={with_main}")
        assert torch.equal(grads[0][0], grads[1][0]) and torch.equal(grads[0][1], grads[1][1])
