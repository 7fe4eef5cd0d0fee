"""Fp8SwiGLUMLP (the decoder's MLP on the FP8 path) through the C ABI.

Each call it makes is checked against the oracle elsewhere; here:
  - its outputs and gradients equal, bit for bit, the same chain of public
    calls made by hand (so the module wires them as documented);
  - they are close to an unquantized float64 MLP (FP8-level differences, far
    below what a swapped gate/up half or a misrouted operand would give);
  - weights carrying an FP32 main_grad receive the sum in the same call."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_03_amd as fp8
from fp8_block_scaled_03_amd import inputs
from helpers import to_dev_bf16

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _setup(T, d, F, key, mfma8=False):
    mlp = fp8.Fp8SwiGLUMLP(d, F, device="cuda", mfma8=mfma8)
    with torch.no_grad():
        mlp.weight_gate_up.copy_(to_dev_bf16(inputs.normal((key, 2 * F, d), (2 * F, d), 0.02)))
        mlp.weight_down.copy_(to_dev_bf16(inputs.normal((key + 1, d, F), (d, F), 0.02)))
    x = to_dev_bf16(inputs.normal((key + 2, T, d), (T, d), 1.0))
    dy = to_dev_bf16(inputs.student_t((key + 3, T, d), (T, d), 3.0, 1e-3))
    return mlp, x, dy


def _by_hand(x, w_gu, w_down, dy, mfma8):
    B = fp8
    fprop = B.fp8_gemm_fprop_mfma8 if mfma8 else B.fp8_gemm_fprop
    dgrad = B.fp8_gemm_dgrad_mfma8 if mfma8 else B.fp8_gemm_dgrad
    wgrad = B.fp8_gemm_wgrad_mfma8 if mfma8 else B.fp8_gemm_wgrad
    xq, xs, xtq, xts = B.fp8_quantize_dual(x)
    gq, gqt, gs = B.fp8_quantize_block(w_gu)
    gu = fprop(xq, xs, gq, gs, out_dtype="bf16")
    hq, hs, htq, hts, _ = B.fp8_swiglu_quantize_dual(gu)
    dq, dqt, dsc = B.fp8_quantize_block(w_down)
    y = fprop(hq, hs, dq, dsc, out_dtype="bf16")
    dyq, dys, dytq, dyts = B.fp8_quantize_dual(dy)
    dh = dgrad(dyq, dys, dqt, dsc, out_dtype="bf16")
    dw_down = wgrad(dytq, dyts, htq, hts, workspace="auto")
    aq, asc, atq, ats, _ = B.fp8_swiglu_backward_quantize_dual(dh, gu)
    dx = dgrad(aq, asc, gqt, gs, out_dtype="bf16")
    dw_gu = wgrad(atq, ats, xtq, xts, workspace="auto")
    return y, dx, dw_gu, dw_down


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.contiguous().view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("mfma8", [False, True])
def test_mlp_equals_the_chain_of_calls(mfma8):
    T, d, F = 512, 256, 384
    mlp, x, dy = _setup(T, d, F, 140, mfma8)
    xg = x.clone().requires_grad_(True)
    y = mlp(xg)
    y.backward(dy)
    ry, rdx, rdw_gu, rdw_down = _by_hand(x, mlp.weight_gate_up.detach(), mlp.weight_down.detach(),
                                         dy, mfma8)
    torch.cuda.synchronize()
    assert _same(y, ry) and _same(xg.grad, rdx)
    # parameter grads are the FP32 results cast to BF16 by autograd
    assert _same(mlp.weight_gate_up.grad, rdw_gu.bfloat16())
    assert _same(mlp.weight_down.grad, rdw_down.bfloat16())


def test_mlp_is_close_to_an_unquantized_mlp():
    T, d, F = 512, 256, 384
    mlp, x, dy = _setup(T, d, F, 144)
    xg = x.clone().requires_grad_(True)
    y = mlp(xg)
    y.backward(dy)
    torch.cuda.synchronize()
    # float64 reference on the CPU, autograd for the gradients
    x64 = x.double().cpu().requires_grad_(True)
    wgu = mlp.weight_gate_up.detach().double().cpu().requires_grad_(True)
    wd = mlp.weight_down.detach().double().cpu().requires_grad_(True)
    gu = x64 @ wgu.T
    h = torch.nn.functional.silu(gu[:, :F]) * gu[:, F:]
    y64 = h @ wd.T
    y64.backward(dy.double().cpu())
    rel = lambda a, b: float((a.detach().double().cpu() - b).norm() / b.norm())
    errs = dict(y=rel(y, y64.detach()), dx=rel(xg.grad, x64.grad), dw_gu=rel(mlp.weight_gate_up.grad, wgu.grad),
                dw_down=rel(mlp.weight_down.grad, wd.grad))
    _say("Fp8SwiGLUMLP vs float64:", {k: f"{v:.3e}" for k, v in errs.items()})
    # one E4M3 quantization per operand gives ~3% per GEMM; two chained GEMMs stay below ~10%
    for k, v in errs.items():
        assert 1e-3 < v < 0.1, (k, v)


def test_mlp_main_grad_accumulates():
    T, d, F = 256, 256, 256
    mlp, x, dy = _setup(T, d, F, 148)
    for w in (mlp.weight_gate_up, mlp.weight_down):
        w.main_grad = torch.zeros(w.shape, dtype=torch.float32, device="cuda")
    for _ in range(2):
        mlp(x.clone().requires_grad_(True)).backward(dy)
    _, _, rdw_gu, rdw_down = _by_hand(x, mlp.weight_gate_up.detach(), mlp.weight_down.detach(), dy,
                                      False)
    torch.cuda.synchronize()
    assert mlp.weight_gate_up.grad is None and mlp.weight_down.grad is None
    # x + x is exact in FP32: two identical backward passes give exactly 2 dW
    assert torch.equal(mlp.weight_gate_up.main_grad, 2 * rdw_gu)
    assert torch.equal(mlp.weight_down.main_grad, 2 * rdw_down)


def test_mlp_batched_shape_and_errors():
    mlp = fp8.Fp8SwiGLUMLP(256, 384, device="cuda")
    x = torch.randn(2, 128, 256, device="cuda").bfloat16()
    assert mlp(x).shape == (2, 128, 256)
    with pytest.raises(ValueError):
        mlp(torch.randn(100, 256, device="cuda").bfloat16())        # tokens not a multiple of 128
    with pytest.raises(ValueError):
        mlp(torch.randn(128, 256, device="cuda"))                   # float32 input
