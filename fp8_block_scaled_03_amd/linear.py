"""Fp8Linear: a bias-free linear layer whose three matmuls run on the
block-scaled FP8 path of this package.

The Puro-2B technical report (lkr-homepage blog, section 2 "FP8") trains the
main linear layers with their matrix multiplications in FP8 under DeepSeek-V3
style fine-grained block quantization, and keeps the rest of the step in BF16
or FP32.  This module is that usage for one layer, over the C ABI only:

  forward   X [T, in] -> fp8_quantize_dual: row tiles for fprop, token-axis
            tiles kept for wgrad (the activation is saved in FP8, not BF16);
            W [out, in] -> fp8_quantize_block (with the transposed codes
            dgrad needs); Y = fp8_gemm_fprop, BF16.
  backward  dY -> fp8_quantize_dual; dX = fp8_gemm_dgrad (BF16);
            dW = fp8_gemm_wgrad (FP32).

dW is returned in FP32 (autograd casts it to the parameter's dtype), or, when
the weight carries an FP32 ``main_grad`` tensor, added into that tensor by the
wgrad GEMM itself (fp8_gemm_wgrad_accumulate) and not returned, the usual home
of weight gradients in mixed-precision training.
T (the flattened token count), ``in`` and ``out`` must be multiples of 128.
There is no fallback: without the HIP library every call raises.
"""
from __future__ import annotations

import math

import torch

from . import _binding as B


def _check_dims(t: int, d_in: int, d_out: int) -> None:
    bad = [f"{n}={v}" for n, v in (("tokens", t), ("in_features", d_in),
                                    ("out_features", d_out)) if v % 128 != 0]
    if bad:
        raise ValueError("Fp8Linear needs multiples of 128: " + ", ".join(bad))


class Fp8LinearFunction(torch.autograd.Function):
    """y = x @ w.T with FP8 block-scaled forward and backward matmuls."""

    @staticmethod
    def forward(ctx, x2d: torch.Tensor, weight: torch.Tensor, workspace, mfma8: bool = False):
        if x2d.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
            raise ValueError("Fp8Linear works on bfloat16 inputs and weights")
        x2d = x2d.contiguous()
        w = weight.detach().contiguous()
        _check_dims(x2d.shape[0], x2d.shape[1], w.shape[0])
        xq, xs, xtq, xts = B.fp8_quantize_dual(x2d)
        wq, wqt, ws = B.fp8_quantize_block(w, with_transpose=True)
        fprop = B.fp8_gemm_fprop_mfma8 if mfma8 else B.fp8_gemm_fprop
        y = fprop(xq, xs, wq, ws, out_dtype=torch.bfloat16)
        ctx.save_for_backward(xtq, xts, wqt, ws)
        ctx.weight = weight
        ctx.workspace = workspace
        ctx.mfma8 = mfma8
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        xtq, xts, wqt, ws = ctx.saved_tensors
        dy = dy.to(torch.bfloat16).contiguous()
        dyq, dys, dytq, dyts = B.fp8_quantize_dual(dy)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dgrad = B.fp8_gemm_dgrad_mfma8 if ctx.mfma8 else B.fp8_gemm_dgrad
            dx = dgrad(dyq, dys, wqt, ws, out_dtype=torch.bfloat16)
        if ctx.needs_input_grad[1]:
            main = getattr(ctx.weight, "main_grad", None)
            ws_arg = ctx.workspace if ctx.workspace is not None else "auto"
            if ctx.mfma8:
                need = B.fp8_gemm_wgrad_mfma8_workspace_bytes(
                    xtq.shape[1], dytq.shape[0], xtq.shape[0])
                if ctx.workspace is not None and ctx.workspace.numel() < need:
                    ws_arg = "auto"
                dw32 = B.fp8_gemm_wgrad_mfma8(dytq, dyts, xtq, xts, workspace=ws_arg)
                if main is not None:
                    main.add_(dw32)      # this mode has no fused accumulation
                else:
                    dw = dw32
            elif main is not None:
                # Summed into main_grad by the GEMM itself (no separate pass).
                need = B.fp8_gemm_wgrad_accumulate_workspace_bytes(
                    xtq.shape[1], dytq.shape[0], xtq.shape[0])
                if ctx.workspace is not None and ctx.workspace.numel() < need:
                    ws_arg = "auto"
                B.fp8_gemm_wgrad_accumulate(dytq, dyts, xtq, xts, main, workspace=ws_arg)
            else:
                dw = B.fp8_gemm_wgrad(dytq, dyts, xtq, xts, workspace=ws_arg)
        return dx, dw, None, None


class Fp8Linear(torch.nn.Module):
    """Bias-free linear layer (weight [out_features, in_features], BF16) whose
    forward and backward matmuls run through the FP8 block-scaled kernels.

    ``workspace``: optional uint8 device tensor for the wgrad split-K slices
    (at least ``fp8_gemm_wgrad_workspace_bytes`` of the layer's shape, or
    ``fp8_gemm_wgrad_accumulate_workspace_bytes`` when the weight carries a
    ``main_grad``); when None or smaller, each backward allocates what the
    library asks for.

    ``mfma8``: run the three GEMMs as fp8_gemm_*_mfma8, whose block sums come
    from the FP8 matrix core (its limited accumulation precision inside each
    128-wide block, at twice the FP16 rate) instead of exactly.
    """

    def __init__(self, in_features: int, out_features: int, device=None, std: float = 0.02,
                 workspace: torch.Tensor | None = None, mfma8: bool = False):
        super().__init__()
        _check_dims(128, in_features, out_features)
        self.in_features = in_features
        self.out_features = out_features
        self.weight = torch.nn.Parameter(
            torch.empty(out_features, in_features, device=device, dtype=torch.bfloat16))
        torch.nn.init.normal_(self.weight, std=std)
        self.workspace = workspace
        self.mfma8 = mfma8

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        y = Fp8LinearFunction.apply(x.reshape(math.prod(lead), self.in_features), self.weight,
                                    self.workspace, self.mfma8)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        mode = "block-scaled, FP8-MFMA block sums" if self.mfma8 else "block-scaled"
        return f"in_features={self.in_features}, out_features={self.out_features}, fp8={mode}"
