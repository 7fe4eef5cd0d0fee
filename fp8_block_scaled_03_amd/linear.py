"""Fp8Linear: a bias-free linear layer whose three matmuls run on the
block-scaled FP8 path of this package; Fp8SwiGLUMLP: the decoder's MLP built
the same way, with its SwiGLU quantizing on produce.

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

Fp8SwiGLUMLP chains two such layers around the MLP's SwiGLU: the gate/up
projection's BF16 output feeds fp8_swiglu_quantize_dual, whose codes are the
down projection's operands, and in the backward fp8_swiglu_backward_quantize_dual
turns the down projection's BF16 input gradient into the gate/up gradient's
codes, so neither H nor its gradient's successor is stored in BF16.
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


def _weight_grad(weight, workspace, mfma8: bool, dytq, dyts, xtq, xts):
    """dW = dY^T X of one linear layer from the token-axis codes of dY and X:
    returned in FP32, or, when the weight carries an FP32 ``main_grad``, added
    into it (by the wgrad GEMM itself on the exact path) and None returned.
    A workspace smaller than the call's query for this shape (or none) is
    replaced by one allocated for the call."""
    main = getattr(weight, "main_grad", None)
    M, N, K = xtq.shape[1], dytq.shape[0], xtq.shape[0]
    if mfma8:
        query = B.fp8_gemm_wgrad_mfma8_workspace_bytes
    elif main is not None:
        query = B.fp8_gemm_wgrad_accumulate_workspace_bytes
    else:
        query = B.fp8_gemm_wgrad_workspace_bytes
    ws_arg = workspace
    if workspace is None or workspace.numel() < query(M, N, K):
        ws_arg = "auto"
    if mfma8:
        dw32 = B.fp8_gemm_wgrad_mfma8(dytq, dyts, xtq, xts, workspace=ws_arg)
        if main is None:
            return dw32
        main.add_(dw32)              # this mode has no fused accumulation
        return None
    if main is not None:
        # Summed into main_grad by the GEMM itself (no separate pass).
        B.fp8_gemm_wgrad_accumulate(dytq, dyts, xtq, xts, main, workspace=ws_arg)
        return None
    return B.fp8_gemm_wgrad(dytq, dyts, xtq, xts, workspace=ws_arg)


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
            dw = _weight_grad(ctx.weight, ctx.workspace, ctx.mfma8, dytq, dyts, xtq, xts)
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


class Fp8SwiGLUMLPFunction(torch.autograd.Function):
    """y = down(silu(x W_g^T) * (x W_u^T)) with every matmul on the FP8 path and
    the SwiGLU's output (forward) and input gradient (backward) quantized on
    produce.

    forward   W_gu, W_down -> fp8_quantize_block_many (one launch);
              X -> fp8_quantize_dual; GU = fprop(X, W_gu) in BF16 [T, 2F]
              (gate | up); fp8_swiglu_quantize_dual(GU) -> H's row tiles (the
              down projection's fprop) and token-axis tiles (its wgrad);
              Y = fprop(H, W_down).  GU is kept for the backward; H is never
              stored in BF16.
    backward  dY -> fp8_quantize_dual; dH = dgrad(dY, W_down) in BF16;
              dW_down = wgrad(dY, H); fp8_swiglu_backward_quantize_dual(dH,
              GU) -> the gate/up gradient's two quantizations; dX = dgrad(dGU,
              W_gu); dW_gu = wgrad(dGU, X).
    """

    @staticmethod
    def forward(ctx, x2d: torch.Tensor, w_gu: torch.Tensor, w_down: torch.Tensor, workspace,
                mfma8: bool = False):
        if x2d.dtype != torch.bfloat16 or w_gu.dtype != torch.bfloat16 or \
                w_down.dtype != torch.bfloat16:
            raise ValueError("Fp8SwiGLUMLP works on bfloat16 inputs and weights")
        x2d = x2d.contiguous()
        wgu, wd = w_gu.detach().contiguous(), w_down.detach().contiguous()
        F = wd.shape[1]
        if wgu.shape != (2 * F, x2d.shape[1]) or wd.shape[0] != x2d.shape[1]:
            raise ValueError(f"Fp8SwiGLUMLP: w_gate_up {tuple(wgu.shape)} and w_down "
                             f"{tuple(wd.shape)} do not fit inputs of width {x2d.shape[1]}")
        _check_dims(x2d.shape[0], x2d.shape[1], 2 * F)
        _check_dims(x2d.shape[0], F, x2d.shape[1])
        fprop = B.fp8_gemm_fprop_mfma8 if mfma8 else B.fp8_gemm_fprop
        (gq, gqt, gs), (dq, dqt, dsc) = B.fp8_quantize_block_many([wgu, wd])   # one launch
        xq, xs, xtq, xts = B.fp8_quantize_dual(x2d)
        gu = fprop(xq, xs, gq, gs, out_dtype=torch.bfloat16)
        hq, hs, htq, hts, _ = B.fp8_swiglu_quantize_dual(gu)
        y = fprop(hq, hs, dq, dsc, out_dtype=torch.bfloat16)
        ctx.save_for_backward(xtq, xts, gqt, gs, gu, htq, hts, dqt, dsc)
        ctx.weights = (w_gu, w_down)
        ctx.workspace = workspace
        ctx.mfma8 = mfma8
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        xtq, xts, gqt, gs, gu, htq, hts, dqt, dsc = ctx.saved_tensors
        w_gu, w_down = ctx.weights
        dgrad = B.fp8_gemm_dgrad_mfma8 if ctx.mfma8 else B.fp8_gemm_dgrad
        dy = dy.to(torch.bfloat16).contiguous()
        dyq, dys, dytq, dyts = B.fp8_quantize_dual(dy)
        dx = dw_gu = dw_down = None
        dh = dgrad(dyq, dys, dqt, dsc, out_dtype=torch.bfloat16)
        if ctx.needs_input_grad[2]:
            dw_down = _weight_grad(w_down, ctx.workspace, ctx.mfma8, dytq, dyts, htq, hts)
        gq, gsc, gtq, gts, _ = B.fp8_swiglu_backward_quantize_dual(dh, gu)
        if ctx.needs_input_grad[0]:
            dx = dgrad(gq, gsc, gqt, gs, out_dtype=torch.bfloat16)
        if ctx.needs_input_grad[1]:
            dw_gu = _weight_grad(w_gu, ctx.workspace, ctx.mfma8, gtq, gts, xtq, xts)
        return dx, dw_gu, dw_down, None, None


class Fp8SwiGLUMLP(torch.nn.Module):
    """The decoder's MLP, y = W_down (silu(W_gate x) * (W_up x)), with its two
    projections on the FP8 block-scaled path and the SwiGLU quantizing its
    output (and, in the backward, its input gradient) on produce.

    ``weight_gate_up`` [2 * ffn, hidden] holds W_gate in its first ``ffn`` rows
    and W_up in the rest; ``weight_down`` is [hidden, ffn].  Both are BF16
    parameters; their gradients follow ``Fp8Linear``'s rules (FP32 returned,
    or added into an FP32 ``main_grad``).  ``workspace`` and ``mfma8`` as for
    ``Fp8Linear``.  The token count, hidden and ffn must be multiples of 128.
    """

    def __init__(self, hidden: int, ffn: int, device=None, std: float = 0.02,
                 workspace: torch.Tensor | None = None, mfma8: bool = False):
        super().__init__()
        _check_dims(128, hidden, ffn)
        self.hidden, self.ffn = hidden, ffn
        self.weight_gate_up = torch.nn.Parameter(
            torch.empty(2 * ffn, hidden, device=device, dtype=torch.bfloat16))
        self.weight_down = torch.nn.Parameter(
            torch.empty(hidden, ffn, device=device, dtype=torch.bfloat16))
        torch.nn.init.normal_(self.weight_gate_up, std=std)
        torch.nn.init.normal_(self.weight_down, std=std)
        self.workspace = workspace
        self.mfma8 = mfma8

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        y = Fp8SwiGLUMLPFunction.apply(x.reshape(math.prod(lead), self.hidden),
                                       self.weight_gate_up, self.weight_down, self.workspace,
                                       self.mfma8)
        return y.reshape(*lead, self.hidden)

    def extra_repr(self) -> str:
        mode = "block-scaled, FP8-MFMA block sums" if self.mfma8 else "block-scaled"
        return f"hidden={self.hidden}, ffn={self.ffn}, fp8={mode}"
