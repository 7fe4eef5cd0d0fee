"""FP8 block-scaled linear-layer path for AMD Instinct MI355X (gfx950).

Quantizers (BF16 -> E4M3 codes + FP32 scales: 1x128 row tiles, 128x128
weight blocks, token-axis tiles; RMSNorm and SwiGLU quantized on produce) and
block-scaled FP8 GEMMs (fprop, dgrad, wgrad) in hand-written HIP kernels
behind the C ABI of include/fp8bs.h.  The Python functions here carry the C
names and only marshal arguments;
``Fp8Linear`` is a bias-free linear layer built on them and ``Fp8SwiGLUMLP``
the decoder's MLP.
"""
from ._binding import (FP8BS_OUT_BF16, FP8BS_OUT_F32, Fp8bsError, bf16_gemm_tn, capi,  # noqa: F401
                       fp8_encode_e4m3, fp8_gemm_dgrad, fp8_gemm_dgrad_mfma8,
                       fp8_gemm_dgrad_quantized, fp8_gemm_fprop, fp8_gemm_fprop_mfma8,
                       fp8_gemm_wgrad, fp8_gemm_wgrad_accumulate, fp8_gemm_wgrad_mfma8,
                       fp8_gemm_wgrad_mfma8_workspace_bytes,
                       fp8_gemm_wgrad_accumulate_workspace_bytes, fp8_gemm_wgrad_noalloc,
                       fp8_gemm_wgrad_workspace_bytes, fp8_quantize_block, fp8_quantize_block_many,
                       fp8_quantize_dual, fp8_quantize_rowtile, fp8_quantize_transposed,
                       fp8_rmsnorm_quantize_dual, fp8_swiglu_backward_quantize_dual,
                       fp8_swiglu_quantize_dual,
                       fp8bs_hbm_rate, fp8bs_mfma_rate, fp8bs_status_string, fp8bs_version)
from .linear import (Fp8Linear, Fp8LinearFunction, Fp8SwiGLUMLP,  # noqa: F401
                     Fp8SwiGLUMLPFunction)
