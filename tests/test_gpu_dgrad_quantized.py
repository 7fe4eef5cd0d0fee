"""dgrad with the row-tile quantizer fused into its epilogue: the BF16 output
passes the dgrad gate against the oracle, and its codes and scales equal the
oracle's row-tile quantization of that BF16 output bit for bit (the fused
quantizer sees exactly the values a separate quantizer pass would read)."""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8
from fp8_block_scaled_03_amd import inputs
from helpers import check_bf16, to_dev_bf16, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _operands(M, N, K, key, kind="student"):
    if kind == "student":
        dyb = inputs.student_t((key, M, N), (M, N), 3.0, 1e-3)
    else:
        dyb = inputs.random_bits((key, M, N), (M, N), kind)
    wb = inputs.normal((key + 1, N, K), (N, K), 0.02)
    dy, w = to_dev_bf16(dyb), to_dev_bf16(wb)
    dyq, dys = fp8.fp8_quantize_rowtile(dy)
    _, wqt, ws = fp8.fp8_quantize_block(w)
    return dyb, wb, dyq, dys, wqt, ws


@pytest.mark.parametrize("M,N,K,kind", [(256, 256, 512, "student"), (300, 640, 384, "wide"),
                                         (1, 128, 256, "student"), (513, 384, 1024, "special"),
                                         (256, 512, 128, "wide")])
def test_dgrad_quantized_matches_oracle(M, N, K, kind):
    _say(f"dgrad quantized {M}x{N}x{K} {kind}")
    dyb, wb, dyq, dys, wqt, ws = _operands(M, N, K, 50, kind)
    dx, dxq, dxs = fp8.fp8_gemm_dgrad_quantized(dyq, dys, wqt, ws)
    _, dxq2, dxs2 = fp8.fp8_gemm_dgrad_quantized(dyq, dys, wqt, ws, with_bf16=False)
    torch.cuda.synchronize()
    dx_bits = to_np(dx)
    # BF16 output: the dgrad gate against the oracle
    odyq, odys = oracle.quantize_rowtile(dyb)
    owq, owqt, ows = oracle.quantize_block(wb)
    ref = oracle.gemm_dgrad(odyq, odys, owqt, ows)
    check_bf16(dx_bits, ref, oracle.dequantize_rows(odyq, odys),
               oracle.dequantize_block(owq, ows).T, "dgrad quantized (bf16)")
    # codes and scales: the oracle's row-tile quantization of this BF16 output
    wq, ws_ = oracle.quantize_rowtile(dx_bits)
    assert np.array_equal(to_np(dxs).view(np.uint32), ws_.view(np.uint32)), "scales differ"
    assert np.array_equal(to_np(dxq), wq), "codes differ"
    # without the BF16 copy the codes are the same
    assert torch.equal(dxq, dxq2) and torch.equal(dxs, dxs2)


def test_dgrad_quantized_bf16_equals_dgrad(monkeypatch):
    """Same kernel, same accumulation: with the 256x256 kernel forced for
    fp8_gemm_dgrad, the BF16 outputs are identical."""
    monkeypatch.setenv("FP8BS_GEMM_KERNEL", "big")
    dyb, wb, dyq, dys, wqt, ws = _operands(512, 1024, 768, 52)
    dx, _, _ = fp8.fp8_gemm_dgrad_quantized(dyq, dys, wqt, ws)
    ref = fp8.fp8_gemm_dgrad(dyq, dys, wqt, ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dx, ref)


def test_dgrad_quantized_full_size():
    """down-projection backward shape of the linear set (16384 x 2048 from a
    6144-wide gradient): codes equal the row-tile quantizer run on dX."""
    M, N, K = 16384, 6144, 2048
    _say(f"dgrad quantized full size {M}x{N}x{K}")
    dy = (torch.randn(M, N, device="cuda") * 1e-3).bfloat16()
    w = (torch.randn(N, K, device="cuda") * 0.02).bfloat16()
    dyq, dys = fp8.fp8_quantize_rowtile(dy)
    _, wqt, ws = fp8.fp8_quantize_block(w)
    dx, dxq, dxs = fp8.fp8_gemm_dgrad_quantized(dyq, dys, wqt, ws)
    q2, s2 = fp8.fp8_quantize_rowtile(dx)
    torch.cuda.synchronize()
    assert torch.equal(dxq, q2) and torch.equal(dxs, s2)
    rows = np.arange(0, M, 997)
    oq, os_ = oracle.quantize_rowtile(to_np(dx)[rows])
    assert np.array_equal(to_np(dxq)[rows], oq) and np.array_equal(to_np(dxs)[rows], os_)


def test_dgrad_quantized_empty():
    z8 = torch.empty((0, 128), dtype=torch.uint8, device="cuda")
    zs = torch.empty((0, 1), dtype=torch.float32, device="cuda")
    wqt = torch.zeros((256, 128), dtype=torch.uint8, device="cuda")
    ws = torch.ones((1, 2), dtype=torch.float32, device="cuda")
    dx, dxq, dxs = fp8.fp8_gemm_dgrad_quantized(z8, zs, wqt, ws)
    assert dx.shape == (0, 256) and dxq.shape == (0, 256) and dxs.shape == (0, 2)
