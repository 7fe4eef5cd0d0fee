"""GPU parity of the unquantized BF16 GEMM (the FP8 path's comparator)
against the oracle's float64-accumulated BF16 GEMM: FP32 output within relF
1e-5 and |err| <= 1e-4 ||a_i|| ||b_j||; BF16 output within one BF16 ulp of
bf16_RNE(oracle), the FP32 bound plus an ulp only where the oracle value is
itself within that bound of zero."""
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


def _run(ab, bb, out):
    c = fp8.bf16_gemm_tn(to_dev_bf16(ab), to_dev_bf16(bb), out_dtype=out)
    torch.cuda.synchronize()
    return to_np(c)


CASES = [(256, 256, 512), (300, 384, 256), (1, 128, 128), (513, 640, 1024), (512, 256, 2048)]


@pytest.mark.parametrize("I,J,K", CASES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_bf16_gemm_parity(I, J, K, out):
    _say(f"bf16 gemm {I}x{J}x{K} {out}")
    ab = inputs.random_bits((30, I, K), (I, K), "wide")
    bb = inputs.normal((31, J, K), (J, K), 0.02)
    c = _run(ab, bb, out)
    ref = oracle.gemm_bf16(ab, bb)
    a64, b64 = oracle.bf16_to_f32(ab).astype(np.float64), oracle.bf16_to_f32(bb).astype(np.float64)
    if out == "f32":
        check_f32(c, ref, a64, b64, "bf16 gemm")
    else:
        check_bf16(c, ref, a64, b64, "bf16 gemm (bf16 out)")


def test_bf16_gemm_exact_small_integers():
    """Small-integer operands give exact FP32 sums: the output must be bit-exact."""
    rng = np.random.default_rng(32)
    I, J, K = 256, 384, 512
    a = rng.integers(-8, 9, size=(I, K)).astype(np.float32)
    b = rng.integers(-8, 9, size=(J, K)).astype(np.float32)
    c = _run(inputs.bf16_bits(a), inputs.bf16_bits(b), "f32")
    assert np.array_equal(c, (a.astype(np.float64) @ b.T.astype(np.float64)).astype(np.float32))


def test_bf16_gemm_empty_and_zero_k():
    a = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    assert fp8.bf16_gemm_tn(a, b).shape == (0, 128)
    a = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((128, 0), dtype=torch.bfloat16, device="cuda")
    c = fp8.bf16_gemm_tn(a, b, out_dtype="f32")
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0


@pytest.mark.parametrize("I,J,K", [(16384, 4096, 2048), (16384, 2048, 6144), (2048, 2048, 16384)])
def test_bf16_gemm_full_size_sampled_rows(I, J, K):
    _say(f"bf16 gemm full size {I}x{J}x{K}")
    ab = inputs.random_bits((33, I, K), (I, K), "normal")
    bb = inputs.normal((34, J, K), (J, K), 0.02)
    c = _run(ab, bb, "f32")
    rows = np.concatenate([np.arange(0, I, I // 61), [I - 1]])
    ref = oracle.gemm_bf16(ab, bb, rows=rows)
    a64 = oracle.bf16_to_f32(ab[rows]).astype(np.float64)
    b64 = oracle.bf16_to_f32(bb).astype(np.float64)
    check_f32(c[rows], ref, a64, b64, "bf16 gemm full size")
