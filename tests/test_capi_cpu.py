"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status before
anything reaches the device (fake pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

from fp8_block_scaled_03_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

OK, NULL, SHAPE, ALIGN, DTYPE = 0, 1, 2, 3, 4


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:fp8|bf16)\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libfp8bs.so is not built (run __graft_entry__.build())")
    return B.capi()


def test_exports_every_header_symbol(L):
    names = header_functions()
    assert len(names) == 14, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.SIGNATURES)


def test_version_and_status_strings(L):
    assert L.fp8bs_version() == 200
    for st in range(8):
        s = L.fp8bs_status_string(st)
        assert s and isinstance(s, bytes)
    assert L.fp8bs_status_string(99) == b"unknown status"


A16 = 0x10000          # a fake, 16-byte aligned address (never dereferenced)
MIS = 0x10001          # a fake misaligned address


def test_quantizer_argument_errors(L):
    assert L.fp8_quantize_rowtile(A16, 4, 100, A16, A16, None) == SHAPE
    assert L.fp8_quantize_rowtile(A16, -1, 128, A16, A16, None) == SHAPE
    assert L.fp8_quantize_rowtile(None, 4, 128, A16, A16, None) == NULL
    assert L.fp8_quantize_rowtile(A16, 4, 128, None, A16, None) == NULL
    assert L.fp8_quantize_rowtile(A16, 4, 128, A16, None, None) == NULL
    assert L.fp8_quantize_rowtile(MIS, 4, 128, A16, A16, None) == ALIGN
    assert L.fp8_quantize_rowtile(A16, 4, 128, MIS, A16, None) == ALIGN
    assert L.fp8_quantize_rowtile(A16, 4, 128, A16, A16 + 2, None) == ALIGN
    # empty tensors are valid and touch nothing
    assert L.fp8_quantize_rowtile(None, 0, 128, None, None, None) == OK
    assert L.fp8_quantize_rowtile(None, 5, 0, None, None, None) == OK

    assert L.fp8_quantize_block(A16, 100, 128, A16, None, A16, None) == SHAPE
    assert L.fp8_quantize_block(A16, 128, 64, A16, None, A16, None) == SHAPE
    assert L.fp8_quantize_block(A16, 128, 128, None, None, A16, None) == NULL
    assert L.fp8_quantize_block(A16, 128, 128, A16, MIS, A16, None) == ALIGN
    assert L.fp8_quantize_block(None, 0, 128, None, None, None, None) == OK

    assert L.fp8_quantize_transposed(A16, 100, 128, A16, A16, None) == SHAPE
    assert L.fp8_quantize_transposed(A16, 128, 96, A16, A16, None) == SHAPE
    assert L.fp8_quantize_transposed(A16, 128, 128, A16, None, None) == NULL
    assert L.fp8_quantize_transposed(None, 0, 0, None, None, None) == OK

    assert L.fp8_quantize_dual(A16, 100, 128, A16, A16, A16, A16, None) == SHAPE
    assert L.fp8_quantize_dual(A16, 128, 64, A16, A16, A16, A16, None) == SHAPE
    assert L.fp8_quantize_dual(A16, 128, 128, A16, A16, None, A16, None) == NULL
    assert L.fp8_quantize_dual(A16, 128, 128, A16, A16, MIS, A16, None) == ALIGN
    assert L.fp8_quantize_dual(None, 0, 128, None, None, None, None, None) == OK

    assert L.fp8_encode_e4m3(A16, -1, A16, None) == SHAPE
    assert L.fp8_encode_e4m3(None, 4, A16, None) == NULL
    assert L.fp8_encode_e4m3(A16, 4, MIS, None) == ALIGN
    assert L.fp8_encode_e4m3(None, 0, None, None) == OK


def test_gemm_argument_errors(L):
    f = L.fp8_gemm_fprop
    assert f(A16, A16, A16, A16, A16, 0, 4, 100, 128, None) == SHAPE
    assert f(A16, A16, A16, A16, A16, 0, 4, 128, 96, None) == SHAPE
    assert f(A16, A16, A16, A16, A16, 0, -4, 128, 128, None) == SHAPE
    assert f(A16, A16, A16, A16, A16, 7, 4, 128, 128, None) == DTYPE
    assert f(None, A16, A16, A16, A16, 0, 4, 128, 128, None) == NULL
    assert f(A16, A16, A16, A16, None, 1, 4, 128, 128, None) == NULL
    assert f(A16, A16, MIS, A16, A16, 0, 4, 128, 128, None) == ALIGN
    assert f(A16, A16 + 1, A16, A16, A16, 0, 4, 128, 128, None) == ALIGN
    assert f(A16, A16, A16, A16, A16 + 8, 0, 4, 128, 128, None) == ALIGN
    assert f(None, None, None, None, None, 0, 0, 128, 128, None) == OK

    d = L.fp8_gemm_dgrad
    assert d(A16, A16, A16, A16, A16, 1, 4, 100, 128, None) == SHAPE
    assert d(A16, A16, A16, A16, A16, 3, 4, 128, 128, None) == DTYPE
    assert d(A16, A16, None, A16, A16, 1, 4, 128, 128, None) == NULL

    w = L.fp8_gemm_wgrad
    assert w(A16, A16, A16, A16, A16, 100, 128, 128, None, 0, None) == SHAPE
    assert w(A16, A16, A16, A16, A16, 128, 100, 128, None, 0, None) == SHAPE
    assert w(A16, A16, A16, A16, None, 128, 128, 128, None, 0, None) == NULL
    assert w(A16, A16, A16, A16, A16, 128, 128, 128, MIS, 64, None) == ALIGN
    assert w(None, None, None, None, None, 128, 0, 128, None, 0, None) == OK
    assert L.fp8_gemm_wgrad_workspace_bytes(100, 128, 128) == 0
    assert L.fp8_gemm_wgrad_workspace_bytes(-128, 128, 128) == 0


def test_dgrad_quantized_argument_errors(L):
    f = L.fp8_gemm_dgrad_quantized
    assert f(A16, A16, A16, A16, A16, A16, A16, 4, 100, 128, None) == SHAPE
    assert f(A16, A16, A16, A16, A16, A16, A16, 4, 128, 96, None) == SHAPE
    assert f(A16, A16, A16, A16, None, None, A16, 4, 128, 128, None) == NULL
    assert f(A16, A16, A16, A16, None, A16, None, 4, 128, 128, None) == NULL
    assert f(A16, A16, A16, A16, A16 + 2, A16, A16, 4, 128, 128, None) == ALIGN
    assert f(A16, A16, A16, A16, None, MIS, A16, 4, 128, 128, None) == ALIGN
    assert f(None, None, None, None, None, None, None, 0, 128, 128, None) == OK


def test_bf16_gemm_argument_errors(L):
    f = L.bf16_gemm_tn
    assert f(A16, A16, A16, 1, 4, 100, 128, None) == SHAPE
    assert f(A16, A16, A16, 1, 4, 128, 96, None) == SHAPE
    assert f(A16, A16, A16, 1, -1, 128, 128, None) == SHAPE
    assert f(A16, A16, A16, 5, 4, 128, 128, None) == DTYPE
    assert f(None, A16, A16, 1, 4, 128, 128, None) == NULL
    assert f(A16, MIS, A16, 1, 4, 128, 128, None) == ALIGN
    assert f(A16, A16, A16 + 8, 0, 4, 128, 128, None) == ALIGN
    assert f(None, None, None, 1, 0, 128, 128, None) == OK


def test_mfma_rate_argument_errors(L):
    f = L.fp8bs_mfma_rate
    assert f(A16, -1, 10, 0.125, None) == SHAPE
    assert f(A16, 4, -1, 0.125, None) == SHAPE
    assert f(A16, 1 << 31, 10, 0.125, None) == SHAPE
    assert f(None, 4, 10, 0.125, None) == NULL
    assert f(MIS, 4, 10, 0.125, None) == ALIGN
    assert f(None, 0, 10, 0.125, None) == OK


def test_binding_names_match_c_names():
    import fp8_block_scaled_03_amd as pkg
    for n in header_functions():
        assert callable(getattr(pkg, n)), n


def test_product_path_never_imports_the_oracle():
    pkg_dir = os.path.join(ROOT, "fp8_block_scaled_03_amd")
    for dirpath, _, files in os.walk(pkg_dir):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src, fn
                assert "fp8bs_oracle" not in src, fn


def test_fp8_linear_has_no_cpu_path():
    """The layer runs only through the device library: CPU tensors are refused
    before any call, there is no host fallback."""
    import torch

    import fp8_block_scaled_03_amd as pkg
    lin = pkg.Fp8Linear(256, 128)
    with pytest.raises(ValueError):
        lin(torch.randn(128, 256).bfloat16())
    with pytest.raises(ValueError):
        pkg.Fp8Linear(200, 128)
