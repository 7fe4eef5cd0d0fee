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
    """The library under test: the built libfp8bs.so, or, when FP8BS_CAPI_LIB
    names one, that build of it (the host-sanitizer build)."""
    alt = os.environ.get("FP8BS_CAPI_LIB")
    if alt:
        lib = ctypes.CDLL(alt)
        for name, (res, args) in B.SIGNATURES.items():
            getattr(lib, name).restype = res
            getattr(lib, name).argtypes = args
        return lib
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libfp8bs.so is not built (run __graft_entry__.build())")
    return B.capi()


def test_exports_every_header_symbol(L):
    names = header_functions()
    assert len(names) == 26, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.SIGNATURES)


def test_version_and_status_strings(L):
    assert L.fp8bs_version() == 300
    for st in range(9):
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

    # several weights in one call: every job is checked before anything runs
    J = B.BlockJob
    def many(*jobs):
        arr = (J * max(len(jobs), 1))(*jobs)
        return L.fp8_quantize_block_many(ctypes.cast(arr, ctypes.c_void_p), len(jobs), None)
    good = J(A16, 128, 256, A16, None, A16)
    assert L.fp8_quantize_block_many(None, -1, None) == SHAPE
    assert L.fp8_quantize_block_many(None, 1, None) == NULL
    assert L.fp8_quantize_block_many(None, 0, None) == OK
    assert many(good, J(A16, 100, 128, A16, None, A16)) == SHAPE
    assert many(good, J(A16, 128, 128, None, None, A16)) == NULL
    assert many(J(A16, 128, 128, A16, MIS, A16), good) == ALIGN
    assert many(good, J(A16, 128, 128, A16, None, A16 + 2)) == ALIGN
    assert many(J(None, 0, 128, None, None, None), J(None, 256, 0, None, None, None)) == OK

    assert L.fp8_quantize_transposed(A16, 100, 128, A16, A16, None) == SHAPE
    assert L.fp8_quantize_transposed(A16, 128, 96, A16, A16, None) == SHAPE
    assert L.fp8_quantize_transposed(A16, 128, 128, A16, None, None) == NULL
    assert L.fp8_quantize_transposed(None, 0, 0, None, None, None) == OK

    assert L.fp8_quantize_dual(A16, 100, 128, A16, A16, A16, A16, None) == SHAPE
    assert L.fp8_quantize_dual(A16, 128, 64, A16, A16, A16, A16, None) == SHAPE
    assert L.fp8_quantize_dual(A16, 128, 128, A16, A16, None, A16, None) == NULL
    assert L.fp8_quantize_dual(A16, 128, 128, A16, A16, MIS, A16, None) == ALIGN
    assert L.fp8_quantize_dual(None, 0, 128, None, None, None, None, None) == OK

    # gate/up [M, 2F] -> H's codes; h (BF16 H) is optional
    assert L.fp8_swiglu_quantize_dual(A16, 100, 128, A16, A16, A16, A16, None, None) == SHAPE
    assert L.fp8_swiglu_quantize_dual(A16, 128, 192, A16, A16, A16, A16, None, None) == SHAPE
    assert L.fp8_swiglu_quantize_dual(None, 128, 128, A16, A16, A16, A16, None, None) == NULL
    assert L.fp8_swiglu_quantize_dual(A16, 128, 128, A16, None, A16, A16, None, None) == NULL
    assert L.fp8_swiglu_quantize_dual(A16, 128, 128, A16, A16, A16, None, None, None) == NULL
    assert L.fp8_swiglu_quantize_dual(MIS, 128, 128, A16, A16, A16, A16, None, None) == ALIGN
    assert L.fp8_swiglu_quantize_dual(A16, 128, 128, A16, A16, A16, A16, MIS, None) == ALIGN
    assert L.fp8_swiglu_quantize_dual(A16, 128, 128, A16, A16 + 2, A16, A16, None, None) == ALIGN
    assert L.fp8_swiglu_quantize_dual(None, 0, 128, None, None, None, None, None, None) == OK
    assert L.fp8_swiglu_quantize_dual(None, 128, 0, None, None, None, None, None, None) == OK

    # x [M, C], gamma [C] -> Y's codes and r; Y in BF16 optional; eps a finite value >= 0
    rn = L.fp8_rmsnorm_quantize_dual
    VALUE = 8
    assert rn(A16, A16, 1e-6, 100, 128, A16, A16, A16, A16, A16, None, None) == SHAPE
    assert rn(A16, A16, 1e-6, 128, 64, A16, A16, A16, A16, A16, None, None) == SHAPE
    assert rn(A16, A16, -1.0, 128, 128, A16, A16, A16, A16, A16, None, None) == VALUE
    assert rn(A16, A16, float("nan"), 128, 128, A16, A16, A16, A16, A16, None, None) == VALUE
    assert rn(A16, A16, float("inf"), 128, 128, A16, A16, A16, A16, A16, None, None) == VALUE
    assert rn(A16, None, 1e-6, 128, 128, A16, A16, A16, A16, A16, None, None) == NULL
    assert rn(A16, A16, 1e-6, 128, 128, A16, A16, A16, A16, None, None, None) == NULL
    assert rn(A16, MIS, 1e-6, 128, 128, A16, A16, A16, A16, A16, None, None) == ALIGN
    assert rn(A16, A16, 1e-6, 128, 128, A16, A16, A16, A16, A16 + 2, None, None) == ALIGN
    assert rn(A16, A16, 1e-6, 128, 128, A16, A16, A16, A16, A16, MIS, None) == ALIGN
    assert rn(None, None, 1e-6, 0, 128, None, None, None, None, None, None, None) == OK
    assert L.fp8bs_status_string(VALUE) == b"scalar argument out of range"

    # dH [M, F] and gate/up [M, 2F] -> the gate/up gradient's codes; its BF16 copy optional
    bw = L.fp8_swiglu_backward_quantize_dual
    assert bw(A16, A16, 100, 128, A16, A16, A16, A16, None, None) == SHAPE
    assert bw(A16, A16, 128, 64, A16, A16, A16, A16, None, None) == SHAPE
    assert bw(None, A16, 128, 128, A16, A16, A16, A16, None, None) == NULL
    assert bw(A16, None, 128, 128, A16, A16, A16, A16, None, None) == NULL
    assert bw(A16, A16, 128, 128, A16, A16, None, A16, None, None) == NULL
    assert bw(A16, MIS, 128, 128, A16, A16, A16, A16, None, None) == ALIGN
    assert bw(A16, A16, 128, 128, A16, A16, A16, A16, MIS, None) == ALIGN
    assert bw(A16, A16, 128, 128, A16, A16, A16, A16 + 1, None, None) == ALIGN
    assert bw(None, None, 0, 128, None, None, None, None, None, None) == OK

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
    n = L.fp8_gemm_wgrad_noalloc
    assert n(A16, A16, A16, A16, A16, 100, 128, 128, None) == SHAPE
    assert n(A16, A16, A16, A16, A16, 128, 128, 96, None) == SHAPE
    assert n(A16, A16, None, A16, A16, 128, 128, 128, None) == NULL
    assert n(A16, A16, A16, A16, None, 128, 128, 128, None) == NULL
    assert n(A16, A16 + 2, A16, A16, A16, 128, 128, 128, None) == ALIGN
    assert n(A16, A16, A16, A16, A16 + 8, 128, 128, 128, None) == ALIGN
    assert n(None, None, None, None, None, 128, 0, 128, None) == OK
    assert L.fp8_gemm_wgrad_workspace_bytes(100, 128, 128) == 0
    assert L.fp8_gemm_wgrad_workspace_bytes(-128, 128, 128) == 0

    for f in (L.fp8_gemm_fprop_mfma8, L.fp8_gemm_dgrad_mfma8):
        assert f(A16, A16, A16, A16, A16, 0, 4, 100, 128, None) == SHAPE
        assert f(A16, A16, A16, A16, A16, 0, -4, 128, 128, None) == SHAPE
        assert f(A16, A16, A16, A16, A16, 7, 4, 128, 128, None) == DTYPE
        assert f(None, A16, A16, A16, A16, 0, 4, 128, 128, None) == NULL
        assert f(A16, A16, MIS, A16, A16, 0, 4, 128, 128, None) == ALIGN
        assert f(A16, A16, A16, A16, A16 + 8, 1, 4, 128, 128, None) == ALIGN
        assert f(None, None, None, None, None, 0, 0, 128, 128, None) == OK
    m = L.fp8_gemm_wgrad_mfma8
    assert m(A16, A16, A16, A16, A16, 100, 128, 128, None, 0, None) == SHAPE
    assert m(A16, A16, A16, A16, None, 128, 128, 128, None, 0, None) == NULL
    assert m(A16, A16, A16, A16, A16, 128, 128, 128, MIS, 64, None) == ALIGN
    assert m(None, None, None, None, None, 128, 0, 128, None, 0, None) == OK
    assert L.fp8_gemm_wgrad_mfma8_workspace_bytes(128, 100, 128) == 0

    a = L.fp8_gemm_wgrad_accumulate
    assert a(A16, A16, A16, A16, A16, 100, 128, 128, None, 0, None) == SHAPE
    assert a(A16, A16, A16, A16, A16, 128, 128, 96, None, 0, None) == SHAPE
    assert a(A16, A16, A16, A16, A16, -128, 128, 128, None, 0, None) == SHAPE
    assert a(A16, A16, None, A16, A16, 128, 128, 128, None, 0, None) == NULL
    assert a(A16, A16, A16, A16, None, 128, 128, 128, None, 0, None) == NULL
    assert a(A16, A16 + 2, A16, A16, A16, 128, 128, 128, None, 0, None) == ALIGN
    assert a(A16, A16, A16, A16, A16 + 8, 128, 128, 128, None, 0, None) == ALIGN
    assert a(A16, A16, A16, A16, A16, 128, 128, 128, MIS, 64, None) == ALIGN
    assert a(None, None, None, None, None, 128, 128, 0, None, 0, None) == OK
    assert L.fp8_gemm_wgrad_accumulate_workspace_bytes(128, 100, 128) == 0
    assert L.fp8_gemm_wgrad_accumulate_workspace_bytes(128, 128, -128) == 0


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


def test_hbm_rate_argument_errors(L):
    f = L.fp8bs_hbm_rate
    assert f(A16, -1, A16, None, None) == SHAPE
    assert f(None, 4, A16, None, None) == NULL
    assert f(A16, 4, None, None, None) == NULL
    assert f(MIS, 4, A16, None, None) == ALIGN
    assert f(A16, 4, A16, MIS, None) == ALIGN
    assert f(None, 0, None, None, None) == OK


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


def _no_library(monkeypatch):
    """Make any call into the C library fail the test: the checks below must
    reject their inputs before one is made."""
    def boom():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(B, "capi", boom)


def test_binding_rejects_mismatched_inputs_before_any_call(monkeypatch):
    import torch

    _no_library(monkeypatch)
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    E = lambda shape, dt: torch.zeros(shape, dtype=dt)
    xq, xs = E((256, 256), u8), E((256, 2), f32)
    wq, ws = E((128, 256), u8), E((1, 2), f32)
    cases = [
        ("wq", lambda: B.fp8_gemm_fprop(xq, xs, E((128, 128), u8), ws)),          # K differs
        ("ws", lambda: B.fp8_gemm_fprop(xq, xs, wq, E((2, 2), f32))),
        ("xq scales", lambda: B.fp8_gemm_fprop(xq, E((256, 1), f32), wq, ws)),
        ("xq", lambda: B.fp8_gemm_fprop(E((256, 256), f32), xs, wq, ws)),         # dtype
        ("xq", lambda: B.fp8_gemm_fprop(xq.t(), xs, wq, ws)),                      # strided
        ("wq_t", lambda: B.fp8_gemm_dgrad(xq, xs, E((128, 128), u8), ws)),
        ("ws", lambda: B.fp8_gemm_dgrad(xq, xs, E((128, 256), u8), E((1, 1), f32))),
        ("dyq scales", lambda: B.fp8_gemm_dgrad_quantized(xq, E((255, 2), f32), E((128, 256), u8), ws)),
        ("xtq", lambda: B.fp8_gemm_wgrad(xq, xs, E((128, 128), u8), E((128, 2), f32))),
        ("xts", lambda: B.fp8_gemm_wgrad(xq, xs, E((128, 256), u8), E((128, 1), f32))),
        ("dytq", lambda: B.fp8_gemm_wgrad(E((256,), u8), xs, E((128, 256), u8), E((128, 2), f32))),
        ("b", lambda: B.bf16_gemm_tn(E((128, 256), bf), E((128, 128), bf))),
        ("a", lambda: B.bf16_gemm_tn(E((128, 256), f32), E((128, 256), bf))),
        ("x", lambda: B.fp8_quantize_rowtile(E((128, 256), bf).t())),
        ("x", lambda: B.fp8_quantize_block(E((128, 256), f32))),
        ("x", lambda: B.fp8_quantize_transposed(E((128, 256, 1), bf))),
        ("x", lambda: B.fp8_quantize_dual(E((256, 128), bf)[:, ::2])),
        ("gate_up", lambda: B.fp8_swiglu_quantize_dual(E((256, 256), f32))),
        ("gate_up", lambda: B.fp8_swiglu_quantize_dual(E((256, 255), bf))),
        ("gate_up", lambda: B.fp8_swiglu_quantize_dual(E((256, 512), bf)[:, ::2])),
        ("h", lambda: B.fp8_swiglu_quantize_dual(E((256, 256), bf), h=E((256, 256), bf))),
        ("qt", lambda: B.fp8_swiglu_quantize_dual(E((256, 256), bf), qt=E((256, 128), u8))),
        ("gate_up", lambda: B.fp8_swiglu_backward_quantize_dual(E((256, 128), bf), E((256, 128), bf))),
        ("w\\[1\\]", lambda: B.fp8_quantize_block_many([E((128, 128), bf), E((128, 128), f32)])),
        ("one flag", lambda: B.fp8_quantize_block_many([E((128, 128), bf)], with_transpose=[True, False])),
        ("gamma", lambda: B.fp8_rmsnorm_quantize_dual(E((256, 128), bf), E((256,), bf))),
        ("gamma", lambda: B.fp8_rmsnorm_quantize_dual(E((256, 128), bf), E((128,), f32))),
        ("rstd", lambda: B.fp8_rmsnorm_quantize_dual(E((256, 128), bf), E((128,), bf),
                                                      rstd=E((128,), f32))),
        ("x", lambda: B.fp8_rmsnorm_quantize_dual(E((256, 256), bf)[:, :128], E((128,), bf))),
        ("dh", lambda: B.fp8_swiglu_backward_quantize_dual(E((256, 128), f32), E((256, 256), bf))),
        ("dgate_up", lambda: B.fp8_swiglu_backward_quantize_dual(
            E((256, 128), bf), E((256, 256), bf), dgate_up=E((256, 128), bf))),
        ("s", lambda: B.fp8_swiglu_backward_quantize_dual(
            E((256, 128), bf), E((256, 256), bf), s=E((256, 1), f32))),
        ("output", lambda: B.fp8_gemm_fprop(xq, xs, wq, ws, y=E((256, 64), bf))),
        ("workspace", lambda: B.fp8_gemm_wgrad(xq, xs, E((128, 256), u8), E((128, 2), f32),
                                               workspace=E((64,), f32))),
        ("wq", lambda: B.fp8_gemm_fprop_mfma8(xq, xs, E((128, 128), u8), ws)),
        ("wq_t", lambda: B.fp8_gemm_dgrad_mfma8(xq, xs, E((128, 128), u8), ws)),
        ("xts", lambda: B.fp8_gemm_wgrad_mfma8(xq, xs, E((128, 256), u8), E((128, 1), f32))),
        ("dw", lambda: B.fp8_gemm_wgrad_accumulate(xq, xs, E((128, 256), u8), E((128, 2), f32),
                                                   E((256, 64), f32))),
        ("dw", lambda: B.fp8_gemm_wgrad_accumulate(xq, xs, E((128, 256), u8), E((128, 2), f32),
                                                   E((256, 128), bf))),
        ("xts", lambda: B.fp8_gemm_wgrad_accumulate(xq, xs, E((128, 256), u8), E((128, 1), f32),
                                                    E((256, 128), f32))),
        ("workspace", lambda: B.fp8_gemm_wgrad_accumulate(
            xq, xs, E((128, 256), u8), E((128, 2), f32), E((256, 128), f32), workspace="big")),
    ]
    for what, call in cases:
        with pytest.raises(ValueError, match=what):
            call()


def test_binding_rejects_host_tensors_before_any_call(monkeypatch):
    import torch

    _no_library(monkeypatch)
    with pytest.raises(ValueError, match="device tensor"):
        B.fp8_quantize_rowtile(torch.zeros((128, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="device tensor"):
        B.fp8_gemm_fprop(torch.zeros((128, 256), dtype=torch.uint8),
                         torch.zeros((128, 2), dtype=torch.float32),
                         torch.zeros((128, 256), dtype=torch.uint8),
                         torch.zeros((1, 2), dtype=torch.float32))
