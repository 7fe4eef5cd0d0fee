"""ctypes binding of libfp8bs (include/fp8bs.h), same names as the C ABI.

Argument marshalling only: every computation runs in the library's HIP
kernels.  torch provides device memory (outputs are allocated with
``torch.empty`` when not passed in) and the stream (the current torch stream
of the tensors' device unless one is given).  If the library has not been
built, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp8bs.so")

FP8BS_OK = 0
STATUS_NAMES = {0: "FP8BS_OK", 1: "FP8BS_ERR_NULL", 2: "FP8BS_ERR_SHAPE", 3: "FP8BS_ERR_ALIGN",
                4: "FP8BS_ERR_DTYPE", 5: "FP8BS_ERR_WORKSPACE", 6: "FP8BS_ERR_HIP",
                7: "FP8BS_ERR_UNSUPPORTED"}
FP8BS_OUT_F32 = 0
FP8BS_OUT_BF16 = 1

# Every symbol include/fp8bs.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
SIGNATURES = {
    "fp8_quantize_rowtile": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "fp8_quantize_block": (_INT, [_P, _I64, _I64, _P, _P, _P, _P]),
    "fp8_quantize_transposed": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "fp8_quantize_dual": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "fp8_gemm_fprop": (_INT, [_P, _P, _P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "fp8_gemm_dgrad": (_INT, [_P, _P, _P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "fp8_gemm_dgrad_quantized": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "fp8_gemm_wgrad": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "fp8_gemm_wgrad_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "bf16_gemm_tn": (_INT, [_P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "fp8_encode_e4m3": (_INT, [_P, _I64, _P, _P]),
    "fp8bs_mfma_rate": (_INT, [_P, _I64, _INT, ctypes.c_float, _P]),
    "fp8bs_status_string": (ctypes.c_char_p, [_INT]),
    "fp8bs_version": (_INT, []),
}

_lib = None


class Fp8bsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} "
                         f"({capi().fp8bs_status_string(status).decode()})")


def capi() -> ctypes.CDLL:
    """The loaded library with argument types set.  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m fp8_block_scaled_03_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != FP8BS_OK:
        raise Fp8bsError(fn, status)


def _stream(t: torch.Tensor, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, shape, what):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{what}: expected contiguous {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    if not t.is_cuda:
        raise ValueError(f"{what}: expected a device tensor")


def _bits16(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


# ------------------------------------------------------------------ quantizers
def fp8_quantize_rowtile(x: torch.Tensor, q=None, s=None, stream=None):
    """x bf16 [M,K] -> (q uint8 [M,K], s float32 [M,K/128])."""
    M, K = x.shape
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if q is None else q
    s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device) if s is None else s
    _need(q, torch.uint8, (M, K), "q")
    _need(s, torch.float32, (M, K // 128), "s")
    _check("fp8_quantize_rowtile", capi().fp8_quantize_rowtile(
        _ptr(x), M, K, _ptr(q), _ptr(s), _stream(x, stream)))
    return q, s


def fp8_quantize_block(w: torch.Tensor, q=None, q_t=None, s=None, with_transpose=True,
                       stream=None):
    """w bf16 [N,K] -> (q uint8 [N,K], q_t uint8 [K,N] or None, s float32 [N/128,K/128])."""
    N, K = w.shape
    if w.dtype != torch.bfloat16:
        raise ValueError("w must be bfloat16")
    dev = w.device
    q = torch.empty((N, K), dtype=torch.uint8, device=dev) if q is None else q
    if with_transpose and q_t is None:
        q_t = torch.empty((K, N), dtype=torch.uint8, device=dev)
    s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev) if s is None else s
    _need(q, torch.uint8, (N, K), "q")
    if q_t is not None:
        _need(q_t, torch.uint8, (K, N), "q_t")
    _need(s, torch.float32, (N // 128, K // 128), "s")
    _check("fp8_quantize_block", capi().fp8_quantize_block(
        _ptr(w), N, K, _ptr(q), _ptr(q_t), _ptr(s), _stream(w, stream)))
    return q, q_t, s


def fp8_quantize_transposed(x: torch.Tensor, qt=None, st=None, stream=None):
    """x bf16 [M,C] -> (qt uint8 [C,M], st float32 [C,M/128])."""
    M, C = x.shape
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    qt = torch.empty((C, M), dtype=torch.uint8, device=x.device) if qt is None else qt
    st = torch.empty((C, M // 128), dtype=torch.float32, device=x.device) if st is None else st
    _need(qt, torch.uint8, (C, M), "qt")
    _need(st, torch.float32, (C, M // 128), "st")
    _check("fp8_quantize_transposed", capi().fp8_quantize_transposed(
        _ptr(x), M, C, _ptr(qt), _ptr(st), _stream(x, stream)))
    return qt, st


def fp8_quantize_dual(x: torch.Tensor, q=None, s=None, qt=None, st=None, stream=None):
    """x bf16 [M,C] -> (q [M,C], s [M,C/128], qt [C,M], st [C,M/128]) in one pass."""
    M, C = x.shape
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    dev = x.device
    q = torch.empty((M, C), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((M, C // 128), dtype=torch.float32, device=dev) if s is None else s
    qt = torch.empty((C, M), dtype=torch.uint8, device=dev) if qt is None else qt
    st = torch.empty((C, M // 128), dtype=torch.float32, device=dev) if st is None else st
    _need(q, torch.uint8, (M, C), "q")
    _need(s, torch.float32, (M, C // 128), "s")
    _need(qt, torch.uint8, (C, M), "qt")
    _need(st, torch.float32, (C, M // 128), "st")
    _check("fp8_quantize_dual", capi().fp8_quantize_dual(
        _ptr(x), M, C, _ptr(q), _ptr(s), _ptr(qt), _ptr(st), _stream(x, stream)))
    return q, s, qt, st


# ----------------------------------------------------------------------- GEMMs
def _out(shape, out_dtype, device, out):
    dt = torch.bfloat16 if out_dtype == FP8BS_OUT_BF16 else torch.float32
    if out is None:
        out = torch.empty(shape, dtype=dt, device=device)
    _need(out, dt, shape, "output")
    return out


def _dtype_code(out_dtype):
    if out_dtype in (torch.bfloat16, "bf16", FP8BS_OUT_BF16):
        return FP8BS_OUT_BF16
    if out_dtype in (torch.float32, "f32", FP8BS_OUT_F32):
        return FP8BS_OUT_F32
    raise ValueError(f"unknown output dtype {out_dtype}")


def fp8_gemm_fprop(xq, xs, wq, ws, out_dtype=torch.bfloat16, y=None, stream=None):
    """Y [M,N] = X W^T from (xq [M,K], xs [M,K/128]) and (wq [N,K], ws [N/128,K/128])."""
    M, K = xq.shape
    N = wq.shape[0]
    code = _dtype_code(out_dtype)
    y = _out((M, N), code, xq.device, y)
    _check("fp8_gemm_fprop", capi().fp8_gemm_fprop(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(y), code, M, N, K, _stream(xq, stream)))
    return y


def fp8_gemm_dgrad(dyq, dys, wq_t, ws, out_dtype=torch.bfloat16, dx=None, stream=None):
    """dX [M,K] = dY W from (dyq [M,N], dys [M,N/128]) and (wq_t [K,N], ws [N/128,K/128])."""
    M, N = dyq.shape
    K = wq_t.shape[0]
    code = _dtype_code(out_dtype)
    dx = _out((M, K), code, dyq.device, dx)
    _check("fp8_gemm_dgrad", capi().fp8_gemm_dgrad(
        _ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws), _ptr(dx), code, M, N, K, _stream(dyq, stream)))
    return dx


def fp8_gemm_dgrad_quantized(dyq, dys, wq_t, ws, with_bf16=True, dx=None, dxq=None, dxs=None,
                             stream=None):
    """dgrad with its BF16 output quantized in 1x128 row tiles in the epilogue:
    returns (dx bf16 [M,K] or None, dxq uint8 [M,K], dxs float32 [M,K/128])."""
    M, N = dyq.shape
    K = wq_t.shape[0]
    dev = dyq.device
    if with_bf16 and dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if dx is not None:
        _need(dx, torch.bfloat16, (M, K), "dx")
    dxq = torch.empty((M, K), dtype=torch.uint8, device=dev) if dxq is None else dxq
    dxs = torch.empty((M, K // 128), dtype=torch.float32, device=dev) if dxs is None else dxs
    _need(dxq, torch.uint8, (M, K), "dxq")
    _need(dxs, torch.float32, (M, K // 128), "dxs")
    _check("fp8_gemm_dgrad_quantized", capi().fp8_gemm_dgrad_quantized(
        _ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws), _ptr(dx), _ptr(dxq), _ptr(dxs), M, N, K,
        _stream(dyq, stream)))
    return dx, dxq, dxs


def fp8_gemm_wgrad_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(capi().fp8_gemm_wgrad_workspace_bytes(M, N, K))


def fp8_gemm_wgrad(dytq, dyts, xtq, xts, dw=None, workspace=None, stream=None):
    """dW [N,K] (float32) = dY^T X from (dytq [N,M], dyts [N,M/128]) and (xtq [K,M], xts [K,M/128]).
    workspace: None (no split), "auto" (allocate the queried size) or a uint8 device tensor."""
    N, M = dytq.shape
    K = xtq.shape[0]
    dw = _out((N, K), FP8BS_OUT_F32, dytq.device, dw)
    if isinstance(workspace, str) and workspace == "auto":
        nbytes = fp8_gemm_wgrad_workspace_bytes(M, N, K)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dytq.device) if nbytes else None
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("fp8_gemm_wgrad", capi().fp8_gemm_wgrad(
        _ptr(dytq), _ptr(dyts), _ptr(xtq), _ptr(xts), _ptr(dw), M, N, K, ws_ptr, ws_bytes,
        _stream(dytq, stream)))
    return dw


def bf16_gemm_tn(a: torch.Tensor, b: torch.Tensor, out_dtype=torch.bfloat16, c=None, stream=None):
    """C [I,J] = A B^T for BF16 A [I,K], B [J,K] (the unquantized comparator)."""
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise ValueError("a and b must be bfloat16")
    I, K = a.shape
    J = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("contraction lengths differ")
    code = _dtype_code(out_dtype)
    c = _out((I, J), code, a.device, c)
    _check("bf16_gemm_tn", capi().bf16_gemm_tn(_bits16(a).data_ptr(), _bits16(b).data_ptr(),
                                               _ptr(c), code, I, J, K, _stream(a, stream)))
    return c


def fp8_encode_e4m3(x: torch.Tensor, q=None, stream=None):
    """Diagnostic: x float32 [n] -> E4M3 codes of clamp(x, -448, 448)."""
    x = x.reshape(-1)
    q = torch.empty(x.numel(), dtype=torch.uint8, device=x.device) if q is None else q
    _check("fp8_encode_e4m3", capi().fp8_encode_e4m3(_ptr(x), x.numel(), _ptr(q),
                                                     _stream(x, stream)))
    return q


def fp8bs_mfma_rate(blocks: int, iters: int, v: float = 0.125, out=None, device="cuda",
                    stream=None):
    """Diagnostic: MFMA-only work of blocks x 256 threads (blocks * 4 * iters *
    128 * 16384 flop); returns the float32 [blocks * 256] results, each
    16384 * v^2 * iters."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device=device) if out is None else out
    _check("fp8bs_mfma_rate", capi().fp8bs_mfma_rate(_ptr(out), blocks, iters, v,
                                                     _stream(out, stream)))
    return out


def fp8bs_status_string(status: int) -> str:
    return capi().fp8bs_status_string(status).decode()


def fp8bs_version() -> int:
    return int(capi().fp8bs_version())
