"""ctypes binding of libfp8bs (include/fp8bs.h), same names as the C ABI.

Argument marshalling only: every computation runs in the library's HIP
kernels.  torch provides device memory (outputs are allocated with
``torch.empty`` when not passed in) and the stream (the current torch stream
of the tensors' device unless one is given).  If the library has not been
built, every call raises; there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp8bs.so")

FP8BS_OK = 0
STATUS_NAMES = {0: "FP8BS_OK", 1: "FP8BS_ERR_NULL", 2: "FP8BS_ERR_SHAPE", 3: "FP8BS_ERR_ALIGN",
                4: "FP8BS_ERR_DTYPE", 5: "FP8BS_ERR_WORKSPACE", 6: "FP8BS_ERR_HIP",
                7: "FP8BS_ERR_UNSUPPORTED", 8: "FP8BS_ERR_VALUE"}
FP8BS_OUT_F32 = 0
FP8BS_OUT_BF16 = 1



class BlockJob(ctypes.Structure):
    """fp8bs_block_job of include/fp8bs.h."""
    _fields_ = [("w", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("q_t", ctypes.c_void_p), ("s", ctypes.c_void_p)]


# Every symbol include/fp8bs.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
SIGNATURES = {
    "fp8_quantize_rowtile": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "fp8_quantize_block": (_INT, [_P, _I64, _I64, _P, _P, _P, _P]),
    "fp8_quantize_transposed": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "fp8_quantize_dual": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "fp8_quantize_block_many": (_INT, [_P, _INT, _P]),
    "fp8_swiglu_quantize_dual": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "fp8_rmsnorm_quantize_dual": (_INT, [_P, _P, ctypes.c_float, _I64, _I64, _P, _P, _P, _P, _P,
                                         _P, _P]),
    "fp8_swiglu_backward_quantize_dual": (_INT, [_P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "fp8_gemm_fprop": (_INT, [_P, _P, _P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "fp8_gemm_dgrad": (_INT, [_P, _P, _P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "fp8_gemm_fprop_mfma8": (_INT, [_P, _P, _P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "fp8_gemm_dgrad_mfma8": (_INT, [_P, _P, _P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "fp8_gemm_wgrad_mfma8": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "fp8_gemm_wgrad_mfma8_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "fp8_gemm_dgrad_quantized": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "fp8_gemm_wgrad": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "fp8_gemm_wgrad_noalloc": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "fp8_gemm_wgrad_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "fp8_gemm_wgrad_accumulate": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t,
                                         _P]),
    "fp8_gemm_wgrad_accumulate_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "bf16_gemm_tn": (_INT, [_P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "fp8_encode_e4m3": (_INT, [_P, _I64, _P, _P]),
    "fp8bs_mfma_rate": (_INT, [_P, _I64, _INT, ctypes.c_float, _P]),
    "fp8bs_hbm_rate": (_INT, [_P, _I64, _P, _P, _P]),
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


def _alloc_on(stream, device):
    """Context in which torch allocates on the stream the kernels run on, so
    that a temporary freed when the call returns (an output or an "auto"
    workspace) is not handed to other work before the kernels are done with
    it (the caching allocator reuses a block only on the stream it was
    allocated on)."""
    if stream is None:
        return contextlib.nullcontext()
    if not hasattr(stream, "cuda_stream"):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    return torch.cuda.stream(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, shape, what):
    """t must be a contiguous tensor of `dtype` and `shape` (a None in `shape`
    matches any size).  Checked before any call, so a mis-shaped or strided
    tensor never reaches a kernel."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what}: expected a tensor, got {type(t).__name__}")
    ok_shape = t.dim() == len(shape) and all(e is None or e == d for e, d in zip(shape, t.shape))
    if t.dtype != dtype or not ok_shape or not t.is_contiguous():
        raise ValueError(f"{what}: expected contiguous {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")


def _on_device(**tensors):
    """Every tensor given (None skipped) must live on one GPU; checked after
    the shapes, right before the call."""
    devs = set()
    for what, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{what}: expected a device tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(map(str, devs))}")


def _dims(t: torch.Tensor, what):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{what}: expected a 2-D tensor")
    return t.shape


def _blocks(n: int):
    """Number of 128-wide blocks of a dimension, or None (any size accepted
    here) when it is not a multiple of 128: the C call then rejects the shape
    with FP8BS_ERR_SHAPE."""
    return n // 128 if n % 128 == 0 else None


def _bits16(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


# ------------------------------------------------------------------ quantizers
def _bf16_input(x, what):
    M, C = _dims(x, what)
    _need(x, torch.bfloat16, (M, C), what)
    return M, C


def fp8_quantize_rowtile(x: torch.Tensor, q=None, s=None, stream=None):
    """x bf16 [M,K] -> (q uint8 [M,K], s float32 [M,K/128])."""
    M, K = _bf16_input(x, "x")
    with _alloc_on(stream, x.device):
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if q is None else q
        s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device) if s is None else s
    _need(q, torch.uint8, (M, K), "q")
    _need(s, torch.float32, (M, _blocks(K)), "s")
    _on_device(x=x, q=q, s=s)
    _check("fp8_quantize_rowtile", capi().fp8_quantize_rowtile(
        _ptr(x), M, K, _ptr(q), _ptr(s), _stream(x, stream)))
    return q, s


def fp8_quantize_block(w: torch.Tensor, q=None, q_t=None, s=None, with_transpose=True,
                       stream=None):
    """w bf16 [N,K] -> (q uint8 [N,K], q_t uint8 [K,N] or None, s float32 [N/128,K/128])."""
    N, K = _bf16_input(w, "w")
    dev = w.device
    with _alloc_on(stream, dev):
        q = torch.empty((N, K), dtype=torch.uint8, device=dev) if q is None else q
        if with_transpose and q_t is None:
            q_t = torch.empty((K, N), dtype=torch.uint8, device=dev)
        s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev) if s is None else s
    _need(q, torch.uint8, (N, K), "q")
    if q_t is not None:
        _need(q_t, torch.uint8, (K, N), "q_t")
    _need(s, torch.float32, (_blocks(N), _blocks(K)), "s")
    _on_device(w=w, q=q, q_t=q_t, s=s)
    _check("fp8_quantize_block", capi().fp8_quantize_block(
        _ptr(w), N, K, _ptr(q), _ptr(q_t), _ptr(s), _stream(w, stream)))
    return q, q_t, s


def fp8_quantize_block_many(ws, with_transpose=True, stream=None):
    """Several weights w bf16 [N,K] through the block quantizer in one launch
    (per 16): returns [(q [N,K], q_t [K,N] or None, s [N/128,K/128]), ...].
    with_transpose: one bool for all weights or one per weight."""
    ws = list(ws)
    flags = ([bool(with_transpose)] * len(ws) if isinstance(with_transpose, bool)
             else [bool(f) for f in with_transpose])
    if len(flags) != len(ws):
        raise ValueError("with_transpose: one flag per weight")
    outs = []
    jobs = (BlockJob * max(len(ws), 1))()
    devs = {}
    for i, (w, t) in enumerate(zip(ws, flags)):
        N, K = _bf16_input(w, f"w[{i}]")
        with _alloc_on(stream, w.device):
            q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
            q_t = torch.empty((K, N), dtype=torch.uint8, device=w.device) if t else None
            s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
        devs[f"w{i}"] = w
        outs.append((q, q_t, s))
        jobs[i] = BlockJob(_ptr(w), N, K, _ptr(q), _ptr(q_t), _ptr(s))
    if not ws:
        return outs
    _on_device(**devs)
    _check("fp8_quantize_block_many", capi().fp8_quantize_block_many(
        ctypes.cast(jobs, ctypes.c_void_p), len(ws), _stream(ws[0], stream)))
    return outs


def fp8_quantize_transposed(x: torch.Tensor, qt=None, st=None, stream=None):
    """x bf16 [M,C] -> (qt uint8 [C,M], st float32 [C,M/128])."""
    M, C = _bf16_input(x, "x")
    with _alloc_on(stream, x.device):
        qt = torch.empty((C, M), dtype=torch.uint8, device=x.device) if qt is None else qt
        st = torch.empty((C, M // 128), dtype=torch.float32, device=x.device) if st is None else st
    _need(qt, torch.uint8, (C, M), "qt")
    _need(st, torch.float32, (C, _blocks(M)), "st")
    _on_device(x=x, qt=qt, st=st)
    _check("fp8_quantize_transposed", capi().fp8_quantize_transposed(
        _ptr(x), M, C, _ptr(qt), _ptr(st), _stream(x, stream)))
    return qt, st


def fp8_quantize_dual(x: torch.Tensor, q=None, s=None, qt=None, st=None, stream=None):
    """x bf16 [M,C] -> (q [M,C], s [M,C/128], qt [C,M], st [C,M/128]) in one pass."""
    M, C = _bf16_input(x, "x")
    dev = x.device
    with _alloc_on(stream, dev):
        q = torch.empty((M, C), dtype=torch.uint8, device=dev) if q is None else q
        s = torch.empty((M, C // 128), dtype=torch.float32, device=dev) if s is None else s
        qt = torch.empty((C, M), dtype=torch.uint8, device=dev) if qt is None else qt
        st = torch.empty((C, M // 128), dtype=torch.float32, device=dev) if st is None else st
    _need(q, torch.uint8, (M, C), "q")
    _need(s, torch.float32, (M, _blocks(C)), "s")
    _need(qt, torch.uint8, (C, M), "qt")
    _need(st, torch.float32, (C, _blocks(M)), "st")
    _on_device(x=x, q=q, s=s, qt=qt, st=st)
    _check("fp8_quantize_dual", capi().fp8_quantize_dual(
        _ptr(x), M, C, _ptr(q), _ptr(s), _ptr(qt), _ptr(st), _stream(x, stream)))
    return q, s, qt, st


def fp8_swiglu_quantize_dual(gate_up: torch.Tensor, q=None, s=None, qt=None, st=None, h=None,
                             with_h: bool = False, stream=None):
    """gate_up bf16 [M,2F] (gate | up) -> H = silu(gate) * up quantized on
    produce: (q [M,F], s [M,F/128], qt [F,M], st [F,M/128], h bf16 [M,F] or None).
    H is returned (and written) only with with_h=True or a given h."""
    M, F2 = _dims(gate_up, "gate_up")
    _need(gate_up, torch.bfloat16, (M, F2), "gate_up")
    if F2 % 2:
        raise ValueError(f"gate_up: expected an even number of columns, got {F2}")
    F = F2 // 2
    dev = gate_up.device
    with _alloc_on(stream, dev):
        q = torch.empty((M, F), dtype=torch.uint8, device=dev) if q is None else q
        s = torch.empty((M, F // 128), dtype=torch.float32, device=dev) if s is None else s
        qt = torch.empty((F, M), dtype=torch.uint8, device=dev) if qt is None else qt
        st = torch.empty((F, M // 128), dtype=torch.float32, device=dev) if st is None else st
        if with_h and h is None:
            h = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    _need(q, torch.uint8, (M, F), "q")
    _need(s, torch.float32, (M, _blocks(F)), "s")
    _need(qt, torch.uint8, (F, M), "qt")
    _need(st, torch.float32, (F, _blocks(M)), "st")
    if h is not None:
        _need(h, torch.bfloat16, (M, F), "h")
    _on_device(gate_up=gate_up, q=q, s=s, qt=qt, st=st, h=h)
    _check("fp8_swiglu_quantize_dual", capi().fp8_swiglu_quantize_dual(
        _ptr(gate_up), M, F, _ptr(q), _ptr(s), _ptr(qt), _ptr(st), _ptr(h),
        _stream(gate_up, stream)))
    return q, s, qt, st, h


def fp8_rmsnorm_quantize_dual(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, q=None,
                              s=None, qt=None, st=None, rstd=None, y=None, with_y: bool = False,
                              stream=None):
    """x bf16 [M,C], gamma bf16 [C] -> Y = RMSNorm(x) * gamma quantized on
    produce: (q [M,C], s [M,C/128], qt [C,M], st [C,M/128], rstd f32 [M],
    y bf16 [M,C] or None).  Y in BF16 only with with_y=True or a given y."""
    M, C = _dims(x, "x")
    _need(x, torch.bfloat16, (M, C), "x")
    _need(gamma, torch.bfloat16, (C,), "gamma")
    dev = x.device
    with _alloc_on(stream, dev):
        q = torch.empty((M, C), dtype=torch.uint8, device=dev) if q is None else q
        s = torch.empty((M, C // 128), dtype=torch.float32, device=dev) if s is None else s
        qt = torch.empty((C, M), dtype=torch.uint8, device=dev) if qt is None else qt
        st = torch.empty((C, M // 128), dtype=torch.float32, device=dev) if st is None else st
        rstd = torch.empty((M,), dtype=torch.float32, device=dev) if rstd is None else rstd
        if with_y and y is None:
            y = torch.empty((M, C), dtype=torch.bfloat16, device=dev)
    _need(q, torch.uint8, (M, C), "q")
    _need(s, torch.float32, (M, _blocks(C)), "s")
    _need(qt, torch.uint8, (C, M), "qt")
    _need(st, torch.float32, (C, _blocks(M)), "st")
    _need(rstd, torch.float32, (M,), "rstd")
    if y is not None:
        _need(y, torch.bfloat16, (M, C), "y")
    _on_device(x=x, gamma=gamma, q=q, s=s, qt=qt, st=st, rstd=rstd, y=y)
    _check("fp8_rmsnorm_quantize_dual", capi().fp8_rmsnorm_quantize_dual(
        _ptr(x), _ptr(gamma), float(eps), M, C, _ptr(q), _ptr(s), _ptr(qt), _ptr(st), _ptr(rstd),
        _ptr(y), _stream(x, stream)))
    return q, s, qt, st, rstd, y


def fp8_swiglu_backward_quantize_dual(dh: torch.Tensor, gate_up: torch.Tensor, q=None, s=None,
                                      qt=None, st=None, dgate_up=None, with_bf16: bool = False,
                                      stream=None):
    """dh bf16 [M,F], gate_up bf16 [M,2F] -> the gate/up gradient dGU [M,2F]
    quantized on produce: (q [M,2F], s [M,2F/128], qt [2F,M], st [2F,M/128],
    dgate_up bf16 [M,2F] or None).  dGU in BF16 only with with_bf16=True or a
    given dgate_up."""
    M, F = _dims(dh, "dh")
    _need(dh, torch.bfloat16, (M, F), "dh")
    _dims(gate_up, "gate_up")
    _need(gate_up, torch.bfloat16, (M, 2 * F), "gate_up")
    dev = dh.device
    with _alloc_on(stream, dev):
        q = torch.empty((M, 2 * F), dtype=torch.uint8, device=dev) if q is None else q
        s = torch.empty((M, 2 * F // 128), dtype=torch.float32, device=dev) if s is None else s
        qt = torch.empty((2 * F, M), dtype=torch.uint8, device=dev) if qt is None else qt
        st = torch.empty((2 * F, M // 128), dtype=torch.float32, device=dev) if st is None else st
        if with_bf16 and dgate_up is None:
            dgate_up = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=dev)
    _need(q, torch.uint8, (M, 2 * F), "q")
    _need(s, torch.float32, (M, _blocks(2 * F)), "s")
    _need(qt, torch.uint8, (2 * F, M), "qt")
    _need(st, torch.float32, (2 * F, _blocks(M)), "st")
    if dgate_up is not None:
        _need(dgate_up, torch.bfloat16, (M, 2 * F), "dgate_up")
    _on_device(dh=dh, gate_up=gate_up, q=q, s=s, qt=qt, st=st, dgate_up=dgate_up)
    _check("fp8_swiglu_backward_quantize_dual", capi().fp8_swiglu_backward_quantize_dual(
        _ptr(dh), _ptr(gate_up), M, F, _ptr(q), _ptr(s), _ptr(qt), _ptr(st), _ptr(dgate_up),
        _stream(dh, stream)))
    return q, s, qt, st, dgate_up


# ----------------------------------------------------------------------- GEMMs
def _out(shape, out_dtype, device, out, stream):
    dt = torch.bfloat16 if out_dtype == FP8BS_OUT_BF16 else torch.float32
    if out is None:
        with _alloc_on(stream, device):
            out = torch.empty(shape, dtype=dt, device=device)
    _need(out, dt, shape, "output")
    return out


def _dtype_code(out_dtype):
    if out_dtype in (torch.bfloat16, "bf16", FP8BS_OUT_BF16):
        return FP8BS_OUT_BF16
    if out_dtype in (torch.float32, "f32", FP8BS_OUT_F32):
        return FP8BS_OUT_F32
    raise ValueError(f"unknown output dtype {out_dtype}")


def _row_operand(q, s, what):
    """Codes [R, L] and scales [R, L/128] of 1x128 tiles along L."""
    R, L = _dims(q, what)
    _need(q, torch.uint8, (R, L), what)
    _need(s, torch.float32, (R, _blocks(L)), what + " scales")
    return R, L


def _fprop(name, xq, xs, wq, ws, out_dtype, y, stream):
    M, K = _row_operand(xq, xs, "xq")
    N, _ = _dims(wq, "wq")
    _need(wq, torch.uint8, (N, K), "wq")
    _need(ws, torch.float32, (_blocks(N), _blocks(K)), "ws")
    code = _dtype_code(out_dtype)
    y = _out((M, N), code, xq.device, y, stream)
    _on_device(xq=xq, xs=xs, wq=wq, ws=ws, y=y)
    _check(name, getattr(capi(), name)(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(y), code, M, N, K, _stream(xq, stream)))
    return y


def fp8_gemm_fprop(xq, xs, wq, ws, out_dtype=torch.bfloat16, y=None, stream=None):
    """Y [M,N] = X W^T from (xq [M,K], xs [M,K/128]) and (wq [N,K], ws [N/128,K/128])."""
    return _fprop("fp8_gemm_fprop", xq, xs, wq, ws, out_dtype, y, stream)


def fp8_gemm_fprop_mfma8(xq, xs, wq, ws, out_dtype=torch.bfloat16, y=None, stream=None):
    """fp8_gemm_fprop with each block's sum formed by the FP8 MFMA (limited
    precision inside the block, see include/fp8bs.h)."""
    return _fprop("fp8_gemm_fprop_mfma8", xq, xs, wq, ws, out_dtype, y, stream)


def _dgrad_operands(dyq, dys, wq_t, ws):
    M, N = _row_operand(dyq, dys, "dyq")
    K, _ = _dims(wq_t, "wq_t")
    _need(wq_t, torch.uint8, (K, N), "wq_t")
    _need(ws, torch.float32, (_blocks(N), _blocks(K)), "ws")
    return M, N, K


def _dgrad(name, dyq, dys, wq_t, ws, out_dtype, dx, stream):
    M, N, K = _dgrad_operands(dyq, dys, wq_t, ws)
    code = _dtype_code(out_dtype)
    dx = _out((M, K), code, dyq.device, dx, stream)
    _on_device(dyq=dyq, dys=dys, wq_t=wq_t, ws=ws, dx=dx)
    _check(name, getattr(capi(), name)(
        _ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws), _ptr(dx), code, M, N, K, _stream(dyq, stream)))
    return dx


def fp8_gemm_dgrad(dyq, dys, wq_t, ws, out_dtype=torch.bfloat16, dx=None, stream=None):
    """dX [M,K] = dY W from (dyq [M,N], dys [M,N/128]) and (wq_t [K,N], ws [N/128,K/128])."""
    return _dgrad("fp8_gemm_dgrad", dyq, dys, wq_t, ws, out_dtype, dx, stream)


def fp8_gemm_dgrad_mfma8(dyq, dys, wq_t, ws, out_dtype=torch.bfloat16, dx=None, stream=None):
    """fp8_gemm_dgrad with each block's sum formed by the FP8 MFMA."""
    return _dgrad("fp8_gemm_dgrad_mfma8", dyq, dys, wq_t, ws, out_dtype, dx, stream)


def fp8_gemm_dgrad_quantized(dyq, dys, wq_t, ws, with_bf16=True, dx=None, dxq=None, dxs=None,
                             stream=None):
    """dgrad with its BF16 output quantized in 1x128 row tiles in the epilogue:
    returns (dx bf16 [M,K] or None, dxq uint8 [M,K], dxs float32 [M,K/128])."""
    M, N, K = _dgrad_operands(dyq, dys, wq_t, ws)
    dev = dyq.device
    with _alloc_on(stream, dev):
        if with_bf16 and dx is None:
            dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dxq = torch.empty((M, K), dtype=torch.uint8, device=dev) if dxq is None else dxq
        dxs = torch.empty((M, K // 128), dtype=torch.float32, device=dev) if dxs is None else dxs
    if dx is not None:
        _need(dx, torch.bfloat16, (M, K), "dx")
    _need(dxq, torch.uint8, (M, K), "dxq")
    _need(dxs, torch.float32, (M, _blocks(K)), "dxs")
    _on_device(dyq=dyq, dys=dys, wq_t=wq_t, ws=ws, dx=dx, dxq=dxq, dxs=dxs)
    _check("fp8_gemm_dgrad_quantized", capi().fp8_gemm_dgrad_quantized(
        _ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws), _ptr(dx), _ptr(dxq), _ptr(dxs), M, N, K,
        _stream(dyq, stream)))
    return dx, dxq, dxs


def fp8_gemm_wgrad_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(capi().fp8_gemm_wgrad_workspace_bytes(M, N, K))


def _wgrad_operands(dytq, dyts, xtq, xts):
    N, M = _row_operand(dytq, dyts, "dytq")
    K, _ = _dims(xtq, "xtq")
    _need(xtq, torch.uint8, (K, M), "xtq")
    _need(xts, torch.float32, (K, _blocks(M)), "xts")
    return M, N, K


def _workspace_arg(workspace):
    """True for "auto"; checks a given workspace tensor."""
    auto = isinstance(workspace, str)
    if auto and workspace != "auto":
        raise ValueError(f"workspace: expected None, 'auto' or a tensor, got {workspace!r}")
    if not auto and workspace is not None:
        _need(workspace, torch.uint8, (None,), "workspace")
    return auto


def _auto_workspace(nbytes, device, stream):
    with _alloc_on(stream, device):
        return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def _wgrad(name, dytq, dyts, xtq, xts, dw, workspace, stream):
    M, N, K = _wgrad_operands(dytq, dyts, xtq, xts)
    auto = _workspace_arg(workspace)
    _on_device(dytq=dytq, dyts=dyts, xtq=xtq, xts=xts)
    dw = _out((N, K), FP8BS_OUT_F32, dytq.device, dw, stream)
    if auto:
        nbytes = int(getattr(capi(), name + "_workspace_bytes")(M, N, K))
        workspace = _auto_workspace(nbytes, dytq.device, stream)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _on_device(dytq=dytq, dyts=dyts, xtq=xtq, xts=xts, dw=dw, workspace=workspace)
    _check(name, getattr(capi(), name)(
        _ptr(dytq), _ptr(dyts), _ptr(xtq), _ptr(xts), _ptr(dw), M, N, K, ws_ptr, ws_bytes,
        _stream(dytq, stream)))
    return dw


def fp8_gemm_wgrad(dytq, dyts, xtq, xts, dw=None, workspace=None, stream=None):
    """dW [N,K] (float32) = dY^T X from (dytq [N,M], dyts [N,M/128]) and (xtq [K,M], xts [K,M/128]).
    workspace: None (no split), "auto" (allocate the queried size) or a uint8 device tensor."""
    return _wgrad("fp8_gemm_wgrad", dytq, dyts, xtq, xts, dw, workspace, stream)


def fp8_gemm_wgrad_mfma8_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(capi().fp8_gemm_wgrad_mfma8_workspace_bytes(M, N, K))


def fp8_gemm_wgrad_mfma8(dytq, dyts, xtq, xts, dw=None, workspace=None, stream=None):
    """fp8_gemm_wgrad with each block's sum formed by the FP8 MFMA; workspace
    as fp8_gemm_wgrad (its query is fp8_gemm_wgrad_mfma8_workspace_bytes)."""
    return _wgrad("fp8_gemm_wgrad_mfma8", dytq, dyts, xtq, xts, dw, workspace, stream)


def fp8_gemm_wgrad_accumulate_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(capi().fp8_gemm_wgrad_accumulate_workspace_bytes(M, N, K))


def fp8_gemm_wgrad_accumulate(dytq, dyts, xtq, xts, dw, workspace=None, stream=None):
    """dw (float32 [N,K], updated in place) += dY^T X, operands as fp8_gemm_wgrad;
    the result equals dw + fp8_gemm_wgrad(...) bit for bit.  workspace: None
    (no split), "auto" or a uint8 device tensor, as fp8_gemm_wgrad (its
    query is fp8_gemm_wgrad_accumulate_workspace_bytes)."""
    M, N, K = _wgrad_operands(dytq, dyts, xtq, xts)
    auto = _workspace_arg(workspace)
    _need(dw, torch.float32, (N, K), "dw")
    _on_device(dytq=dytq, dyts=dyts, xtq=xtq, xts=xts, dw=dw)
    if auto:
        workspace = _auto_workspace(fp8_gemm_wgrad_accumulate_workspace_bytes(M, N, K),
                                    dytq.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _on_device(dytq=dytq, dyts=dyts, xtq=xtq, xts=xts, dw=dw, workspace=workspace)
    _check("fp8_gemm_wgrad_accumulate", capi().fp8_gemm_wgrad_accumulate(
        _ptr(dytq), _ptr(dyts), _ptr(xtq), _ptr(xts), _ptr(dw), M, N, K, _ptr(workspace),
        ws_bytes, _stream(dytq, stream)))
    return dw


NOALLOC_SCRATCH_BYTES = 128 << 20     # FP8BS_NOALLOC_SCRATCH_BYTES


def fp8_gemm_wgrad_noalloc(dytq, dyts, xtq, xts, dw, stream=None):
    """fp8_gemm_wgrad with its split-K slices in the library's static device
    scratch: the C call allocates nothing, so dw (float32 [N,K]) must be
    given.  Calls that may overlap on one device race on the scratch."""
    M, N, K = _wgrad_operands(dytq, dyts, xtq, xts)
    _need(dw, torch.float32, (N, K), "dw")
    _on_device(dytq=dytq, dyts=dyts, xtq=xtq, xts=xts, dw=dw)
    _check("fp8_gemm_wgrad_noalloc", capi().fp8_gemm_wgrad_noalloc(
        _ptr(dytq), _ptr(dyts), _ptr(xtq), _ptr(xts), _ptr(dw), M, N, K, _stream(dytq, stream)))
    return dw


def bf16_gemm_tn(a: torch.Tensor, b: torch.Tensor, out_dtype=torch.bfloat16, c=None, stream=None):
    """C [I,J] = A B^T for BF16 A [I,K], B [J,K] (the unquantized comparator)."""
    I, K = _bf16_input(a, "a")
    J, _ = _dims(b, "b")
    _need(b, torch.bfloat16, (J, K), "b")
    code = _dtype_code(out_dtype)
    c = _out((I, J), code, a.device, c, stream)
    _on_device(a=a, b=b, c=c)
    _check("bf16_gemm_tn", capi().bf16_gemm_tn(_bits16(a).data_ptr(), _bits16(b).data_ptr(),
                                               _ptr(c), code, I, J, K, _stream(a, stream)))
    return c


def fp8_encode_e4m3(x: torch.Tensor, q=None, stream=None):
    """Diagnostic: x float32 [n] -> E4M3 codes of clamp(x, -448, 448)."""
    if not isinstance(x, torch.Tensor):
        raise ValueError("x: expected a tensor")
    x = x.reshape(-1)
    _need(x, torch.float32, (x.numel(),), "x")
    with _alloc_on(stream, x.device):
        q = torch.empty(x.numel(), dtype=torch.uint8, device=x.device) if q is None else q
    _need(q, torch.uint8, (x.numel(),), "q")
    _on_device(x=x, q=q)
    _check("fp8_encode_e4m3", capi().fp8_encode_e4m3(_ptr(x), x.numel(), _ptr(q),
                                                     _stream(x, stream)))
    return q


def fp8bs_mfma_rate(blocks: int, iters: int, v: float = 0.125, out=None, device="cuda",
                    stream=None):
    """Diagnostic: MFMA-only work of blocks x 256 threads (blocks * 4 * iters *
    128 * 16384 flop); returns the float32 [blocks * 256] results, each
    16384 * v^2 * iters."""
    if out is None:
        with _alloc_on(stream, device):
            out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    _need(out, torch.float32, (blocks * 256,), "out")
    _on_device(out=out)
    _check("fp8bs_mfma_rate", capi().fp8bs_mfma_rate(_ptr(out), blocks, iters, v,
                                                     _stream(out, stream)))
    return out


def fp8bs_hbm_rate(x: torch.Tensor, y0=None, y1=None, two_outputs=False, stream=None):
    """Diagnostic: the quantizers' streaming traffic (2 bytes read, 1 or 2
    written per element) without their arithmetic.  x is viewed as n BF16
    bit patterns; returns (y0, y1): the high bytes and (two_outputs) the low
    bytes of x, uint8 [n]."""
    if not isinstance(x, torch.Tensor) or x.dtype not in (torch.bfloat16, torch.int16):
        raise ValueError("x: expected a bfloat16 or int16 tensor")
    x = x.reshape(-1)
    _need(x, x.dtype, (x.numel(),), "x")
    n = x.numel()
    with _alloc_on(stream, x.device):
        y0 = torch.empty(n, dtype=torch.uint8, device=x.device) if y0 is None else y0
        if two_outputs and y1 is None:
            y1 = torch.empty(n, dtype=torch.uint8, device=x.device)
    _need(y0, torch.uint8, (n,), "y0")
    if y1 is not None:
        _need(y1, torch.uint8, (n,), "y1")
    _on_device(x=x, y0=y0, y1=y1)
    _check("fp8bs_hbm_rate", capi().fp8bs_hbm_rate(_ptr(x), n, _ptr(y0), _ptr(y1),
                                                   _stream(x, stream)))
    return y0, y1


def fp8bs_status_string(status: int) -> str:
    return capi().fp8bs_status_string(status).decode()


def fp8bs_version() -> int:
    return int(capi().fp8bs_version())
