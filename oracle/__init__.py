"""CPU oracle for the FP8 block-scaled linear-layer path (test infrastructure).

Only ``tests/``, the package smoke check and the benchmark's CPU-baseline leg
use this module.  The product path never imports it.  The arithmetic lives in
``fp8bs_oracle.c`` (plain C, built with gcc); this file only marshals numpy
arrays into it and computes error metrics in float64.

What the oracle computes follows the Puro-2B technical report (lkr-homepage
blog, section 2 "FP8"): FP8 matmuls for the main linear layers with
DeepSeek-V3-style fine-grained block quantization, sensitive work in BF16/FP32.
The format and tile choices (OCP E4M3FN codes, 1x128 activation/gradient
tiles, 128x128 weight blocks, FP32 scales, scale fold at every 128-wide
contraction step) are this library's reading of that passage.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_fp8bs.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source, for
# a host sanitizer run of the CPU tests (FP8BS_ORACLE_SANITIZE=1, with gcc's
# libasan and libubsan preloaded into the Python process).
ASAN_LIB_PATH = os.path.join(_HERE, "liboracle_fp8bs_asan.so")
SRC_PATH = os.path.join(_HERE, "fp8bs_oracle.c")

MODE_BLOCK = 0     # fprop: weight scales ws[j/128][kb]
MODE_BLOCK_T = 1   # dgrad: weight scales read transposed ws[kb][j/128]
MODE_ROW = 2       # wgrad: per-row token-axis scales s[j][kb]

_ERRORS = {-1: "shape", -2: "non-finite input", -3: "argument", -4: "out of memory"}


def _sanitized() -> bool:
    return os.environ.get("FP8BS_ORACLE_SANITIZE", "") == "1"


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction); with
    sanitize, the ASan/UBSan build (-O1, every UB report fatal)."""
    out = ASAN_LIB_PATH if sanitize else LIB_PATH
    if force or not os.path.exists(out) or (os.path.getmtime(out) < os.path.getmtime(SRC_PATH)):
        opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=all"] if sanitize else ["-O2"])
        cmd = ["gcc", *opt, "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-o", out + ".tmp", SRC_PATH, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return out


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = ASAN_LIB_PATH if _sanitized() else LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC_PATH):
            build(sanitize=_sanitized())
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_units.restype = ctypes.c_int32
        L.oracle_e4m3_units.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_e4m3_encode_array.argtypes = [P, i64, P]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16_array.restype = None
        L.oracle_f32_to_bf16_array.argtypes = [P, i64, P]
        L.oracle_quantize_rowtile.restype = ctypes.c_int
        L.oracle_quantize_rowtile.argtypes = [P, i64, i64, P, P, ctypes.c_int]
        L.oracle_quantize_block.restype = ctypes.c_int
        L.oracle_quantize_block.argtypes = [P, i64, i64, P, P, P, ctypes.c_int]
        L.oracle_quantize_transposed.restype = ctypes.c_int
        L.oracle_quantize_transposed.argtypes = [P, i64, i64, P, P, ctypes.c_int]
        L.oracle_gemm.restype = ctypes.c_int
        L.oracle_gemm.argtypes = [ctypes.c_int, P, P, P, P, i64, i64, i64, P, i64, P, ctypes.c_int]
        L.oracle_swiglu_bf16.restype = ctypes.c_int
        L.oracle_swiglu_bf16.argtypes = [P, i64, i64, P, ctypes.c_int]
        L.oracle_swiglu_backward_bf16.restype = ctypes.c_int
        L.oracle_swiglu_backward_bf16.argtypes = [P, P, i64, i64, P, ctypes.c_int]
        L.oracle_rmsnorm_bf16.restype = ctypes.c_int
        L.oracle_rmsnorm_bf16.argtypes = [P, P, ctypes.c_double, i64, i64, P, P, ctypes.c_int]
        L.oracle_gemm_bf16.restype = ctypes.c_int
        L.oracle_gemm_bf16.argtypes = [P, P, i64, i64, i64, P, i64, P, ctypes.c_int]
        L.oracle_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _u16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("BF16 inputs are passed as uint16 bit patterns")
    return x


# --------------------------------------------------------------------------- codec
def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def e4m3_table() -> np.ndarray:
    """float64 values of all 256 codes (NaN for 0x7F / 0xFF)."""
    return np.array([lib().oracle_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def f32_to_bf16(v) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------- quantizers
def quantize_rowtile(x: np.ndarray, threads: int = 0):
    """x bf16 bits [M,K] -> (q uint8 [M,K], s float32 [M,K/128])."""
    x = _u16(x)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 128), dtype=np.float32)
    _check(lib().oracle_quantize_rowtile(_ptr(x), M, K, _ptr(q), _ptr(s), threads), "rowtile")
    return q, s


def quantize_block(w: np.ndarray, with_transpose: bool = True, threads: int = 0):
    """w bf16 bits [N,K] -> (q [N,K], q_t [K,N] or None, s [N/128,K/128])."""
    w = _u16(w)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    qt = np.empty((K, N), dtype=np.uint8) if with_transpose else None
    s = np.empty((N // 128, K // 128), dtype=np.float32)
    _check(lib().oracle_quantize_block(_ptr(w), N, K, _ptr(q), _ptr(qt), _ptr(s), threads), "block")
    return q, qt, s


def quantize_transposed(x: np.ndarray, threads: int = 0):
    """x bf16 bits [M,C] -> (qt uint8 [C,M], st float32 [C,M/128])."""
    x = _u16(x)
    M, C = x.shape
    qt = np.empty((C, M), dtype=np.uint8)
    st = np.empty((C, M // 128), dtype=np.float32)
    _check(lib().oracle_quantize_transposed(_ptr(x), M, C, _ptr(qt), _ptr(st), threads),
           "transposed")
    return qt, st


# ------------------------------------------------------------------ SwiGLU
def swiglu(gu: np.ndarray, threads: int = 0) -> np.ndarray:
    """gate/up bf16 bits [M, 2F] -> H = silu(gate) * up, bf16 bits [M, F]
    (gate = the first F columns, up = the last F; exact in double, one
    rounding to BF16)."""
    gu = _u16(gu)
    M, F2 = gu.shape
    if F2 % 2:
        raise ValueError("gate/up input needs an even number of columns")
    h = np.empty((M, F2 // 2), dtype=np.uint16)
    _check(lib().oracle_swiglu_bf16(_ptr(gu), M, F2 // 2, _ptr(h), threads), "swiglu")
    return h


def swiglu_backward(dh: np.ndarray, gu: np.ndarray, threads: int = 0) -> np.ndarray:
    """dH bf16 bits [M, F] and gate/up bf16 bits [M, 2F] -> the gate/up
    gradient [M, 2F] as bf16 bits: d_gate = dH * up * silu'(gate) in the first
    F columns, d_up = dH * silu(gate) in the last F (double, one rounding)."""
    dh, gu = _u16(dh), _u16(gu)
    M, F = dh.shape
    if gu.shape != (M, 2 * F):
        raise ValueError("gate/up input must be [M, 2F] for dH [M, F]")
    out = np.empty((M, 2 * F), dtype=np.uint16)
    _check(lib().oracle_swiglu_backward_bf16(_ptr(dh), _ptr(gu), M, F, _ptr(out), threads),
           "swiglu backward")
    return out


# ------------------------------------------------------------------ RMSNorm
def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, threads: int = 0):
    """x bf16 bits [M, C], gamma bf16 bits [C] -> (y bf16 bits [M, C],
    r float32 [M]) with y = x * r * gamma, r = 1/sqrt(mean(x^2) + eps)
    (double, one rounding of each output)."""
    x, gamma = _u16(x), _u16(gamma)
    M, C = x.shape
    if gamma.shape != (C,):
        raise ValueError("gamma must have one entry per channel")
    y = np.empty((M, C), dtype=np.uint16)
    r = np.empty(M, dtype=np.float32)
    _check(lib().oracle_rmsnorm_bf16(_ptr(x), _ptr(gamma), float(eps), M, C, _ptr(y), _ptr(r),
                                     threads), "rmsnorm")
    return y, r


# ------------------------------------------------------------------------- GEMMs
def gemm(mode: int, A: np.ndarray, sA: np.ndarray, B: np.ndarray, sB: np.ndarray,
         rows=None, threads: int = 0) -> np.ndarray:
    """TN block-scaled GEMM; returns float32 [len(rows) or I, J]."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sA = np.ascontiguousarray(sA, dtype=np.float32)
    sB = np.ascontiguousarray(sB, dtype=np.float32)
    I, Kc = A.shape
    J, Kc2 = B.shape
    if Kc2 != Kc:
        raise ValueError("contraction lengths differ")
    r = None
    n = I
    if rows is not None:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = r.size
    out = np.empty((n, J), dtype=np.float32)
    _check(lib().oracle_gemm(mode, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), I, J, Kc, _ptr(r), n,
                             _ptr(out), threads), "gemm")
    return out


def gemm_fprop(xq, xs, wq, ws, rows=None, threads: int = 0):
    """Y[M,N] = X W^T from xq [M,K], xs [M,K/128], wq [N,K], ws [N/128,K/128]."""
    return gemm(MODE_BLOCK, xq, xs, wq, ws, rows, threads)


def gemm_dgrad(dyq, dys, wq_t, ws, rows=None, threads: int = 0):
    """dX[M,K] = dY W from dyq [M,N], dys [M,N/128], wq_t [K,N], ws [N/128,K/128]."""
    return gemm(MODE_BLOCK_T, dyq, dys, wq_t, ws, rows, threads)


def gemm_wgrad(dytq, dyts, xtq, xts, rows=None, threads: int = 0):
    """dW[N,K] = dY^T X from dytq [N,M], dyts [N,M/128], xtq [K,M], xts [K,M/128]."""
    return gemm(MODE_ROW, dytq, dyts, xtq, xts, rows, threads)


def gemm_bf16(a_bits: np.ndarray, b_bits: np.ndarray, rows=None, threads: int = 0) -> np.ndarray:
    """Unquantized comparator: out [I or len(rows), J] float32 = A B^T for BF16
    bit patterns A [I,K], B [J,K]; products exact, sum in float64, one rounding."""
    A = _u16(a_bits)
    B = _u16(b_bits)
    I, K = A.shape
    J, K2 = B.shape
    if K2 != K:
        raise ValueError("contraction lengths differ")
    r = None
    n = I
    if rows is not None:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = r.size
    out = np.empty((n, J), dtype=np.float32)
    _check(lib().oracle_gemm_bf16(_ptr(A), _ptr(B), I, J, K, _ptr(r), n, _ptr(out), threads),
           "gemm_bf16")
    return out


# ----------------------------------------------------------------------- metrics
def dequantize_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 dec(q)*s with one scale per row and 128-wide block (row-tile layout)."""
    t = e4m3_table()
    v = t[q]
    R, K = q.shape
    return (v.reshape(R, K // 128, 128) * s.astype(np.float64)[:, :, None]).reshape(R, K)


def dequantize_block(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    t = e4m3_table()
    v = t[q]
    N, K = q.shape
    return v * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:N, :K]


def rel_frobenius(y: np.ndarray, ref: np.ndarray) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / den) if den > 0 else float(np.linalg.norm(y - ref))


def elementwise_bound_ratio(y, ref, a_rows: np.ndarray, b_rows: np.ndarray,
                            c: float = 1e-4) -> float:
    """max |y-ref| / (c * ||a_i|| * ||b_j||) over elements (<= 1 passes).
    a_rows / b_rows are the dequantized contraction vectors (float64)."""
    na = np.linalg.norm(a_rows, axis=1)
    nb = np.linalg.norm(b_rows, axis=1)
    bound = c * np.outer(na, nb)
    err = np.abs(np.asarray(y, np.float64) - np.asarray(ref, np.float64))
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0
