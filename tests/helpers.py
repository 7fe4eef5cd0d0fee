"""Shared helpers for the tests: device tensors from seeded BF16 bits, the
parity gates, and a check that the HIP library is the code under test."""
from __future__ import annotations

import numpy as np
import torch

import oracle

RELF_GATE = 1e-5          # FP32 output: relative Frobenius error
ELEM_C = 1e-4             # FP32 output: |err| <= 1e-4 * ||a_i|| * ||b_j||


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_to_f32(bits).astype(np.float64)


def dequant_rowtile(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return oracle.dequantize_rows(q, s)


def check_f32(y: np.ndarray, ref: np.ndarray, a_deq: np.ndarray, b_deq: np.ndarray, what=""):
    """FP32 gate: relF <= 1e-5 and the per-element bound.  a_deq / b_deq are
    the dequantized contraction vectors behind the compared rows / columns."""
    rel = oracle.rel_frobenius(y, ref)
    ratio = oracle.elementwise_bound_ratio(y, ref, a_deq, b_deq, ELEM_C)
    assert rel <= RELF_GATE, f"{what}: relF {rel:.3e} > {RELF_GATE}"
    assert ratio <= 1.0, f"{what}: per-element bound exceeded ({ratio:.3e})"
    return rel, ratio


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """One BF16 ulp at the magnitude of each float64 value (the smallest
    normal's ulp below it)."""
    mag = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(mag)) - 7)


def check_bf16(y_bits: np.ndarray, ref_f32: np.ndarray, a_deq, b_deq, what=""):
    """BF16 gate: every element within one BF16 ulp of bf16_RNE(oracle).

    The one exception is an element whose oracle value is itself no larger
    than the FP32 per-element bound (1e-4 ||a_i|| ||b_j||): there an FP32
    difference the FP32 gate allows can span many BF16 ulps of so small a
    value, so it may differ by up to that bound plus one ulp of the larger
    of the two values.  Returns the number of elements that needed it."""
    ref_bits = oracle.f32_to_bf16(ref_f32)
    y = bf16_to_f64(y_bits)
    r = bf16_to_f64(ref_bits)
    ref = np.asarray(ref_f32, dtype=np.float64)
    bound = ELEM_C * np.outer(np.linalg.norm(a_deq, axis=1), np.linalg.norm(b_deq, axis=1))
    err = np.abs(y - r)
    near_zero = np.abs(ref) <= bound
    ok = (err <= bf16_ulp(r)) | (near_zero & (err <= bound + bf16_ulp(np.maximum(np.abs(r), np.abs(y)))))
    assert ok.all(), f"{what}: {int((~ok).sum())} BF16 elements off (max err {err.max():.3e})"
    return int((near_zero & (err > bf16_ulp(r))).sum())


def check_bf16_is_rne_of_f32(y_bits: np.ndarray, y_f32: np.ndarray, what=""):
    """The BF16 output of a kernel equals round-to-nearest-even of the same
    kernel's FP32 output, bit for bit."""
    want = oracle.f32_to_bf16(np.ascontiguousarray(y_f32, dtype=np.float32))
    bad = int((np.asarray(y_bits) != want).sum())
    assert bad == 0, f"{what}: {bad} BF16 outputs differ from RNE of the FP32 output"


def loaded_native_libs():
    """Paths of the libfp8bs copies mapped into this process."""
    libs = []
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libfp8bs" in line:
                    libs.append(line.split()[-1])
    except OSError:
        pass
    return sorted(set(libs))
