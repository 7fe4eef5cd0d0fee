"""Seeded synthetic inputs for the FP8 block-scaled linear-layer path.

This module holds no arithmetic of the method: it only draws random numbers
(numpy PCG64, keyed by ``SeedSequence([config, layer, tensor])``) and rounds
them to BF16 with torch's CPU cast.  Both the HIP path's tests and the CPU
oracle's tests take their inputs from here.

Shapes follow a Qwen3-1.7B-like decoder (hidden 2048, FFN 6144, 16 query and
8 key/value heads of width 128, 28 layers), the model size the Puro-2B
technical report trains in FP8 (lkr-homepage blog, section 2 "FP8": the 1.7B
rung of its scaling ladder).  Every value is synthetic; no dataset or trained
weight is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

HIDDEN = 2048
FFN = 6144
Q_WIDTH = 16 * 128
KV_WIDTH = 8 * 128
QKV_WIDTH = Q_WIDTH + 2 * KV_WIDTH      # 4096
LAYERS = 28
TOKENS_FULL = 4 * 4096                  # micro-batch of 4 sequences of 4096 tokens


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> BF16 bit patterns (uint16), rounded by torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _rng(key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def normal(key, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) drawn in float32, scaled in float32, as BF16 bits."""
    x = _rng(key).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


def student_t(key, shape, nu: float, scale: float) -> np.ndarray:
    """scale * Student-t(nu), drawn in float64, rounded to float32, as BF16 bits."""
    x = _rng(key).standard_t(nu, size=shape) * scale
    return bf16_bits(x.astype(np.float32))


def normal_with_outliers(key, shape, n_outliers: int, factor: float):
    """N(0,1) with ``n_outliers`` channels (columns) multiplied by ``factor``.
    Returns (bits, channel indices); the channels are drawn without
    replacement from the same seed."""
    rng = _rng(key)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    cols = np.sort(rng.choice(shape[1], size=n_outliers, replace=False))
    x[:, cols] *= np.float32(factor)
    return bf16_bits(x), cols


# ------------------------------------------------------------------ configurations
@dataclass(frozen=True)
class Gemm:
    """One GEMM of a configuration.  kind is fprop / dgrad / wgrad; a, b name the
    BF16 tensors it quantizes; out is 'f32' or 'bf16'."""
    name: str
    kind: str
    a: str
    b: str
    M: int
    N: int
    K: int
    out: str

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


@dataclass(frozen=True)
class Config:
    key: int
    name: str
    tensors: dict = field(default_factory=dict)   # name -> (shape, distribution spec)
    gemms: tuple = ()
    layers: int = 1
    per_layer: tuple = ()                          # tensor names drawn per layer


def _c5_gemms(T: int):
    g = []
    lin = (("qkv", QKV_WIDTH, HIDDEN, "X_qkv", "dY_qkv", "W_qkv"),
           ("o", HIDDEN, HIDDEN, "X_o", "dY_o", "W_o"),
           ("gu", 2 * FFN, HIDDEN, "X_mlp", "dY_gu", "W_gu"),
           ("down", HIDDEN, FFN, "H", "dY_d", "W_d"))
    for nm, n_out, k_in, x, dy, w in lin:
        # fprop: Y[T, n_out] = X[T, k_in] W[n_out, k_in]^T
        g.append(Gemm(f"{nm}.fprop", "fprop", x, w, T, n_out, k_in, "bf16"))
        # dgrad: dX[T, k_in] = dY[T, n_out] W[n_out, k_in]
        g.append(Gemm(f"{nm}.dgrad", "dgrad", dy, w, T, n_out, k_in, "bf16"))
        # wgrad: dW[n_out, k_in] = dY^T X, contraction over T tokens
        g.append(Gemm(f"{nm}.wgrad", "wgrad", dy, x, T, n_out, k_in, "f32"))
    return tuple(g)


CONFIGS = {
    "tiny": Config(1, "Tiny fprop", {
        "X": ((256, 512), ("normal", 1.0)),
        "W": ((256, 512), ("normal", 0.02)),
    }, (Gemm("fprop", "fprop", "X", "W", 256, 256, 512, "f32"),)),
    "qkv": Config(2, "QKV projection fprop", {
        "X": ((8192, HIDDEN), ("outliers", 8, 20.0)),
        "W": ((QKV_WIDTH, HIDDEN), ("normal", 0.02)),
    }, (Gemm("fprop", "fprop", "X", "W", 8192, QKV_WIDTH, HIDDEN, "bf16"),)),
    "mlp": Config(3, "MLP fprop pair", {
        "X": ((8192, HIDDEN), ("normal", 1.0)),
        "W_gu": ((2 * FFN, HIDDEN), ("normal", 0.02)),
        "H": ((8192, FFN), ("t", 4.0, 0.5 / np.sqrt(2.0))),
        "W_d": ((HIDDEN, FFN), ("normal", 0.02)),
    }, (Gemm("gu.fprop", "fprop", "X", "W_gu", 8192, 2 * FFN, HIDDEN, "bf16"),
        Gemm("down.fprop", "fprop", "H", "W_d", 8192, HIDDEN, FFN, "bf16"))),
    "down_bwd": Config(4, "MLP down-projection backward", {
        "dY": ((8192, HIDDEN), ("t", 3.0, 1e-3)),
        "W_d": ((HIDDEN, FFN), ("normal", 0.02)),
        "H": ((8192, FFN), ("t", 4.0, 0.5 / np.sqrt(2.0))),
    }, (Gemm("down.dgrad", "dgrad", "dY", "W_d", 8192, HIDDEN, FFN, "bf16"),
        Gemm("down.wgrad", "wgrad", "dY", "H", 8192, HIDDEN, FFN, "f32"))),
    "linear_set": Config(5, "Full linear set, 28 layers", {
        "X_qkv": ((TOKENS_FULL, HIDDEN), ("normal", 1.0)),
        "X_o": ((TOKENS_FULL, HIDDEN), ("normal", 1.0)),
        "X_mlp": ((TOKENS_FULL, HIDDEN), ("normal", 1.0)),
        "H": ((TOKENS_FULL, FFN), ("normal", 1.0)),
        "dY_qkv": ((TOKENS_FULL, QKV_WIDTH), ("normal", 1.0)),
        "dY_o": ((TOKENS_FULL, HIDDEN), ("normal", 1.0)),
        "dY_gu": ((TOKENS_FULL, 2 * FFN), ("normal", 1.0)),
        "dY_d": ((TOKENS_FULL, HIDDEN), ("normal", 1.0)),
        "W_qkv": ((QKV_WIDTH, HIDDEN), ("normal", 0.02)),
        "W_o": ((HIDDEN, HIDDEN), ("normal", 0.02)),
        "W_gu": ((2 * FFN, HIDDEN), ("normal", 0.02)),
        "W_d": ((HIDDEN, FFN), ("normal", 0.02)),
    }, _c5_gemms(TOKENS_FULL), LAYERS, ("W_qkv", "W_o", "W_gu", "W_d")),
}

_TENSOR_IDS = {}


def _tensor_id(name: str) -> int:
    # stable small integer per tensor name (sorted order of every name used)
    if not _TENSOR_IDS:
        names = sorted({n for c in CONFIGS.values() for n in c.tensors})
        _TENSOR_IDS.update({n: i for i, n in enumerate(names)})
    return _TENSOR_IDS[name]


def tensor(config: str, name: str, layer: int = 0, rows: int | None = None) -> np.ndarray:
    """BF16 bits of tensor ``name`` of ``config`` (for per-layer tensors, of
    ``layer``; shared tensors ignore ``layer``).  ``rows`` draws a shorter
    tensor with the same distribution (used for reduced-size cases)."""
    cfg = CONFIGS[config]
    shape, dist = cfg.tensors[name]
    if rows is not None:
        shape = (rows, shape[1])
    lay = layer if name in cfg.per_layer else 0
    key = (cfg.key, lay, _tensor_id(name), 0 if rows is None else rows)
    if dist[0] == "normal":
        return normal(key, shape, dist[1])
    if dist[0] == "t":
        return student_t(key, shape, dist[1], dist[2])
    if dist[0] == "outliers":
        return normal_with_outliers(key, shape, dist[1], dist[2])[0]
    raise KeyError(dist[0])


def outlier_channels(config: str = "qkv", name: str = "X") -> np.ndarray:
    cfg = CONFIGS[config]
    shape, dist = cfg.tensors[name]
    return normal_with_outliers((cfg.key, 0, _tensor_id(name), 0), shape, dist[1], dist[2])[1]


def random_bits(key, shape, kind: str = "normal") -> np.ndarray:
    """Edge-case generators for parity tests (all seeded, BF16 bits).

    normal      N(0,1)
    wide        N(0,1) times 2^u with u uniform in [-30, 30] per 128-element tile
    special     a mix of zeros, signed zeros, BF16 subnormals, exact E4M3 grid
                values times powers of two, and values at E4M3 rounding ties
    """
    rng = _rng(key)
    if kind == "normal":
        return bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))
    if kind == "wide":
        x = rng.standard_normal(size=shape).astype(np.float64)
        flat = x.reshape(-1)
        n_t = (flat.size + 127) // 128
        e = rng.integers(-30, 31, size=n_t)
        flat *= np.repeat(np.exp2(e.astype(np.float64)), 128)[: flat.size]
        return bf16_bits(flat.reshape(shape).astype(np.float32))
    if kind == "special":
        n = int(np.prod(shape))
        choice = rng.integers(0, 6, size=n)
        mant = rng.integers(0, 16, size=n)            # 4-bit significands hit E4M3 ties
        expo = rng.integers(-12, 9, size=n)
        sign = np.where(rng.integers(0, 2, size=n) == 1, -1.0, 1.0)
        grid = sign * (8 + mant) / 8.0 * np.exp2(expo)
        sub = sign * rng.integers(1, 128, size=n) * 2.0 ** -133   # BF16 subnormals
        vals = np.select(
            [choice == 0, choice == 1, choice == 2, choice == 3],
            [np.zeros(n), np.full(n, -0.0), sub, grid],
            rng.standard_normal(n))
        return bf16_bits(vals.reshape(shape).astype(np.float32))
    raise KeyError(kind)
