"""Pins of the oracle's unquantized BF16 GEMM (the comparator the FP8 path is
timed against) by routes that do not use it:

* exact rational sums (fractions) on tiny inputs spanning many binades: the
  result is the correctly rounded FP32 value of the exact sum, up to the
  float64 summation error;
* numpy's float64 matmul of the widened operands (library routine);
* one-hot rows (closed form) and the transpose identity;
* row subsets and thread counts give identical bits.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp8_block_scaled_03_amd import inputs


def _spread_bits(key, shape, lo=-20, hi=20):
    rng = np.random.default_rng(key)
    x = rng.standard_normal(shape) * np.exp2(rng.integers(lo, hi + 1, size=shape))
    return inputs.bf16_bits(x.astype(np.float32))


def _f64(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def test_exact_rational_sums_correctly_rounded():
    I, J, K = 3, 5, 40
    a, b = _spread_bits(1, (I, K)), _spread_bits(2, (J, K))
    got = oracle.gemm_bf16(a, b)
    af, bf = _f64(a), _f64(b)
    for i in range(I):
        for j in range(J):
            terms = [Fraction(float(af[i, k])) * Fraction(float(bf[j, k])) for k in range(K)]
            exact = sum(terms, Fraction(0))
            absum = float(sum(abs(t) for t in terms))
            want = np.float32(float(exact))
            ulp = float(np.spacing(np.float32(abs(want)))) if want != 0 else 2.0 ** -149
            err = abs(Fraction(float(got[i, j])) - exact)
            assert float(err) <= 0.5 * ulp + K * 2.0 ** -53 * absum * 1.01, (i, j)


def test_matches_float64_numpy_matmul():
    I, J, K = 64, 48, 384
    a, b = _spread_bits(3, (I, K), -4, 4), _spread_bits(4, (J, K), -4, 4)
    got = oracle.gemm_bf16(a, b).astype(np.float64)
    ref = _f64(a) @ _f64(b).T
    # both sum exact products in float64 (in different orders), then one rounding
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1.01 * ulp + 1e-12 * np.abs(_f64(a)) @ np.abs(_f64(b)).T)
    assert np.mean(got == ref.astype(np.float32)) > 0.99


def test_one_hot_rows_pick_columns_and_transpose_identity():
    J, K = 16, 256
    b = _spread_bits(5, (J, K))
    a = np.zeros((K, K), dtype=np.uint16)
    a[np.arange(K), np.arange(K)] = 0x3F80                     # BF16 1.0
    got = oracle.gemm_bf16(a, b)
    assert np.array_equal(got, oracle.bf16_to_f32(b).T)
    x, y = _spread_bits(6, (40, 128)), _spread_bits(7, (24, 128))
    assert np.array_equal(oracle.gemm_bf16(x, y), oracle.gemm_bf16(y, x).T)


def test_rows_and_threads_bitwise_stable():
    a, b = _spread_bits(8, (50, 256)), _spread_bits(9, (30, 256))
    full = oracle.gemm_bf16(a, b, threads=1)
    assert np.array_equal(full, oracle.gemm_bf16(a, b, threads=4))
    rows = np.array([49, 0, 17, 17])
    assert np.array_equal(oracle.gemm_bf16(a, b, rows=rows), full[rows])


def test_non_finite_rejected():
    a = np.zeros((2, 128), dtype=np.uint16)
    a[1, 5] = 0x7F80                                           # +inf
    b = np.zeros((2, 128), dtype=np.uint16)
    with pytest.raises(Exception):
        oracle.gemm_bf16(a, b)
