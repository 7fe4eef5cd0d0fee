"""Pins for the oracle's RMSNorm (y = x * r * gamma, r = 1/sqrt(mean(x^2) +
eps), double, one rounding of y to BF16 and of r to FP32): closed forms
(constant rows, zero rows), invariants (exact scale invariance without eps,
linearity in gamma, unit mean square, channel permutation) and torch's own
RMSNorm in float64.  A sum in place of the mean, eps outside the square root,
a dropped or misindexed gamma, or r not inverted fails one of them."""
import numpy as np
import pytest
import torch

import oracle


def _bits(v):
    t = torch.as_tensor(np.asarray(v, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _val(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def _ulp(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _case(M, C, key, xstd=1.0):
    rng = np.random.default_rng(key)
    return _bits(rng.normal(0, xstd, (M, C))), _bits(rng.uniform(0.5, 1.5, C))


def test_constant_rows_give_signed_gamma():
    C = 256
    vals = [3.0, -0.75, 1024.0, -2.0 ** -20]
    x = _bits(np.repeat(np.array(vals)[:, None], C, axis=1))
    gamma = _bits(np.random.default_rng(1).normal(0, 1, C))
    y, r = oracle.rmsnorm(x, gamma, 0.0)
    for i, v in enumerate(vals):
        assert np.array_equal(_val(y[i]), np.sign(v) * _val(gamma))
        assert r[i] == np.float32(1.0 / abs(v))


def test_zero_rows_and_the_role_of_eps():
    """A zero row gives y = 0 and r = 1/sqrt(eps); with eps far above
    mean(x^2), r is within a relative 1e-6 of 1/sqrt(eps) (eps under the root)."""
    C = 128
    gamma = _bits(np.ones(C))
    y, r = oracle.rmsnorm(np.zeros((1, C), dtype=np.uint16), gamma, 0.25)
    assert np.all(_val(y) == 0.0) and r[0] == np.float32(2.0)
    x = _bits(np.random.default_rng(2).normal(0, 1e-3, (4, C)))
    y, r = oracle.rmsnorm(x, gamma, 1e6)
    assert np.allclose(r, 1e-3, rtol=1e-6)
    assert np.all(np.abs(_val(y) - _val(x) * 1e-3) <= _ulp(_val(x) * 1e-3))


def test_scale_invariance_without_eps():
    x, gamma = _case(64, 512, 3)
    y, r = oracle.rmsnorm(x, gamma, 0.0)
    for k in (-7, 1, 9):
        y2, r2 = oracle.rmsnorm(_bits(_val(x) * 2.0 ** k), gamma, 0.0)
        assert np.array_equal(y2, y)
        assert np.array_equal(r2, (r.astype(np.float64) * 2.0 ** -k).astype(np.float32))


def test_linear_in_gamma():
    x, gamma = _case(32, 256, 4)
    y, _ = oracle.rmsnorm(x, gamma, 1e-5)
    y2, _ = oracle.rmsnorm(x, _bits(-4.0 * _val(gamma)), 1e-5)
    assert np.array_equal(_val(y2), -4.0 * _val(y))


def test_unit_mean_square():
    """With gamma = 1 and no eps every row of y has mean square 1, up to the
    BF16 rounding of its elements (each within a relative 2^-9)."""
    x, _ = _case(64, 1024, 5, xstd=7.0)
    y, _ = oracle.rmsnorm(x, _bits(np.ones(1024)), 0.0)
    ms = np.mean(_val(y) ** 2, axis=1)
    assert np.all(np.abs(ms - 1.0) <= 2 * 2.0 ** -9)


def test_channel_permutation():
    x, gamma = _case(16, 384, 6)
    p = np.random.default_rng(7).permutation(384)
    y, r = oracle.rmsnorm(x, gamma, 1e-6)
    yp, rp = oracle.rmsnorm(np.ascontiguousarray(x[:, p]), np.ascontiguousarray(gamma[p]), 1e-6)
    assert np.array_equal(yp, y[:, p])
    assert np.allclose(rp, r, rtol=2 ** -22)       # the sum of squares only changes order


@pytest.mark.parametrize("eps", [1e-6, 1e-5])
def test_against_torch_rms_norm(eps):
    """torch.nn.functional.rms_norm in float64 rounded to BF16 by torch (its
    float64 -> float32 -> BF16 path may differ by one unit at near ties only)."""
    M, C = 128, 2048
    x, gamma = _case(M, C, 8)
    y, r = oracle.rmsnorm(x, gamma, eps)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_val(x)), (C,),
                                       weight=torch.from_numpy(_val(gamma)), eps=eps).numpy()
    want = _bits(ref)
    diff = y != want
    if diff.any():
        u = np.abs(ref[diff]) / _ulp(ref[diff])
        assert np.all(np.abs(u - np.floor(u) - 0.5) < 2.0 ** -15)
        assert np.all(np.abs(_val(y[diff]) - _val(want[diff])) <= _ulp(ref[diff]))
    assert diff.mean() < 1e-3
    rr = 1.0 / np.sqrt(np.mean(_val(x) ** 2, axis=1) + eps)
    assert np.allclose(r, rr, rtol=2 ** -23)


def test_rejects_bad_arguments():
    x, gamma = _case(2, 128, 9)
    with pytest.raises(ValueError):
        oracle.rmsnorm(x, gamma, -1.0)
    with pytest.raises(ValueError):
        oracle.rmsnorm(x, gamma[:64], 1e-6)
    bad = x.copy()
    bad[0, 0] = 0x7F80                                # +inf
    with pytest.raises(ValueError):
        oracle.rmsnorm(bad, gamma, 1e-6)
