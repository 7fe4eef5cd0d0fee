"""Pins for the oracle's SwiGLU (H = silu(gate) * up, one rounding to BF16),
against facts that do not come from the oracle itself: closed forms at the
ends of the exponential, the odd-symmetry identity silu(g) - silu(-g) = g,
exact scaling by powers of two, and scipy's logistic function in float64
rounded to BF16 by torch.  A swapped gate/up half, a sign error in the
exponent or a plain sigmoid in place of silu fails one of them."""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle


def _bits(v):
    """float values -> BF16 bits, rounding once by torch (float64 -> bf16)."""
    t = torch.as_tensor(np.asarray(v, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _gu(g_bits, u_bits):
    g = np.asarray(g_bits, dtype=np.uint16).reshape(1, -1)
    u = np.asarray(u_bits, dtype=np.uint16).reshape(1, -1)
    return np.concatenate([g, u], axis=1)


def _val(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def _ulp(x):
    """Spacing of BF16 values at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def test_zero_gate_or_zero_up_gives_signed_zero():
    g = _bits([0.0, 0.0, 1.5, -1.5, -0.0])
    u = _bits([2.0, -2.0, 0.0, 0.0, 3.0])
    h = oracle.swiglu(_gu(g, u))[0]
    # 0/(1+1)*u keeps the sign of u; silu(g)*0 keeps the sign of silu(g) = sign of g
    assert list(h) == [0x0000, 0x8000, 0x0000, 0x8000, 0x8000]


def test_large_gate_is_the_plain_product():
    """e^-g < 2^-129 for g >= 90, so 1 + e^-g is 1 in double and h = g * u,
    an exact FP32 product of two BF16 values, rounded to BF16 by torch."""
    rng = np.random.default_rng(1)
    g = _bits(rng.uniform(90, 3000, 64))
    u = _bits(rng.normal(0, 4, 64))
    h = oracle.swiglu(_gu(g, u))[0]
    prod = torch.from_numpy((_val(g) * _val(u)).astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(h, prod.view(torch.int16).numpy().view(np.uint16))


def test_very_negative_gate_flushes_to_signed_zero():
    """|g u e^g| < 2^-134 (half the smallest BF16 subnormal) for g <= -150
    and |u| <= 1000, so h is a zero carrying the sign of g * u."""
    rng = np.random.default_rng(2)
    g = _bits(rng.uniform(-3000, -150, 64))
    u = _bits(rng.uniform(-1000, 1000, 64))
    h = oracle.swiglu(_gu(g, u))[0]
    sign = (np.signbit(_val(g) * _val(u))).astype(np.uint16) << 15
    assert np.array_equal(h, sign)


def test_odd_symmetry():
    """silu(g) - silu(-g) = g exactly; each side is rounded once to BF16, so
    with u = 1 the rounded values differ from g by at most half a unit of each."""
    rng = np.random.default_rng(3)
    gv = rng.normal(0, 4, 4096)
    g, gn = _bits(gv), _bits(-_val(_bits(gv)))
    one = _bits(np.ones(gv.size))
    hp = _val(oracle.swiglu(_gu(g, one))[0])
    hn = _val(oracle.swiglu(_gu(gn, one))[0])
    err = np.abs((hp - hn) - _val(g))
    assert np.all(err <= 0.5 * _ulp(hp) + 0.5 * _ulp(hn))


def test_doubling_up_doubles_h_exactly():
    rng = np.random.default_rng(4)
    g = _bits(rng.normal(0, 3, 4096))
    u = _bits(rng.normal(0, 1, 4096))
    u2 = _bits(2.0 * _val(u))
    h = oracle.swiglu(_gu(g, u))[0]
    h2 = oracle.swiglu(_gu(g, u2))[0]
    assert np.array_equal(_val(h2), 2.0 * _val(h))


@pytest.mark.parametrize("sigma", [0.5, 3.0, 12.0])
def test_against_scipy_logistic(sigma):
    """h == BF16(g * expit(g) * u) computed in float64 with scipy.  torch
    rounds float64 -> float32 -> BF16, which differs from one rounding only
    when the value lies within a float32 unit of a BF16 tie; such elements may
    differ by one BF16 unit and nothing else may differ."""
    rng = np.random.default_rng(5)
    M, F = 64, 256
    gu = _bits(np.concatenate([rng.normal(0, sigma, (M, F)), rng.normal(0, 1, (M, F))], axis=1))
    h = oracle.swiglu(gu)
    g, u = _val(gu[:, :F]), _val(gu[:, F:])
    exact = g * expit(g) * u
    ref = _bits(exact)
    diff = h != ref
    if diff.any():
        x = exact[diff]
        units = np.abs(x) / _ulp(x)
        near_tie = np.abs(units - np.floor(units) - 0.5) < 2.0 ** -15
        assert near_tie.all()
        assert np.all(np.abs(_val(h[diff]) - _val(ref[diff])) <= _ulp(x))
    assert diff.mean() < 1e-2      # large gates give exact products g*u, so near ties are common


def test_gate_is_the_first_half():
    """With the up half all ones, h is silu of the first half; with the gate
    half all ones, h is silu(1) times the second half."""
    rng = np.random.default_rng(6)
    v = _bits(rng.normal(0, 2, 256))
    one = _bits(np.ones(256))
    h1 = oracle.swiglu(_gu(v, one))[0]
    h2 = oracle.swiglu(_gu(one, v))[0]
    gv = _val(v)
    assert np.array_equal(h1, _bits(gv * expit(gv)))
    assert np.array_equal(h2, _bits(expit(1.0) * gv))


def test_rejects_non_finite_and_odd_width():
    bad = _gu(_bits([np.inf]), _bits([1.0]))
    with pytest.raises(ValueError):
        oracle.swiglu(bad)
    with pytest.raises(ValueError):
        oracle.swiglu(np.zeros((2, 3), dtype=np.uint16))


# ------------------------------------------------------------------ backward
def _bwd(dh_bits, g_bits, u_bits):
    return oracle.swiglu_backward(np.asarray(dh_bits, dtype=np.uint16).reshape(1, -1),
                                  _gu(g_bits, u_bits))[0]


def _silu64(g):
    return g * expit(g)


def test_backward_at_zero_gate():
    """silu'(0) = 1/2 and silu(0) = 0: d_gate = dh*u/2 (an exact product
    halved, rounded by torch) and d_up is a signed zero."""
    rng = np.random.default_rng(7)
    n = 512
    dh, u = _bits(rng.normal(0, 1, n)), _bits(rng.normal(0, 1, n))
    g = _bits(np.zeros(n))
    out = _bwd(dh, g, u)
    half = torch.from_numpy((_val(dh) * _val(u) / 2).astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(out[:n], half.view(torch.int16).numpy().view(np.uint16))
    assert np.all(_val(out[n:]) == 0.0)


def test_backward_large_and_very_negative_gates():
    rng = np.random.default_rng(8)
    n = 256
    dh, u = _bits(rng.normal(0, 1, n)), _bits(rng.normal(0, 1, n))
    big = _bits(rng.uniform(90, 3000, n))
    out = _bwd(dh, big, u)
    as_bf16 = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out[:n], as_bf16(_val(dh) * _val(u)))      # silu' = 1
    assert np.array_equal(out[n:], as_bf16(_val(dh) * _val(big)))    # silu = g
    neg = _bits(rng.uniform(-3000, -150, n))
    out = _bwd(dh, neg, u)
    assert np.all(_val(out) == 0.0)


def test_backward_up_gradient_is_forward_with_unit_up():
    """d_up = dh * silu(g): with dh = 1 it is the forward H for u = 1."""
    rng = np.random.default_rng(9)
    n = 2048
    g = _bits(rng.normal(0, 3, n))
    one = _bits(np.ones(n))
    out = _bwd(one, g, _bits(rng.normal(0, 1, n)))
    fwd = oracle.swiglu(_gu(g, one))[0]
    assert np.array_equal(out[n:], fwd)


@pytest.mark.parametrize("sigma", [0.5, 2.0, 6.0])
def test_backward_against_central_differences(sigma):
    """d_gate against dh*u*(silu(g+e) - silu(g-e))/(2e) in float64 (scipy's
    logistic, e = 2^-20: truncation error ~1e-13 relative), d_up against
    dh*g*expit(g); both within one BF16 unit, equal away from near ties."""
    rng = np.random.default_rng(10)
    n = 8192
    dh, g, u = (_bits(rng.normal(0, 1, n)), _bits(rng.normal(0, sigma, n)),
                _bits(rng.normal(0, 1, n)))
    out = _bwd(dh, g, u)
    gv, eps = _val(g), 2.0 ** -20
    d_gate = _val(dh) * _val(u) * (_silu64(gv + eps) - _silu64(gv - eps)) / (2 * eps)
    d_up = _val(dh) * _silu64(gv)
    for got, want in ((out[:n], d_gate), (out[n:], d_up)):
        diff = np.abs(_val(got) - want)
        assert np.all(diff <= _ulp(want))
        assert np.mean(got != _bits(want)) < 1e-2


def test_backward_is_linear_in_dh():
    rng = np.random.default_rng(11)
    n = 2048
    dh, g, u = (_bits(rng.normal(0, 1, n)), _bits(rng.normal(0, 2, n)),
                _bits(rng.normal(0, 1, n)))
    a = _bwd(dh, g, u)
    b = _bwd(_bits(-2.0 * _val(dh)), g, u)
    assert np.array_equal(_val(b), -2.0 * _val(a))
