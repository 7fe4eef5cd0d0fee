"""fp8_swiglu_quantize_dual and fp8_swiglu_backward_quantize_dual through the
C ABI, against the oracle.

The kernel forms H = silu(gate) * up in FP32 with the hardware exponential and
reciprocal and rounds it to BF16; the oracle forms it in double and rounds
once.  The gate on H: every element within one BF16 unit of the oracle's
(nearly all equal).  The codes and scales are a decision taken from H, so they
are compared bit for bit with the oracle's quantization of the H the kernel
formed (returned through the optional h output): row tiles as
oracle.quantize_rowtile(H), token-axis tiles as oracle.quantize_transposed(H).
Without h the codes are the same bytes, and they equal fp8_quantize_dual of
that H on the GPU.  The backward (the gate/up gradient from dH) is checked the
same way, against the oracle's double-precision backward."""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8
from fp8_block_scaled_03_amd import inputs
from helpers import bf16_to_f64, bf16_ulp, to_dev_bf16, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _gate_up(M, F, key, gate_std=1.0):
    g = inputs.normal((key, M, F), (M, F), gate_std)
    u = inputs.normal((key + 1, M, F), (M, F), 1.0)
    return np.ascontiguousarray(np.concatenate([g, u], axis=1))


def _check(gu_bits, what, full_h_equal_frac=0.99):
    M, F = gu_bits.shape[0], gu_bits.shape[1] // 2
    gu = to_dev_bf16(gu_bits)
    q, s, qt, st, h = fp8.fp8_swiglu_quantize_dual(gu, with_h=True)
    q2, s2, qt2, st2, none = fp8.fp8_swiglu_quantize_dual(gu)
    dq, ds, dqt, dst = fp8.fp8_quantize_dual(h)
    torch.cuda.synchronize()
    assert none is None
    hk = to_np(h)
    ho = oracle.swiglu(gu_bits)
    diff = np.abs(bf16_to_f64(hk) - bf16_to_f64(ho))
    ok = diff <= bf16_ulp(bf16_to_f64(ho))
    eq = float((hk == ho).mean())
    _say(f"{what} {M}x{F}: H equal {eq:.6f}, max diff/ulp "
         f"{float((diff / bf16_ulp(bf16_to_f64(ho))).max()):.2f}")
    assert ok.all(), f"{what}: {int((~ok).sum())} H elements more than one BF16 unit off"
    assert eq >= full_h_equal_frac
    oq, os_ = oracle.quantize_rowtile(hk)
    oqt, ost = oracle.quantize_transposed(hk)
    for name, got, want in (("q", q, oq), ("s", s, os_), ("qt", qt, oqt), ("st", st, ost)):
        g = to_np(got)
        if g.dtype == np.float32:
            g, want = g.view(np.uint32), want.view(np.uint32)
        assert np.array_equal(g, want), f"{what}: {name} differs from the oracle's quantization of H"
    for a, b, name in ((q, q2, "q"), (s, s2, "s"), (qt, qt2, "qt"), (st, st2, "st"),
                       (q, dq, "q vs dual"), (s, ds, "s vs dual"), (qt, dqt, "qt vs dual"),
                       (st, dst, "st vs dual")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: {name}"


@pytest.mark.parametrize("M,F,std", [(256, 384, 1.0), (1024, 768, 3.0), (128, 128, 0.25)])
def test_swiglu_dual_parity(M, F, std):
    _check(_gate_up(M, F, 110, std), "swiglu")


def test_swiglu_dual_special_values():
    """Zero gates and ups (signed zeros), gates large enough that H is the
    plain product, gates negative enough that H is a signed zero, and a
    tile of all zeros (the amax floor)."""
    M, F = 256, 256
    gu = _gate_up(M, F, 112).copy()
    gate, up = gu[:, :F], gu[:, F:]
    bits = lambda v: inputs.bf16_bits(np.full(1, v, dtype=np.float32))[0]
    gate[0, :64] = bits(0.0)
    gate[0, 64:128] = bits(-0.0)
    up[1, :128] = bits(0.0)
    gate[2, :128] = bits(100.0)
    gate[3, :128] = bits(-100.0)
    gate[128:, 128:] = bits(0.0)                  # token-axis and row tiles that are all zero
    _check(gu, "swiglu special", full_h_equal_frac=0.99)


def test_swiglu_dual_empty():
    for M, F in ((0, 256), (256, 0)):
        gu = torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda")
        q, s, qt, st, h = fp8.fp8_swiglu_quantize_dual(gu, with_h=True)
        torch.cuda.synchronize()
        assert q.numel() == 0 and qt.numel() == 0 and h.numel() == 0


def test_swiglu_dual_mlp_size():
    """The down projection's input at the 8192-token MLP shape: gate/up
    [8192, 12288] from N(0,1) activations, every element compared."""
    _check(_gate_up(8192, inputs.FFN, 114), "swiglu mlp")


# ------------------------------------------------------------------ backward
def _check_bwd(dh_bits, gu_bits, what, equal_frac=0.99):
    M, F = dh_bits.shape
    dh, gu = to_dev_bf16(dh_bits), to_dev_bf16(gu_bits)
    q, s, qt, st, d = fp8.fp8_swiglu_backward_quantize_dual(dh, gu, with_bf16=True)
    q2, s2, qt2, st2, none = fp8.fp8_swiglu_backward_quantize_dual(dh, gu)
    dq, ds, dqt, dst = fp8.fp8_quantize_dual(d)
    torch.cuda.synchronize()
    assert none is None
    dk = to_np(d)
    do = oracle.swiglu_backward(dh_bits, gu_bits)
    want = bf16_to_f64(do)
    diff = np.abs(bf16_to_f64(dk) - want)
    ok = diff <= bf16_ulp(want)
    eq_gate, eq_up = float((dk[:, :F] == do[:, :F]).mean()), float((dk[:, F:] == do[:, F:]).mean())
    _say(f"{what} {M}x{F}: dGU equal gate {eq_gate:.6f} up {eq_up:.6f}")
    assert ok.all(), f"{what}: {int((~ok).sum())} gradient elements more than one BF16 unit off"
    assert min(eq_gate, eq_up) >= equal_frac
    oq, os_ = oracle.quantize_rowtile(dk)
    oqt, ost = oracle.quantize_transposed(dk)
    for name, got, want_q in (("q", q, oq), ("s", s, os_), ("qt", qt, oqt), ("st", st, ost)):
        g = to_np(got)
        if g.dtype == np.float32:
            g, want_q = g.view(np.uint32), want_q.view(np.uint32)
        assert np.array_equal(g, want_q), f"{what}: {name} differs from the oracle's quantization"
    for a, b, name in ((q, q2, "q"), (s, s2, "s"), (qt, qt2, "qt"), (st, st2, "st"),
                       (q, dq, "q vs dual"), (s, ds, "s vs dual"), (qt, dqt, "qt vs dual"),
                       (st, dst, "st vs dual")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: {name}"


@pytest.mark.parametrize("M,F,std", [(256, 384, 1.0), (512, 256, 4.0)])
def test_swiglu_backward_dual_parity(M, F, std):
    dh = inputs.student_t((120, M, F), (M, F), 3.0, 1e-3)
    _check_bwd(dh, _gate_up(M, F, 121, std), "swiglu backward")


def test_swiglu_backward_dual_special_values():
    M, F = 256, 256
    dh = inputs.normal((123, M, F), (M, F), 1.0).copy()
    gu = _gate_up(M, F, 124).copy()
    bits = lambda v: inputs.bf16_bits(np.full(1, v, dtype=np.float32))[0]
    gu[0, :128] = bits(0.0)                  # silu'(0) = 1/2, silu(0) = 0
    gu[1, :128] = bits(100.0)                # silu' = 1
    gu[2, :128] = bits(-100.0)               # both zero
    gu[3, :128] = bits(-1.28125)             # next to the root of silu'
    dh[4, :] = bits(0.0)
    dh[128:, 128:] = bits(0.0)               # an all-zero tile of both halves
    _check_bwd(dh, gu, "swiglu backward special")


def test_swiglu_backward_dual_mlp_size():
    """The gate/up projection's output gradient at the 8192-token MLP shape:
    dH [8192, 6144] (Student-t, nu = 3, x 1e-3) and gate/up [8192, 12288]."""
    M, F = 8192, inputs.FFN
    dh = inputs.student_t((126, M, F), (M, F), 3.0, 1e-3)
    _check_bwd(dh, _gate_up(M, F, 127), "swiglu backward mlp")


def _low_gate_case(key):
    """Gates from -300 to -64.5 (below -87 e^-g overflows FP32 and
    sigmoid(g) is an FP32 denormal or zero, while g * sigmoid(g) * u can still
    be a normal BF16 value), with up values of every magnitude from 1e-30 to
    1e30 and a quarter of the rows N(0, 1)."""
    M, F = 256, 256
    rng = np.random.default_rng(key)
    gate = -np.exp(rng.uniform(np.log(64.5), np.log(300.0), (M, F)))
    mag = 10.0 ** rng.uniform(-30, 30, (M, F))
    up = np.where(rng.random((M, F)) < 0.5, -mag, mag)
    up[:, :64] = rng.normal(0, 1, (M, 64))
    as_bits = lambda v: inputs.bf16_bits(np.asarray(v, dtype=np.float32))
    return np.ascontiguousarray(np.concatenate([as_bits(gate), as_bits(up)], axis=1))


def test_swiglu_dual_very_negative_gates():
    _check(_low_gate_case(115), "swiglu low gates", full_h_equal_frac=0.95)


def test_swiglu_backward_dual_very_negative_gates():
    gu = _low_gate_case(128)
    M, F = gu.shape[0], gu.shape[1] // 2
    rng = np.random.default_rng(129)
    mag = 10.0 ** rng.uniform(-20, 20, (M, F))
    dh = inputs.bf16_bits(np.where(rng.random((M, F)) < 0.5, -mag, mag).astype(np.float32))
    _check_bwd(dh, gu, "swiglu backward low gates", equal_frac=0.95)


def test_swiglu_backward_dual_overflowing_dh_times_up():
    """Gates from -64 to -40, where silu'(g) is 1e-26 to 1e-16, with dH and
    up values from 1e15 to 1e25: dH * u overflows FP32 on many elements while
    the gate gradient dH * u * silu'(g) stays finite (below 1e35)."""
    M, F = 256, 256
    rng = np.random.default_rng(130)
    gate = rng.uniform(-64.0, -40.0, (M, F))
    mag = lambda: 10.0 ** rng.uniform(15, 25, (M, F)) * np.where(rng.random((M, F)) < 0.5, -1, 1)
    as_bits = lambda v: inputs.bf16_bits(np.asarray(v, dtype=np.float32))
    gu = np.ascontiguousarray(np.concatenate([as_bits(gate), as_bits(mag())], axis=1))
    dh = as_bits(mag())
    prod = oracle.bf16_to_f32(dh).astype(np.float64) * oracle.bf16_to_f32(gu[:, F:]).astype(np.float64)
    assert (np.abs(prod) > 3.4e38).mean() > 0.2
    _check_bwd(dh, gu, "swiglu backward dh*u overflow", equal_frac=0.95)
