"""fp8_rmsnorm_quantize_dual through the C ABI, against the oracle.

The kernel sums each row's squares in FP32 and forms Y = x * r * gamma in FP32;
the oracle works in double and rounds once.  Gates: r within a relative 2^-20
of the oracle's; every element of Y within one BF16 unit of the oracle's
(nearly all equal); the codes and scales bit for bit equal to the oracle's
quantization of the Y the kernel formed, the same bytes without the BF16 Y,
and equal to fp8_quantize_dual of that Y on the GPU."""
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


def _gamma(C, key):
    g = np.random.default_rng(key).uniform(0.5, 1.5, C).astype(np.float32)
    return inputs.bf16_bits(g)


def _check(x_bits, g_bits, eps, what):
    M, C = x_bits.shape
    x, gamma = to_dev_bf16(x_bits), to_dev_bf16(g_bits)
    q, s, qt, st, r, y = fp8.fp8_rmsnorm_quantize_dual(x, gamma, eps, with_y=True)
    q2, s2, qt2, st2, r2, none = fp8.fp8_rmsnorm_quantize_dual(x, gamma, eps)
    dq, ds, dqt, dst = fp8.fp8_quantize_dual(y)
    torch.cuda.synchronize()
    assert none is None
    yo, ro = oracle.rmsnorm(x_bits, g_bits, eps)
    rk = to_np(r).astype(np.float64)
    rel_r = float(np.max(np.abs(rk - ro) / ro))
    yk = to_np(y)
    want = bf16_to_f64(yo)
    diff = np.abs(bf16_to_f64(yk) - want)
    ok = diff <= bf16_ulp(want)
    eq = float((yk == yo).mean())
    _say(f"{what} {M}x{C}: r rel err {rel_r:.2e}, Y equal {eq:.6f}")
    assert rel_r <= 2.0 ** -20, f"{what}: r off by {rel_r:.3e}"
    assert ok.all(), f"{what}: {int((~ok).sum())} elements of Y more than one BF16 unit off"
    assert eq >= 0.99
    assert torch.equal(r, r2)
    oq, os_ = oracle.quantize_rowtile(yk)
    oqt, ost = oracle.quantize_transposed(yk)
    for name, got, want_q in (("q", q, oq), ("s", s, os_), ("qt", qt, oqt), ("st", st, ost)):
        g = to_np(got)
        if g.dtype == np.float32:
            g, want_q = g.view(np.uint32), want_q.view(np.uint32)
        assert np.array_equal(g, want_q), f"{what}: {name} differs from the oracle's quantization"
    for a, b, name in ((q, q2, "q"), (s, s2, "s"), (qt, qt2, "qt"), (st, st2, "st"),
                       (q, dq, "q vs dual"), (s, ds, "s vs dual"), (qt, dqt, "qt vs dual"),
                       (st, dst, "st vs dual")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: {name}"


@pytest.mark.parametrize("M,C,std,eps", [(256, 384, 1.0, 1e-6), (1024, 2048, 30.0, 1e-5),
                                         (128, 128, 0.01, 1e-6)])
def test_rmsnorm_dual_parity(M, C, std, eps):
    x = inputs.normal((130, M, C), (M, C), std)
    _check(x, _gamma(C, 131), eps, "rmsnorm")


def test_rmsnorm_dual_special_rows():
    """Zero rows (Y = 0, r = 1/sqrt(eps)), constant rows (Y = sign * gamma up
    to eps), one huge and one tiny row, and an all-zero 128 x 128 tile."""
    M, C = 256, 512
    x = inputs.normal((132, M, C), (M, C), 1.0).copy()
    bits = lambda v: inputs.bf16_bits(np.full(1, v, dtype=np.float32))[0]
    x[0, :] = bits(0.0)
    x[1, :] = bits(-3.0)
    x[2, :] = bits(1.0e15)
    x[3, :] = bits(1.0e-30)
    x[128:, :128] = bits(0.0)
    _check(x, _gamma(C, 133), 1e-6, "rmsnorm special")


def test_rmsnorm_dual_empty():
    for M, C in ((0, 256), (256, 0)):
        x = torch.empty((M, C), dtype=torch.bfloat16, device="cuda")
        g = torch.ones((C,), dtype=torch.bfloat16, device="cuda")
        q, s, qt, st, r, y = fp8.fp8_rmsnorm_quantize_dual(x, g, 1e-6, with_y=True)
        torch.cuda.synchronize()
        assert q.numel() == 0 and qt.numel() == 0 and y.numel() == 0


def test_rmsnorm_dual_rejects_bad_eps():
    x = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.ones((128,), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fp8.Fp8bsError):
        fp8.fp8_rmsnorm_quantize_dual(x, g, -1e-6)


def test_rmsnorm_dual_qkv_input_size():
    """The QKV projection's input at 8192 tokens: N(0,1) with 8 outlier
    channels x20 (they dominate some rows' RMS), every element compared."""
    c = inputs.CONFIGS["qkv"]
    g = next(g for g in c.gemms if g.kind == "fprop")
    x = inputs.tensor("qkv", g.a)
    _check(x, _gamma(x.shape[1], 134), 1e-6, "rmsnorm qkv input")


def test_rmsnorm_dual_rows_past_one_grid_pass():
    """4,194,688 rows of 128 channels: the per-row 1/RMS kernel runs a capped
    grid of 2^20 workgroups (4 rows each), so rows past 2^22 are taken on a
    second pass.  Row m holds row (7919 m) mod 8192 of a seeded base (a
    permutation of every 8192-row window): r is compared on every row, Y and
    the row-tile codes on 12,288 rows (first, last, random), the token-axis
    codes on the 128-row blocks around 2^22 and at the end."""
    M, C, B = (1 << 22) + 384, 128, 8192
    base = inputs.normal((135, B, C), (B, C), 1.0)
    g_bits = _gamma(C, 136)
    idx = (np.arange(M, dtype=np.int64) * 7919) % B
    x = to_dev_bf16(base)[torch.from_numpy(idx).cuda()]
    gamma = to_dev_bf16(g_bits)
    _say(f"rmsnorm {M}x{C} (two grid passes)")
    q, s, qt, st, r, y = fp8.fp8_rmsnorm_quantize_dual(x, gamma, 1e-6, with_y=True)
    torch.cuda.synchronize()
    yo, ro = oracle.rmsnorm(base, g_bits, 1e-6)
    rk = to_np(r).astype(np.float64)
    assert float(np.max(np.abs(rk - ro[idx]) / ro[idx])) <= 2.0 ** -20
    rng = np.random.default_rng(137)
    rows = np.unique(np.concatenate([np.arange(4096), np.arange(M - 4096, M),
                                     rng.integers(0, M, 4096)]))
    rows_t = torch.from_numpy(rows).cuda()
    yk = to_np(y[rows_t])
    want = bf16_to_f64(yo[idx[rows]])
    assert np.all(np.abs(bf16_to_f64(yk) - want) <= bf16_ulp(want))
    oq, os_ = oracle.quantize_rowtile(yk)
    assert np.array_equal(to_np(q[rows_t]), oq)
    assert np.array_equal(to_np(s[rows_t]).view(np.uint32), os_.view(np.uint32))
    for mb in ((1 << 22) // 128 - 1, (1 << 22) // 128, M // 128 - 1):
        yb = to_np(y[128 * mb:128 * (mb + 1)])
        oqt, ost = oracle.quantize_transposed(yb)
        assert np.array_equal(to_np(qt[:, 128 * mb:128 * (mb + 1)]), oqt), f"qt block {mb}"
        assert np.array_equal(to_np(st[:, mb:mb + 1]).view(np.uint32), ost.view(np.uint32))
    del x, q, s, qt, st, r, y
    torch.cuda.empty_cache()


def test_rmsnorm_dual_rows_outside_fp32_squares():
    """Rows whose sum of squares leaves FP32's range are summed again at a
    power-of-two scale: rows of N(0,1) x 1e25 (the squares overflow), x 1e36,
    x 1e-25 and x 1e-35 (the squares underflow) with eps = 0, the tiny rows
    also with eps = 1e-6 (which then dominates), beside ordinary rows."""
    M, C = 256, 384
    base = inputs.normal((138, M, C), (M, C), 1.0)
    vals = oracle.bf16_to_f32(base).astype(np.float64)
    scale = np.ones(M)
    scale[0:32], scale[32:64], scale[64:96], scale[96:128] = 1e25, 1e36, 1e-25, 1e-35
    x = inputs.bf16_bits((vals * scale[:, None]).astype(np.float32))
    g = _gamma(C, 139)
    _check(x, g, 0.0, "rmsnorm extreme rows eps=0")
    _check(np.ascontiguousarray(x[64:192]), g, 1e-6, "rmsnorm tiny rows eps=1e-6")
