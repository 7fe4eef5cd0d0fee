"""Pins of the oracle's E4M3 codec and BF16 rounding against things other than
itself: the OCP E4M3 format points (golden file), torch's float8_e4m3fn decode
and cast (an independent library routine with the same round-to-nearest-even
semantics in range), and torch's BF16 cast."""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_encode(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_view_of_all_codes():
    t = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    assert set(np.flatnonzero(np.isnan(t))) == {0x7F, 0xFF}
    fin = ~np.isnan(t)
    assert np.array_equal(t[fin], ref[fin])
    # signed zeros
    assert np.signbit(t[0x80]) and not np.signbit(t[0x00])


def test_decode_golden_format_points():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "e4m3_format_points.txt"))
             if l.strip() and not l.startswith("#")]
    assert len(lines) >= 10
    t = oracle.e4m3_table()
    for code_s, val_s, *_ in lines:
        c = int(code_s, 16)
        if val_s == "nan":
            assert np.isnan(t[c])
        else:
            assert t[c] == float(val_s), (code_s, val_s, t[c])
            assert np.signbit(t[c]) == val_s.startswith("-")


def test_units_are_exact_multiples_of_2pow_minus9():
    L = oracle.lib()
    for c in range(256):
        v = oracle.e4m3_value(c)
        u = L.oracle_e4m3_units(c)
        if np.isnan(v):
            assert u == -2**31
        else:
            assert u == v * 512
    assert max(abs(L.oracle_e4m3_units(c)) for c in range(256) if c not in (0x7F, 0xFF)) == 229376


def test_encode_every_finite_value_roundtrips():
    t = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    got = oracle.e4m3_encode(t[codes].astype(np.float32))
    assert np.array_equal(got, codes)


def test_encode_ties_and_neighbours_match_torch():
    t = oracle.e4m3_table()
    mags = np.sort(t[:127])
    mids = 0.5 * (mags[:-1] + mags[1:])                 # exact in float32
    pts = np.concatenate([mags, mids]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(-np.inf))
    v = np.concatenate([pts, up, dn])
    v = v[np.abs(v) <= 448]
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.e4m3_encode(v), _torch_encode(v))


def test_encode_strided_sweep_matches_torch():
    # every 61st FP32 bit pattern with magnitude <= 448*(1+2^-22), both signs
    hi = np.float32(448.0).view(np.uint32) + 2
    pats = np.arange(0, hi, 61, dtype=np.uint32)
    v = pats.view(np.float32)
    for sgn in (1, -1):
        vv = (v * np.float32(sgn)).astype(np.float32)
        assert np.array_equal(oracle.e4m3_encode(vv), _torch_encode(vv))


def test_encode_special_values():
    v = np.array([0.0, -0.0, -1e-30, 1e-30, 449.0, -1000.0, np.inf, np.nan], dtype=np.float32)
    got = oracle.e4m3_encode(v)
    assert list(got[:6]) == [0x00, 0x80, 0x80, 0x00, 0x7E, 0xFE]
    assert got[6] == 0x7E          # saturating encoder (the quantizer clamps before it)
    assert got[7] == 0x7F


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    pats = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties (low half 0x8000) and near-ties
    pats[::3] = (pats[::3] & 0xFFFF0000) | 0x8000
    pats[1::7] = (pats[1::7] & 0xFFFF0000) | 0x7FFF
    v = pats.view(np.float32)
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(v), ref)


def test_bf16_to_f32_is_exact():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(f[fin].view(np.uint32), ref[fin].view(np.uint32))


@pytest.mark.slow
def test_encode_exhaustive_matches_torch():
    """Every FP32 pattern with |v| <= 448*(1+2^-22); about a minute."""
    hi = int(np.float32(448.0).view(np.uint32)) + 2
    step = 1 << 25
    for lo in range(0, hi, step):
        pats = np.arange(lo, min(lo + step, hi), dtype=np.uint32)
        v = pats.view(np.float32)
        assert np.array_equal(oracle.e4m3_encode(v), _torch_encode(v)), lo
        assert np.array_equal(oracle.e4m3_encode(-v), _torch_encode(-v)), lo
