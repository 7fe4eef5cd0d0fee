"""Pins of the oracle's tile quantizers (row tiles, weight blocks, token-axis
tiles) against invariants and closed forms that do not reuse its code:

* hand-worked tiles (tests/golden/quant_tile_worked.txt),
* the amax element of every tile encodes to +-448,
* tiles of E4M3 grid values times 2^j round-trip exactly with s = 2^j,
* sign symmetry, 2^j equivariance, permutation within a tile,
* transposition identities between the three quantizers,
* correct rounding of the scale (exact rationals),
* nearest-code optimality by brute force over all 254 finite codes,
* the per-element dequantization error bound of a 3-bit-mantissa format.
"""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp8_block_scaled_03_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _worked_tiles():
    tiles = {}
    for line in open(os.path.join(GOLDEN, "quant_tile_worked.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "tile":
            tiles.setdefault(f[1], {"elems": []})["scale"] = int(f[3], 16)
        else:
            tiles.setdefault(f[0], {"elems": []})["elems"].append((int(f[1]), float(f[2]), int(f[3], 16)))
    return tiles


def test_worked_tiles_golden():
    tiles = _worked_tiles()
    assert set(tiles) == {"A", "B", "C"}
    for name, t in tiles.items():
        x = np.zeros(128, dtype=np.float32)
        want = np.zeros(128, dtype=np.uint8)
        for i, v, c in t["elems"]:
            x[i] = v
            want[i] = c
        bits = inputs.bf16_bits(x.reshape(1, 128))
        assert np.array_equal(oracle.bf16_to_f32(bits).reshape(128).view(np.uint32),
                              x.view(np.uint32)), "fixture values must be exact in BF16"
        q, s = oracle.quantize_rowtile(bits)
        assert _f32_bits(float(s[0, 0])) == t["scale"], name
        assert np.array_equal(q.reshape(128), want), (name, q.reshape(128)[:20], want[:20])


def _tiles_of(kind, seed, shape=(64, 1024)):
    return inputs.random_bits((99, seed), shape, kind)


@pytest.mark.parametrize("kind", ["normal", "wide", "special"])
def test_amax_element_maps_to_448(kind):
    x = _tiles_of(kind, 1)
    q, s = oracle.quantize_rowtile(x)
    xf = oracle.bf16_to_f32(x).reshape(x.shape[0], -1, 128)
    qt = q.reshape(x.shape[0], -1, 128)
    amax = np.abs(xf).max(axis=2)
    arg = np.abs(xf).argmax(axis=2)
    code_at = np.take_along_axis(qt, arg[..., None], axis=2)[..., 0]
    live = amax >= 2.0 ** -100
    assert live.any()
    assert np.all((code_at[live] & 0x7F) == 0x7E)
    # every code is within the finite range, never NaN
    assert not np.any((q & 0x7F) == 0x7F)


def test_scale_is_correctly_rounded_quotient():
    x = _tiles_of("wide", 2, (16, 512))
    q, s = oracle.quantize_rowtile(x)
    xf = oracle.bf16_to_f32(x).reshape(16, 4, 128)
    amax = np.abs(xf).max(axis=2)
    for a, sc in zip(amax.reshape(-1), s.reshape(-1)):
        a = max(float(a), 2.0 ** -100)
        exact = Fraction(a) / 448
        sc = float(sc)
        lo = np.nextafter(np.float32(sc), np.float32(0))
        hi = np.nextafter(np.float32(sc), np.float32(np.inf))
        # sc is nearest: the exact quotient lies within half an ulp on either side
        assert abs(Fraction(sc) - exact) <= abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(sc) - exact) <= abs(Fraction(float(hi)) - exact)


def test_exactly_representable_tiles_round_trip():
    rng = np.random.default_rng(3)
    t = oracle.e4m3_table()
    finite = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    for j in (-20, -7, 0, 5, 30):
        codes = rng.choice(finite, size=(8, 128))
        codes[:, 17] = 0x7E                      # +448 in every tile
        codes[3, 17] = 0xFE                      # one tile with -448 as its amax
        x = (t[codes] * 2.0 ** j).astype(np.float32)
        bits = inputs.bf16_bits(x)
        assert np.array_equal(oracle.bf16_to_f32(bits).view(np.uint32), x.view(np.uint32))
        q, s = oracle.quantize_rowtile(bits)
        assert np.all(s == np.float32(2.0 ** j))
        # zero codes keep their sign; everything else must match exactly
        assert np.array_equal(q, codes)


def test_sign_symmetry_and_power_of_two_equivariance():
    x = _tiles_of("normal", 4, (32, 512))
    q, s = oracle.quantize_rowtile(x)
    qn, sn = oracle.quantize_rowtile(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, q ^ 0x80)
    assert np.array_equal(sn, s)
    xf = oracle.bf16_to_f32(x)
    for j in (-9, 11):
        xs = inputs.bf16_bits(xf * np.float32(2.0 ** j))
        qj, sj = oracle.quantize_rowtile(xs)
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, s * np.float32(2.0 ** j))


def test_permutation_within_tile_permutes_codes():
    x = _tiles_of("special", 5, (8, 256))
    q, s = oracle.quantize_rowtile(x)
    perm = np.random.default_rng(5).permutation(128)
    xp = x.reshape(8, 2, 128)[:, :, perm].reshape(8, 256)
    qp, sp = oracle.quantize_rowtile(xp)
    assert np.array_equal(qp.reshape(8, 2, 128), q.reshape(8, 2, 128)[:, :, perm])
    assert np.array_equal(sp, s)


def test_codes_are_nearest_by_brute_force():
    """Brute force: each code is the finite E4M3 value nearest to fl32(x*inv)
    (ties to the even code), with inv = fl32(448/a)."""
    x = _tiles_of("special", 6, (4, 256))
    q, s = oracle.quantize_rowtile(x)
    t = oracle.e4m3_table()
    finite = [c for c in range(127)]
    xf = oracle.bf16_to_f32(x).reshape(4, 2, 128)
    for r in range(4):
        for b in range(2):
            a = max(float(np.abs(xf[r, b]).max()), 2.0 ** -100)
            inv = np.float32(np.float32(448.0) / np.float32(a))
            for e in range(128):
                p = np.float32(xf[r, b, e] * inv)
                p = min(max(float(p), -448.0), 448.0)
                mag = abs(p)
                d = [abs(t[c] - mag) for c in finite]
                best = min(d)
                cands = [c for c in finite if d[c] == best]
                want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
                if np.signbit(p) or (p == 0 and np.signbit(xf[r, b, e])):
                    want |= 0x80
                assert q[r, b * 128 + e] == want, (r, b, e, p)


@pytest.mark.parametrize("cfg,name", [("qkv", "X"), ("mlp", "H"), ("down_bwd", "dY"),
                                      ("tiny", "W")])
def test_dequantization_error_bound_and_rho(cfg, name):
    """|dec(q)*s - x| <= max(2^-4 |x|, 2^-10 s): half an ulp of a 3-bit mantissa
    in the normal range, half the subnormal step below it.  rho (relative
    Frobenius error of the dequantized tensor) stays below 3e-2."""
    rows = 256
    x = inputs.tensor(cfg, name, rows=rows) if cfg != "tiny" else inputs.tensor(cfg, name)
    q, s = oracle.quantize_rowtile(x)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    deq = oracle.dequantize_rows(q, s)
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(deq - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)
    rho = np.linalg.norm(deq - xf) / np.linalg.norm(xf)
    assert rho <= 3e-2, rho


def test_transposed_equals_rowtile_of_transpose():
    x = _tiles_of("wide", 7, (384, 200))                 # C not a multiple of 128 is fine
    qt, st = oracle.quantize_transposed(x)
    q2, s2 = oracle.quantize_rowtile(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q2) and np.array_equal(st, s2)


def test_block_of_transpose_is_transpose_of_block():
    w = _tiles_of("normal", 8, (256, 384))
    q, qt, s = oracle.quantize_block(w)
    assert np.array_equal(qt, q.T)
    q2, qt2, s2 = oracle.quantize_block(np.ascontiguousarray(w.T))
    assert np.array_equal(q2, q.T) and np.array_equal(s2, s.T) and np.array_equal(qt2, q)


def test_block_amax_and_scale():
    w = inputs.tensor("tiny", "W")
    q, _, s = oracle.quantize_block(w, with_transpose=False)
    wf = oracle.bf16_to_f32(w).reshape(2, 128, 4, 128)
    amax = np.abs(wf).max(axis=(1, 3))
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    # each block's amax element encodes to +-448
    for bi in range(2):
        for bj in range(4):
            blk = oracle.bf16_to_f32(w)[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            r, c = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert q[bi * 128 + r, bj * 128 + c] & 0x7F == 0x7E


def test_zero_tile_uses_floor_and_encodes_zero():
    x = np.zeros((3, 256), dtype=np.uint16)
    x[1, :128] = 0x8000                                   # -0.0 tile
    q, s = oracle.quantize_rowtile(x)
    assert np.all(s.view(np.uint32) == 0x09124925)
    assert np.all(q[1, :128] == 0x80) and np.all(q[0] == 0) and np.all(q[1, 128:] == 0)


def test_empty_and_ragged_rows():
    q, s = oracle.quantize_rowtile(np.zeros((0, 256), dtype=np.uint16))
    assert q.shape == (0, 256) and s.shape == (0, 2)
    x = _tiles_of("normal", 9, (77, 256))
    q, s = oracle.quantize_rowtile(x)
    q1, s1 = oracle.quantize_rowtile(x[:13])
    assert np.array_equal(q[:13], q1) and np.array_equal(s[:13], s1)


def test_errors_non_finite_and_shape():
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 5] = 0x7F80                                      # +inf
    with pytest.raises(ValueError, match="non-finite"):
        oracle.quantize_rowtile(x)
    with pytest.raises(ValueError, match="shape"):
        oracle.quantize_rowtile(np.zeros((2, 100), dtype=np.uint16))
    with pytest.raises(ValueError, match="shape"):
        oracle.quantize_transposed(np.zeros((100, 128), dtype=np.uint16))


def test_thread_count_does_not_change_results():
    x = _tiles_of("wide", 10, (64, 1024))
    a = oracle.quantize_rowtile(x, threads=1)
    b = oracle.quantize_rowtile(x, threads=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
