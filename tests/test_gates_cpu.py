"""The parity gates themselves, on hand-made values: the BF16 gate accepts
one BF16 ulp and nothing more away from zero, and its wider allowance only
applies where the oracle value is within the FP32 per-element bound of zero;
the FP32 gate catches a relative error above 1e-5."""
import numpy as np
import pytest

import oracle
from helpers import check_bf16, check_bf16_is_rne_of_f32, check_f32


def _case():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((4, 256))
    b = rng.standard_normal((6, 256))
    ref = (a @ b.T).astype(np.float32)
    return a, b, ref


def test_bf16_gate_is_one_ulp_away_from_zero():
    a, b, ref = _case()
    bits = oracle.f32_to_bf16(ref)
    check_bf16(bits, ref, a, b)                               # exact: passes
    one = bits.copy()
    one[1, 2] += np.uint16(1)                                 # one ulp: passes
    check_bf16(one, ref, a, b)
    two = bits.copy()
    two[1, 2] += np.uint16(2)                                 # two ulps: fails
    with pytest.raises(AssertionError):
        check_bf16(two, ref, a, b)


def test_bf16_gate_near_zero_allowance_is_bounded():
    a, b, ref = _case()
    bound = 1e-4 * np.linalg.norm(a[0]) * np.linalg.norm(b[0])
    ref = ref.copy()
    ref[0, 0] = np.float32(bound / 8)                         # an oracle value close to zero
    bits = oracle.f32_to_bf16(ref)
    near = bits.copy()
    near[0, 0] = oracle.f32_to_bf16(np.float32(bound / 8 + bound / 2))[0]   # many ulps, within bound
    assert check_bf16(near, ref, a, b) == 1
    far = bits.copy()
    far[0, 0] = oracle.f32_to_bf16(np.float32(bound / 8 + 3 * bound))[0]
    with pytest.raises(AssertionError):
        check_bf16(far, ref, a, b)
    # the same absolute difference where the oracle value is 8x the bound
    # (so not near zero; there bound/2 is about eight ulps) is refused
    bound23 = 1e-4 * np.linalg.norm(a[2]) * np.linalg.norm(b[3])
    ref[2, 3] = np.float32(8 * bound23)
    bits = oracle.f32_to_bf16(ref)
    away = bits.copy()
    away[2, 3] = oracle.f32_to_bf16(np.float32(8 * bound23 + bound23 / 2))[0]
    with pytest.raises(AssertionError):
        check_bf16(away, ref, a, b)


def test_f32_gate_and_rne_identity():
    a, b, ref = _case()
    check_f32(ref.copy(), ref, a, b)
    bad = ref * np.float32(1 + 3e-5)
    with pytest.raises(AssertionError):
        check_f32(bad, ref, a, b)
    check_bf16_is_rne_of_f32(oracle.f32_to_bf16(ref), ref)
    off = oracle.f32_to_bf16(ref)
    off[3, 1] ^= np.uint16(1)
    with pytest.raises(AssertionError):
        check_bf16_is_rne_of_f32(off, ref)
