"""The seeded input recipes: every configuration's GEMMs refer to tensors of
consistent shapes, draws are reproducible, and the distributions are the
stated ones (checked on small draws)."""
import numpy as np
import pytest

import oracle
from fp8_block_scaled_03_amd import inputs


@pytest.mark.parametrize("name", sorted(inputs.CONFIGS))
def test_config_shapes_are_consistent(name):
    c = inputs.CONFIGS[name]
    for g in c.gemms:
        sa = c.tensors[g.a][0]
        sb = c.tensors[g.b][0]
        if g.kind == "fprop":
            assert sa == (g.M, g.K) and sb == (g.N, g.K), g
        elif g.kind == "dgrad":
            assert sa == (g.M, g.N) and sb == (g.N, g.K), g
        else:
            assert sa == (g.M, g.N) and sb == (g.M, g.K), g
        assert g.out in ("f32", "bf16")
        for d in (g.N, g.K):
            assert d % 128 == 0
    for t in c.per_layer:
        assert t in c.tensors


def test_linear_set_totals():
    c = inputs.CONFIGS["linear_set"]
    assert len(c.gemms) == 12 and c.layers == 28
    assert sum(g.flops for g in c.gemms) * c.layers == 138_538_465_099_776
    assert {g.kind for g in c.gemms} == {"fprop", "dgrad", "wgrad"}


def test_draws_are_reproducible_and_layer_keyed():
    a = inputs.tensor("linear_set", "W_o", layer=3)
    b = inputs.tensor("linear_set", "W_o", layer=3)
    c = inputs.tensor("linear_set", "W_o", layer=4)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # shared activations ignore the layer
    x0 = inputs.tensor("tiny", "X", layer=0)
    x5 = inputs.tensor("tiny", "X", layer=5)
    assert np.array_equal(x0, x5)


def test_distributions():
    w = oracle.bf16_to_f32(inputs.tensor("tiny", "W")).astype(np.float64)
    assert abs(w.std() - 0.02) < 0.001 and abs(w.mean()) < 0.001
    h = oracle.bf16_to_f32(inputs.tensor("mlp", "H", rows=512)).astype(np.float64)
    assert abs(h.std() - 0.5) < 0.05                       # t(4) scaled to std 0.5
    dy = oracle.bf16_to_f32(inputs.tensor("down_bwd", "dY", rows=512)).astype(np.float64)
    assert 1e-3 < np.median(np.abs(dy)) / 0.765 * 1.3 < 2e-3   # 1e-3 * t(3), median |t3| ~ 0.765
    x = oracle.bf16_to_f32(inputs.tensor("qkv", "X")).astype(np.float64)
    cols = inputs.outlier_channels()
    assert len(cols) == 8
    std = x.std(axis=0)
    assert np.all(std[cols] > 15) and np.median(std) < 1.1
