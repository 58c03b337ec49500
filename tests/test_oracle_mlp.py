"""Pins for the dense MLP oracle (CPU only)."""

import math

import numpy as np
import pytest

from oracle import mlp as om


def test_silu_closed_forms():
    ln3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert om.silu(0.0) == 0.0
    assert abs(om.silu(ln3) - 0.75 * ln3) < 1e-15
    assert abs(om.silu(-ln3) + 0.25 * ln3) < 1e-15
    z = np.linspace(-12, 12, 97)
    assert np.allclose(om.silu(z) - om.silu(-z), z, rtol=0, atol=1e-13)
    # asymptotes: SiLU(z) -> z for z >> 0 and -> 0 for z << 0
    assert abs(om.silu(60.0) - 60.0) < 1e-20 * 60 + 1e-12
    assert abs(om.silu(-60.0)) < 1e-20


def _ints(rng, shape, lo=-3, hi=3):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def test_integer_gate_up_exact():
    rng = np.random.default_rng(5)
    B, H, I = 3, 7, 5          # non-square so transposed operands fail
    x, wg, wu = _ints(rng, (B, H)), _ints(rng, (H, I)), _ints(rng, (H, I))
    wd = _ints(rng, (I, H))
    y, g, u, h = om.mlp(x, wg, wu, wd, return_intermediates=True)
    for b in range(B):
        for i in range(I):
            assert g[b, i] == sum(int(x[b, t]) * int(wg[t, i]) for t in range(H))
            assert u[b, i] == sum(int(x[b, t]) * int(wu[t, i]) for t in range(H))
            if g[b, i] == 0 or u[b, i] == 0:
                assert h[b, i] == 0


def test_one_hot_down_selects_h_columns():
    rng = np.random.default_rng(6)
    B, H, I = 4, 6, 9
    x = rng.standard_normal((B, H)).astype(np.float32)
    wg = rng.standard_normal((H, I)).astype(np.float32)
    wu = rng.standard_normal((H, I)).astype(np.float32)
    sel = rng.integers(0, I, size=H)
    wd = np.zeros((I, H), np.float32)
    wd[sel, np.arange(H)] = 1.0
    y, g, u, h = om.mlp(x, wg, wu, wd, return_intermediates=True)
    assert (y == h[:, sel]).all()


def test_gate_is_the_silu_operand():
    # u == 1 and two gate columns +2 / -2: h0 - h1 = SiLU(2) - SiLU(-2) = 2 exactly
    # in exact arithmetic; a swapped gate/up gives SiLU(1) * 4 instead.
    H, I = 3, 2
    x = np.array([[1, 0, 0]], np.float32)
    wg = np.zeros((H, I), np.float32); wg[0] = [2, -2]
    wu = np.zeros((H, I), np.float32); wu[0] = [1, 1]
    wd = np.eye(I, H, dtype=np.float32)
    y = om.mlp(x, wg, wu, wd)
    assert abs((y[0, 0] - y[0, 1]) - 2.0) < 1e-14


def test_linear_in_down_weights():
    rng = np.random.default_rng(8)
    B, H, I = 2, 5, 3
    x = rng.standard_normal((B, H))
    wg, wu = rng.standard_normal((H, I)), rng.standard_normal((H, I))
    d1, d2 = rng.standard_normal((I, H)), rng.standard_normal((I, H))
    assert np.allclose(om.mlp(x, wg, wu, d1 + d2), om.mlp(x, wg, wu, d1) + om.mlp(x, wg, wu, d2))


def test_shape_errors():
    with pytest.raises(ValueError):
        om.mlp(np.zeros((1, 4)), np.zeros((4, 3)), np.zeros((4, 3)), np.zeros((4, 3)))
