"""Oracle: the dense SiLU-gated MLP chain (test infrastructure only).

The pages name the dense MLP of the served models (Event Tensor notes,
sections "计算通信融合" and "端到端低 batch serving": MLP shapes of Qwen3 /
LLaMA 3.1 / Gemma 2 / GPT-3, and the dense-MLP GEMM pipelined across stages)
but do not write it out.  The plainest reading, used for the models the pages
name, is the gated MLP

    g = x @ Wg,  u = x @ Wu,  h = SiLU(g) * u,  y = h @ Wd,
    SiLU(z) = z / (1 + exp(-z)),

with logical layouts x [B, H], Wg/Wu [H, I], Wd [I, H].  Everything is
evaluated in float64 from the exact input values, with no intermediate
rounding.

Pins (tests/test_oracle_mlp.py): SiLU at closed-form points (0, +-ln 3) and
its odd-part identity SiLU(z) - SiLU(-z) = z together with its two
asymptotes; integer-valued x/W checked exactly against brute-force integer
dot products; one-hot Wu / Wd selection structures that expose transposed or
swapped operands.
"""

import numpy as np


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def mlp(x, wg, wu, wd, return_intermediates=False):
    """y = (SiLU(x Wg) * (x Wu)) Wd.

    x: [B, H]; wg, wu: [H, I]; wd: [I, H] (logical layouts, any float dtype;
    values are widened exactly to float64).  Returns y [B, H] float64, or
    (y, g, u, h) when ``return_intermediates``.
    """
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(wg, dtype=np.float64)
    wu = np.asarray(wu, dtype=np.float64)
    wd = np.asarray(wd, dtype=np.float64)
    if x.ndim != 2 or wg.shape != wu.shape or wg.shape[0] != x.shape[1] \
            or wd.shape != (wg.shape[1], x.shape[1]):
        raise ValueError("mlp: shapes must be x[B,H], wg/wu[H,I], wd[I,H]")
    g = x @ wg
    u = x @ wu
    h = silu(g) * u
    y = h @ wd
    if return_intermediates:
        return y, g, u, h
    return y
