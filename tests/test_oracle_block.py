"""Pins for the router -> MoE -> dense MLP chain oracle (CPU only)."""

import math

import numpy as np

from oracle import block


def _loops_matmul(a, b):
    n, kk = len(a), len(a[0])
    m = len(b[0])
    return [[math.fsum(float(a[i][t]) * float(b[t][j]) for t in range(kk)) for j in range(m)]
            for i in range(n)]


def test_router_integer_exact():
    rng = np.random.default_rng(21)
    x = rng.integers(-4, 5, size=(7, 13)).astype(np.float32)
    w = rng.integers(-3, 4, size=(13, 6)).astype(np.float32)
    got = block.router(x, w)
    ref = _loops_matmul(x.tolist(), w.tolist())
    assert np.array_equal(got, np.array(ref))
    # transposed operands would fail the shape check or the values
    assert got.shape == (7, 6)


def test_router_against_correctly_rounded_sums():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((5, 40)).astype(np.float32)
    w = rng.standard_normal((40, 9)).astype(np.float32)
    got = block.router(x, w)
    ref = np.array(_loops_matmul(x.tolist(), w.tolist()))
    assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max()


def _silu(v):
    return v / (1.0 + math.exp(-v))


def _brute_block(x, wr, k, wg, wu, wd, mg, mu, md):
    """Everything by explicit loops: logits, top-k by exhaustive ranking
    (descending, ties to the lower index), softmax over the kept logits,
    each selected expert's gated MLP per token, the weighted sum, then the
    dense gated MLP of that sum."""
    T, H = len(x), len(x[0])
    E = len(wr[0])
    logits = _loops_matmul(x, wr)
    ys = []
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t][e], e))[:k]
        m = max(logits[t][e] for e in order)
        ex = [math.exp(logits[t][e] - m) for e in order]
        s = math.fsum(ex)
        z = [0.0] * H
        for e, p in zip(order, ex):
            g = _loops_matmul([x[t]], wg[e])[0]
            u = _loops_matmul([x[t]], wu[e])[0]
            h = [_silu(a) * b for a, b in zip(g, u)]
            ye = _loops_matmul([h], wd[e])[0]
            z = [zz + (p / s) * v for zz, v in zip(z, ye)]
        g = _loops_matmul([z], mg)[0]
        u = _loops_matmul([z], mu)[0]
        h = [_silu(a) * b for a, b in zip(g, u)]
        ys.append((logits[t], z, _loops_matmul([h], md)[0]))
    return ys


def test_chain_brute_force_tiny():
    rng = np.random.default_rng(23)
    T, H, E, k, I, Im = 5, 6, 4, 2, 3, 5
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((H, E))
    wg, wu = rng.standard_normal((E, H, I)) * 0.5, rng.standard_normal((E, H, I)) * 0.5
    wd = rng.standard_normal((E, I, H)) * 0.5
    mg, mu, md = rng.standard_normal((H, Im)), rng.standard_normal((H, Im)), rng.standard_normal((Im, H))
    res = block.block(x, wr, k, (wg, wu, wd), (mg, mu, md))
    brute = _brute_block(x.tolist(), wr.tolist(), k, wg.tolist(), wu.tolist(), wd.tolist(),
                         mg.tolist(), mu.tolist(), md.tolist())
    for t in range(T):
        lg, z, y = brute[t]
        assert np.allclose(res["logits"][t], lg, rtol=1e-13, atol=1e-13)
        assert np.allclose(res["z"][t], z, rtol=1e-12, atol=1e-12)
        assert np.allclose(res["y"][t], y, rtol=1e-11, atol=1e-11)


def test_route_logits_override_decides_ties():
    """Ranking on the float32 logits a kernel produced: two experts whose
    fp64 logits differ below float32 resolution are ranked as the float32
    values say (equal -> lower index)."""
    x = np.array([[1.0, 1.0]])
    wr = np.array([[0.5, 0.5 + 2.0 ** -30, -1.0], [0.25, 0.25, -1.0]])
    lg = block.router(x, wr)
    assert lg[0, 1] > lg[0, 0]                       # fp64 prefers expert 1
    f32 = lg.astype(np.float32)
    assert f32[0, 0] == f32[0, 1]                    # float32 ties them
    wg = np.ones((3, 2, 1)); wu = np.ones((3, 2, 1)); wd = np.ones((3, 1, 2))
    m = (np.eye(2, 1), np.eye(2, 1), np.eye(1, 2))
    r64 = block.block(x, wr, 1, (wg, wu, wd), m)
    r32 = block.block(x, wr, 1, (wg, wu, wd), m, route_logits=f32)
    assert r64["ids"][0, 0] == 1 and r32["ids"][0, 0] == 0
