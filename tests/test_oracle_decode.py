"""Pins for the decode attention-front oracle (CPU only)."""

import cmath
import math

import numpy as np

from oracle import decode


def test_rms_norm_closed_forms():
    D = 8
    w = np.arange(1, D + 1, dtype=np.float64)
    # constant input c: mean(x^2) = c^2, so n = c / sqrt(c^2 + eps) * w
    for c in (2.0, -0.5):
        got = decode.rms_norm(np.full(D, c), w, 1e-6)
        assert np.allclose(got, c / math.sqrt(c * c + 1e-6) * w, rtol=1e-15, atol=0)
    # x = (3, 4): mean of squares 12.5
    got = decode.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(got, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    # scale invariance without eps
    x = np.random.default_rng(1).standard_normal(16)
    assert np.allclose(decode.rms_norm(7 * x, np.ones(16), 0.0), decode.rms_norm(x, np.ones(16), 0.0))


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(2)
    D, theta = 16, 10000.0
    x = rng.standard_normal(D)
    for pos in (0, 1, 7, 300):
        got = decode.rope(x, pos, theta)
        for i in range(D // 2):
            z = complex(x[i], x[i + D // 2]) * cmath.exp(1j * pos * theta ** (-2.0 * i / D))
            assert abs(got[i] - z.real) < 1e-12 and abs(got[i + D // 2] - z.imag) < 1e-12
    assert np.array_equal(decode.rope(x, 0, theta), x)


def test_rope_norm_and_additivity():
    rng = np.random.default_rng(3)
    D, theta = 32, 1e6
    x = rng.standard_normal((3, D))
    r = decode.rope(x, np.array([5, 11, 400]), theta)
    h = D // 2
    assert np.allclose(x[:, :h] ** 2 + x[:, h:] ** 2, r[:, :h] ** 2 + r[:, h:] ** 2)
    two = decode.rope(decode.rope(x, 17, theta), 25, theta)
    assert np.allclose(two, decode.rope(x, 42, theta), atol=1e-12)


def _loops_attention(qn, K, V, n):
    Hq, D = len(qn), len(qn[0])
    Hk = len(K[0])
    G = Hq // Hk
    out = []
    for j in range(Hq):
        h = j // G
        s = [math.fsum(qn[j][d] * K[p][h][d] for d in range(D)) / math.sqrt(D) for p in range(n)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        tot = math.fsum(e)
        out.append([math.fsum(e[p] * V[p][h][d] for p in range(n)) / tot for d in range(D)])
    return out


def test_attention_against_loops():
    rng = np.random.default_rng(4)
    Hq, Hk, D, S = 4, 2, 6, 9
    qn = rng.standard_normal((Hq, D))
    K, V = rng.standard_normal((S, Hk, D)), rng.standard_normal((S, Hk, D))
    for n in (1, 5, 9):
        got = decode.attention(qn, K, V, n)
        ref = _loops_attention(qn.tolist(), K.tolist(), V.tolist(), n)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    Hq, Hk, D, S = 4, 1, 8, 6
    K, V = rng.standard_normal((S, Hk, D)), rng.standard_normal((S, Hk, D))
    qn = rng.standard_normal((Hq, D))
    # one position: every head returns that value row
    assert np.allclose(decode.attention(qn, K, V, 1), np.repeat(V[0], Hq, axis=0))
    # zero query: uniform weights, the mean of the value rows
    assert np.allclose(decode.attention(np.zeros((Hq, D)), K, V, S), np.repeat(V[:, 0].mean(0)[None], Hq, 0))


def test_decode_step_appends_at_pos():
    rng = np.random.default_rng(6)
    B, Hq, Hk, D, S = 2, 4, 2, 8, 5
    q, k, v = rng.standard_normal((B, Hq, D)), rng.standard_normal((B, Hk, D)), rng.standard_normal((B, Hk, D))
    kc, vc = rng.standard_normal((B, S, Hk, D)), rng.standard_normal((B, S, Hk, D))
    pos = np.array([0, 3])
    kc0, vc0 = kc.copy(), vc.copy()
    qr, kr, out = decode.decode_step(q, k, v, np.ones(D), np.ones(D), pos, 1e4, 1e-6, kc, vc)
    # sequence 0 attends to its new token only
    for j in range(Hq):
        assert np.allclose(out[0, j], v[0, j // 2])
    # sequence 1: the appended key replaces position 3, earlier positions are the cache's
    K = kc[1, :4].copy(); K[3] = kr[1]
    V = vc[1, :4].copy(); V[3] = v[1]
    assert np.allclose(out[1], decode.attention(qr[1], K, V, 4))
    assert np.array_equal(kc, kc0) and np.array_equal(vc, vc0)   # inputs untouched
