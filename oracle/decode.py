"""Oracle: one decode step's attention front -- query and key branches,
cache append and attention (test infrastructure only).

Follows Event Tensor notes, section "端到端低 batch serving": the megakernel
covers the decoding pipeline (attention, RoPE, KV cache, norm), and one of
the cross-operator optimisations it names is running the query branch's
Norm + RoPE in parallel with the key branch's Norm + RoPE + cache append.
The models it serves are Qwen3 (30B-A3B, 32B), whose attention normalises
each query and key head before the rotary embedding.

Readings taken where the pages are silent (each also listed in the design doc):

* Norm is RMSNorm over one head's D elements with a learned weight:
  n(x) = x / sqrt(mean(x^2) + eps) * w;
* RoPE rotates element pairs (i, i + D/2) by the angle pos * theta^(-2i/D)
  (the half-split pairing of the Qwen / NeoX layout);
* the new token of sequence b sits at position pos[b]: its rotated key and
  its value are appended at that index of the cache, which already holds
  positions 0 .. pos[b]-1;
* grouped-query attention: query head j reads key/value head j // G with
  G = Hq / Hk; scores are scaled by 1 / sqrt(D); softmax over positions
  0 .. pos[b] inclusive; the output is the probability-weighted sum of the
  value rows.

Everything is float64 from the exact input values.

Pins (tests/test_oracle_decode.py): RMSNorm closed forms; RoPE against the
complex-multiplication form of the same rotation, its identity at position
0, norm preservation per pair and additivity of angles; attention against
explicit loops, a single cached position (output = the value row) and
uniform scores (output = the mean of the value rows).
"""

import numpy as np


def rms_norm(x, w, eps):
    """x[..., D] / sqrt(mean(x^2) + eps) * w, float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * w


def rope(x, pos, theta):
    """Rotate pairs (i, i + D/2) of x[..., D] by pos * theta^(-2i/D); pos
    broadcasts against x's leading dimensions."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    inv = float(theta) ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(qn, K, V, n):
    """One sequence: qn [Hq, D]; K, V [S, Hk, D] (positions 0..n-1 used).
    Returns [Hq, D]."""
    Hq, D = qn.shape
    Hk = K.shape[1]
    G = Hq // Hk
    out = np.zeros((Hq, D))
    for j in range(Hq):
        h = j // G
        s = K[:n, h] @ qn[j] / np.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        out[j] = p @ V[:n, h]
    return out


def decode_step(q, k, v, wq, wk, pos, theta, eps, k_cache, v_cache):
    """q [B, Hq, D], k and v [B, Hk, D], wq / wk [D], pos [B] int, caches
    [B, S, Hk, D].  Returns (q_rot [B, Hq, D], k_rot [B, Hk, D], out
    [B, Hq, D]) in float64; the caches passed in are not modified."""
    pos = np.asarray(pos, dtype=np.int64)
    qn = rope(rms_norm(q, wq, eps), pos[:, None], theta)
    kn = rope(rms_norm(k, wk, eps), pos[:, None], theta)
    B = qn.shape[0]
    out = np.zeros(qn.shape)
    for b in range(B):
        p = int(pos[b])
        K = np.array(k_cache[b, :p + 1], dtype=np.float64)
        V = np.array(v_cache[b, :p + 1], dtype=np.float64)
        K[p] = kn[b]
        V[p] = np.asarray(v[b], dtype=np.float64)
        out[b] = attention(qn[b], K, V, p + 1)
    return qn, kn, out
