"""Pins for the MoE oracle (CPU only)."""

import itertools
import math

import numpy as np
import torch

from oracle import moe, mlp as om, events
from event_driven_moe_amd import synth


def _brute_topk(row, k):
    """Exhaustive search: the ordered k-tuple of distinct experts whose key
    sequence (-logit, index) is lexicographically smallest."""
    best, best_key = None, None
    for tup in itertools.permutations(range(len(row)), k):
        key = [(-float(row[e]) + 0.0, e) for e in tup]   # + 0.0 folds -0.0
        if best_key is None or key < best_key:
            best, best_key = tup, key
    return list(best)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(11)
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 1.0], np.float32)
    for E in (3, 4, 5, 6):
        for k in range(1, min(E, 3) + 1):
            L = rng.choice(vals, size=(20, E)).astype(np.float32)
            ids, _ = moe.route(L, k)
            for t in range(20):
                assert list(ids[t]) == _brute_topk(L[t], k), (E, k, L[t])


def test_signed_zero_ties_to_lower_index():
    ids, _ = moe.route(np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32), 1)
    assert ids[:, 0].tolist() == [0, 0]


def test_renormalised_weights_closed_form():
    # kept logits ln 3 and 0 -> weights 3/4 and 1/4 whatever the dropped logits are
    L = np.array([[math.log(3.0), 0.0, -5.0, -7.0]], np.float32)
    ids, w = moe.route(L, 2)
    assert ids.tolist() == [[0, 1]]
    l0 = float(np.float32(math.log(3.0)))
    assert abs(w[0, 0] - math.exp(l0) / (math.exp(l0) + 1)) < 1e-15
    assert abs(w[0, 0] - 0.75) < 1e-7
    # general: softmax restricted to the kept logits
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 16)).astype(np.float32)
    ids, w = moe.route(L, 4)
    for t in range(50):
        kept = [float(L[t, e]) for e in ids[t]]
        z = [math.exp(v - max(kept)) for v in kept]
        ref = [v / math.fsum(z) for v in z]
        assert np.allclose(w[t], ref, rtol=1e-14, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-14
        assert all(w[t, s] >= w[t, s + 1] for s in range(3))


def test_k_equals_E_and_k_one():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((10, 6)).astype(np.float32)
    ids, w = moe.route(L, 6)
    for t in range(10):
        p = np.exp(L[t].astype(np.float64) - L[t].max())
        p /= p.sum()
        assert np.allclose(w[t], p[ids[t]], rtol=1e-14, atol=0)
        assert sorted(ids[t].tolist()) == list(range(6))
    ids, w = moe.route(L, 1)
    assert (w == 1.0).all()
    assert (ids[:, 0] == L.argmax(axis=1)).all()


def test_grouping_invariants_and_brute_force():
    rng = np.random.default_rng(9)
    for T, E, k in ((1, 4, 2), (7, 5, 3), (33, 8, 2), (64, 16, 4)):
        L = rng.standard_normal((T, E)).astype(np.float32)
        ids, _ = moe.route(L, k)
        g = moe.group(ids, E)
        assert g["counts"].sum() == T * k
        assert g["tok_indptr"][0] == 0 and g["tok_indptr"][-1] == T * k
        assert sorted(g["perm"].tolist()) == list(range(T * k))
        flat = ids.reshape(-1)
        brute = [t * k + s for e in range(E) for t in range(T) for s in range(k) if ids[t, s] == e]
        assert g["perm"].tolist() == brute
        for e in range(E):
            seg = g["perm"][g["tok_indptr"][e]:g["tok_indptr"][e + 1]]
            assert (flat[seg] == e).all()
            assert (np.diff(seg // k) > 0).all()        # ascending tokens
        for t in range(T):
            for s in range(k):
                assert g["perm"][g["inv"][t, s]] == t * k + s


def test_task_indptr_brute_force():
    counts = np.array([0, 1, 16, 17, 40, 0, 3])
    for bm, nt in ((16, 1), (16, 11), (64, 2)):
        ip = moe.task_indptr(counts, bm, nt)
        tasks = [(e, b, n) for e in range(len(counts)) for b in range(-(-counts[e] // bm))
                 for n in range(nt)]
        assert ip[-1] == len(tasks)
        for e in range(len(counts)):
            assert ip[e + 1] - ip[e] == sum(1 for t in tasks if t[0] == e)
        tab = events.moe_table(counts, bm, nt * 16, 16, 32, 32, 4)
        assert tab["tasks"]["gate_up"] == ip[-1]
        assert (tab["events"]["E_exp"]["wait_count"] == counts).all()
        # E_he[e]: one notify per gate/up task of expert e (brute-force count)
        he = events.notify_counts([(t, t[0]) for t in tasks], (len(counts),))
        assert (tab["events"]["E_he"]["wait_count"] == he).all()
        assert tab["events"]["E_he"]["wait_count"].sum() == tab["tasks"]["gate_up"]


def test_combine_group_events_brute_force():
    """E_cg[g, c]: enumerate every (routed row, down tile, combine tile)
    triple whose columns overlap and count the notifies per combine tile."""
    rng = np.random.default_rng(3)
    for T, k, H, dc, cc in ((37, 3, 512, 256, 64), (50, 2, 256, 16, 64), (16, 8, 768, 64, 256),
                            (1, 1, 320, 64, 256)):
        E = max(6, k + 1)
        ids, _ = moe.route(rng.standard_normal((T, E)).astype(np.float32), k)
        counts = np.bincount(ids.reshape(-1), minlength=E)
        tab = events.moe_table(counts, 16, 64, 16, H, dc, 2, tokens=T, top_k=k, comb_tok=16,
                               comb_cols=cc)
        pairs = []
        for t in range(T):
            for s in range(k):
                for n2 in range(H // dc):
                    for c in range(-(-H // cc)):
                        if n2 * dc < min(H, (c + 1) * cc) and c * cc < (n2 + 1) * dc:
                            pairs.append(((t, s, n2), (t // 16, c)))
        cg = events.notify_counts(pairs, tab["events"]["E_cg"]["shape"])
        assert (tab["events"]["E_cg"]["wait_count"] == cg).all()
        assert cg.sum() == T * k * (H // dc) * max(1, dc // cc)


def _rand_experts(rng, E, H, I):
    return (rng.standard_normal((E, H, I)) * 0.3, rng.standard_normal((E, H, I)) * 0.3,
            rng.standard_normal((E, I, H)) * 0.3)


def test_k1_is_argmax_expert():
    rng = np.random.default_rng(12)
    T, E, H, I = 9, 5, 6, 4
    L = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, H))
    W = _rand_experts(rng, E, H, I)
    r = moe.moe_layer(L, x, 1, W)
    for t in range(T):
        e = int(L[t].argmax())
        assert np.allclose(r["out"][t], om.mlp(x[t:t + 1], W[0][e], W[1][e], W[2][e])[0],
                           rtol=1e-13, atol=1e-13)


def test_identical_experts_reduce_to_dense_mlp():
    rng = np.random.default_rng(13)
    T, E, k, H, I = 11, 6, 3, 8, 5
    L = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, H))
    wg, wu, wd = rng.standard_normal((H, I)), rng.standard_normal((H, I)), rng.standard_normal((I, H))
    W = (np.stack([wg] * E), np.stack([wu] * E), np.stack([wd] * E))
    r = moe.moe_layer(L, x, k, W)
    assert np.allclose(r["out"], om.mlp(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


def test_zero_expert_drops_out():
    # With one of the two kept experts zeroed, out = w_other * y_other.
    rng = np.random.default_rng(14)
    T, E, H, I = 5, 4, 6, 3
    L = np.tile(np.array([2.0, 1.0, -3.0, -4.0], np.float32), (T, 1))
    x = rng.standard_normal((T, H))
    W = list(_rand_experts(rng, E, H, I))
    for m in W:
        m[1] = 0.0
    r = moe.moe_layer(L, x, 2, W)
    w0 = 1.0 / (1.0 + math.exp(-1.0))
    ref = w0 * om.mlp(x, W[0][0], W[1][0], W[2][0])
    assert np.allclose(r["out"], ref, rtol=1e-13, atol=1e-13)


def test_sampled_tokens_match_full():
    cfg = dict(synth.MOE_SMALL, hidden=64, inter=32)
    logits, x = synth.moe_activations(cfg, 10)
    wg, wu, wd = zip(*[synth.moe_expert_weights(cfg, e) for e in range(cfg["n_experts"])])
    W = tuple(torch.stack(m).float().numpy() for m in (wg, wu, wd))
    full = moe.moe_layer(logits.numpy(), x.float().numpy(), 2, W)
    part = moe.moe_layer(logits.numpy(), x.float().numpy(), 2,
                         lambda e: (W[0][e], W[1][e], W[2][e]), tokens=[7, 2, 9])
    # equal up to the BLAS's fp64 rounding order (row blocking differs)
    assert np.allclose(part["out"], full["out"][[7, 2, 9]], rtol=1e-13, atol=1e-16)
    assert full["n_active"] == int((full["counts"] > 0).sum())
