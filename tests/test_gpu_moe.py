"""GPU parity: the MoE layer vs the oracle (small and skewed layers)."""

import functools

import numpy as np
import pytest
import torch

from event_driven_moe_amd import et, synth
from oracle import moe as omoe, events as oev
from gpu_helpers import DEV, SCHEDS, say, assert_rel, to_np, moe_weights, moe_oracle_weights

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=4)
def _ws(name, max_tokens):
    cfg = synth.MOE_PRESETS[name]
    return et.Workspace(et.WL_MOE, max_tokens, cfg["hidden"], cfg["inter"], cfg["n_experts"],
                        cfg["top_k"], device=DEV)


def run_moe(name, T, sched, ws=None, **opts):
    cfg = synth.MOE_PRESETS[name]
    wg, wu, wd = moe_weights(name)
    logits, x = synth.moe_activations(cfg, T, device=DEV)
    ws = ws or _ws(name, max(cfg["tokens"]))
    out = torch.full((T, cfg["hidden"]), float("nan"), device=DEV)
    say("moe", name, T, sched, opts)
    et.moe_layer(logits, x, wg, wu, wd, out, ws, sched, **opts)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == 0, st
    aux = {k: v.cpu().numpy() for k, v in et.moe_aux(ws, T).items()}
    return cfg, logits, x, (wg, wu, wd), out.cpu().numpy(), aux, ws


@functools.lru_cache(maxsize=8)
def _oracle(name, T):
    cfg = synth.MOE_PRESETS[name]
    wg, wu, wd = moe_weights(name)
    logits, x = synth.moe_activations(cfg, T, device=DEV)
    return omoe.moe_layer(to_np(logits), to_np(x), cfg["top_k"], moe_oracle_weights(wg, wu, wd))


def check_against_oracle(name, T, out, aux):
    ref = _oracle(name, T)
    assert np.array_equal(aux["ids"], ref["ids"]), "topk ids"
    assert np.array_equal(aux["counts"], ref["counts"]), "counts"
    assert np.array_equal(aux["tok_indptr"], ref["tok_indptr"]), "tok_indptr"
    assert np.array_equal(aux["perm"], ref["perm"]), "perm"
    assert np.array_equal(aux["inv"], ref["inv"]), "inv"
    assert np.abs(aux["w"] - ref["w"]).max() <= 1e-5 * np.abs(ref["w"]).max(), "topk_w"
    assert_rel(out, ref["out"], 1e-2, "out")
    return ref


CASES = [("moe_small", 1), ("moe_small", 8), ("moe_small", 32),
         ("moe_skewed", 64), ("moe_skewed", 256), ("moe_skewed", 1024)]


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("name,T", CASES)
def test_parity(name, T, sched):
    _, _, _, _, out, aux, _ = run_moe(name, T, sched)
    check_against_oracle(name, T, out, aux)


@pytest.mark.parametrize("name,T", [("moe_small", 32), ("moe_skewed", 256)])
def test_modes_bit_identical(name, T):
    outs = [run_moe(name, T, s)[4] for s in SCHEDS]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def moe_tiling(T, k, tile=-1):
    """(rows per block, h columns per gate/up task, columns per down task) of
    the library's tile variant for T tokens routed to k experts each (or the
    forced variant)."""
    tv = tile if tile >= 0 else ((5 if T * k >= 16 else 0) if T <= 32 else 2 if T * k <= 256 else
                                 3 if T <= 512 else 4)
    return {0: (16, 16, 16), 1: (32, 16, 16), 2: (64, 16, 16), 3: (64, 128, 256),
            4: (128, 128, 256), 5: (16, 16, 64)}[tv]


@pytest.mark.parametrize("sched", ["static", "dynamic"])
@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("T", [64, 1024])
def test_tile_variants(tile, sched, T):
    _, _, _, _, out, aux, _ = run_moe("moe_skewed", T, sched, tile=tile)
    check_against_oracle("moe_skewed", T, out, aux)


@pytest.mark.parametrize("fetch", [1, 8])
def test_fetch_batches(fetch):
    _, _, _, _, out, aux, _ = run_moe("moe_skewed", 256, "dynamic", fetch_batch=fetch)
    check_against_oracle("moe_skewed", 256, out, aux)


@pytest.mark.parametrize("T", [16, 64, 256, 1024])
@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_event_invariants(sched, T):
    """Each task ran once; the data-dependent expert events ended at their
    run-time wait counts (rows routed to each expert; dynamic: also the
    gate/up tiles over each expert's blocks), the static schedule's block
    events at the number of gate/up tiles of a block, and every combine
    tile's event at its rows times overlapping down tiles."""
    name = "moe_skewed"
    ws = _ws(name, 1024)
    ws.runs().zero_()
    cfg, _, _, _, out, aux, _ = run_moe(name, T, sched, ws=ws, debug=et.DEBUG_COUNTS)
    st = ws.status()
    E, k, H, I = cfg["n_experts"], cfg["top_k"], cfg["hidden"], cfg["inter"]
    nr = min(128, 8192 // E, -(-T // 8))   # routing chunks of about 8 tokens
    rows, bn1, bn2 = moe_tiling(T, k)
    ccols = 256 if -(-T // 16) * -(-H // 256) >= et.num_workers() else 64
    tab = oev.moe_table(aux["counts"], rows, I, bn1, H, bn2, nr, tokens=T, top_k=k,
                        comb_tok=16, comb_cols=ccols)
    ncomb = -(-T // 16) * -(-H // ccols)   # combine tiles of 16 tokens x ccols columns
    total = sum(tab["tasks"].values()) + ncomb
    runs = ws.runs().cpu().numpy()
    assert (runs[:total] == 1).all() and (runs[total:] == 0).all()
    cnt = ws.counters(1 - st["bank"]).cpu().numpy()
    assert cnt[0] == -nr                                   # all routing tasks notified
    ev_exp, ev_he, ev_h = 8, 8 + E, 8 + 2 * E
    ev_c = ev_h + -(-1024 * k // 16) + E                   # after the block events (T_max 1024)
    nb = tab["blocks"]
    cg = tab["events"]["E_cg"]
    ncg = int(np.prod(cg["shape"]))
    if sched == "static" and T >= 256 and tab["tasks"]["down"] <= 4 * et.num_workers():
        # shallow down phase: every combine tile waited on its own event
        assert cnt[4] == 0
        assert (cnt[ev_c:ev_c + ncg] == -cg["wait_count"].reshape(-1)).all()
    else:
        assert cnt[4] == -tab["tasks"]["down"]            # all down tiles done
        assert (cnt[ev_c:ev_c + ncg] == 0).all()
    if sched == "dynamic":
        # data-dependent: rows per expert, and gate/up tiles over its blocks
        assert (cnt[ev_exp:ev_exp + E] == -tab["events"]["E_exp"]["wait_count"]).all()
        assert (cnt[ev_he:ev_he + E] == -tab["events"]["E_he"]["wait_count"]).all()
        assert (cnt[ev_h:ev_h + nb] == 0).all()
        # chunk 0 fires the scan event for the other chunks' pushes
        assert cnt[1] == (-1 if nr >= 16 else 0) and cnt[2] == 0
    else:
        assert (cnt[ev_h:ev_h + nb] == -tab["events"]["E_h"]["wait_count"]).all()
        assert (cnt[ev_he:ev_he + E] == 0).all()
        assert cnt[1] == -1 and cnt[2] == -nr
    check_against_oracle(name, T, out, aux)


def _exact_case(k, E=4, H=256, I=256, T=50, seed=0):
    """Integer experts: x in {0,1} with x[:,0]=1; gate row 0 in [16,40) so
    SiLU(g) == g below bf16 precision; |u| <= 3, so h = g*u exactly (|h| <=
    117); two +-1 entries per down column, so every y is an integer with
    |y| <= 234, exact in bf16 (the layer keeps y, the down projection's rows,
    in bf16 like h).  Logits make the kept weights exactly 1 (k = 1) or 1/2
    (two tied maxima, k = 2)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randint(0, 2, (T, H), generator=g).float()
    x[:, 0] = 1
    wg = torch.zeros(E, H, I)
    wg[:, 0, :] = torch.randint(16, 40, (E, I), generator=g).float()
    wu = torch.zeros(E, H, I)
    for e in range(E):
        for i in range(I):
            r = torch.randperm(H - 1, generator=g)[:3] + 1
            wu[e, r, i] = torch.randint(0, 2, (3,), generator=g).float() * 2 - 1
    wd = torch.zeros(E, I, H)
    for e in range(E):
        for j in range(H):
            r = torch.randperm(I, generator=g)[:2]
            wd[e, r, j] = torch.randint(0, 2, (2,), generator=g).float() * 2 - 1
    logits = torch.randn(T, E, generator=g) - 4.0
    for t in range(T):
        logits[t, torch.randperm(E, generator=g)[:k]] = 1.0   # ties between k distinct experts
    return x, wg, wu, wd, logits


@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_integer_exact(k, sched):
    x, wg, wu, wd, logits = _exact_case(k)
    E, H, I = wg.shape[0], wg.shape[1], wg.shape[2]
    T = x.shape[0]
    ws = et.Workspace(et.WL_MOE, 64, H, I, E, k, device=DEV)
    out = torch.full((T, H), float("nan"), device=DEV)
    dev = lambda t: t.to(torch.bfloat16).to(DEV)
    say("moe integer", k, sched)
    et.moe_layer(logits.to(DEV), dev(x), synth.k_major(dev(wg)), synth.k_major(dev(wu)),
                 synth.k_major(dev(wd)), out, ws, sched)
    torch.cuda.synchronize()
    assert ws.status()["status"] == 0
    ref = omoe.moe_layer(logits.numpy(), x.numpy(), k, (wg.numpy(), wu.numpy(), wd.numpy()))
    ids, w = ref["ids"], ref["w"]
    assert set(np.unique(w).tolist()) <= {1.0, 0.5}
    exact = np.zeros((T, H))
    for t in range(T):
        for s in range(k):
            e = ids[t, s]
            gg = x[t].numpy().astype(np.float64) @ wg[e].numpy()
            uu = x[t].numpy().astype(np.float64) @ wu[e].numpy()
            exact[t] += w[t, s] * ((gg * uu) @ wd[e].numpy())
    assert np.array_equal(out.cpu().numpy(), exact.astype(np.float32))
    aux = {kk: v.cpu().numpy() for kk, v in et.moe_aux(ws, T).items()}
    assert np.array_equal(aux["ids"], ids) and np.array_equal(aux["perm"], ref["perm"])


def test_symbolic_token_counts_one_workspace():
    """One workspace, token counts changing call to call (and the tile variant
    with them): every call still matches the oracle."""
    ws = _ws("moe_skewed", 1024)
    for T in (64, 1, 1024, 17, 33):
        for sched in ("dynamic", "static"):
            _, _, _, _, out, aux, _ = run_moe("moe_skewed", T, sched, ws=ws)
            check_against_oracle("moe_skewed", T, out, aux)


def test_schedules_interleaved_one_workspace():
    """All four schedules in turn on one workspace, with the token count
    changing: the coarse events' broadcast flags hold the generation of the
    call that fired them, which grows with every call except the
    per-operator baseline's (it runs no epilogue and waits on no event), so
    a flag left by an earlier call must never pass for a fired event.  With
    64 and 32 routing chunks (T=1024, 256) the routing event is a broadcast
    event too; with 8 (T=64) it is polled on its counter."""
    ws = _ws("moe_skewed", 1024)
    seq = [("static", 1024), ("per_op", 256), ("static", 256), ("barrier", 1024),
           ("per_op", 64), ("barrier", 64), ("dynamic", 1024), ("static", 1024),
           ("per_op", 1024), ("dynamic", 256), ("static", 64)]
    calls0 = ws.status()["calls"]
    for sched, T in seq:
        _, _, _, _, out, aux, _ = run_moe("moe_skewed", T, sched, ws=ws)
        check_against_oracle("moe_skewed", T, out, aux)
    assert ws.status()["calls"] == calls0 + sum(s != "per_op" for s, _ in seq)


@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_cooperative_launch(sched):
    """The cooperative launch mode runs the same kernel: same results."""
    _, _, _, _, out0, aux0, _ = run_moe("moe_skewed", 256, sched)
    _, _, _, _, out1, aux1, _ = run_moe("moe_skewed", 256, sched, cooperative=True)
    assert np.array_equal(out0, out1)
    check_against_oracle("moe_skewed", 256, out1, aux1)


@pytest.mark.parametrize("T", [64, 1024])
def test_central_queue(T):
    """One central ready queue instead of one shard per XCD: same results."""
    _, _, _, _, out8, aux8, _ = run_moe("moe_skewed", T, "dynamic")
    _, _, _, _, out1, aux1, _ = run_moe("moe_skewed", T, "dynamic", queue_shards=1)
    assert np.array_equal(out8, out1)
    check_against_oracle("moe_skewed", T, out1, aux1)
