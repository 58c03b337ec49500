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


def check_routing(aux, ref, k, inter, T, tile=-1, hidden=2048):
    """Integer outputs bit-exact (ids, counts, CSR offsets of rows and of the
    gate/up tasks of the tiling the call used, the permutation and its
    inverse); routing weights within 1e-5 of the largest."""
    assert np.array_equal(aux["ids"], ref["ids"]), "topk ids"
    assert np.array_equal(aux["counts"], ref["counts"]), "counts"
    assert np.array_equal(aux["tok_indptr"], ref["tok_indptr"]), "tok_indptr"
    assert np.array_equal(aux["perm"], ref["perm"]), "perm"
    assert np.array_equal(aux["inv"], ref["inv"]), "inv"
    rows, bn1, _ = moe_tiling(T, k, tile, hidden)
    assert np.array_equal(aux["task_indptr"], omoe.task_indptr(ref["counts"], rows, inter // bn1)), \
        "task_indptr"
    assert np.abs(aux["w"] - ref["w"]).max() <= 1e-5 * np.abs(ref["w"]).max(), "topk_w"


def check_against_oracle(name, T, out, aux, tile=-1):
    cfg = synth.MOE_PRESETS[name]
    ref = _oracle(name, T)
    check_routing(aux, ref, cfg["top_k"], cfg["inter"], T, tile, cfg["hidden"])
    assert_rel(out, ref["out"], 1e-2, "out")
    return ref


CASES = [("moe_small", 1), ("moe_small", 8), ("moe_small", 32),
         ("moe_skewed", 64), ("moe_skewed", 256), ("moe_skewed", 1024),
         ("moe_skewed_cal", 64), ("moe_skewed_cal", 256), ("moe_skewed_cal", 1024)]


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


def moe_tiling(T, k, tile=-1, hidden=2048):
    """(rows per block, h columns per gate/up task, columns per down task) of
    the library's tile variant for T tokens routed to k experts each (or the
    forced variant); the wide variants need a hidden size divisible by 256."""
    tv = tile if tile >= 0 else ((5 if T * k >= 16 else 0) if T <= 32 else
                                 2 if T * k <= 256 or hidden % 256 else 3 if T <= 512 else 4)
    return {0: (16, 16, 16), 1: (32, 16, 16), 2: (64, 16, 16), 3: (64, 128, 256),
            4: (128, 128, 256), 5: (16, 16, 64)}[tv]


@pytest.mark.parametrize("sched", ["static", "dynamic"])
@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("T", [64, 1024])
def test_tile_variants(tile, sched, T):
    _, _, _, _, out, aux, _ = run_moe("moe_skewed", T, sched, tile=tile)
    check_against_oracle("moe_skewed", T, out, aux, tile=tile)


@pytest.mark.parametrize("name,T", [("moe_small", 8), ("moe_small", 32), ("moe_skewed", 64),
                                    ("moe_skewed", 1024), ("moe_skewed_cal", 256)])
@pytest.mark.parametrize("tile", [-1, 3, 4])
@pytest.mark.parametrize("fetch,shards", [(1, 0), (8, 0), (2, 1)])
def test_static_order_queue(name, T, tile, fetch, shards):
    """Dynamic schedule with every GEMM task an implicit queue entry in the
    static order (claims of one entry whatever the fetch batch), on every tile
    kind, with per-XCD shards and with one central queue."""
    _, _, _, _, out, aux, _ = run_moe(name, T, "dynamic", queue_order="static", tile=tile,
                                      fetch_batch=fetch, queue_shards=shards)
    check_against_oracle(name, T, out, aux, tile)


@pytest.mark.parametrize("fetch", [1, 8])
def test_fetch_batches(fetch):
    _, _, _, _, out, aux, _ = run_moe("moe_skewed", 256, "dynamic", fetch_batch=fetch)
    check_against_oracle("moe_skewed", 256, out, aux)


@pytest.mark.parametrize("T", [16, 64, 256, 1024])
@pytest.mark.parametrize("sched", ["static", "dynamic", "dynamic_ready", "dynamic_static"])
def test_event_invariants(sched, T):
    """Each task ran once; the data-dependent expert events ended at their
    run-time wait counts (rows routed to each expert; dynamic, tasks pushed
    as they become ready: also the gate/up tiles over each expert's blocks),
    the block events (static schedule and the dynamic static-order queue) at
    the number of gate/up tiles of a block, and every combine tile's event at
    its rows times overlapping down tiles.  "dynamic" lets the scan choose
    the queue order: ready when one expert is chosen by at least 90% of the
    tokens and holds at least 4 row blocks, else static (the literal skew
    preset routes every token to one expert, so the choice flips between
    T = 64, one block, and T = 256)."""
    name = "moe_skewed"
    ws = _ws(name, 1024)
    ws.runs().zero_()
    order = {"dynamic": "auto", "dynamic_ready": "ready", "dynamic_static": "static"}.get(sched, "auto")
    if sched.startswith("dynamic"):
        sched = "dynamic"
    cfg, _, _, _, out, aux, _ = run_moe(name, T, sched, ws=ws, debug=et.DEBUG_COUNTS,
                                        queue_order=order)
    st = ws.status()
    E, k, H, I = cfg["n_experts"], cfg["top_k"], cfg["hidden"], cfg["inter"]
    nr = min(128, 8192 // E, -(-T // 8))   # routing chunks of about 8 tokens
    rows, bn1, bn2 = moe_tiling(T, k)
    cts = aux["counts"].astype(np.int64)
    mr = int(cts[-(-cts // rows) >= 4].max(initial=0))
    qstatic = order == "static" or (order == "auto" and not 10 * mr >= 9 * T)
    if order == "auto":
        assert qstatic == (T <= 64), (T, mr)
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
    if sched == "dynamic" and qstatic:
        # data-dependent rows per expert; down tiles wait on their block
        assert (cnt[ev_exp:ev_exp + E] == -tab["events"]["E_exp"]["wait_count"]).all()
        assert (cnt[ev_h:ev_h + nb] == -tab["events"]["E_h"]["wait_count"]).all()
        assert (cnt[ev_he:ev_he + E] == 0).all()
        assert cnt[1] == (-1 if nr >= 16 else 0) and cnt[2] == 0
    elif sched == "dynamic":
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


def _exact_case(k, mode, E=4, H=512, I=256, T=50, seed=0):
    """Integer experts whose every intermediate is exact: x in {0,1} with
    x[:,0] = 1, so the gate row 0 of W_gate sets g exactly; g >= 16 makes
    SiLU(g) equal g far below bf16 precision, so h = g*u and y = h Wd are
    exact whenever they are representable in bf16 (the layer rounds h and
    the down projection's rows y to bf16).

    mode "mixed": g in [16, 40), three +-1 entries per up column (|u| <= 3),
    two +-1 entries per down column (|y| <= 234).
    mode "up_dense": g = 16, the up projection dense in {-1, 0, 1} (every
    K-block of the gate/up tile contributes; h = 16 u), one +-1 entry per
    down column (y_j = +-h_i).
    mode "down_dense": g = 16, one +-1 entry per up column (h in {0, +-16}),
    the down projection dense in {-1, 0, 1} over I = 256 (y = 16 n with
    |n| <= 256, so every K-block of the down tile contributes exactly).

    Logits make the kept weights exactly 1 (k = 1) or 1/2 (two tied maxima,
    k = 2), so the combine is exact too."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randint(0, 2, (T, H), generator=g).float()
    x[:, 0] = 1
    wg = torch.zeros(E, H, I)
    if mode == "mixed":
        wg[:, 0, :] = torch.randint(16, 40, (E, I), generator=g).float()
    else:
        wg[:, 0, :] = 16.0
    wu = torch.zeros(E, H, I)
    if mode == "up_dense":
        wu[:, 1:, :] = torch.randint(-1, 2, (E, H - 1, I), generator=g).float()
    else:
        nu = 3 if mode == "mixed" else 1
        for e in range(E):
            for i in range(I):
                r = torch.randperm(H - 1, generator=g)[:nu] + 1
                wu[e, r, i] = torch.randint(0, 2, (nu,), generator=g).float() * 2 - 1
    wd = torch.zeros(E, I, H)
    if mode == "down_dense":
        wd[:] = torch.randint(-1, 2, (E, I, H), generator=g).float()
    else:
        nd = 2 if mode == "mixed" else 1
        for e in range(E):
            for j in range(H):
                r = torch.randperm(I, generator=g)[:nd]
                wd[e, r, j] = torch.randint(0, 2, (nd,), generator=g).float() * 2 - 1
    logits = torch.randn(T, E, generator=g) - 4.0
    for t in range(T):
        logits[t, torch.randperm(E, generator=g)[:k]] = 1.0   # ties between k distinct experts
    return x, wg, wu, wd, logits


def _bf16_exact(a):
    a = np.asarray(a, dtype=np.float64)
    return np.array_equal(torch.from_numpy(a).to(torch.bfloat16).double().numpy(), a)


@pytest.mark.parametrize("mode,T,tile", [
    ("mixed", 50, -1), ("up_dense", 50, -1), ("down_dense", 50, -1),
    ("mixed", 300, 3), ("up_dense", 300, 3), ("down_dense", 300, 3),
    ("mixed", 300, 4), ("up_dense", 300, 4), ("down_dense", 300, 4)])
@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_integer_exact(k, sched, mode, T, tile):
    """Bit-exact layer output on integer experts, through the stream tiles
    (T = 50: the 64-row variant) and the LDS-ring tiles forced (64 and 128
    rows: several row blocks per expert and a partial last block)."""
    x, wg, wu, wd, logits = _exact_case(k, mode, T=T)
    E, H, I = wg.shape[0], wg.shape[1], wg.shape[2]
    ws = et.Workspace(et.WL_MOE, 512, H, I, E, k, device=DEV)
    out = torch.full((T, H), float("nan"), device=DEV)
    dev = lambda t: t.to(torch.bfloat16).to(DEV)
    say("moe integer", k, sched, mode, T, tile)
    et.moe_layer(logits.to(DEV), dev(x), synth.k_major(dev(wg)), synth.k_major(dev(wu)),
                 synth.k_major(dev(wd)), out, ws, sched, tile=tile)
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
            assert gg.min() >= 16
            hh = gg * uu
            yy = hh @ wd[e].numpy()
            assert _bf16_exact(hh) and _bf16_exact(yy)   # the premise of exactness
            exact[t] += w[t, s] * yy
    assert np.array_equal(out.cpu().numpy(), exact.astype(np.float32))
    aux = {kk: v.cpu().numpy() for kk, v in et.moe_aux(ws, T).items()}
    check_routing(aux, ref, k, I, T, tile, hidden=H)
    if mode != "mixed":
        assert np.abs(exact).max() > 256      # beyond what the narrow case reaches


@pytest.mark.parametrize("tile", [3, 4])
def test_wide_tile_needs_hidden_multiple_of_256(tile):
    """A forced wide variant on a hidden size its 256-column down tiles do not
    divide is refused before any launch; the automatic choice falls back to
    the 64-row stream variant and matches the oracle."""
    T, E, k, H, I = 300, 4, 2, 384, 256
    ws = et.Workspace(et.WL_MOE, 512, H, I, E, k, device=DEV)
    logits = synth.normal_bf16((T, E), 1.0, 5, DEV).float()
    x = synth.normal_bf16((T, H), 1.0, 6, DEV)
    wg = synth.normal_bf16((E, H, I), 0.02, 7, DEV)
    wu = synth.normal_bf16((E, H, I), 0.02, 8, DEV)
    wd = synth.normal_bf16((E, I, H), 0.02, 9, DEV)
    out = torch.full((T, H), float("nan"), device=DEV)
    args = (logits, x, synth.k_major(wg), synth.k_major(wu), synth.k_major(wd), out, ws)
    with pytest.raises(et.EtError) as err:
        et.moe_layer(*args, "static", tile=tile)
    assert err.value.code == et.EUNSUPPORTED
    say("moe H=384 automatic tile")
    et.moe_layer(*args, "dynamic")
    torch.cuda.synchronize()
    assert ws.status()["status"] == 0
    ref = omoe.moe_layer(to_np(logits), to_np(x), k, (to_np(wg), to_np(wu), to_np(wd)))
    aux = {kk: v.cpu().numpy() for kk, v in et.moe_aux(ws, T).items()}
    check_routing(aux, ref, k, I, T, hidden=H)
    assert moe_tiling(T, k, hidden=H)[:2] == (64, 16)
    assert_rel(out.cpu().numpy(), ref["out"], 1e-2, "out")


_TIE_VALUES = np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 1.0], np.float32)


@pytest.mark.parametrize("E,k", [(5, 1), (5, 3), (8, 2), (16, 3), (16, 1)])
@pytest.mark.parametrize("T", [64, 200])
@pytest.mark.parametrize("sched", SCHEDS)
def test_routing_ties_and_signed_zeros(E, k, T, sched):
    """Logits drawn from {-1, -0.0, +0.0, 0.5, 1}: most tokens have ties that
    straddle the k-th place and zeros of both signs.  The GPU's order-preserving
    keys must pick exactly the oracle's experts (descending logit, ties to the
    lower index, -0.0 equal to +0.0), and the grouping built on them must be
    bit-exact.  T = 200 routes in 25 chunks (broadcast events, chunk 0
    publishes the scan), T = 64 in 8; E = 5 is not a multiple of 4."""
    H, I = 256, 256
    rng = np.random.default_rng(1000 * E + 10 * k + T)
    L = rng.choice(_TIE_VALUES, size=(T, E)).astype(np.float32)
    n_tie_k = sum(1 for t in range(T) if k < E and
                  np.float32(sorted(L[t], reverse=True)[k - 1]) == sorted(L[t], reverse=True)[k])
    assert n_tie_k >= T // 4                 # the boundary ties are really exercised
    assert (np.signbit(L) & (L == 0)).any() and ((~np.signbit(L)) & (L == 0)).any()
    logits = torch.from_numpy(L).to(DEV)
    x = synth.normal_bf16((T, H), 1.0, 11, DEV)
    wg = synth.normal_bf16((E, H, I), 0.02, 12, DEV)
    wu = synth.normal_bf16((E, H, I), 0.02, 13, DEV)
    wd = synth.normal_bf16((E, I, H), 0.02, 14, DEV)
    ws = _ws_dims(256, H, I, E, k)
    out = torch.full((T, H), float("nan"), device=DEV)
    say("moe routing ties", E, k, T, sched)
    et.moe_layer(logits, x, synth.k_major(wg), synth.k_major(wu), synth.k_major(wd), out, ws, sched)
    torch.cuda.synchronize()
    assert ws.status()["status"] == 0
    ref = omoe.moe_layer(L, to_np(x), k, (to_np(wg), to_np(wu), to_np(wd)))
    aux = {kk: v.cpu().numpy() for kk, v in et.moe_aux(ws, T).items()}
    check_routing(aux, ref, k, I, T, hidden=H)
    assert_rel(out.cpu().numpy(), ref["out"], 1e-2, "out")


@functools.lru_cache(maxsize=4)
def _ws_dims(max_tokens, H, I, E, k):
    return et.Workspace(et.WL_MOE, max_tokens, H, I, E, k, device=DEV)


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


@pytest.mark.parametrize("sched", ["static", "dynamic", "barrier"])
def test_watchdog_timeout_is_reported(sched):
    """A one-tick watchdog (forced from the host, checked at every poll) makes
    the first wait not satisfied at its first poll end the call: the device records ET_ETIMEOUT, every
    workgroup leaves (the call completes), later calls do nothing until the
    workspace is re-initialised, and then the layer matches the oracle again."""
    ws = et.Workspace(et.WL_MOE, 1024, 2048, 768, 128, 8, device=DEV)
    cfg, logits, x, (wg, wu, wd), _, _, _ = run_moe("moe_skewed", 1024, sched, ws=ws)
    out = torch.zeros((1024, cfg["hidden"]), device=DEV)
    say("moe watchdog tick", sched)
    et.moe_layer(logits, x, wg, wu, wd, out, ws, sched, debug=et.DEBUG_WATCHDOG_TICK)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == et.ETIMEOUT, st
    calls = st["calls"]
    et.moe_layer(logits, x, wg, wu, wd, out, ws, sched)       # sticky: no work done
    torch.cuda.synchronize()
    assert ws.status()["status"] == et.ETIMEOUT and ws.status()["calls"] == calls
    ws.init()
    _, _, _, _, out2, aux, _ = run_moe("moe_skewed", 1024, sched, ws=ws)
    check_against_oracle("moe_skewed", 1024, out2, aux)


@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_clock_stamps(sched):
    """ET_DEBUG_CLOCK records every workgroup's start / end stamps (real time
    and shader clock) and no per-task records; the output is unchanged, and
    the clock the stamps give lies in the device's range."""
    name, T = "moe_skewed", 256
    ws = _ws(name, 1024)
    tr, _ = ws.trace()
    tr.zero_()
    cfg, logits, x, (wg, wu, wd), out, aux, _ = run_moe(name, T, sched, ws=ws, debug=et.DEBUG_CLOCK)
    G = et.num_workers()
    st = ws.clock_stamps()[:G].cpu().long()
    d_rt = (st[:, 1, 0] - st[:, 0, 0]) & 0xFFFFFFFF
    d_sc = (st[:, 1, 1] - st[:, 0, 1]) & 0xFFFFFFFF
    assert (d_rt > 0).all() and (d_sc > 0).all()
    ghz = float(d_sc.sum()) / float(d_rt.sum()) * 0.1
    assert 0.3 < ghz < 3.0, ghz
    assert int(tr.abs().sum()) == 0                     # no per-task records
    check_against_oracle(name, T, out, aux)
