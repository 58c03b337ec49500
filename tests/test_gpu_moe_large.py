"""GPU parity at the large MoE layer's full size (hidden 7168, 256 experts,
top-8, intermediate 2048: 22.5 GB of expert weights) in the launch
configuration the benchmark uses.

Routing and grouping over all T tokens are compared bit-exactly with the
oracle.  The layer output is compared on a token sample that covers every
row block of the grouped GEMMs: for each expert's row blocks (64 rows at
T = 512, 128 rows from T = 2048 on) at least one token with a row in the
block is checked, the last row of each block first, so every expert's
partial last block is among them; since whole output rows are compared,
every gate/up and down column tile of each block is covered.  At T = 512
every token is compared.  The fp64 oracle evaluates each expert once per T
and the result serves every schedule."""

import numpy as np
import pytest
import torch

from event_driven_moe_amd import et, synth
from oracle import moe as omoe
from gpu_helpers import DEV, say, assert_rel, to_np, moe_weights, moe_oracle_weights

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

NAME = "moe_large"
_REF = {}


@pytest.fixture(scope="module")
def ws():
    cfg = synth.MOE_PRESETS[NAME]
    return et.Workspace(et.WL_MOE, max(cfg["tokens"]), cfg["hidden"], cfg["inter"],
                        cfg["n_experts"], cfg["top_k"], device=DEV)


def block_cover(g, k, rows):
    """Tokens such that every row block (rows per block ``rows``) of every
    expert segment holds a row of one of them; returns (tokens, blocks)."""
    counts, tip, perm, inv = g["counts"], g["tok_indptr"], g["perm"], g["inv"]
    first_blk = np.concatenate([[0], np.cumsum(-(-counts // rows))])

    def block_of(pos):
        e = np.searchsorted(tip, pos, side="right") - 1
        return first_blk[e] + (pos - tip[e]) // rows

    covered = np.zeros(first_blk[-1], dtype=bool)
    chosen = []
    for e in np.nonzero(counts)[0]:
        for b in range(-(-int(counts[e]) // rows)):
            if covered[first_blk[e] + b]:
                continue
            last = min(tip[e] + (b + 1) * rows, tip[e + 1]) - 1
            t = int(perm[last]) // k
            chosen.append(t)
            covered[block_of(inv[t])] = True
    assert covered.all()
    return np.array(sorted(set(chosen))), int(first_blk[-1])


def reference(T):
    if T not in _REF:
        cfg = synth.MOE_PRESETS[NAME]
        k, E = cfg["top_k"], cfg["n_experts"]
        wg, wu, wd = moe_weights(NAME)
        logits, x = synth.moe_activations(cfg, T, device=DEV)
        ids, w = omoe.route(to_np(logits), k)
        g = omoe.group(ids, E)
        rows = 64 if T <= 512 else 128
        if T <= 512:
            sample, nblk = np.arange(T), None
        else:
            sample, nblk = block_cover(g, k, rows)
        say("oracle moe_large T=%d: %d tokens (%s row blocks)" % (T, len(sample), nblk))
        out = omoe.experts_and_combine(to_np(x), ids, w, moe_oracle_weights(wg, wu, wd),
                                       tokens=sample)
        _REF[T] = (ids, w, g, sample, out)
    return _REF[T]


# "dynamic" takes the queue order the library picks (tasks pushed as they
# become ready at T = 512, the static-order queue from T = 2048 on);
# "dynamic_ready" / "dynamic_static" force one order.
@pytest.mark.parametrize("T", [512, 2048, 8192])
@pytest.mark.parametrize("sched", ["static", "dynamic", "barrier", "per_op", "dynamic_ready",
                                   "dynamic_static"])
def test_full_size_block_cover(ws, T, sched):
    cfg = synth.MOE_PRESETS[NAME]
    wg, wu, wd = moe_weights(NAME)
    logits, x = synth.moe_activations(cfg, T, device=DEV)
    out = torch.full((T, cfg["hidden"]), float("nan"), device=DEV)
    say("moe_large", T, sched)
    if sched.startswith("dynamic_"):
        et.moe_layer(logits, x, wg, wu, wd, out, ws, "dynamic", queue_order=sched[8:])
    else:
        et.moe_layer(logits, x, wg, wu, wd, out, ws, sched)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == 0, st
    aux = {kk: v.cpu().numpy() for kk, v in et.moe_aux(ws, T).items()}

    ids, w, g, sample, ref = reference(T)
    assert np.array_equal(aux["ids"], ids), "topk ids"
    for key in ("counts", "tok_indptr", "perm", "inv"):
        assert np.array_equal(aux[key], g[key]), key
    rows, bn1 = (64, 128) if T <= 512 else (128, 128)
    assert np.array_equal(aux["task_indptr"],
                          omoe.task_indptr(g["counts"], rows, cfg["inter"] // bn1)), "task_indptr"
    assert np.abs(aux["w"] - w).max() <= 1e-5 * np.abs(w).max(), "topk_w"
    got = out[torch.as_tensor(sample, device=DEV)].cpu().numpy()
    assert np.isfinite(got).all()
    assert_rel(got, ref, 1e-2, "out (%d tokens)" % len(sample))
    if T == 512:
        assert np.isfinite(out.cpu().numpy()).all()


@pytest.mark.parametrize("T", [2048, 8192])
@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_full_size_event_invariants(ws, T, sched):
    """At the benchmark's sizes (about 12,000 and 33,000 tasks): every task
    ran exactly once, every row block's E_h ended at its gate/up tiles (both
    schedules: the dynamic schedule takes the static-order queue here), every
    expert's E_exp at its routed rows (dynamic), and EV_DOWN at the number of
    down tiles."""
    cfg = synth.MOE_PRESETS[NAME]
    H, I, E, k = cfg["hidden"], cfg["inter"], cfg["n_experts"], cfg["top_k"]
    wg, wu, wd = moe_weights(NAME)
    logits, x = synth.moe_activations(cfg, T, device=DEV)
    out = torch.empty((T, H), device=DEV)
    ws.runs().zero_()
    say("moe_large invariants", T, sched)
    et.moe_layer(logits, x, wg, wu, wd, out, ws, sched, debug=et.DEBUG_COUNTS)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == 0, st
    counts = et.moe_aux(ws, T)["counts"].cpu().numpy().astype(np.int64)
    nr = min(128, 8192 // E, -(-T // 8))
    rows, nt1, nt2 = 128, I // 128, H // 256
    nb = int((-(-counts // rows)).sum())
    ccols = 1024 if -(-T // 16) * -(-H // 1024) >= 4 * et.num_workers() else 256
    ncomb = -(-T // 16) * -(-H // ccols)
    total = 2 * nr + 1 + nb * (nt1 + nt2) + ncomb
    runs = ws.runs().cpu().numpy()
    assert (runs[:total] == 1).all() and (runs[total:] == 0).all()
    cnt = ws.counters(1 - st["bank"]).cpu().numpy()
    ev_exp, ev_he, ev_h = 8, 8 + E, 8 + 2 * E
    assert cnt[0] == -nr
    assert cnt[4] == -nb * nt2
    assert (cnt[ev_h:ev_h + nb] == -nt1).all()
    assert (cnt[ev_he:ev_he + E] == 0).all()
    if sched == "dynamic":
        assert (cnt[ev_exp:ev_exp + E] == -counts).all()
    else:
        assert (cnt[ev_exp:ev_exp + E] == 0).all() and cnt[2] == -nr
