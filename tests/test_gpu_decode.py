"""GPU parity: the decode attention front (query and key branches, cache
append, grouped-query attention) in one launch vs the oracle.

Shapes are Qwen3-32B's attention (64 query heads, 8 key/value heads, head
dimension 128) and Qwen3-30B-A3B's (32 / 4), with ragged cache lengths:
positions drawn per sequence, the extremes 0 (an empty cache) and
max_seq - 1 (a full one) always among them, and the pages' serving mix
(512-token prompts, up to 100 generated tokens)."""

import functools

import numpy as np
import pytest
import torch

from event_driven_moe_amd import et, synth
from oracle import decode as odec
from gpu_helpers import DEV, SCHEDS, say, assert_rel, to_np

pytestmark = pytest.mark.gpu

THETA, EPS, S = 1e6, 1e-6, 1024


@functools.lru_cache(maxsize=4)
def _ws(Hq, Hk):
    return et.Workspace(et.WL_DECODE, 64, device=DEV, n_heads=Hq, n_kv_heads=Hk, head_dim=128)


def inputs(B, Hq, Hk, mix="uniform", seed=0):
    D = 128
    q = synth.normal_bf16((B, Hq, D), 1.0, 800 + seed, DEV)
    k = synth.normal_bf16((B, Hk, D), 1.0, 801 + seed, DEV)
    v = synth.normal_bf16((B, Hk, D), 1.0, 802 + seed, DEV)
    wq = (1.0 + synth.normal_bf16((D,), 0.1, 803 + seed, DEV).float()).to(torch.bfloat16)
    wk = (1.0 + synth.normal_bf16((D,), 0.1, 804 + seed, DEV).float()).to(torch.bfloat16)
    kc = synth.normal_bf16((B, S, Hk, D), 1.0, 805 + seed, DEV)
    vc = synth.normal_bf16((B, S, Hk, D), 1.0, 806 + seed, DEV)
    g = torch.Generator(device="cpu").manual_seed(807 + seed)
    if mix == "serving":
        pos = torch.randint(512, 612, (B,), generator=g)
    else:
        pos = torch.randint(0, S, (B,), generator=g)
    pos[0] = 0
    if B > 1:
        pos[-1] = S - 1
    return q, k, v, wq, wk, pos.to(torch.int32).to(DEV), kc, vc


def run(B, Hq, Hk, sched, mix="uniform", seed=0, **opts):
    q, k, v, wq, wk, pos, kc, vc = inputs(B, Hq, Hk, mix, seed)
    kc0, vc0 = kc.clone(), vc.clone()
    out = torch.full((B, Hq, 128), float("nan"), device=DEV)
    ws = _ws(Hq, Hk)
    say("decode", B, Hq, Hk, sched, mix, opts)
    et.decode_attention(q, k, v, wq, wk, pos, kc, vc, out, ws, sched, rope_theta=THETA, eps=EPS,
                        **opts)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == 0, st
    qr = et.decode_q_rot(ws, B).cpu().numpy()
    return (q, k, v, wq, wk, pos, kc0, vc0), (kc, vc, out.cpu().numpy(), qr)


def check(inp, res):
    q, k, v, wq, wk, pos, kc0, vc0 = inp
    kc, vc, out, qr = res
    P = pos.cpu().numpy()
    rq, rk, rout = odec.decode_step(to_np(q), to_np(k), to_np(v), to_np(wq), to_np(wk), P,
                                    THETA, EPS, to_np(kc0), to_np(vc0))
    # fp32 angles: |error| <= 2 * pos * 2^-24 rad per pair, far below 1e-3 of the values
    assert_rel(qr, rq, 1e-3, "rotated queries")
    b = np.arange(len(P))
    knew, vnew = to_np(kc[b, P]), to_np(vc[b, P])
    # the appended key is rounded to bf16: within half an ulp of bf16 plus the fp32 error
    assert (np.abs(knew - rk) <= 2.0 ** -8 * np.abs(rk) + 1e-3 * np.abs(rk).max()).all(), "key append"
    assert np.array_equal(vnew, to_np(v)), "value append"
    keep = torch.ones(kc.shape[:2], dtype=torch.bool)
    keep[b, P] = False
    assert torch.equal(kc[keep.to(DEV)], kc0[keep.to(DEV)]) and torch.equal(vc[keep.to(DEV)], vc0[keep.to(DEV)])
    assert_rel(out, rout, 1e-2, "attention")
    return rout


CASES = [(1, 64, 8, "uniform"), (8, 64, 8, "uniform"), (64, 64, 8, "serving"),
         (64, 64, 8, "uniform"), (16, 32, 4, "uniform"), (5, 32, 2, "uniform")]


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("B,Hq,Hk,mix", CASES)
def test_decode_parity(B, Hq, Hk, mix, sched):
    inp, res = run(B, Hq, Hk, sched, mix)
    check(inp, res)


def test_decode_schedules_bit_identical():
    outs = [run(16, 64, 8, s, seed=3)[1][2] for s in SCHEDS]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_decode_event_invariants(sched):
    """Every task ran once; every E_qk event received its two notifies (one
    from each branch) and every E_att event one per attention split (24
    sequences x 8 heads = 192 pairs on 256 workgroups: one split; 2
    sequences: 16 pairs, 8 splits of 128 positions)."""
    for B, NS in ((24, 1), (2, 8)):
        _invariants(B, NS, sched)


def _invariants(B, NS, sched):
    Hq, Hk = 64, 8
    assert et.num_workers() == 256
    ws = _ws(Hq, Hk)
    ws.runs().zero_()
    inp, res = run(B, Hq, Hk, sched, debug=et.DEBUG_COUNTS)
    st = ws.status()
    N = B * Hk
    total = 2 * N + N * NS + N
    runs = ws.runs().cpu().numpy()
    assert st["last_tasks"] == total
    assert (runs[:total] == 1).all() and (runs[total:] == 0).all()
    cnt = ws.counters(1 - st["bank"]).cpu().numpy()
    assert (cnt[8:8 + N] == -2).all() and (cnt[8 + N:8 + 2 * N] == -NS).all()
    assert (cnt[:8] == 0).all()
    check(inp, res)


def test_decode_position_out_of_range_is_reported():
    """A position at or past the cache length is refused by the kernel's own
    bounds check: the call records ET_ERANGE (sticky until re-init), writes
    no cache row, and the workspace works again after et_workspace_init."""
    B, Hq, Hk = 4, 64, 8
    q, k, v, wq, wk, pos, kc, vc = inputs(B, Hq, Hk, seed=5)
    pos[2] = S
    kc0 = kc.clone()
    out = torch.zeros((B, Hq, 128), device=DEV)
    ws = _ws(Hq, Hk)
    et.decode_attention(q, k, v, wq, wk, pos, kc, vc, out, ws, "static", rope_theta=THETA, eps=EPS)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == et.ERANGE and st["err_info"][1] == 2 and st["err_info"][2] == S
    assert torch.equal(kc[2], kc0[2])
    ws.init()
    inp, res = run(B, Hq, Hk, "static", seed=5)
    check(inp, res)
