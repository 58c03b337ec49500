"""GPU parity: dense SiLU-gated MLP chain vs the oracle."""

import numpy as np
import pytest
import torch

from event_driven_moe_amd import et, synth
from oracle import mlp as om, events as oev
from gpu_helpers import DEV, SCHEDS, say, assert_rel, to_np

pytestmark = pytest.mark.gpu

H, I = 2048, 5632


@pytest.fixture(scope="module")
def weights():
    _, wg, wu, wd = synth.mlp_inputs(1, H, I, device=DEV)
    return wg, wu, wd, synth.k_major(wg), synth.k_major(wu), synth.k_major(wd)


@pytest.fixture(scope="module")
def ws():
    return et.Workspace(et.WL_MLP, 64, H, I, device=DEV)


def _run(ws, x, wgT, wuT, wdT, sched, **opts):
    y = torch.full((x.shape[0], H), float("nan"), device=DEV)
    say("mlp", sched, tuple(x.shape), opts)
    et.mlp(x, wgT, wuT, wdT, y, ws, sched, **opts)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == 0, st
    return y.cpu().numpy()


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("B", [1, 4, 16, 64])
def test_parity(ws, weights, sched, B):
    wg, wu, wd, wgT, wuT, wdT = weights
    x = synth.mlp_inputs(B, H, I, device=DEV)[0]
    y = _run(ws, x, wgT, wuT, wdT, sched)
    ref = om.mlp(to_np(x), to_np(wg), to_np(wu), to_np(wd))
    assert_rel(y, ref, 1e-2, "y")


@pytest.mark.parametrize("B", [3, 17, 33, 63])
def test_ragged_batches(ws, weights, B):
    wg, wu, wd, wgT, wuT, wdT = weights
    x = synth.normal_bf16((B, H), 1.0, 900 + B, DEV)
    y = _run(ws, x, wgT, wuT, wdT, "static")
    ref = om.mlp(to_np(x), to_np(wg), to_np(wu), to_np(wd))
    assert_rel(y, ref, 1e-2, "y")


@pytest.mark.parametrize("tile", [0, 1, 2])
def test_integer_exact_layout(ws, tile):
    """Small-integer operands: g >= 16 makes SiLU(g) = g to far below bf16
    precision, so h = g*u exactly (|g*u| < 256) and y = h Wd is an exact
    integer in fp32.  Any slip in tiling, indexing or layout breaks equality."""
    g = torch.Generator(device="cpu").manual_seed(3)
    B, Hs, Is = 40, 256, 384
    x = torch.randint(0, 2, (B, Hs), generator=g).float()
    x[:, 0] = 1.0
    wg = torch.zeros(Hs, Is)
    wg[0, :] = torch.randint(16, 40, (Is,), generator=g).float()      # g = 16..39
    wu = torch.zeros(Hs, Is)                                          # |u| <= 6
    for i in range(Is):
        rows = torch.randperm(Hs - 1, generator=g)[:6] + 1
        wu[rows, i] = torch.randint(0, 2, (6,), generator=g).float() * 2 - 1
    wd = torch.randint(-2, 3, (Is, Hs), generator=g).float()
    ws2 = et.Workspace(et.WL_MLP, 64, Hs, Is, device=DEV)
    xd, wgd, wud, wdd = (t.to(torch.bfloat16).to(DEV) for t in (x, wg, wu, wd))
    y = torch.full((B, Hs), float("nan"), device=DEV)
    say("mlp integer", tile)
    et.mlp(xd, synth.k_major(wgd), synth.k_major(wud), synth.k_major(wdd), y, ws2, "static",
           tile=tile)
    torch.cuda.synchronize()
    yo, go, uo, ho = om.mlp(x.numpy(), wg.numpy(), wu.numpy(), wd.numpy(), return_intermediates=True)
    assert np.abs(go * uo).max() < 256 and go.min() >= 16
    exact = (go * uo) @ wd.numpy().astype(np.float64)         # h = g*u exactly in bf16
    assert np.array_equal(y.cpu().numpy(), exact.astype(np.float32))
    # the oracle itself agrees to SiLU's distance from the identity at g >= 16
    assert np.abs(yo - exact).max() <= 1e-5 * max(1.0, np.abs(exact).max())


def test_modes_bit_identical(ws, weights):
    wg, wu, wd, wgT, wuT, wdT = weights
    x = synth.normal_bf16((16, H), 1.0, 77, DEV)
    outs = [_run(ws, x, wgT, wuT, wdT, s) for s in SCHEDS]
    for y in outs[1:]:
        assert np.array_equal(y, outs[0])


def test_invariants(ws, weights):
    """Each task ran exactly once and every E_h counter ended at its wait
    count, both as the oracle's event table states for the library's tiling
    (rows per block 16/32/64 for B <= 16/32/64, 16-column gate/up and down
    tiles, one event per 128-column h tile, the down tile covering all of K)."""
    wg, wu, wd, wgT, wuT, wdT = weights
    for B, sched in ((64, "static"), (5, "dynamic"), (16, "static"), (33, "dynamic")):
        ws.runs().zero_()
        x = synth.normal_bf16((B, H), 1.0, B, DEV)
        _run(ws, x, wgT, wuT, wdT, sched, debug=et.DEBUG_COUNTS)
        st = ws.status()
        rows = 16 if B <= 16 else (32 if B <= 32 else 64)
        tab = oev.mlp_table(B, H, I, rows, 16, 128, 16, 1)
        ntask = sum(tab["tasks"].values())
        assert st["last_tasks"] == ntask
        runs = ws.runs().cpu().numpy()
        assert (runs[:ntask] == 1).all() and (runs[ntask:] == 0).all()
        cnt = ws.counters(1 - st["bank"]).cpu().numpy()
        wc = tab["events"]["E_h"]["wait_count"].reshape(-1)
        assert (cnt[:wc.size] == -wc).all() and (cnt[wc.size:-1] == 0).all()


@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_cooperative_launch(ws, weights, sched):
    """The cooperative launch mode runs the same kernel: same results."""
    wg, wu, wd, wgT, wuT, wdT = weights
    x = synth.mlp_inputs(16, H, I, device=DEV)[0]
    y0 = _run(ws, x, wgT, wuT, wdT, sched)
    y1 = _run(ws, x, wgT, wuT, wdT, sched, cooperative=True)
    assert np.array_equal(y0, y1)
    assert_rel(y1, om.mlp(to_np(x), to_np(wg), to_np(wu), to_np(wd)), 1e-2, "y")
