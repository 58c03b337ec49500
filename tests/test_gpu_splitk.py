"""GPU parity: split-K two-stage reduction vs the oracle, all schedule modes."""

import numpy as np
import pytest
import torch

from event_driven_moe_amd import et, synth
from oracle import splitk as osk, events as oev
from gpu_helpers import DEV, SCHEDS, say, assert_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ws():
    return et.Workspace(et.WL_SPLITK, 2048, device=DEV)


def _run(ws, A, sched, **opts):
    rows = A.shape[0]
    B = torch.full((rows, 4), float("nan"), device=DEV)
    C = torch.full((rows,), float("nan"), device=DEV)
    say("splitk", sched, rows, opts)
    et.splitk_reduce(A, B, C, ws, sched, **opts)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == 0, st
    return B.cpu().numpy(), C.cpu().numpy()


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("rows", [32, 96, 2048])
def test_parity_uniform(ws, sched, rows):
    A = synth.splitk_inputs(rows=rows, seed=101, device=DEV)
    B, C = _run(ws, A, sched)
    Bref, Cref = osk.splitk_reduce(A.cpu().numpy())
    assert_rel(B, Bref, 1e-5, "B")
    assert_rel(C, Cref, 1e-5, "C")


@pytest.mark.parametrize("sched", SCHEDS)
def test_integer_inputs_bit_exact(ws, sched):
    A = synth.splitk_inputs(rows=2048, seed=111, device=DEV, integer=True)
    B, C = _run(ws, A, sched)
    Bref, Cref = osk.splitk_reduce(A.cpu().numpy())
    assert np.array_equal(B, Bref) and np.array_equal(C, Cref)


def test_modes_bit_identical(ws):
    A = synth.splitk_inputs(rows=2048, seed=5, device=DEV)
    outs = [_run(ws, A, s) for s in SCHEDS]
    for B, C in outs[1:]:
        assert np.array_equal(B, outs[0][0]) and np.array_equal(C, outs[0][1])


@pytest.mark.parametrize("sched", ["static", "dynamic", "barrier"])
def test_event_invariants(ws, sched):
    """Every task runs once; every counter of the used bank ends at its wait count
    (stored relative to it: -wait_count); unused events stay armed (0)."""
    for rows in (2048, 320, 64):       # symbolic shape: n changes between calls
        n = rows // 32
        ws.runs().zero_()
        A = synth.splitk_inputs(rows=rows, seed=rows, device=DEV)
        st0 = ws.status()
        B, C = _run(ws, A, sched, debug=et.DEBUG_COUNTS)
        st = ws.status()
        assert st["calls"] == st0["calls"] + 1
        used = 1 - st["bank"]
        cnt = ws.counters(used).cpu().numpy()
        runs = ws.runs().cpu().numpy()
        tab = oev.splitk_table(rows)
        assert (runs[:5 * n] == 1).all() and (runs[5 * n:] == 0).all()
        assert runs[:5 * n].sum() == sum(tab["tasks"].values())
        if sched == "barrier":
            assert cnt[2048 // 32] == -4 * n and (cnt[:64] == 0).all()
        else:
            assert (cnt[:n] == -tab["events"]["E"]["wait_count"]).all()
            assert (cnt[n:64] == 0).all()
        assert st["q_head"] == 0 and st["q_push"] == 0
        Bref, Cref = osk.splitk_reduce(A.cpu().numpy())
        assert_rel(C, Cref, 1e-5, "C")


@pytest.mark.parametrize("fetch", [1, 2, 8])
def test_dynamic_fetch_batches(ws, fetch):
    A = synth.splitk_inputs(rows=2048, seed=9, device=DEV)
    B, C = _run(ws, A, "dynamic", fetch_batch=fetch)
    _, Cref = osk.splitk_reduce(A.cpu().numpy())
    assert_rel(C, Cref, 1e-5, "C")


def test_bad_rows_rejected(ws):
    A = torch.zeros((48, 128), device=DEV)
    with pytest.raises(et.EtError) as e:
        et.splitk_reduce(A, torch.zeros((48, 4), device=DEV), torch.zeros(48, device=DEV), ws)
    assert e.value.code == et.EUNSUPPORTED
    A = torch.zeros((4096, 128), device=DEV)
    with pytest.raises(et.EtError) as e:
        et.splitk_reduce(A, torch.zeros((4096, 4), device=DEV), torch.zeros(4096, device=DEV), ws)
    assert e.value.code == et.EWORKSPACE


@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_cooperative_launch(ws, sched):
    """The cooperative launch mode runs the same kernel: same results."""
    A = synth.splitk_inputs(rows=2048, seed=12, device=DEV)
    B0, C0 = _run(ws, A, sched)
    B1, C1 = _run(ws, A, sched, cooperative=True)
    assert np.array_equal(B0, B1) and np.array_equal(C0, C1)
    _, Cref = osk.splitk_reduce(A.cpu().numpy())
    assert_rel(C1, Cref, 1e-5, "C")


def test_central_queue(ws):
    """One central ready queue instead of one shard per XCD: same results."""
    A = synth.splitk_inputs(rows=2048, seed=13, device=DEV)
    B8, C8 = _run(ws, A, "dynamic")
    B1, C1 = _run(ws, A, "dynamic", queue_shards=1)
    assert np.array_equal(C8, C1) and np.array_equal(B8, B1)


def test_init_leaves_queue_total_unknown(ws):
    """et_workspace_init writes every header word exactly once: the ready
    queue's task total (header word 160) reads "unknown" (INT32_MAX) after
    init, so the first dynamic call's workers wait for pushed slots instead
    of giving up claimed ones (a stray zero there would leave stage-2 rows
    unwritten).  Init, check the word, then a dynamic call against the
    oracle, several times over."""
    A = synth.splitk_inputs(rows=2048, seed=121, device=DEV, integer=True)
    Bref, Cref = osk.splitk_reduce(A.cpu().numpy())
    for _ in range(8):
        ws.init()
        torch.cuda.synchronize()
        hdr = ws.view(0, torch.int32, 256).cpu()
        assert int(hdr[160]) == 0x7FFFFFFF
        B, C = _run(ws, A, "dynamic")
        assert np.array_equal(B, Bref) and np.array_equal(C, Cref)
