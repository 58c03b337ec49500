"""Host-side checks of the C ABI (no GPU needed: no compute call is made)."""

import ctypes

import pytest

from event_driven_moe_amd import et


def test_library_exports_every_declared_symbol():
    L = et.lib()
    names = et.header_functions()
    assert {"et_splitk_reduce", "et_mlp", "et_moe_layer", "et_plan_workspace",
            "et_workspace_init", "et_read_status"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in range(7):
        assert et.status_str(code)
    assert "unknown" in et.status_str(99)


def test_plan_validation():
    with pytest.raises(et.EtError) as e:
        et.plan_workspace(et.WL_SPLITK, 33)
    assert e.value.code == et.EUNSUPPORTED
    with pytest.raises(et.EtError) as e:
        et.plan_workspace(et.WL_MLP, 4, 2048, 1000)          # I not a multiple of 128
    assert e.value.code == et.EUNSUPPORTED
    with pytest.raises(et.EtError) as e:
        et.plan_workspace(et.WL_MOE, 4, 2048, 768, 8, 9)     # top_k > E
    assert e.value.code == et.EINVAL
    with pytest.raises(et.EtError) as e:
        et.plan_workspace(99, 4)
    assert e.value.code == et.EINVAL


def test_plan_layout_is_consistent():
    for args in ((et.WL_SPLITK, 2048), (et.WL_MLP, 64, 2048, 5632),
                 (et.WL_MOE, 1024, 2048, 768, 128, 8), (et.WL_MOE, 8192, 7168, 2048, 256, 8)):
        p = et.plan_workspace(*args)
        assert p.off_counters >= 1024
        assert p.off_slots >= p.off_counters + 2 * 4 * p.n_events
        assert p.off_runs >= p.off_slots + 4 * p.max_tasks
        assert p.off_aux >= p.off_runs + 4 * p.max_tasks
        assert p.bytes >= p.off_aux + p.aux_bytes
        for off in (p.off_counters, p.off_slots, p.off_runs, p.off_aux, p.bytes):
            assert off % 256 == 0


def test_call_errors_enqueue_nothing():
    # Argument errors are reported synchronously, before any device work:
    # a null workspace and a wrong workload are rejected without touching HIP.
    L = et.lib()
    p = et.plan_workspace(et.WL_SPLITK, 64)
    r = L.et_splitk_reduce(None, 64, None, None, None, ctypes.byref(p), 0, None, None)
    assert r == et.EWORKSPACE
    pm = et.plan_workspace(et.WL_MLP, 4, 256, 256)
    r = L.et_splitk_reduce(None, 64, None, None, ctypes.c_void_p(256), ctypes.byref(pm), 0,
                           None, None)
    assert r == et.EWORKSPACE


def test_option_errors_enqueue_nothing():
    # Out-of-range options are rejected before any HIP call: queue order,
    # claim batch, queue shards and tile variant.
    L = et.lib()
    p = et.plan_workspace(et.WL_MOE, 64, 2048, 768, 128, 8)
    fake_ws = ctypes.c_void_p(256)   # aligned, never dereferenced on the host
    for kw in ({"queue_order": "static"}, {"fetch_batch": 9}, {"queue_shards": 3}, {"tile": 99}):
        o = et._opts(**kw)
        if "queue_order" in kw:
            o.queue_order = 7
        r = L.et_moe_layer(None, None, 8, None, None, None, None, fake_ws, ctypes.byref(p),
                           et.SCHED_DYNAMIC, ctypes.byref(o), None)
        assert r == et.EINVAL, (kw, r)
