"""The allocation-free MoE entry point (library-held scratch array) against
the workspace entry point: same kernels, so the outputs and routing results
must be identical, on consecutive calls whose token counts shrink and grow
(the scratch keeps the last call's state between them)."""

import ctypes

import numpy as np
import pytest
import torch

from event_driven_moe_amd import et, synth
from gpu_helpers import DEV, say, moe_weights

pytestmark = pytest.mark.gpu


def _both(name, T, sched, ws):
    cfg = synth.MOE_PRESETS[name]
    wg, wu, wd = moe_weights(name)
    logits, x = synth.moe_activations(cfg, T, device=DEV)
    out_ws = torch.full((T, cfg["hidden"]), float("nan"), device=DEV)
    out_na = torch.full((T, cfg["hidden"]), float("nan"), device=DEV)
    say("moe noalloc", name, T, sched)
    et.moe_layer(logits, x, wg, wu, wd, out_ws, ws, sched)
    et.moe_layer_noalloc(logits, x, wg, wu, wd, out_na, sched, top_k=cfg["top_k"])
    torch.cuda.synchronize()
    assert ws.status()["status"] == 0
    return out_ws.cpu().numpy(), out_na.cpu().numpy()


@pytest.mark.parametrize("sched", ["dynamic", "static"])
@pytest.mark.parametrize("name,sizes", [("moe_skewed", (256, 64, 1024, 1)),
                                        ("moe_small", (32, 8, 1))])
def test_noalloc_matches_workspace_entry(name, sizes, sched):
    cfg = synth.MOE_PRESETS[name]
    ws = et.Workspace(et.WL_MOE, max(sizes), cfg["hidden"], cfg["inter"], cfg["n_experts"],
                      cfg["top_k"], device=DEV)
    for T in sizes:          # the second call is smaller than the first
        a, b = _both(name, T, sched, ws)
        assert np.isfinite(a).all()
        assert np.array_equal(a, b), (name, T, sched)


def test_noalloc_rejects_oversized_layer():
    """A layer whose workspace exceeds the 64 MiB scratch is refused before
    anything is enqueued (the pointers are never read)."""
    L = et.lib()
    dummy = torch.zeros(16, device=DEV)
    p = ctypes.c_void_p(dummy.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    r = L.et_moe_layer_noalloc(p, p, 4096, 7168, 2048, 256, 8, p, p, p, p, 1, None, s)
    assert r == et.EWORKSPACE
    r = L.et_moe_layer_noalloc(p, p, -1, 7168, 2048, 256, 8, p, p, p, p, 1, None, s)
    assert r == et.EINVAL
    torch.cuda.synchronize()
    assert (dummy == 0).all()


def test_noalloc_reset_flag():
    """ET_SCRATCH_RESET clears the scratch state before the call; the result
    is unchanged."""
    name, T = "moe_skewed", 64
    cfg = synth.MOE_PRESETS[name]
    wg, wu, wd = moe_weights(name)
    logits, x = synth.moe_activations(cfg, T, device=DEV)
    outs = []
    for flags in (0, et.SCRATCH_RESET, 0):
        out = torch.full((T, cfg["hidden"]), float("nan"), device=DEV)
        et.moe_layer_noalloc(logits, x, wg, wu, wd, out, "dynamic", top_k=cfg["top_k"],
                             debug=flags)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
