"""GPU parity at the large MoE layer's full size (hidden 7168, 256 experts,
top-8, intermediate 2048: 22.5 GB of expert weights) in the launch
configuration the benchmark uses.  Routing and grouping over all T tokens
are compared bit-exactly with the oracle; the layer output is compared on
sampled tokens (the fp64 oracle evaluates one token's 8 experts at a time)."""

import numpy as np
import pytest
import torch

from event_driven_moe_amd import et, synth
from oracle import moe as omoe
from gpu_helpers import DEV, say, assert_rel, to_np, moe_weights, moe_oracle_weights

pytestmark = pytest.mark.gpu

NAME = "moe_large"


@pytest.fixture(scope="module")
def ws():
    cfg = synth.MOE_PRESETS[NAME]
    return et.Workspace(et.WL_MOE, max(cfg["tokens"]), cfg["hidden"], cfg["inter"],
                        cfg["n_experts"], cfg["top_k"], device=DEV)


@pytest.mark.parametrize("sched", ["static", "dynamic"])
@pytest.mark.parametrize("T", [512, 2048, 8192])
def test_full_size_sampled(ws, T, sched):
    cfg = synth.MOE_PRESETS[NAME]
    k, E = cfg["top_k"], cfg["n_experts"]
    wg, wu, wd = moe_weights(NAME)
    logits, x = synth.moe_activations(cfg, T, device=DEV)
    out = torch.full((T, cfg["hidden"]), float("nan"), device=DEV)
    say("moe_large", T, sched)
    et.moe_layer(logits, x, wg, wu, wd, out, ws, sched)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == 0, st
    aux = {kk: v.cpu().numpy() for kk, v in et.moe_aux(ws, T).items()}

    ids, w = omoe.route(to_np(logits), k)
    g = omoe.group(ids, E)
    assert np.array_equal(aux["ids"], ids), "topk ids"
    for key in ("counts", "tok_indptr", "perm", "inv"):
        assert np.array_equal(aux[key], g[key]), key
    assert np.abs(aux["w"] - w).max() <= 1e-5 * np.abs(w).max(), "topk_w"

    # sampled tokens: two random ones and one routed to the most loaded expert
    rng = np.random.default_rng(T)
    hot = int(np.argmax(g["counts"]))
    t_hot = int(g["perm"][g["tok_indptr"][hot]] // k)
    sample = np.unique(np.concatenate([rng.choice(T, 2, replace=False), [t_hot]]))
    ref = omoe.experts_and_combine(to_np(x), ids, w, moe_oracle_weights(wg, wu, wd),
                                   tokens=sample)
    got = out[torch.as_tensor(sample, device=DEV)].cpu().numpy()
    assert np.isfinite(got).all()
    assert_rel(got, ref, 1e-2, "out (sampled tokens %s)" % sample.tolist())
