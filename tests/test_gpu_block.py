"""GPU parity: the router GEMM -> MoE layer -> dense MLP chain in one launch
vs the oracle, at the small and skewed MoE layers' shapes with the dense
MLP workload's intermediate size (5632).

The router logits are compared against the fp64 oracle within the error
bound of fp32 accumulation; the routing decision is then taken on the GPU's
fp32 logits on both sides, so ids, counts and the permutation are compared
bit-exactly; the MoE output z and the dense MLP output y within
1e-2 * max|ref| (bf16 inputs, fp32 accumulation, h and the MLP input
rounded to bf16)."""

import functools

import numpy as np
import pytest
import torch

from event_driven_moe_amd import et, synth
from oracle import block as oblock, moe as omoe
from gpu_helpers import DEV, SCHEDS, say, assert_rel, to_np, moe_weights, moe_oracle_weights

pytestmark = pytest.mark.gpu

IM = 5632
ROUTER_STD = 0.02


@functools.lru_cache(maxsize=1)
def mlp_weights():
    _, wg, wu, wd = synth.mlp_inputs(1, 2048, IM, device=DEV)
    return wg, wu, wd, synth.k_major(wg), synth.k_major(wu), synth.k_major(wd)


@functools.lru_cache(maxsize=2)
def router_weights(E):
    return synth.normal_bf16((2048, E), ROUTER_STD, 700 + E, DEV)


@functools.lru_cache(maxsize=2)
def _ws(name):
    cfg = synth.MOE_PRESETS[name]
    return et.Workspace(et.WL_BLOCK, max(cfg["tokens"]), cfg["hidden"], cfg["inter"],
                        cfg["n_experts"], cfg["top_k"], device=DEV, mlp_inter=IM)


def run_block(name, T, sched, **opts):
    cfg = synth.MOE_PRESETS[name]
    wg, wu, wd = moe_weights(name)
    _, _, _, mgT, muT, mdT = mlp_weights()
    wr = router_weights(cfg["n_experts"])
    _, x = synth.moe_activations(cfg, T, device=DEV)
    ws = _ws(name)
    z = torch.full((T, cfg["hidden"]), float("nan"), device=DEV)
    y = torch.full((T, cfg["hidden"]), float("nan"), device=DEV)
    say("block", name, T, sched, opts)
    et.moe_block(x, synth.k_major(wr), wg, wu, wd, mgT, muT, mdT, z, y, ws, sched, **opts)
    torch.cuda.synchronize()
    st = ws.status()
    assert st["status"] == 0, st
    aux = {k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy()
           for k, v in et.block_aux(ws, T).items()}
    return cfg, x, wr, z.cpu().numpy(), y.cpu().numpy(), aux


def check(name, T, x, wr, z, y, aux):
    cfg = synth.MOE_PRESETS[name]
    wg, wu, wd = moe_weights(name)
    mg, mu, md, _, _, _ = mlp_weights()
    X, WR = to_np(x).astype(np.float64), to_np(wr).astype(np.float64)
    ref = oblock.block(X, WR, cfg["top_k"], moe_oracle_weights(wg, wu, wd),
                       (to_np(mg), to_np(mu), to_np(md)), route_logits=aux["logits"])
    # fp32 accumulation of H products: |err| <= H * 2^-23 * sum_h |x w|
    bound = X.shape[1] * 2.0 ** -23 * (np.abs(X) @ np.abs(WR))
    assert (np.abs(aux["logits"] - ref["logits"]) <= bound).all(), "router logits"
    for key in ("ids", "counts", "tok_indptr", "perm", "inv"):
        assert np.array_equal(aux[key], ref[key]), key
    assert np.abs(aux["w"] - ref["w"]).max() <= 1e-5 * np.abs(ref["w"]).max(), "topk_w"
    assert_rel(z, ref["z"], 1e-2, "moe out")
    assert np.array_equal(aux["z"], torch.from_numpy(z).to(torch.bfloat16).float().numpy()), \
        "bf16 copy of the MoE output"
    assert_rel(y, ref["y"], 1e-2, "mlp out")


CASES = [("moe_small", 1), ("moe_small", 8), ("moe_small", 32),
         ("moe_skewed", 64), ("moe_skewed", 256)]


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("name,T", CASES)
def test_block_parity(name, T, sched):
    _, x, wr, z, y, aux = run_block(name, T, sched)
    check(name, T, x, wr, z, y, aux)


@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_block_parity_1024(sched):
    _, x, wr, z, y, aux = run_block("moe_skewed", 1024, sched)
    check("moe_skewed", 1024, x, wr, z, y, aux)


@pytest.mark.parametrize("name,T", [("moe_small", 8), ("moe_skewed", 1024)])
def test_block_static_order_queue(name, T):
    """The chain under the dynamic schedule with the MoE GEMM tasks queued at
    the scan in the static order."""
    _, x, wr, z, y, aux = run_block(name, T, "dynamic", queue_order="static")
    check(name, T, x, wr, z, y, aux)


@pytest.mark.parametrize("name,T", [("moe_small", 8), ("moe_skewed", 256)])
def test_block_schedules_bit_identical(name, T):
    outs = [run_block(name, T, s)[3:5] for s in SCHEDS]
    for z, y in outs[1:]:
        assert np.array_equal(z, outs[0][0]) and np.array_equal(y, outs[0][1])


@pytest.mark.parametrize("sched", ["static", "dynamic"])
def test_block_event_invariants(sched):
    """Each task ran once; every E_z counter ended at its wait count (16-token
    combine groups of the block times combine column tiles) and every dense
    MLP h event at 8 gate/up tiles."""
    name, T = "moe_skewed", 256
    ws = _ws(name)
    ws.runs().zero_()
    cfg, x, wr, z, y, aux = run_block(name, T, sched, debug=et.DEBUG_COUNTS)
    st = ws.status()
    H, I, E, k = cfg["hidden"], cfg["inter"], cfg["n_experts"], cfg["top_k"]
    rows, bn1, bn2 = 64, 128, 256          # the 64-row LDS-ring variant at 256 tokens
    nr = min(128, 8192 // E, -(-T // 8))
    nb = int((-(-aux["counts"] // rows)).sum())
    ccols = 256 if -(-T // 16) * -(-H // 256) >= et.num_workers() else 64
    ncomb = -(-T // 16) * -(-H // ccols)
    nmb = -(-T // 64)
    total = 2 * nr + 1 + nb * (I // bn1 + H // bn2) + ncomb + nmb * (IM // 16 + H // 16)
    runs = ws.runs().cpu().numpy()
    assert st["last_tasks"] in (0, total)
    assert (runs[:total] == 1).all() and (runs[total:] == 0).all()
    cnt = ws.counters(1 - st["bank"]).cpu().numpy()
    moe_events = ws.plan.n_events - (-(-1024 // 16)) * (1 + IM // 128)
    ez = cnt[moe_events:moe_events + nmb]
    groups = [min(-(-T // 16), (b + 1) * 4) - b * 4 for b in range(nmb)]
    assert (ez == -np.array(groups) * -(-H // ccols)).all()
    ehm = cnt[moe_events + 64:moe_events + 64 + nmb * (IM // 128)]
    assert (ehm == -8).all()
    check(name, T, x, wr, z, y, aux)
