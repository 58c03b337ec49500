"""Benchmark of the Event Tensor MoE megakernel on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tokens T]
                [--sched dynamic|static|barrier|per_op] [--modes] [--no-cpu]

Prints ONE JSON line.  A step is one whole MoE layer (routing -> grouping ->
grouped gate/up GEMM -> grouped down GEMM -> combine) on one batch of seeded
synthetic input already resident in HBM.  The default workload is the
Qwen3-30B-A3B-shaped layer of the Event Tensor MoE experiment (hidden 2048,
128 experts, top-8, expert intermediate 768) at 1024 tokens with Zipf-skewed
routing, under the dynamic schedule with 4 slots claimed per atomic.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer µs & tokens/s vs tokens (static/dynamic); % HBM BW / % MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "event_driven_moe_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic(cfg, T, n_active):
    """Bytes the layer must move (each active expert's weights once, plus x,
    logits and out) and flops of the routed rows (2 per MAC, 3 projections)."""
    H, I, E, k = cfg["hidden"], cfg["inter"], cfg["n_experts"], cfg["top_k"]
    per_expert = 3 * H * I * 2
    io = T * H * 2 + T * E * 4 + T * H * 4
    return {"bytes": n_active * per_expert + io, "per_expert_bytes": per_expert,
            "io_bytes": io, "flops": 2 * 3 * H * I * T * k}


def time_calls(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]   # ms, per launch
    return per, wall


def cpu_baseline(cfg, logits, x, wg, wu, wd, T, target_s=15.0):
    """The oracle (fp64, numpy) on a bounded sample of the same workload's
    tokens; tokens/s scaled from the sample."""
    import numpy as np
    from oracle import moe as omoe
    try:
        import threadpoolctl
        threads = max([d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    L = logits.cpu().numpy()
    X = x.float().cpu().numpy()
    cache = {}

    def weights(e):
        if e not in cache:
            cache[e] = (wg[e].t().float().cpu().numpy(), wu[e].t().float().cpu().numpy(),
                        wd[e].t().float().cpu().numpy())
        return cache[e]
    # host copies of every expert's weights first (not oracle work)
    for e in range(cfg["n_experts"]):
        weights(e)
    rng = np.random.default_rng(0)
    n = min(T, 16)
    t0 = time.perf_counter()
    omoe.moe_layer(L, X, cfg["top_k"], weights, tokens=rng.choice(T, n, replace=False))
    dt = time.perf_counter() - t0
    # a token sample sized for about target_s of oracle work, repeated
    # until that much time has passed
    n2 = int(min(T, max(n, n * target_s / max(dt, 1e-3))))
    sample = np.sort(rng.choice(T, n2, replace=False))
    reps = 0
    t0 = time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < target_s:
        omoe.moe_layer(L, X, cfg["top_k"], weights, tokens=sample)
        reps += 1
    dt = time.perf_counter() - t0
    return {"value": reps * n2 / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d pass(es) over %d of %d tokens (each pass routes and groups all %d), "
                      "fp64 numpy, %.1f s" % (reps, n2, T, T, dt)}


COPY_BYTES = 1 << 30   # calibration copy: reads and writes 1 GiB


def copy_calibration():
    """A plain device copy of known size, so that one profiled run holds both
    the MoE kernel and a reference for the HBM byte counters."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def _pmc_per_dispatch(db, counter):
    """{kernel name: [per-dispatch value]} of one counter in a rocprofv3 DB."""
    import sqlite3
    con = sqlite3.connect(db)
    out = {}
    for _, kn, v in con.execute(
            "select dispatch_id, kernel_name, sum(value) from counters_collection "
            "where counter_name = ? group by dispatch_id order by dispatch_id", (counter,)):
        out.setdefault(kn, []).append(v)
    return out


def kernel_stats(db):
    """Per-kernel launch statistics of a rocprofv3 --kernel-trace database, in
    the form the profiles keep (the stats CSV is not always written when the
    profiled process exits)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = {}
    for name, dur, vgpr, agpr, lds, scr in con.execute(
            "select name, duration, vgpr_count, accum_vgpr_count, lds_size, scratch_size from kernels"):
        r = rows.setdefault(name, {"d": [], "res": (vgpr, agpr, lds, scr)})
        r["d"].append(dur / 1000.0)
    total = sum(sum(r["d"]) for r in rows.values())
    print("| kernel | calls | total us | avg us | median us | min us | max us | % | VGPR/AGPR/LDS B/scratch B |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, r in sorted(rows.items(), key=lambda kv: -sum(kv[1]["d"])):
        d = sorted(r["d"])
        short = name if len(name) < 60 else name[:57] + "..."
        print("| %s | %d | %.1f | %.2f | %.2f | %.2f | %.2f | %.1f | %s |" % (
            short, len(d), sum(d), sum(d) / len(d), d[len(d) // 2], d[0], d[-1],
            100.0 * sum(d) / total, "/".join(str(x) for x in r["res"])))


def traffic_summary(fetch_db, write_db, key):
    """HBM bytes per launch of the MoE kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (both KiB per dispatch), each scaled by what the counter
    reads for the calibration copy; stores the figure for later bench lines."""
    res = {}
    for name, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        d = _pmc_per_dispatch(db, name)
        moe = [v for k, vs in d.items() if "moe_kernel" in k for v in vs]
        cpy = [v for k, vs in d.items() if "moe_kernel" not in k for v in vs
               if abs(v * 1024 - COPY_BYTES) < 0.6 * COPY_BYTES]
        if not moe or not cpy:
            raise SystemExit("%s: no MoE kernel or calibration copy dispatches in %s" % (name, db))
        cal = COPY_BYTES / (1024.0 * sum(cpy) / len(cpy))
        res[name] = {"kib_per_dispatch": sum(moe) / len(moe), "dispatches": len(moe),
                     "copy_kib": sum(cpy) / len(cpy), "scale": cal,
                     "bytes": 1024.0 * cal * sum(moe) / len(moe)}
    ent = {"kernel_hash": kernel_source_hash(),
           "hbm_bytes_per_launch": int(res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]),
           "read_bytes": int(res["FETCH_SIZE"]["bytes"]), "write_bytes": int(res["WRITE_SIZE"]["bytes"]),
           "counters": res}
    try:
        with open(TRAFFIC_FILE) as fh:
            tj = json.load(fh)
    except (OSError, ValueError):
        tj = {}
    tj[key] = ent
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(tj, fh, indent=1, sort_keys=True)
    print(json.dumps({key: ent}, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moe_skewed")
    ap.add_argument("--tokens", type=int, default=1024)
    ap.add_argument("--sched", default="dynamic")
    ap.add_argument("--fetch", type=int, default=4)
    ap.add_argument("--modes", action="store_true", help="also time the other schedules")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy before timing (reference for HBM counters)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="no GPU work: read two rocprofv3 --pmc databases (FETCH_SIZE, "
                         "WRITE_SIZE) of this command and record the MoE kernel's HBM bytes")
    ap.add_argument("--kernel-stats", metavar="DB",
                    help="no GPU work: print per-kernel statistics of a rocprofv3 --kernel-trace database")
    args = ap.parse_args()
    if args.kernel_stats:
        kernel_stats(args.kernel_stats)
        return
    if args.traffic:
        traffic_summary(args.traffic[0], args.traffic[1],
                        "%s:T%d:%s" % (args.workload, args.tokens, args.sched))
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from event_driven_moe_amd import et, synth

    dev = "cuda"
    cfg = synth.MOE_PRESETS[args.workload]
    T = args.tokens
    logits, x = synth.moe_activations(cfg, T, device=dev)
    wg, wu, wd = synth.moe_weights_k_major(cfg, device=dev)
    ws = et.Workspace(et.WL_MOE, T, cfg["hidden"], cfg["inter"], cfg["n_experts"],
                      cfg["top_k"], device=dev)
    out = torch.empty((T, cfg["hidden"]), device=dev)

    def step(sched=args.sched):
        et.moe_layer(logits, x, wg, wu, wd, out, ws, sched, fetch_batch=args.fetch)

    step()
    torch.cuda.synchronize()
    st = ws.status()
    if st["status"] != 0:
        raise SystemExit("device fault: %s" % st)
    aux = et.moe_aux(ws, T)
    n_active = int((aux["counts"] > 0).sum().item())
    max_rows = int(aux["counts"].max().item())
    alg = algorithmic(cfg, T, n_active)

    if args.copy_calibration:
        copy_calibration()
    torch.cuda.synchronize()
    per, wall = time_calls(step, args.steps, args.warmup)
    torch.cuda.synchronize()
    if ws.status()["status"] != 0:
        raise SystemExit("device fault during timing")
    ms = sum(per) / len(per)
    per_sorted = sorted(per)
    value = T / (ms * 1e-3)
    achieved_gbs = alg["bytes"] / (ms * 1e-3) / 1e9
    achieved_tfs = alg["flops"] / (ms * 1e-3) / 1e12
    ai = alg["flops"] / alg["bytes"]
    bound = "hbm" if ai < MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"

    traffic = None
    try:
        with open(TRAFFIC_FILE) as fh:
            tj = json.load(fh)
        key = "%s:T%d:%s" % (args.workload, T, args.sched)
        ent = tj.get(key)
        if ent and ent.get("kernel_hash") == kernel_source_hash():
            traffic = ent["hbm_bytes_per_launch"]
    except (OSError, ValueError):
        pass

    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved_tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved_tfs / MFMA_BF16_PEAK_TFS, 4),
                "traffic": traffic}

    modes = {}
    if args.modes:
        for s in ("static", "dynamic", "barrier", "per_op"):
            p, _ = time_calls(lambda: step(s), max(10, args.steps // 2), 3)
            modes[s] = round(1e3 * sum(p) / len(p), 2)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random-init bf16 expert weights ~N(0,0.02))",
        "config": {
            "workload": "%s: MoE layer, %d tokens, hidden %d, %d experts, top-%d, "
                        "intermediate %d%s" % (args.workload, T, cfg["hidden"], cfg["n_experts"],
                                               cfg["top_k"], cfg["inter"],
                                               ", Zipf-skewed router bias" if cfg["bias"] == "zipf" else ""),
            "tokens": T, "schedule": args.sched, "fetch_batch": args.fetch,
            "active_experts": n_active, "max_rows_per_expert": max_rows,
            "us_per_layer_median": round(1e3 * per_sorted[len(per) // 2], 2),
            "us_per_layer_p10": round(1e3 * per_sorted[len(per) // 10], 2),
            "us_per_layer_p90": round(1e3 * per_sorted[(9 * len(per)) // 10], 2),
            "algorithmic_bytes": alg["bytes"], "flops": alg["flops"],
            "mfma_frac": round(achieved_tfs / MFMA_BF16_PEAK_TFS, 4),
            "hbm_frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "kernel": "moe_kernel (one persistent launch per layer)",
        },
        "roofline": roof,
    }
    if modes:
        res["config"]["us_per_layer_by_schedule"] = modes
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(cfg, logits, x, wg, wu, wd, T)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
