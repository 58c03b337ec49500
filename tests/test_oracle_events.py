"""Pins for the event semantics and the scheduler simulator (CPU only)."""

import os
import random

import pytest

from oracle import events as ev

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _steps(name):
    out = []
    for line in open(os.path.join(GOLD, name), encoding="utf-8"):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(tuple(line.split()))
    return out


def _walk_graph():
    return ev.TaskGraph(
        tasks=["gemm0", "gemm1", "gemm2", "rs"],
        waits={"rs": ["E"]},
        notifies={"gemm0": ["E"], "gemm1": ["E"]},
        wait_count={"E": 2},
    )


def _dur(t):
    return {"gemm0": 1.0, "gemm1": 2.0, "gemm2": 5.0, "rs": 1.0}[t]


def _match(trace, expected):
    """Every expected step appears in the trace, in order."""
    it = iter(trace)
    for exp in expected:
        for step in it:
            act = step[0]
            if act != exp[0]:
                continue
            if act in ("notify", "spin"):
                ok = (str(step[1]) == exp[1] and step[2] == exp[2] and str(step[4]) == exp[3])
            elif act in ("run", "push"):
                ok = (exp[1] == "*" or str(step[1]) == exp[1]) and step[2] == exp[2]
            else:
                ok = False
            if ok:
                break
        else:
            return False
    return True


def test_static_walkthrough():
    g = _walk_graph()
    g.tasks.remove("gemm2")
    trace, cnt, runs = ev.run_static(g, [["gemm0", "rs"], ["gemm1"]], _dur)
    assert _match(trace, _steps("static_walkthrough.txt")), trace
    assert cnt["E"] == 0 and all(v == 1 for v in runs.values())


def test_dynamic_walkthrough():
    g = _walk_graph()
    trace, cnt, runs = ev.run_dynamic(g, 2, ["gemm0", "gemm1", "gemm2"], _dur)
    assert _match(trace, _steps("dynamic_walkthrough.txt")), trace
    # the producer never waits: no spin steps exist in dynamic mode
    assert not any(s[0] == "spin" for s in trace)
    assert cnt["E"] == 0 and all(v == 1 for v in runs.values())
    # exactly one push of the consumer, by the notifier that zeroed the counter
    pushes = [s for s in trace if s[0] == "push"]
    assert pushes == [("push", 1, "rs")]


def _random_layered(seed, layers=4, width=6):
    rnd = random.Random(seed)
    tasks, waits, notifies, wc = [], {}, {}, {}
    prev = []
    for L in range(layers):
        cur = ["t%d_%d" % (L, i) for i in range(rnd.randint(1, width))]
        for t in cur:
            tasks.append(t)
            if prev:
                e = "e_" + t
                producers = rnd.sample(prev, rnd.randint(1, len(prev)))
                for p in producers:
                    notifies.setdefault(p, []).append(e)
                waits[t] = [e]
                wc[e] = len(producers)
        prev = cur
    return ev.TaskGraph(tasks, waits, notifies, wc)


@pytest.mark.parametrize("seed", range(12))
def test_random_graphs_exactly_once(seed):
    g = _random_layered(seed)
    rnd = random.Random(100 + seed)
    dur = lambda t: 1.0 + (hash((seed, t)) % 7)
    # static: round-robin over workers, each list in topological (layer) order
    nw = rnd.randint(1, 4)
    lists = [g.tasks[w::nw] for w in range(nw)]
    _, cnt, runs = ev.run_static(g, lists, dur)
    assert all(v == 0 for v in cnt.values()) and all(v == 1 for v in runs.values())
    # dynamic, fetch 1 and 4
    init = [t for t in g.tasks if not g.waits[t]]
    for fetch in (1, 4):
        _, cnt, runs = ev.run_dynamic(g, nw, init, dur, fetch=fetch)
        assert all(v == 0 for v in cnt.values()) and all(v == 1 for v in runs.values())


def test_wrong_wait_count_is_detected():
    g = _walk_graph()
    g.tasks.remove("gemm2")
    g.wait_count["E"] = 3      # one notify too few will ever arrive
    with pytest.raises(ev.Deadlock):
        ev.run_static(g, [["gemm0", "rs"], ["gemm1"]], _dur)
    _, cnt, runs = ev.run_dynamic(g, 2, ["gemm0", "gemm1"], _dur)
    assert cnt["E"] == 1 and runs["rs"] == 0     # consumer never pushed


def test_list_out_of_topological_order_deadlocks():
    g = _walk_graph()
    g.tasks.remove("gemm2")
    with pytest.raises(ev.Deadlock):
        ev.run_static(g, [["rs", "gemm0", "gemm1"]], _dur)


@pytest.mark.parametrize("batch,rows,gate_cols,h_tile,down_cols,k_slices", [
    (1, 16, 16, 128, 16, 1), (64, 16, 16, 128, 16, 1), (40, 32, 32, 128, 64, 2),
    (17, 64, 64, 256, 128, 4), (100, 16, 128, 128, 32, 3)])
def test_mlp_table_brute_force(batch, rows, gate_cols, h_tile, down_cols, k_slices):
    """Enumerate every task of the dense MLP chain under a tiling and count
    the notifies each event receives: gate/up tile (m, n) covers h columns
    [n*gate_cols, (n+1)*gate_cols) of row block m and notifies the E_h[m, c]
    of the h tile holding them; down tile (m, n2, s) covers K-slice s of the
    output columns of tile n2 and, with several K-slices, notifies E_y[m, n2].
    The table's task counts and wait counts must equal the enumeration."""
    hidden, inter = 512, 768
    tab = ev.mlp_table(batch, hidden, inter, rows, gate_cols, h_tile, down_cols, k_slices)
    mb = -(-batch // rows)
    gate = [(m, n) for m in range(mb) for n in range(inter // gate_cols)]
    down = [(m, n2, s) for m in range(mb) for n2 in range(hidden // down_cols)
            for s in range(k_slices)]
    assert tab["tasks"]["gate_up"] == len(gate)
    assert tab["tasks"]["down"] == len(down)
    # every h column is produced by exactly one gate/up tile
    cols = sorted(c for (m, n) in gate if m == 0 for c in range(n * gate_cols, (n + 1) * gate_cols))
    assert cols == list(range(inter))
    eh = ev.notify_counts([(t, (t[0], t[1] * gate_cols // h_tile)) for t in gate],
                          (mb, inter // h_tile))
    assert tab["events"]["E_h"]["shape"] == (mb, inter // h_tile)
    assert (tab["events"]["E_h"]["wait_count"] == eh).all()
    if k_slices > 1:
        ey = ev.notify_counts([(t, (t[0], t[1])) for t in down], (mb, hidden // down_cols))
        assert (tab["events"]["E_y"]["wait_count"] == ey).all()
        assert tab["tasks"]["reduce"] == mb * (hidden // down_cols)
    else:
        assert "E_y" not in tab["events"] and tab["tasks"]["reduce"] == 0


def test_mlp_table_symbolic_batch():
    """One event table shape per row-block count: the E_h shape grows with
    ceil(B / rows) and nothing else (the symbolic batch dimension)."""
    shapes = {B: ev.mlp_table(B, 2048, 5632, 16, 16, 128, 16, 1)["events"]["E_h"]["shape"]
              for B in (1, 4, 16, 17, 64)}
    assert shapes == {1: (1, 44), 4: (1, 44), 16: (1, 44), 17: (2, 44), 64: (4, 44)}
