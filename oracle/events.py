"""Oracle: Event Tensor semantics, expected event tables and a small
scheduler simulator (test infrastructure only).

Follows Event Tensor notes:
* section "Event Tensor 抽象": an Event Tensor is an array of events; each
  element has an initial wait count; notify() atomically decrements it; wait()
  holds until it is zero; under dynamic scheduling the consumers of an event
  are pushed to the ready queue when its count reaches zero; producer/consumer
  coordinate maps are einsum-like ("ij->i", "i->i");
* section "静态调度": per-SM task lists fixed before launch, notify at the end
  of a producer, wait at the start of a consumer, no run-time push/pop; the
  walkthrough with one Reduce-Scatter tile fed by two GEMM tiles (counter
  2 -> 1, SM0 spins, SM1 brings it to 0, SM0 runs);
* section "动态调度": a ready-task queue on the GPU; an idle SM pops; the
  producer whose notify zeroes a counter pushes the consumers; in the same
  walkthrough SM0 does not wait but pops another producer;
* section "两类动态性如何进入依赖表示": symbolic event shapes and
  data-dependent wait counts (the expert event starts at the number of rows
  routed to it) and fan-out (tasks[exp_indptr[e]:exp_indptr[e+1]]).

The table functions restate, for a given tiling, how many tasks of each kind
a workload has and what every event's initial count is; debug runs of the
GPU path are compared against them (every task runs exactly once, every
counter ends at zero).  The simulator replays the two walkthroughs of the
page (tests/golden/*walkthrough*.txt) and checks deadlock freedom and
exactly-once execution on random task graphs.

Pins: the walkthrough traces printed by the page; brute-force enumeration of
the producer maps (each event receives exactly its wait count of notifies).
"""

import heapq

import numpy as np


# --------------------------------------------------------------------------
# Expected tables
# --------------------------------------------------------------------------

def splitk_table(rows):
    """Split-K example: E shape (n,), wait count 4; 4n stage-1 tasks (map
    "ij->i"), n stage-2 tasks (map "i->i")."""
    if rows % 32:
        raise ValueError("rows must be a multiple of 32")
    n = rows // 32
    return {
        "tasks": {"stage1": 4 * n, "stage2": n},
        "events": {"E": {"shape": (n,), "wait_count": np.full(n, 4, np.int64)}},
        "producer_map": [((i, j), i) for i in range(n) for j in range(4)],
    }


def mlp_table(batch, hidden, inter, rows_per_tile, gate_cols, h_tile, down_cols, k_slices):
    """Dense MLP chain under a tiling: gate/up tiles of ``gate_cols`` columns of
    the intermediate dimension notify E_h[m, c] (one event per ``h_tile``
    columns of h, symbolic in the number of row blocks m = ceil(B/rows));
    down tiles (m, n, s) wait on the E_h events of their K-slice and, when
    ``k_slices`` > 1, notify E_y[m, n] which gates a reduce tile."""
    mb = -(-batch // rows_per_tile)
    n_h = inter // h_tile
    n_down = hidden // down_cols
    tab = {
        "tasks": {
            "gate_up": mb * (inter // gate_cols),
            "down": mb * n_down * k_slices,
            "reduce": mb * n_down if k_slices > 1 else 0,
        },
        "events": {
            "E_h": {"shape": (mb, n_h),
                    "wait_count": np.full((mb, n_h), h_tile // gate_cols, np.int64)},
        },
    }
    if k_slices > 1:
        tab["events"]["E_y"] = {"shape": (mb, n_down),
                                "wait_count": np.full((mb, n_down), k_slices, np.int64)}
    return tab


def moe_table(counts, rows_per_tile, inter, gate_cols, hidden, down_cols, n_route,
              tokens=None, top_k=None, comb_tok=16, comb_cols=None):
    """MoE layer under a tiling: ``n_route`` routing tasks, one scan task,
    ``n_route`` grouping tasks; expert e owns ceil(counts[e]/rows) row blocks;
    each block has inter/gate_cols gate/up tiles and hidden/down_cols down
    tiles.  E_exp[e] starts at counts[e] (data-dependent); E_h[block] at the
    number of gate/up tiles of a block; E_he[e] (the dynamic schedule's
    per-expert edge from gate/up to down tiles) at the number of gate/up
    tiles over all of expert e's blocks (data-dependent).

    With ``tokens`` given: E_cg[g, c], the edge from the down tiles to the
    combine tile of tokens [g*comb_tok, (g+1)*comb_tok) and columns
    [c*comb_cols, (c+1)*comb_cols).  Each down tile notifies it once per row
    of its block that belongs to a token of group g (a notify target read
    from the run-time permutation) when the tile's columns overlap the
    combine tile's, so it starts at top_k rows per token of the group times
    the number of down column tiles overlapping the combine tile."""
    counts = np.asarray(counts, dtype=np.int64)
    blocks = -(-counts // rows_per_tile)
    nb = int(blocks.sum())
    tab = {
        "tasks": {
            "route": n_route, "scan": 1, "group": n_route,
            "gate_up": nb * (inter // gate_cols),
            "down": nb * (hidden // down_cols),
        },
        "blocks": nb,
        "events": {
            "E_exp": {"shape": (counts.shape[0],), "wait_count": counts.copy()},
            "E_h": {"shape": (nb,),
                    "wait_count": np.full(nb, inter // gate_cols, np.int64)},
            "E_he": {"shape": (counts.shape[0],),
                     "wait_count": blocks * (inter // gate_cols)},
        },
    }
    if tokens is not None:
        ng, nc = -(-tokens // comb_tok), -(-hidden // comb_cols)
        g0 = np.arange(ng) * comb_tok
        ntok = np.minimum(tokens, g0 + comb_tok) - g0
        c0 = np.arange(nc) * comb_cols
        c1 = np.minimum(hidden, c0 + comb_cols)
        ndown = (c1 - 1) // down_cols - c0 // down_cols + 1
        tab["events"]["E_cg"] = {"shape": (ng, nc),
                                 "wait_count": np.outer(ntok * top_k, ndown).astype(np.int64)}
    return tab


def notify_counts(producer_map, shape):
    """Brute force: apply a producer map (list of (task, event index)) and
    count the notifies each event receives."""
    c = np.zeros(shape, dtype=np.int64)
    for _, ev in producer_map:
        c[ev] += 1
    return c


# --------------------------------------------------------------------------
# Scheduler simulator (discrete events; models the protocol, not timing)
# --------------------------------------------------------------------------

class Deadlock(RuntimeError):
    pass


class TaskGraph:
    """tasks: names; waits[t]: events t waits on; notifies[t]: events t
    notifies (once each); wait_count[ev]: initial count; the consumers of an
    event are the tasks that wait on it."""

    def __init__(self, tasks, waits, notifies, wait_count):
        self.tasks = list(tasks)
        self.waits = {t: list(waits.get(t, ())) for t in self.tasks}
        self.notifies = {t: list(notifies.get(t, ())) for t in self.tasks}
        self.wait_count = dict(wait_count)
        self.consumers = {ev: [] for ev in self.wait_count}
        for t in self.tasks:
            for ev in self.waits[t]:
                self.consumers[ev].append(t)


def run_static(g, lists, duration):
    """Static schedule: worker w runs lists[w] in order; before a task it
    spins until every event it waits on is zero; after it, it notifies.
    Returns (trace, counters, runs).  Raises Deadlock if no worker can move."""
    cnt = dict(g.wait_count)
    pos = [0] * len(lists)
    clock = [0.0] * len(lists)
    trace, runs = [], {t: 0 for t in g.tasks}
    spinning = set()
    # event queue of (finish_time, worker, task)
    running = []
    idle = list(range(len(lists)))
    while True:
        progressed = False
        for w in list(idle):
            if pos[w] >= len(lists[w]):
                idle.remove(w)
                continue
            t = lists[w][pos[w]]
            blocked = [ev for ev in g.waits[t] if cnt[ev] != 0]
            if blocked:
                if (w, t) not in spinning:
                    trace.append(("spin", w, t, blocked[0], cnt[blocked[0]]))
                    spinning.add((w, t))
                continue
            spinning.discard((w, t))
            trace.append(("run", w, t))
            runs[t] += 1
            idle.remove(w)
            heapq.heappush(running, (clock[w] + duration(t), w, t))
            progressed = True
        if running:
            tfin, w, t = heapq.heappop(running)
            clock[w] = tfin
            for other in idle:
                clock[other] = max(clock[other], tfin)
            for ev in g.notifies[t]:
                cnt[ev] -= 1
                trace.append(("notify", w, t, ev, cnt[ev]))
            pos[w] += 1
            idle.append(w)
            idle.sort()
            continue
        if not progressed:
            if any(pos[w] < len(lists[w]) for w in range(len(lists))):
                raise Deadlock("static lists deadlock")
            return trace, cnt, runs


def run_dynamic(g, n_workers, initial, duration, fetch=1):
    """Dynamic schedule: a FIFO ready queue seeded with ``initial``; an idle
    worker pops up to ``fetch`` tasks per claim and runs them in order; the
    notify that zeroes an event pushes its consumers whose other events are
    already zero.  A worker never waits on an event.  Returns
    (trace, counters, runs)."""
    cnt = dict(g.wait_count)
    queue = list(initial)
    head = 0
    trace, runs = [], {t: 0 for t in g.tasks}
    running = []
    local = {w: [] for w in range(n_workers)}
    idle = list(range(n_workers))
    now = 0.0
    while True:
        for w in list(idle):
            if not local[w]:
                if head < len(queue):
                    local[w] = queue[head:head + fetch]
                    head += len(local[w])
                    trace.append(("pop", w, tuple(local[w])))
                else:
                    continue
            t = local[w].pop(0)
            if any(cnt[ev] != 0 for ev in g.waits[t]):
                raise Deadlock("dynamic queue held a task that is not ready")
            trace.append(("run", w, t))
            runs[t] += 1
            idle.remove(w)
            heapq.heappush(running, (now + duration(t), w, t))
        if not running:
            if head < len(queue) or any(local.values()):
                continue
            return trace, cnt, runs
        now, w, t = heapq.heappop(running)
        for ev in g.notifies[t]:
            cnt[ev] -= 1
            trace.append(("notify", w, t, ev, cnt[ev]))
            if cnt[ev] == 0:
                for c in g.consumers[ev]:
                    if all(cnt[e2] == 0 for e2 in g.waits[c]):
                        queue.append(c)
                        trace.append(("push", w, c))
        idle.append(w)
        idle.sort()
