"""Pins for the split-K oracle (CPU only)."""

import math
import os

import numpy as np

from oracle import splitk, events
from event_driven_moe_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLD, name), encoding="utf-8"):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(None, 1)
            out[k] = v
    return out


def test_page_example_constants():
    g = _golden("splitk_example.txt")
    assert int(g["input_cols"]) == splitk.SLICES * splitk.SLICE_W
    assert int(g["k_slices"]) == splitk.SLICES
    assert int(g["slice_width"]) == splitk.SLICE_W
    assert int(g["rows_per_event"]) == splitk.ROWS_PER_BLOCK
    tab = events.splitk_table(64 * 32)
    assert tab["events"]["E"]["shape"] == (64,)
    assert (tab["events"]["E"]["wait_count"] == int(g["wait_count"])).all()
    assert g["producer_map"] == "ij->i" and g["consumer_map"] == "i->i"


def test_event_table_brute_force():
    # Enumerate producer tasks (i, j) -> E[i] and count notifies per event.
    for n in (1, 3, 64):
        tab = events.splitk_table(n * 32)
        cnt = events.notify_counts(tab["producer_map"], (n,))
        assert (cnt == tab["events"]["E"]["wait_count"]).all()
        assert tab["tasks"] == {"stage1": 4 * n, "stage2": n}


def test_against_fsum():
    A = synth.splitk_inputs(rows=256, seed=7).numpy()
    B, C = splitk.splitk_reduce(A)
    for r in range(0, 256, 17):
        row = [float(v) for v in A[r]]
        assert abs(C[r] - math.fsum(row)) <= 1e-14 * max(1.0, abs(math.fsum(row)))
        for j in range(4):
            ref = math.fsum(row[32 * j:32 * j + 32])
            assert abs(B[r, j] - ref) <= 1e-14 * max(1.0, abs(ref))


def test_integer_exact():
    A = synth.splitk_inputs(rows=128, seed=111, integer=True).numpy()
    B, C = splitk.splitk_reduce(A)
    Ai = A.astype(np.int64)
    for r in range(128):
        assert C[r] == sum(int(v) for v in Ai[r])
        for j in range(4):
            assert B[r, j] == sum(int(v) for v in Ai[r, 32 * j:32 * j + 32])


def test_all_ones():
    B, C = splitk.splitk_reduce(np.ones((64, 128), np.float32))
    assert (B == 32).all() and (C == 128).all()


def test_index_closed_forms():
    # A[r, c] = c: B[r, j] = sum of the arithmetic series 32j .. 32j+31.
    A = np.tile(np.arange(128, dtype=np.float32), (32, 1))
    B, C = splitk.splitk_reduce(A)
    for j in range(4):
        assert (B[:, j] == 1024 * j + 496).all()
    assert (C == 127 * 128 / 2).all()
    # A[r, c] = r: C[r] = 128 r (rows are not mixed up).
    A = np.repeat(np.arange(96, dtype=np.float32)[:, None], 128, axis=1)
    B, C = splitk.splitk_reduce(A)
    assert (C == 128 * np.arange(96)).all()
