"""Shared helpers for the GPU parity tests (inputs from event_driven_moe_amd.synth,
expected values from oracle/ on host copies of the same tensors)."""

import functools
import sys

import numpy as np
import torch

from event_driven_moe_amd import et, synth

DEV = "cuda"
SCHEDS = ("static", "dynamic", "barrier", "per_op")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    return err / scale if scale > 0 else err


def assert_rel(got, ref, tol, what=""):
    r = max_rel_err(got, ref)
    assert r <= tol, "%s: max|err| / max|ref| = %.3e > %.1e" % (what, r, tol)


def to_np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def moe_weights(name):
    """Device weights of a preset, cached per weight set (presets that differ
    only in their router bias share one copy)."""
    cfg = synth.MOE_PRESETS[name]
    return _moe_weights(cfg["hidden"], cfg["inter"], cfg["n_experts"], cfg["seed_w"])


@functools.lru_cache(maxsize=2)
def _moe_weights(hidden, inter, n_experts, seed_w):
    cfg = dict(hidden=hidden, inter=inter, n_experts=n_experts, seed_w=seed_w)
    return synth.moe_weights_k_major(cfg, device=DEV)


def moe_oracle_weights(wg, wu, wd):
    """Callable e -> logical fp64-ready host arrays of expert e (from the device tensors)."""
    def get(e):
        return (wg[e].t().float().cpu().numpy(), wu[e].t().float().cpu().numpy(),
                wd[e].t().float().cpu().numpy())
    return get
