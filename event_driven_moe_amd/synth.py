"""Seeded synthetic inputs for the three workloads.

This module only draws numbers: it holds none of the method's arithmetic, so
both the HIP path and the CPU oracle can be fed from it.  Every draw comes
from a ``torch.Generator`` seeded per tensor (and per expert), on the device
the caller names: the same seed on the same device type gives the same
values.  Parity checks on a GPU draw the inputs there and hand the oracle a
host copy of the very same tensors.

Distributions follow the workloads the pages measure, with synthetic values
standing in for trained weights and real routing (no checkpoints or traces
are used):

* split-K example: A float32 (n*32, 128) uniform in [-1, 1), or small
  integers for exactness checks;
* dense MLP: x bf16 [B, H] ~ N(0, 1); weights bf16 ~ N(0, 0.02) (0.02 is the
  standard deviation), drawn in float32 and rounded to bf16 to nearest-even;
* MoE: router logits float32 [T, E] ~ N(0, 1) plus an optional per-expert
  bias; x bf16 [T, H] ~ N(0, 1); expert weights bf16 ~ N(0, 0.02).

Weights are drawn in their logical layout (gate/up [H, I], down [I, H]);
``k_major`` returns the K-contiguous copy the library takes.
"""

import torch

# Workload presets (sizes of the workloads the pages evaluate; the MoE presets
# mirror the Qwen3-30B-A3B-shaped layer of the Event Tensor MoE experiment and
# a small and a large layer around it).
SPLITK = dict(name="splitk", rows=2048, cols=128, seed=101, int_seed=111)
MLP = dict(name="mlp", hidden=2048, inter=5632, batches=(1, 4, 16, 64),
           seed_x=201, seed_wg=202, seed_wu=203, seed_wd=204)
MOE_SMALL = dict(name="moe_small", hidden=2048, inter=1408, n_experts=8, top_k=2,
                 tokens=(1, 8, 32), seed_logits=301, seed_x=302, seed_w=303,
                 bias="none")
MOE_SKEWED = dict(name="moe_skewed", hidden=2048, inter=768, n_experts=128, top_k=8,
                  tokens=(64, 256, 1024), seed_logits=401, seed_x=402, seed_w=403,
                  bias="zipf", zipf_scale=1.5, zipf_exp=1.2)
# The skewed layer's bias formula taken literally (scale 1.5) gives the
# hottest expert every token (max/mean load E/k = 16); the same formula with
# scale 0.15 gives the 3-4x max/mean load its description states.  Both are
# kept: same shapes, seeds and weights, only the bias scale differs.
MOE_SKEWED_CAL = dict(MOE_SKEWED, name="moe_skewed_cal", zipf_scale=0.15)
MOE_LARGE = dict(name="moe_large", hidden=7168, inter=2048, n_experts=256, top_k=8,
                 tokens=(512, 2048, 8192), seed_logits=501, seed_x=502, seed_w=503,
                 seed_bias=504, bias="random")
MOE_PRESETS = {c["name"]: c for c in (MOE_SMALL, MOE_SKEWED, MOE_SKEWED_CAL, MOE_LARGE)}

WEIGHT_STD = 0.02


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, std, seed, device):
    g = _gen(seed, device)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(torch.bfloat16)


def splitk_inputs(rows=2048, seed=101, device="cpu", integer=False):
    """A float32 [rows, 128]: uniform [-1, 1), or integers in [-8, 8]."""
    g = _gen(seed, device)
    if integer:
        return torch.randint(-8, 9, (rows, 128), generator=g, device=device).to(torch.float32)
    return torch.rand((rows, 128), generator=g, device=device, dtype=torch.float32) * 2 - 1


def mlp_inputs(batch, hidden=2048, inter=5632, device="cpu", seeds=(201, 202, 203, 204)):
    """x [B,H], wg [H,I], wu [H,I], wd [I,H] (bf16, logical layout)."""
    sx, sg, su, sd = seeds
    x = normal_bf16((batch, hidden), 1.0, sx + batch, device)
    wg = normal_bf16((hidden, inter), WEIGHT_STD, sg, device)
    wu = normal_bf16((hidden, inter), WEIGHT_STD, su, device)
    wd = normal_bf16((inter, hidden), WEIGHT_STD, sd, device)
    return x, wg, wu, wd


def expert_bias(cfg, tokens, device="cpu"):
    """Per-expert router bias [E] float32 (zeros when the preset has none).

    zipf: bias_e = scale * ln((e + 1) ** -exponent), expert e having Zipf rank
    e + 1.  random: one N(0, 1) vector per call, seeded by the token count."""
    E = cfg["n_experts"]
    if cfg["bias"] == "none":
        return torch.zeros(E, dtype=torch.float32, device=device)
    if cfg["bias"] == "zipf":
        r = torch.arange(1, E + 1, dtype=torch.float64)
        b = cfg["zipf_scale"] * torch.log(r ** (-cfg["zipf_exp"]))
        return b.to(torch.float32).to(device)
    if cfg["bias"] == "random":
        g = _gen(cfg["seed_bias"] + tokens, device)
        return torch.randn(E, generator=g, device=device, dtype=torch.float32)
    raise ValueError(cfg["bias"])


def moe_activations(cfg, tokens, device="cpu"):
    """logits float32 [T, E] (N(0,1) + bias) and x bf16 [T, H] ~ N(0, 1)."""
    E, H = cfg["n_experts"], cfg["hidden"]
    g = _gen(cfg["seed_logits"] + tokens, device)
    logits = torch.randn((tokens, E), generator=g, device=device, dtype=torch.float32)
    logits += expert_bias(cfg, tokens, device)[None, :]
    x = normal_bf16((tokens, H), 1.0, cfg["seed_x"] + tokens, device)
    return logits, x


def expert_seed(cfg, e, which):
    """Seed of expert e's gate (0), up (1) or down (2) matrix."""
    return cfg["seed_w"] * 1_000_003 + 3 * e + which


def moe_expert_weights(cfg, e, device="cpu"):
    """Expert e's logical weights: wg [H,I], wu [H,I], wd [I,H] (bf16)."""
    H, I = cfg["hidden"], cfg["inter"]
    return (normal_bf16((H, I), WEIGHT_STD, expert_seed(cfg, e, 0), device),
            normal_bf16((H, I), WEIGHT_STD, expert_seed(cfg, e, 1), device),
            normal_bf16((I, H), WEIGHT_STD, expert_seed(cfg, e, 2), device))


def moe_weights_k_major(cfg, device="cpu", experts=None):
    """All experts' weights directly in the library's K-contiguous layout:
    w_gate [E, I, H], w_up [E, I, H], w_down [E, H, I] (bf16).  Expert e holds
    the transposes of ``moe_expert_weights(cfg, e)``."""
    E, H, I = cfg["n_experts"], cfg["hidden"], cfg["inter"]
    alloc = torch.empty if experts is None else torch.zeros   # unlisted experts: zeros
    experts = range(E) if experts is None else experts
    wg = alloc((E, I, H), dtype=torch.bfloat16, device=device)
    wu = alloc((E, I, H), dtype=torch.bfloat16, device=device)
    wd = alloc((E, H, I), dtype=torch.bfloat16, device=device)
    for e in experts:
        g, u, d = moe_expert_weights(cfg, e, device)
        wg[e].copy_(g.t())
        wu[e].copy_(u.t())
        wd[e].copy_(d.t())
    return wg, wu, wd


def k_major(w):
    """Logical [K, N] (or [E, K, N]) -> K-contiguous [N, K] ([E, N, K])."""
    return w.transpose(-1, -2).contiguous()
