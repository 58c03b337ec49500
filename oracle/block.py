"""Oracle: router GEMM -> MoE layer -> dense MLP, the cross-stage chain of
one decoder step (test infrastructure only).

Follows Event Tensor notes, section "端到端低 batch serving": the megakernel
covers the whole decoding pipeline, and among the cross-operator
optimisations it names are the pipelining of the MoE GroupGEMM with the dense
MLP GEMM across stages and fetching the next stage's weights before its
activations arrive.  The router GEMM is the step that turns hidden states
into the router logits the MoE layer takes (Weave MoE article section 1.1:
each token's router scores select its experts).

Readings taken where the pages are silent (each also listed in the design doc):

* the router is a bias-free linear map, logits = x @ W_router with x [T, H]
  and W_router [H, E];
* the dense MLP consumes the MoE layer's output of the same tokens:
  y = MLP(z) with z = MoE(x) (the gated MLP of ``oracle.mlp``); no residual
  or normalisation sits between them (the pages do not name one);
* routing ranks the logits as ``oracle.moe.route`` does.  When the caller
  passes ``route_logits`` (the float32 logits another implementation
  computed), routing ranks those instead: a top-k decision taken on
  float32 values is compared in float32, where fp64 logits could order two
  nearly tied experts differently.

Everything else is float64 from the exact inputs, with no intermediate
rounding.

Pins (tests/test_oracle_block.py): the router matmul against explicit
Python sums, exactly on integer inputs; the whole chain against a
pure-Python brute force on tiny inputs (its own loops for the matmuls, the
top-k, the grouping-free per-token expert evaluation and the combine).
"""

import numpy as np

from . import moe, mlp as omlp


def router(x, w_router):
    """logits[t, e] = sum_h x[t, h] * W_router[h, e], float64.
    x: [T, H]; w_router: [H, E] (logical layout)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[0]:
        raise ValueError("router: shapes must be x[T,H], w_router[H,E]")
    return x @ w


def block(x, w_router, k, expert_weights, mlp_weights, route_logits=None, tokens=None):
    """The chain.  expert_weights as for ``oracle.moe.moe_layer``;
    mlp_weights = (wg [H, Im], wu [H, Im], wd [Im, H]).  Returns a dict with
    logits (float64 [T, E]), the routing and grouping results of
    ``oracle.moe.moe_layer``, z (the MoE output, float64) and y (the MLP
    output, float64), rows for ``tokens`` (default all)."""
    logits = router(x, w_router)
    ranked = logits if route_logits is None else np.asarray(route_logits)
    res = moe.moe_layer(ranked, x, k, expert_weights, tokens=tokens)
    z = res.pop("out")
    wg, wu, wd = mlp_weights
    res.update(logits=logits, z=z, y=omlp.mlp(z, wg, wu, wd))
    return res
