"""Oracle: the MoE layer -- routing, token grouping, expert MLPs, combine
(test infrastructure only).

Follows Event Tensor notes, section "两类动态性如何进入依赖表示" (the MoE chain
TopK routing -> token grouping -> GroupGEMM, grouping tasks notifying the
events of the experts named by the runtime top-k tensor, and the CSR
``exp_indptr`` of tasks per expert), section "完整 MoE layer" (grouping and the
two-stage GroupGEMM), and Weave MoE article section 1.1 (each token keeps the
top-k experts by router probability; tokens bound for one expert are gathered
into one compact matrix, "token permutation").

Readings taken where the pages are silent (each also listed in the design doc):

* routing: softmax over all experts, keep the k largest, renormalise the kept
  weights to sum to 1 (the usual top-k router; equal to a softmax over the
  kept logits);
* ranking is on the float32 logits (softmax is monotone), descending, ties go
  to the lower expert index, and -0.0 ranks equal to +0.0; slot s of a token
  is its rank;
* grouping is a stable counting sort of the flat index t*k+s by expert, so
  inside one expert's segment rows appear in ascending token order;
* each expert is the gated MLP of ``oracle.mlp`` with its own weights;
* out[t] = sum_{s=0}^{k-1} w[t, s] * y[t, s], summed in slot order.

Pins (tests/test_oracle_moe.py): brute-force search over all ordered k-tuples
for the top-k (with engineered ties and signed zeros), the closed form of the
renormalised weights (softmax restricted to the kept logits) and exact
hand-picked values, grouping invariants plus brute force, k = 1 (out is the
argmax expert's MLP), k = E (weights are the full softmax), identical experts
(the layer reduces to the dense MLP), and sampled-token evaluation equal to
the full evaluation.
"""

import numpy as np

from .mlp import mlp


def route(logits, k):
    """Top-k routing.  logits: [T, E] float32 values.  Returns
    (ids int32 [T, k], w float64 [T, k])."""
    L = np.asarray(logits, dtype=np.float64)
    if L.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # Descending logit, ties -> lower index.  np.lexsort sorts by the last key
    # first; float comparison treats -0.0 and +0.0 as equal, so the index key
    # decides between them.
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -L), axis=-1)
    ids = order[:, :k].astype(np.int32)
    # softmax over all experts, then renormalise the kept probabilities
    m = L.max(axis=1, keepdims=True)
    p = np.exp(L - m)
    p /= p.sum(axis=1, keepdims=True)
    kept = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = kept / kept.sum(axis=1, keepdims=True)
    return ids, w


def group(ids, n_experts):
    """Token grouping.  Returns dict with
    counts [E] (rows routed to each expert), tok_indptr [E+1] (exclusive scan),
    perm [T*k] (perm[pos] = t*k+s, stable by flat index within an expert),
    inv [T, k] (inv[t, s] = pos), all int32."""
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=n_experts)
    if counts.shape[0] != n_experts:
        raise ValueError("expert id out of range")
    tok_indptr = np.zeros(n_experts + 1, dtype=np.int64)
    tok_indptr[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable")
    inv = np.empty(T * k, dtype=np.int64)
    inv[perm] = np.arange(T * k)
    return {
        "counts": counts.astype(np.int32),
        "tok_indptr": tok_indptr.astype(np.int32),
        "perm": perm.astype(np.int32),
        "inv": inv.reshape(T, k).astype(np.int32),
    }


def task_indptr(counts, rows_per_tile, tiles_per_block):
    """CSR of GroupGEMM tasks per expert (the ``exp_indptr`` of Event Tensor
    notes, data-dependent task triggering): expert e owns
    ceil(counts[e] / rows_per_tile) row blocks, each split into
    ``tiles_per_block`` column tiles."""
    counts = np.asarray(counts, dtype=np.int64)
    per = -(-counts // rows_per_tile) * tiles_per_block
    out = np.zeros(counts.shape[0] + 1, dtype=np.int64)
    out[1:] = np.cumsum(per)
    return out.astype(np.int32)


def _expert_weights(weights, e):
    if callable(weights):
        return weights(e)
    wg, wu, wd = weights
    return wg[e], wu[e], wd[e]


def experts_and_combine(x, ids, w, weights, tokens=None):
    """out[t] = sum_s w[t, s] * MLP_{ids[t, s]}(x[t]) for t in ``tokens``
    (default: all tokens).

    weights: either (wg [E,H,I], wu [E,H,I], wd [E,I,H]) logical arrays or a
    callable e -> (wg_e [H,I], wu_e [H,I], wd_e [I,H]), so large expert sets can
    be supplied one expert at a time.  Returns float64 [len(tokens), H]."""
    x = np.asarray(x)
    T, k = ids.shape
    sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    H = x.shape[1]
    y = np.zeros((sel.shape[0], k, H), dtype=np.float64)
    sel_ids = ids[sel]
    for e in np.unique(sel_ids):
        rows, slots = np.nonzero(sel_ids == e)
        wg, wu, wd = _expert_weights(weights, int(e))
        y[rows, slots] = mlp(x[sel[rows]], wg, wu, wd)
    out = np.zeros((sel.shape[0], H), dtype=np.float64)
    wsel = np.asarray(w, dtype=np.float64)[sel]
    for s in range(k):
        out += wsel[:, s:s + 1] * y[:, s, :]
    return out


def moe_layer(logits, x, k, weights, tokens=None):
    """The whole layer.  Returns a dict with ids, w, counts, tok_indptr, perm,
    inv, n_active and out (rows for ``tokens``, default all)."""
    ids, w = route(logits, k)
    E = np.asarray(logits).shape[1]
    g = group(ids, E)
    out = experts_and_combine(x, ids, w, weights, tokens)
    res = {"ids": ids, "w": w, "out": out,
           "n_active": int((g["counts"] > 0).sum())}
    res.update(g)
    return res
