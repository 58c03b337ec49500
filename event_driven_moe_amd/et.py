"""Thin Python binding of the C ABI in include/et.h (argument marshalling only).

Every function here checks dtypes, devices and shapes, then passes raw device
pointers and the current HIP stream to libet.so.  All computation happens in
the library's kernels; if libet.so is missing or cannot be loaded the calls
raise, there is no fallback.
"""

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libet.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "et.h")

SCHED_STATIC, SCHED_DYNAMIC, SCHED_BARRIER, SCHED_PER_OP = 0, 1, 2, 3
SCHEDS = {"static": 0, "dynamic": 1, "barrier": 2, "per_op": 3}
OK, EINVAL, EWORKSPACE, EHIP, ETIMEOUT, EUNSUPPORTED, ESTATE, ERANGE = range(8)
WL_SPLITK, WL_MLP, WL_MOE, WL_BLOCK, WL_DECODE = 1, 2, 3, 4, 5
DEBUG_COUNTS, DEBUG_TRACE, SCRATCH_RESET, DEBUG_WATCHDOG_TICK, DEBUG_CLOCK = 1, 2, 4, 8, 16

c_int, c_size_t, c_void_p = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p


class Opts(ctypes.Structure):
    _fields_ = [("fetch_batch", c_int), ("debug_flags", c_int), ("timeout_ms", c_int),
                ("tile", c_int), ("launch", c_int), ("queue_shards", c_int), ("queue_order", c_int)]


class Plan(ctypes.Structure):
    _fields_ = [("workload", c_int), ("max_tokens", c_int), ("hidden", c_int), ("inter", c_int),
                ("n_experts", c_int), ("top_k", c_int), ("n_events", c_int),
                ("max_tasks", c_int), ("bytes", c_size_t), ("off_counters", c_size_t),
                ("off_slots", c_size_t), ("off_runs", c_size_t), ("off_trace", c_size_t),
                ("off_aux", c_size_t),
                ("aux_bytes", c_size_t), ("mlp_inter", c_int), ("n_heads", c_int),
                ("n_kv_heads", c_int)]


class Layout(ctypes.Structure):
    _fields_ = [("counters_bank", c_size_t * 2), ("n_events", c_int), ("runs", c_size_t),
                ("trace", c_size_t),
                ("topk_ids", c_size_t), ("topk_w", c_size_t), ("counts", c_size_t),
                ("tok_indptr", c_size_t), ("perm", c_size_t), ("inv", c_size_t),
                ("task_indptr", c_size_t), ("h", c_size_t), ("y", c_size_t),
                ("logits", c_size_t), ("z", c_size_t), ("h2", c_size_t), ("q_rot", c_size_t)]


class Report(ctypes.Structure):
    _fields_ = [("status", c_int), ("err_info", c_int * 3), ("bank", c_int), ("calls", c_int),
                ("last_tasks", c_int), ("q_head", c_int), ("q_push", c_int),
                ("last_extent", c_int)]


class EtError(RuntimeError):
    def __init__(self, code, what):
        super().__init__("%s: %s (status %d)" % (what, status_str(code), code))
        self.code = code


_lib = None


def lib():
    """Loads libet.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libet.so is not built; run __graft_entry__.build() or "
                               "python -m event_driven_moe_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.et_plan_workspace.argtypes = [c_int] * 6 + [P(Plan)]
        L.et_workspace_init.argtypes = [c_void_p, P(Plan), c_void_p]
        L.et_workspace_layout.argtypes = [P(Plan), c_int, P(Layout)]
        L.et_splitk_reduce.argtypes = [c_void_p, c_int, c_void_p, c_void_p, c_void_p, P(Plan),
                                       c_int, P(Opts), c_void_p]
        L.et_mlp.argtypes = [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             P(Plan), c_int, P(Opts), c_void_p]
        L.et_moe_layer.argtypes = [c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, P(Plan), c_int, P(Opts), c_void_p]
        L.et_plan_block.argtypes = [c_int] * 6 + [P(Plan)]
        L.et_plan_decode.argtypes = [c_int] * 4 + [P(Plan)]
        L.et_decode_attention.argtypes = ([c_void_p] * 6 + [c_int, ctypes.c_float, ctypes.c_float] +
                                          [c_void_p, c_void_p, c_int, c_void_p, c_void_p, P(Plan),
                                           c_int, P(Opts), c_void_p])
        L.et_moe_block.argtypes = [c_void_p, c_int] + [c_void_p] * 10 + [P(Plan), c_int, P(Opts),
                                                                       c_void_p]
        L.et_moe_layer_noalloc.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                           P(Opts), c_void_p]
        L.et_ceiling_mfma.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_void_p]
        L.et_ceiling_stream.argtypes = [c_void_p, c_size_t, c_void_p, c_int, c_void_p]
        L.et_read_status.argtypes = [c_void_p, P(Plan), c_void_p, P(Report)]
        L.et_status_str.argtypes = [c_int]
        L.et_status_str.restype = ctypes.c_char_p
        L.et_num_workers.argtypes = []
        for f in ("et_plan_workspace", "et_workspace_init", "et_workspace_layout",
                  "et_splitk_reduce", "et_mlp", "et_moe_layer", "et_moe_layer_noalloc",
                  "et_plan_block", "et_moe_block", "et_plan_decode", "et_decode_attention",
                  "et_read_status", "et_num_workers", "et_ceiling_mfma", "et_ceiling_stream"):
            getattr(L, f).restype = c_int
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/et.h declares."""
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(et_[a-z_0-9]+)\s*\(", src)))


def status_str(code):
    try:
        return lib().et_status_str(int(code)).decode()
    except RuntimeError:
        return "status %d" % code


def _check(code, what):
    if code != OK:
        raise EtError(code, what)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _ptr(t, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return c_void_p(t.data_ptr())


LAUNCH_ORDINARY, LAUNCH_COOPERATIVE = 0, 1


QORDER = {"auto": 0, "ready": 1, "static": 2}


def _opts(fetch_batch=2, debug=0, timeout_ms=2000, tile=-1, cooperative=False, queue_shards=0,
          queue_order="auto"):
    return Opts(fetch_batch, debug, timeout_ms, tile,
                LAUNCH_COOPERATIVE if cooperative else LAUNCH_ORDINARY, queue_shards,
                QORDER[queue_order])


def plan_workspace(workload, max_tokens, hidden=0, inter=0, n_experts=0, top_k=0, mlp_inter=0,
                   n_heads=0, n_kv_heads=0, head_dim=0):
    p = Plan()
    if workload == WL_DECODE:    # max_tokens: sequences
        _check(lib().et_plan_decode(max_tokens, n_heads, n_kv_heads, head_dim, ctypes.byref(p)),
               "et_plan_decode")
    elif workload == WL_BLOCK:
        _check(lib().et_plan_block(max_tokens, hidden, inter, n_experts, top_k, mlp_inter,
                                   ctypes.byref(p)), "et_plan_block")
    else:
        _check(lib().et_plan_workspace(workload, max_tokens, hidden, inter, n_experts, top_k,
                                       ctypes.byref(p)), "et_plan_workspace")
    return p


class Workspace:
    """Device memory for one workload's event counters, ready queue and
    intermediates, sized by et_plan_workspace and cleared by et_workspace_init."""

    def __init__(self, workload, max_tokens, hidden=0, inter=0, n_experts=0, top_k=0,
                 device="cuda", stream=None, mlp_inter=0, n_heads=0, n_kv_heads=0, head_dim=0):
        self.plan = plan_workspace(workload, max_tokens, hidden, inter, n_experts, top_k,
                                   mlp_inter, n_heads, n_kv_heads, head_dim)
        self.buf = torch.empty(self.plan.bytes, dtype=torch.uint8, device=device)
        self.init(stream)

    def init(self, stream=None):
        _check(lib().et_workspace_init(c_void_p(self.buf.data_ptr()), ctypes.byref(self.plan),
                                       _stream(stream)), "et_workspace_init")

    @property
    def ptr(self):
        return c_void_p(self.buf.data_ptr())

    def layout(self, n_tokens=0):
        lay = Layout()
        _check(lib().et_workspace_layout(ctypes.byref(self.plan), n_tokens, ctypes.byref(lay)),
               "et_workspace_layout")
        return lay

    def view(self, offset, dtype, count):
        """A typed view of `count` elements at byte `offset` of the workspace."""
        nbytes = torch.empty((), dtype=dtype).element_size() * count
        return self.buf[offset:offset + nbytes].view(dtype)

    def status(self, stream=None):
        r = Report()
        _check(lib().et_read_status(self.ptr, ctypes.byref(self.plan), _stream(stream),
                                    ctypes.byref(r)), "et_read_status")
        return {"status": r.status, "err_info": list(r.err_info), "bank": r.bank,
                "calls": r.calls, "last_tasks": r.last_tasks, "q_head": r.q_head,
                "q_push": r.q_push, "last_extent": r.last_extent}

    def counters(self, bank):
        lay = self.layout()
        return self.view(lay.counters_bank[bank], torch.int32, lay.n_events)

    def runs(self):
        lay = self.layout()
        return self.view(lay.runs, torch.int32, self.plan.max_tasks)

    def trace(self):
        """(tasks [max_tasks, 4]: workgroup, start, end, valid; workgroups [1024, 2]:
        start, end) in 100 MHz ticks (low 32 bits), from ET_DEBUG_TRACE calls."""
        lay = self.layout()
        n = self.plan.max_tasks
        t = self.view(lay.trace, torch.int32, 4 * n + 4096)
        return t[:4 * n].view(n, 4), t[4 * n:4 * n + 2048].view(1024, 2)

    def clock_stamps(self):
        """Workgroups [1024, 2, 2]: (start, end) x (100 MHz real-time counter,
        shader clock counter), low 32 bits, from ET_DEBUG_TRACE or
        ET_DEBUG_CLOCK calls."""
        lay = self.layout()
        n = self.plan.max_tasks
        t = self.view(lay.trace, torch.int32, 4 * n + 4096)
        return torch.stack([t[4 * n:4 * n + 2048].view(1024, 2),
                            t[4 * n + 2048:].view(1024, 2)], dim=2)


def splitk_reduce(A, Bpart, C, ws, sched="static", stream=None, **opts):
    rows = A.shape[0]
    a = _ptr(A, torch.float32, "A", (rows, 128))
    b = _ptr(Bpart, torch.float32, "Bpart", (rows, 4))
    c = _ptr(C, torch.float32, "C", (rows,))
    o = _opts(**opts)
    _check(lib().et_splitk_reduce(a, rows, b, c, ws.ptr, ctypes.byref(ws.plan),
                                  SCHEDS.get(sched, sched), ctypes.byref(o), _stream(stream)),
           "et_splitk_reduce")


def mlp(x, w_gate, w_up, w_down, y, ws, sched="static", stream=None, **opts):
    """x bf16 [B,H]; w_gate/w_up bf16 [I,H] (K-contiguous); w_down bf16 [H,I]; y f32 [B,H]."""
    B, H = x.shape
    I = w_gate.shape[0]
    args = (_ptr(x, torch.bfloat16, "x", (B, H)), B,
            _ptr(w_gate, torch.bfloat16, "w_gate", (I, H)),
            _ptr(w_up, torch.bfloat16, "w_up", (I, H)),
            _ptr(w_down, torch.bfloat16, "w_down", (H, I)),
            _ptr(y, torch.float32, "y", (B, H)))
    if (H, I) != (ws.plan.hidden, ws.plan.inter):
        raise ValueError("weights do not match the workspace plan")
    o = _opts(**opts)
    _check(lib().et_mlp(*args, ws.ptr, ctypes.byref(ws.plan), SCHEDS.get(sched, sched),
                        ctypes.byref(o), _stream(stream)), "et_mlp")


def moe_layer(logits, x, w_gate, w_up, w_down, out, ws, sched="dynamic", stream=None, **opts):
    """logits f32 [T,E]; x bf16 [T,H]; w_gate/w_up bf16 [E,I,H]; w_down bf16 [E,H,I];
    out f32 [T,H]."""
    T, E = logits.shape
    H = x.shape[1]
    I = w_gate.shape[1]
    args = (_ptr(logits, torch.float32, "logits", (T, E)), _ptr(x, torch.bfloat16, "x", (T, H)),
            T, _ptr(w_gate, torch.bfloat16, "w_gate", (E, I, H)),
            _ptr(w_up, torch.bfloat16, "w_up", (E, I, H)),
            _ptr(w_down, torch.bfloat16, "w_down", (E, H, I)),
            _ptr(out, torch.float32, "out", (T, H)))
    if (H, I, E) != (ws.plan.hidden, ws.plan.inter, ws.plan.n_experts):
        raise ValueError("weights do not match the workspace plan")
    o = _opts(**opts)
    _check(lib().et_moe_layer(*args, ws.ptr, ctypes.byref(ws.plan), SCHEDS.get(sched, sched),
                              ctypes.byref(o), _stream(stream)), "et_moe_layer")


def moe_block(x, w_router, w_gate, w_up, w_down, mlp_gate, mlp_up, mlp_down, moe_out, y, ws,
              sched="static", stream=None, **opts):
    """x bf16 [T,H]; w_router bf16 [E,H]; experts as for moe_layer; dense MLP
    mlp_gate/mlp_up bf16 [Im,H], mlp_down bf16 [H,Im]; moe_out, y f32 [T,H]."""
    T, H = x.shape
    E = w_router.shape[0]
    I = w_gate.shape[1]
    Im = mlp_gate.shape[0]
    if (H, I, E, Im) != (ws.plan.hidden, ws.plan.inter, ws.plan.n_experts, ws.plan.mlp_inter):
        raise ValueError("weights do not match the workspace plan")
    args = (_ptr(x, torch.bfloat16, "x", (T, H)), T,
            _ptr(w_router, torch.bfloat16, "w_router", (E, H)),
            _ptr(w_gate, torch.bfloat16, "w_gate", (E, I, H)),
            _ptr(w_up, torch.bfloat16, "w_up", (E, I, H)),
            _ptr(w_down, torch.bfloat16, "w_down", (E, H, I)),
            _ptr(mlp_gate, torch.bfloat16, "mlp_gate", (Im, H)),
            _ptr(mlp_up, torch.bfloat16, "mlp_up", (Im, H)),
            _ptr(mlp_down, torch.bfloat16, "mlp_down", (H, Im)),
            _ptr(moe_out, torch.float32, "moe_out", (T, H)),
            _ptr(y, torch.float32, "y", (T, H)))
    o = _opts(**opts)
    _check(lib().et_moe_block(*args, ws.ptr, ctypes.byref(ws.plan), SCHEDS.get(sched, sched),
                              ctypes.byref(o), _stream(stream)), "et_moe_block")


def decode_attention(q, k, v, q_norm_w, k_norm_w, pos, k_cache, v_cache, out, ws,
                     sched="static", rope_theta=1e6, eps=1e-6, stream=None, **opts):
    """q bf16 [B,Hq,D]; k, v bf16 [B,Hk,D]; norm weights bf16 [D]; pos int32 [B];
    caches bf16 [B,S,Hk,D] (updated in place); out f32 [B,Hq,D]."""
    B, Hq, D = q.shape
    Hk = k.shape[1]
    S = k_cache.shape[1]
    if (Hq, Hk, D) != (ws.plan.n_heads, ws.plan.n_kv_heads, ws.plan.hidden):
        raise ValueError("heads do not match the workspace plan")
    args = (_ptr(q, torch.bfloat16, "q", (B, Hq, D)), _ptr(k, torch.bfloat16, "k", (B, Hk, D)),
            _ptr(v, torch.bfloat16, "v", (B, Hk, D)), _ptr(q_norm_w, torch.bfloat16, "q_norm_w", (D,)),
            _ptr(k_norm_w, torch.bfloat16, "k_norm_w", (D,)), _ptr(pos, torch.int32, "pos", (B,)),
            B, float(rope_theta), float(eps),
            _ptr(k_cache, torch.bfloat16, "k_cache", (B, S, Hk, D)),
            _ptr(v_cache, torch.bfloat16, "v_cache", (B, S, Hk, D)), S,
            _ptr(out, torch.float32, "out", (B, Hq, D)))
    o = _opts(**opts)
    _check(lib().et_decode_attention(*args, ws.ptr, ctypes.byref(ws.plan), SCHEDS.get(sched, sched),
                                     ctypes.byref(o), _stream(stream)), "et_decode_attention")


def decode_q_rot(ws, B):
    """The normalised, rotated queries of the last decode call (float [B, Hq, D])."""
    lay = ws.layout(B)
    Hq, D = ws.plan.n_heads, ws.plan.hidden
    return ws.view(lay.q_rot, torch.float32, B * Hq * D).view(B, Hq, D)


def block_aux(ws, T):
    """The chain's intermediates of the last call: router logits (float
    [T, E]), the MoE output in bf16 (the dense MLP's input, [T, H]) and the
    dense MLP's h (bf16 [T, Im]), plus the MoE routing views of moe_aux."""
    lay = ws.layout(T)
    E, H, Im = ws.plan.n_experts, ws.plan.hidden, ws.plan.mlp_inter
    aux = moe_aux(ws, T)
    aux["logits"] = ws.view(lay.logits, torch.float32, T * E).view(T, E)
    aux["z"] = ws.view(lay.z, torch.bfloat16, T * H).view(T, H)
    aux["h2"] = ws.view(lay.h2, torch.bfloat16, T * Im).view(T, Im)
    return aux


def moe_layer_noalloc(logits, x, w_gate, w_up, w_down, out, sched="dynamic", stream=None,
                      **opts):
    """The allocation-free entry point: same tensors as moe_layer, no
    workspace (the library holds a fixed 64 MiB scratch array per device)."""
    T, E = logits.shape
    H = x.shape[1]
    I = w_gate.shape[1]
    k = opts.pop("top_k")
    args = (_ptr(logits, torch.float32, "logits", (T, E)), _ptr(x, torch.bfloat16, "x", (T, H)),
            T, H, I, E, k, _ptr(w_gate, torch.bfloat16, "w_gate", (E, I, H)),
            _ptr(w_up, torch.bfloat16, "w_up", (E, I, H)),
            _ptr(w_down, torch.bfloat16, "w_down", (E, H, I)),
            _ptr(out, torch.float32, "out", (T, H)))
    o = _opts(**opts)
    _check(lib().et_moe_layer_noalloc(*args, SCHEDS.get(sched, sched), ctypes.byref(o),
                                      _stream(stream)), "et_moe_layer_noalloc")


def moe_aux(ws, T, intermediates=False):
    """Routing results and grouping of the last call (views into the workspace);
    with ``intermediates``, also h (bf16 [T*k, I]) and y (bf16 [T*k, H]), the
    grouped rows of the two projections."""
    lay = ws.layout(T)
    k, E = ws.plan.top_k, ws.plan.n_experts
    aux = {
        "ids": ws.view(lay.topk_ids, torch.int32, T * k).view(T, k),
        "w": ws.view(lay.topk_w, torch.float32, T * k).view(T, k),
        "counts": ws.view(lay.counts, torch.int32, E),
        "tok_indptr": ws.view(lay.tok_indptr, torch.int32, E + 1),
        "perm": ws.view(lay.perm, torch.int32, T * k),
        "inv": ws.view(lay.inv, torch.int32, T * k).view(T, k),
        "task_indptr": ws.view(lay.task_indptr, torch.int32, E + 1),
    }
    if intermediates:
        aux["h"] = ws.view(lay.h, torch.bfloat16, T * k * ws.plan.inter).view(T * k, ws.plan.inter)
        aux["y"] = ws.view(lay.y, torch.bfloat16, T * k * ws.plan.hidden).view(T * k, ws.plan.hidden)
    return aux


def ceiling_mfma(out, iters, operands=None, stamps=None, stream=None):
    """Enqueues the MFMA-only microbenchmark (out: float32 [G*4] device tensor;
    operands: None or a bf16 device tensor of G*256*16 elements, the
    fragments each lane loads; stamps: None or an int64 [G*4] device tensor
    that receives shader-clock / real-time stamps around the loop)."""
    if operands is not None and (operands.dtype != torch.bfloat16 or not operands.is_cuda
                                 or not operands.is_contiguous()
                                 or operands.numel() < num_workers() * 256 * 16):
        raise ValueError("operands must be a contiguous bf16 device tensor of G*256*16 elements")
    if stamps is not None and stamps.numel() < num_workers() * 4:
        raise ValueError("stamps must hold G*4 int64 values")
    ops = c_void_p(operands.data_ptr()) if operands is not None else None
    st = _ptr(stamps, torch.int64, "stamps") if stamps is not None else None
    _check(lib().et_ceiling_mfma(ops, _ptr(out, torch.float32, "out"), st, iters, _stream(stream)),
           "et_ceiling_mfma")


def ceiling_stream(src, out, wgs_per_cu=4, stream=None):
    """Enqueues the streaming-read microbenchmark over the bytes of ``src``
    (out: int32 [G*wgs_per_cu*4] device tensor)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _check(lib().et_ceiling_stream(c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                   _ptr(out, torch.int32, "out"), wgs_per_cu, _stream(stream)),
           "et_ceiling_stream")


def num_workers():
    n = lib().et_num_workers()
    if n < 0:
        raise EtError(-n, "et_num_workers")
    return n
