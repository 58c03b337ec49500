// et_api.hip -- the C ABI: workspace planning, argument validation and launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/et.h"
#include "et_device.hpp"
#include "et_launch.hpp"
#include "et_plan.hpp"

namespace et {

RunArgs LaunchCommon::run_args() const {
  RunArgs a;
  std::memset(&a, 0, sizeof(a));
  a.hdr = reinterpret_cast<int*>(ws);
  a.counters = reinterpret_cast<int*>(ws + plan->off_counters);
  a.n_events = plan->n_events;
  a.qctl = reinterpret_cast<int*>(ws + plan->off_slots);
  a.slots = reinterpret_cast<int*>(ws + plan->off_slots + kQCtlBytes);
  a.q_cap = plan->max_tasks;
  a.nq = shards;
  a.runs = (debug & ET_DEBUG_COUNTS) ? reinterpret_cast<int*>(ws + plan->off_runs) : nullptr;
  a.trace = (debug & (ET_DEBUG_TRACE | ET_DEBUG_CLOCK)) ? reinterpret_cast<int*>(ws + plan->off_trace)
                                                       : nullptr;
  a.trace_tasks = (debug & ET_DEBUG_TRACE) ? 1 : 0;
  a.sched = sched;
  a.fetch = fetch;
  a.phase = -1;
  a.timeout = (debug & ET_DEBUG_WATCHDOG_TICK) ? 1 : (long long)timeout_ms * 100000ll;
  a.n_init = 0;
  a.impl_base = 0;
  a.total_hint = kUnknownTotal;
  a.extent = 0;
  return a;
}

// Clears [0, bytes) of the workspace and writes the header (no memset node,
// so the call can also sit in a captured graph).
// Every word is written exactly once, by the one thread whose grid-stride
// loop reaches it, so no two stores to a word race.
__global__ void ws_init_kernel(int* ws, size_t words, int workload) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    ws[i] = i == HDR_MAGIC ? kMagic : i == HDR_WORKLOAD ? workload
          : i == HDR_QTOTAL || i == HDR_QIMPL ? kUnknownTotal : 0;
}

namespace {

std::atomic<int> g_workers[64];   // cached workgroups per device (0 = not yet known)

int workers_for_current_device(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ET_EHIP;
  if (dev < 0 || dev >= 64) return ET_EHIP;
  int g = g_workers[dev].load(std::memory_order_relaxed);
  if (g == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return ET_EHIP;
    if (cus <= 0) return ET_EHIP;
    g = cus;   // one persistent workgroup per compute unit
    g_workers[dev].store(g, std::memory_order_relaxed);
  }
  *out = g;
  return ET_OK;
}

bool valid_sched(int s) { return s >= ET_SCHED_STATIC && s <= ET_SCHED_PER_OP; }

int fill_common(LaunchCommon& lc, void* ws, const et_plan* plan, int sched, const et_opts* o,
                hipStream_t stream, int workload) {
  if (!ws || !plan) return ET_EWORKSPACE;
  if (plan->workload != workload) return ET_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return ET_EWORKSPACE;
  if (!valid_sched(sched)) return ET_EINVAL;
  lc.plan = plan;
  lc.ws = static_cast<char*>(ws);
  lc.sched = sched;
  lc.fetch = o && o->fetch_batch > 0 ? o->fetch_batch : 2;
  if (lc.fetch > kMaxFetch) return ET_EINVAL;
  lc.debug = o ? o->debug_flags : 0;
  lc.timeout_ms = o && o->timeout_ms > 0 ? o->timeout_ms : 2000;
  lc.tile = o ? o->tile : -1;
  if (o && (o->tile < -1 || o->tile >= TV_COUNT)) return ET_EINVAL;
  lc.coop = o ? o->launch : ET_LAUNCH_ORDINARY;
  if (lc.coop != ET_LAUNCH_ORDINARY && lc.coop != ET_LAUNCH_COOPERATIVE) return ET_EINVAL;
  lc.shards = o && o->queue_shards ? o->queue_shards : kMaxShards;
  if (lc.shards != 1 && lc.shards != kMaxShards) return ET_EINVAL;
  lc.qorder = o ? o->queue_order : ET_QORDER_AUTO;
  if (lc.qorder < ET_QORDER_AUTO || lc.qorder > ET_QORDER_STATIC) return ET_EINVAL;
  lc.stream = stream;
  return workers_for_current_device(&lc.G);
}

// Byte offsets of the common regions (header, counters, queue, debug) and the
// total, once n_events, max_tasks and the aux bytes are known.
void finish_plan(et_plan* plan, size_t aux) {
  size_t o = kHdrBytes;
  plan->off_counters = o;
  o = align_up(o + (size_t)2 * plan->n_events * 4, 256);
  plan->off_slots = o;
  o = align_up(o + kQCtlBytes + (size_t)kMaxShards * plan->max_tasks * 4, 256);
  plan->off_runs = o;
  o = align_up(o + (size_t)plan->max_tasks * 4, 256);
  plan->off_trace = o;
  o = align_up(o + (size_t)plan->max_tasks * 16 + 1024 * 16, 256);
  plan->off_aux = o;
  plan->aux_bytes = aux;
  plan->bytes = align_up(o + aux, 256);
}

// MoE dimension checks shared by the MoE layer and the chain.
int check_moe_dims(int max_tokens, int hidden, int inter, int n_experts, int top_k) {
  if (hidden <= 0 || inter <= 0 || n_experts <= 0 || top_k <= 0) return ET_EINVAL;
  if (top_k > n_experts) return ET_EINVAL;
  if (hidden % 128 || inter % 128) return ET_EUNSUPPORTED;
  if (n_experts > kMaxExperts || top_k > kMaxTopK) return ET_EUNSUPPORTED;
  const size_t tk = (size_t)max_tokens * top_k;
  if (tk * inter * 2 >= (1ull << 31) || (size_t)max_tokens * hidden * 2 >= (1ull << 31) ||
      (size_t)inter * hidden * 2 >= (1ull << 31) || tk * hidden * 4 >= (1ull << 31))
    return ET_EUNSUPPORTED;
  MoePlan p{max_tokens, hidden, inter, n_experts, top_k, moe_n_route(n_experts)};
  if ((size_t)p.n_events_max() >= (1ull << 30) || (size_t)p.max_tasks() >= (1ull << 30))
    return ET_EUNSUPPORTED;
  return ET_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Library-held scratch of the allocation-free MoE entry point: the workspace
// (header, counter banks, ready queue, intermediates) of callers that cannot
// allocate device memory.  One copy per device, held until the process ends.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;

}  // namespace et

static __device__ __align__(256) unsigned char scratch[et::kScratchBytes];

namespace et {
namespace {

struct ScratchState {
  void* ptr = nullptr;   // device address of `scratch` on this device
  et_plan plan{};        // plan the scratch is laid out for (bytes == 0: none yet)
};
std::mutex g_scratch_mu;
ScratchState g_scratch[64];

// Address of this device's copy of `scratch`, looked up once per device with
// that device current (the array's name is only a host-side stand-in).
int scratch_for_device(int dev, ScratchState** out) {
  ScratchState& st = g_scratch[dev];
  if (!st.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ET_EHIP;
    if ((reinterpret_cast<uintptr_t>(p) & 255) != 0) return ET_EHIP;
    st.ptr = p;
  }
  *out = &st;
  return ET_OK;
}

}  // namespace
}  // namespace et

using namespace et;

extern "C" {

int et_plan_workspace(int workload, int max_tokens, int hidden, int inter, int n_experts,
                      int top_k, et_plan* plan) {
  if (!plan) return ET_EINVAL;
  std::memset(plan, 0, sizeof(*plan));
  if (max_tokens <= 0) return ET_EINVAL;
  plan->workload = workload;
  plan->max_tokens = max_tokens;
  size_t aux = 0;
  if (workload == ET_WL_SPLITK) {
    if (max_tokens % 32 != 0) return ET_EUNSUPPORTED;
    if (hidden != 0 && hidden != 128) return ET_EUNSUPPORTED;
    if (max_tokens > (1 << 24)) return ET_EUNSUPPORTED;
    SplitKPlan p{max_tokens / 32};
    plan->hidden = 128;
    plan->n_events = p.n_events();
    plan->max_tasks = p.max_tasks();
  } else if (workload == ET_WL_MLP) {
    if (hidden <= 0 || inter <= 0) return ET_EINVAL;
    if (hidden % 128 || inter % 128) return ET_EUNSUPPORTED;
    if ((size_t)inter * hidden * 2 >= (1ull << 31)) return ET_EUNSUPPORTED;
    if ((size_t)max_tokens * (hidden > inter ? hidden : inter) * 4 >= (1ull << 31))
      return ET_EUNSUPPORTED;
    MlpPlan p{max_tokens, hidden, inter};
    plan->hidden = hidden;
    plan->inter = inter;
    plan->n_events = p.n_events_max();
    plan->max_tasks = p.max_tasks();
    aux = (size_t)max_tokens * inter * 2;
  } else if (workload == ET_WL_MOE) {
    const int e = check_moe_dims(max_tokens, hidden, inter, n_experts, top_k);
    if (e) return e;
    MoePlan p{max_tokens, hidden, inter, n_experts, top_k, moe_n_route(n_experts)};
    plan->hidden = hidden;
    plan->inter = inter;
    plan->n_experts = n_experts;
    plan->top_k = top_k;
    plan->n_events = p.n_events_max();
    plan->max_tasks = p.max_tasks();
    aux = moe_aux_layout(p).bytes;
  } else {
    return ET_EINVAL;
  }
  finish_plan(plan, aux);
  return ET_OK;
}

int et_plan_block(int max_tokens, int hidden, int inter, int n_experts, int top_k, int mlp_inter,
                  et_plan* plan) {
  if (!plan) return ET_EINVAL;
  std::memset(plan, 0, sizeof(*plan));
  if (max_tokens <= 0 || mlp_inter <= 0) return ET_EINVAL;
  int e = check_moe_dims(max_tokens, hidden, inter, n_experts, top_k);
  if (e) return e;
  if (mlp_inter % 128) return ET_EUNSUPPORTED;
  if ((size_t)mlp_inter * hidden * 2 >= (1ull << 31) ||
      (size_t)max_tokens * mlp_inter * 2 >= (1ull << 31) ||
      (size_t)max_tokens * n_experts * 4 >= (1ull << 31))
    return ET_EUNSUPPORTED;
  const BlockPlan p{MoePlan{max_tokens, hidden, inter, n_experts, top_k, moe_n_route(n_experts)},
                    mlp_inter};
  if ((size_t)p.n_events_max() >= (1ull << 30) || (size_t)p.max_tasks() >= (1ull << 30))
    return ET_EUNSUPPORTED;
  plan->workload = ET_WL_BLOCK;
  plan->max_tokens = max_tokens;
  plan->hidden = hidden;
  plan->inter = inter;
  plan->n_experts = n_experts;
  plan->top_k = top_k;
  plan->mlp_inter = mlp_inter;
  plan->n_events = p.n_events_max();
  plan->max_tasks = p.max_tasks();
  finish_plan(plan, block_aux_layout(p).bytes);
  return ET_OK;
}

int et_workspace_init(void* ws, const et_plan* plan, hipStream_t stream) {
  if (!ws || !plan || plan->bytes == 0) return ET_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return ET_EWORKSPACE;
  const size_t words = plan->off_aux / 4;   // header, counters, slots, run counts
  hipLaunchKernelGGL(ws_init_kernel, dim3(256), dim3(256), 0, stream, static_cast<int*>(ws),
                     words, plan->workload);
  return hipGetLastError() == hipSuccess ? ET_OK : ET_EHIP;
}

int et_workspace_layout(const et_plan* plan, int n_tokens, et_layout* out) {
  if (!plan || !out) return ET_EINVAL;
  std::memset(out, 0, sizeof(*out));
  out->counters_bank[0] = plan->off_counters;
  out->counters_bank[1] = plan->off_counters + (size_t)plan->n_events * 4;
  out->n_events = plan->n_events;
  out->runs = plan->off_runs;
  out->trace = plan->off_trace;
  if (plan->workload == ET_WL_DECODE) {
    out->q_rot = plan->off_aux;
  } else if (plan->workload == ET_WL_MLP) {
    out->h = plan->off_aux;
  } else if (plan->workload == ET_WL_MOE || plan->workload == ET_WL_BLOCK) {
    MoePlan p{plan->max_tokens, plan->hidden, plan->inter, plan->n_experts, plan->top_k,
              moe_n_route(plan->n_experts)};
    const MoeAux a = moe_aux_layout(p);
    const size_t b = plan->off_aux;
    if (plan->workload == ET_WL_BLOCK) {
      const BlockAux ba = block_aux_layout(BlockPlan{p, plan->mlp_inter});
      out->logits = b + ba.logits;
      out->z = b + ba.zb;
      out->h2 = b + ba.h2;
    }
    out->topk_ids = b + a.topk_ids;
    out->topk_w = b + a.topk_w;
    out->counts = b + a.counts;
    out->tok_indptr = b + a.tok_indptr;
    out->perm = b + a.perm;
    out->inv = b + a.inv;
    out->task_indptr = b + a.task_indptr;
    out->h = b + a.h;
    out->y = b + a.y;
  }
  (void)n_tokens;
  return ET_OK;
}

int et_splitk_reduce(const float* A, int rows, float* Bpart, float* C, void* ws,
                     const et_plan* plan, int sched, const et_opts* opts, hipStream_t stream) {
  LaunchCommon lc;
  int e = fill_common(lc, ws, plan, sched, opts, stream, ET_WL_SPLITK);
  if (e) return e;
  if (rows < 0 || rows % 32 != 0) return ET_EUNSUPPORTED;
  if (rows > plan->max_tokens) return ET_EWORKSPACE;
  if (rows == 0) return ET_OK;
  if (!A || !Bpart || !C) return ET_EINVAL;
  return launch_splitk(lc, A, rows, Bpart, C);
}

int et_mlp(const uint16_t* x, int n_tokens, const uint16_t* w_gate, const uint16_t* w_up,
           const uint16_t* w_down, float* y, void* ws, const et_plan* plan, int sched,
           const et_opts* opts, hipStream_t stream) {
  LaunchCommon lc;
  int e = fill_common(lc, ws, plan, sched, opts, stream, ET_WL_MLP);
  if (e) return e;
  if (n_tokens < 0) return ET_EINVAL;
  if (n_tokens > plan->max_tokens) return ET_EWORKSPACE;
  if (n_tokens == 0) return ET_OK;
  if (!x || !w_gate || !w_up || !w_down || !y) return ET_EINVAL;
  return launch_mlp(lc, x, n_tokens, w_gate, w_up, w_down, y);
}

int et_moe_layer(const float* logits, const uint16_t* x, int n_tokens, const uint16_t* w_gate,
                 const uint16_t* w_up, const uint16_t* w_down, float* out, void* ws,
                 const et_plan* plan, int sched, const et_opts* opts, hipStream_t stream) {
  LaunchCommon lc;
  int e = fill_common(lc, ws, plan, sched, opts, stream, ET_WL_MOE);
  if (e) return e;
  if (n_tokens < 0) return ET_EINVAL;
  if (n_tokens > plan->max_tokens) return ET_EWORKSPACE;
  if (n_tokens == 0) return ET_OK;
  if (!logits || !x || !w_gate || !w_up || !w_down || !out) return ET_EINVAL;
  return launch_moe(lc, logits, x, n_tokens, w_gate, w_up, w_down, out);
}

int et_plan_decode(int max_batch, int n_heads, int n_kv_heads, int head_dim, et_plan* plan) {
  if (!plan) return ET_EINVAL;
  std::memset(plan, 0, sizeof(*plan));
  if (max_batch <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0) return ET_EINVAL;
  if (n_heads % n_kv_heads) return ET_EINVAL;
  if (head_dim != 128 || n_heads / n_kv_heads > 16) return ET_EUNSUPPORTED;
  if ((size_t)max_batch * n_heads * head_dim * 4 >= (1ull << 31) ||
      (size_t)max_batch * n_kv_heads * 11 >= (1ull << 30))
    return ET_EUNSUPPORTED;
  plan->workload = ET_WL_DECODE;
  plan->max_tokens = max_batch;
  plan->hidden = head_dim;
  plan->n_heads = n_heads;
  plan->n_kv_heads = n_kv_heads;
  // events: E_qk and E_att per (sequence, key/value head); tasks: two
  // branches, up to 8 attention splits and a merge per (sequence, head);
  // workspace: rotated queries, then the splits' partial outputs (8 per
  // query head) and their running maxima and sums
  plan->n_events = 8 + 2 * max_batch * n_kv_heads;
  plan->max_tasks = 11 * max_batch * n_kv_heads;
  const size_t qr = (size_t)max_batch * n_heads * head_dim * 4;
  finish_plan(plan, qr + 8 * qr + (size_t)max_batch * n_heads * 8 * 2 * 4);
  return ET_OK;
}

int et_decode_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* q_norm_w, const uint16_t* k_norm_w, const int32_t* pos,
                        int n_seqs, float rope_theta, float eps, uint16_t* k_cache,
                        uint16_t* v_cache, int max_seq, float* out, void* ws,
                        const et_plan* plan, int sched, const et_opts* opts, hipStream_t stream) {
  LaunchCommon lc;
  int e = fill_common(lc, ws, plan, sched, opts, stream, ET_WL_DECODE);
  if (e) return e;
  if (n_seqs < 0 || max_seq <= 0 || !(rope_theta > 1.0f) || !(eps >= 0.0f)) return ET_EINVAL;
  if (n_seqs > plan->max_tokens) return ET_EWORKSPACE;
  if (n_seqs == 0) return ET_OK;
  if (!q || !k || !v || !q_norm_w || !k_norm_w || !pos || !k_cache || !v_cache || !out)
    return ET_EINVAL;
  if ((size_t)n_seqs * max_seq * plan->n_kv_heads * plan->hidden * 2 >= (1ull << 32))
    return ET_EUNSUPPORTED;
  return launch_decode(lc, q, k, v, q_norm_w, k_norm_w, pos, n_seqs, rope_theta, eps, k_cache,
                       v_cache, max_seq, out);
}

int et_moe_block(const uint16_t* x, int n_tokens, const uint16_t* w_router,
                 const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                 const uint16_t* mlp_gate, const uint16_t* mlp_up, const uint16_t* mlp_down,
                 float* moe_out, float* y, void* ws, const et_plan* plan, int sched,
                 const et_opts* opts, hipStream_t stream) {
  LaunchCommon lc;
  int e = fill_common(lc, ws, plan, sched, opts, stream, ET_WL_BLOCK);
  if (e) return e;
  if (n_tokens < 0) return ET_EINVAL;
  if (n_tokens > plan->max_tokens) return ET_EWORKSPACE;
  if (n_tokens == 0) return ET_OK;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !mlp_gate || !mlp_up || !mlp_down ||
      !moe_out || !y)
    return ET_EINVAL;
  return launch_block(lc, x, n_tokens, w_router, w_gate, w_up, w_down, mlp_gate, mlp_up, mlp_down,
                      moe_out, y);
}

int et_read_status(const void* ws, const et_plan* plan, hipStream_t stream, et_report* out) {
  if (!ws || !plan || !out) return ET_EINVAL;
  if (hipStreamSynchronize(stream) != hipSuccess) return ET_EHIP;
  int h[HDR_WORDS];
  if (hipMemcpy(h, ws, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return ET_EHIP;
  std::memset(out, 0, sizeof(*out));
  if (h[HDR_MAGIC] != kMagic) return ET_EWORKSPACE;
  out->status = h[HDR_ERR];
  out->err_info[0] = h[HDR_ERR_A];
  out->err_info[1] = h[HDR_ERR_B];
  out->err_info[2] = h[HDR_ERR_C];
  out->bank = h[HDR_BANK];
  out->calls = h[HDR_CALLS];
  out->last_tasks = h[HDR_LAST_TASKS];
  int qc[kMaxShards * kQCtlStride];
  if (hipMemcpy(qc, static_cast<const char*>(ws) + plan->off_slots, sizeof(qc),
                hipMemcpyDeviceToHost) != hipSuccess)
    return ET_EHIP;
  out->q_head = h[HDR_QHEAD];
  out->q_push = 0;
  for (int q = 0; q < kMaxShards; ++q) {
    out->q_head += qc[q * kQCtlStride];
    out->q_push += qc[q * kQCtlStride + 32];
  }
  out->last_extent = h[HDR_EXT0 + (1 - (h[HDR_BANK] & 1))];
  return ET_OK;
}

int et_moe_layer_noalloc(const float* logits, const uint16_t* x, int n_tokens, int hidden,
                         int inter, int n_experts, int top_k, const uint16_t* w_gate,
                         const uint16_t* w_up, const uint16_t* w_down, float* out, int sched,
                         const et_opts* opts, hipStream_t stream) {
  if (n_tokens < 0) return ET_EINVAL;
  if (n_tokens == 0) return ET_OK;
  if (!logits || !x || !w_gate || !w_up || !w_down || !out) return ET_EINVAL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ET_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState* st = nullptr;
  int e = scratch_for_device(dev, &st);
  if (e) return e;
  const et_plan& cur = st->plan;
  const bool same_dims = cur.bytes != 0 && cur.hidden == hidden && cur.inter == inter &&
                         cur.n_experts == n_experts && cur.top_k == top_k;
  bool init = (opts && (opts->debug_flags & ET_SCRATCH_RESET)) != 0;
  if (!same_dims || n_tokens > cur.max_tokens) {
    // lay the scratch out for a power-of-two token bound (at least 16), so
    // that nearby token counts reuse the layout; fall back to the exact count
    // when the rounded plan does not fit
    int bound = 16;
    while (bound < n_tokens) bound *= 2;
    if (same_dims && cur.max_tokens > bound) bound = cur.max_tokens;
    et_plan p;
    e = et_plan_workspace(ET_WL_MOE, bound, hidden, inter, n_experts, top_k, &p);
    if (e == ET_OK && p.bytes > kScratchBytes)
      e = et_plan_workspace(ET_WL_MOE, n_tokens, hidden, inter, n_experts, top_k, &p);
    if (e) return e;
    if (p.bytes > kScratchBytes) return ET_EWORKSPACE;
    st->plan = p;
    init = true;
  }
  if (init) {
    // header, counter banks, queue and run counts start cleared (a kernel,
    // not a memset node, so the call can also be captured in a graph)
    hipLaunchKernelGGL(ws_init_kernel, dim3(256), dim3(256), 0, stream,
                       static_cast<int*>(st->ptr), st->plan.off_aux / 4, st->plan.workload);
    if (hipGetLastError() != hipSuccess) return ET_EHIP;
  }
  return et_moe_layer(logits, x, n_tokens, w_gate, w_up, w_down, out, st->ptr, &st->plan, sched,
                      opts, stream);
}

const char* et_status_str(int s) {
  switch (s) {
    case ET_OK: return "ok";
    case ET_EINVAL: return "invalid argument";
    case ET_EWORKSPACE: return "workspace missing, too small or planned for other dimensions";
    case ET_EHIP: return "HIP runtime error";
    case ET_ETIMEOUT: return "device wait exceeded the watchdog";
    case ET_EUNSUPPORTED: return "unsupported dimensions";
    case ET_ESTATE: return "event over-notified or ready queue overflow";
    case ET_ERANGE: return "device input index out of range";
    default: return "unknown status";
  }
}

int et_num_workers(void) {
  int g = 0;
  int e = workers_for_current_device(&g);
  return e ? -e : g;
}

}  // extern "C"
