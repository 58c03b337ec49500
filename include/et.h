/*
 * et.h -- C ABI of the Event Tensor megakernel library for MI355X (gfx950).
 *
 * Three operations, each run as ONE persistent HIP kernel whose workgroups
 * (one per compute unit) execute tiled tasks of several operators with no
 * kernel boundary between them.  Tasks synchronise through Event Tensors:
 * device-resident int32 counters with an initial wait count, a notify() that
 * atomically decrements and a wait() that holds until the count is zero
 * (Event Tensor notes = the page "Event Tensor：用“事件张量”编译动态
 * Megakernel", notes.kuangjux.top, section "Event Tensor 抽象").  Tasks are
 * dispatched from per-CU static lists (section "静态调度") or from an on-device
 * ready queue with atomic, batched pop (section "动态调度"; Weave MoE article
 * = "MoE Kernel动态SM调度：从静态分配到任务池", icman.com.cn, section 2.2).
 *
 * Conventions for every entry point below:
 *  - All tensor pointers are DEVICE pointers, owned by the caller.  The
 *    library never allocates, frees or synchronises; work is enqueued on
 *    `stream` and the call returns.
 *  - Scratch state (event counters, ready queue, intermediates) lives in a
 *    caller-allocated workspace described by an et_plan.  Size it with
 *    et_plan_workspace(), allocate plan.bytes of device memory (256-byte
 *    aligned), then call et_workspace_init() once before the first call.
 *    One workspace must not be used by two calls that can overlap in time.
 *  - Synchronous errors (bad arguments, a workspace plan that does not fit
 *    the call) return a nonzero et_status and enqueue nothing.
 *  - Asynchronous faults found on the device (a wait that exceeded the
 *    watchdog, an event that received too many notifies, a full queue) are
 *    recorded in the workspace and reported by et_read_status().  They are
 *    sticky: later calls on that workspace do no work until
 *    et_workspace_init() is called again.
 *  - The token count of a call is a run-time value <= plan.max_tokens: one
 *    compiled library serves every batch size (Event Tensor notes, section
 *    "Shape dynamism").
 *  - bf16 is IEEE bfloat16 stored as uint16_t.
 */
#ifndef ET_H_
#define ET_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Schedule modes. */
enum {
  ET_SCHED_STATIC = 0,  /* per-CU task lists fixed before launch; consumers spin in wait()
                           (data-dependent MoE edges fall back to one coarse event, as the
                           static lowering of the Event Tensor notes does) */
  ET_SCHED_DYNAMIC = 1, /* on-device ready queue; the notify that zeroes an event pushes its
                           consumers; workers claim `fetch_batch` queue slots per atomic */
  ET_SCHED_BARRIER = 2, /* same tasks and code, but one event per operator, i.e. a global
                           barrier between operators (the unfused-megakernel ablation baseline
                           of the Event Tensor notes, section "静态与动态调度的消融") */
  ET_SCHED_PER_OP = 3   /* the same device functions launched as one kernel per operator */
};

/* Status codes. */
enum {
  ET_OK = 0,
  ET_EINVAL = 1,        /* bad argument */
  ET_EWORKSPACE = 2,    /* workspace missing, too small, or planned for other dimensions */
  ET_EHIP = 3,          /* a HIP runtime call failed */
  ET_ETIMEOUT = 4,      /* device: a wait or a queue slot exceeded the watchdog */
  ET_EUNSUPPORTED = 5,  /* dimensions the kernels do not tile (see each entry point) */
  ET_ESTATE = 6         /* device: an event was over-notified or the ready queue overflowed */
};

/* Workloads (a workspace is planned for one of them). */
enum { ET_WL_SPLITK = 1, ET_WL_MLP = 2, ET_WL_MOE = 3 };

/* Debug flags. */
enum {
  ET_DEBUG_COUNTS = 1,  /* count how many times each task ran (et_layout.runs) */
  ET_DEBUG_TRACE = 2    /* record each task's workgroup and start / end time (et_layout.trace) */
};

/* Launch modes of the persistent kernels.  Every workgroup of a persistent
 * launch must be resident at the same time, since tasks wait on each other.
 * The kernels launch one workgroup per compute unit and are sized so that one
 * fits per unit, so an ordinary launch makes them all resident whenever no
 * other kernel holds compute units indefinitely.  A cooperative launch
 * guarantees co-residency even on a shared device, but the runtime separates
 * it from the previous kernel by a device-wide drain (about 20 us on MI355X).
 * Under either mode a workgroup that never becomes resident makes the others'
 * waits end in ET_ETIMEOUT, not a hang. */
enum {
  ET_LAUNCH_ORDINARY = 0,     /* default */
  ET_LAUNCH_COOPERATIVE = 1
};

/* Per-call options; pass NULL for the defaults. */
typedef struct et_opts {
  int fetch_batch;   /* dynamic mode: queue slots claimed per atomic (1..8; default 4) */
  int debug_flags;   /* ET_DEBUG_* (default 0) */
  int timeout_ms;    /* watchdog for every wait / queue spin (default 2000 ms) */
  int tile;          /* MoE / MLP tile-variant override (-1 = chosen from the token count) */
  int launch;        /* ET_LAUNCH_* (default ET_LAUNCH_ORDINARY) */
  int queue_shards;  /* dynamic mode: ready-queue shards, 1 (one central queue) or 8 (one per
                        XCD: a pushed task goes to the shard its weight tile hashes to, workers
                        pop their own XCD's shard first and take from the others when it is
                        empty); 0 = default (8) */
} et_opts;

/* Workspace plan: dimensions and byte offsets of every region.  Filled by
 * et_plan_workspace(); passed unchanged to every call on that workspace. */
typedef struct et_plan {
  int workload;
  int max_tokens;      /* split-K: max rows; MLP: max batch B; MoE: max tokens T */
  int hidden, inter, n_experts, top_k;
  int n_events;        /* counters per bank */
  int max_tasks;       /* upper bound of tasks per call (ready-queue capacity) */
  size_t bytes;        /* total workspace bytes */
  size_t off_counters; /* int32 [2][n_events] event counters (two banks) */
  size_t off_slots;    /* ready queue: int32 [8][64] shard control words (claim and push
                          counters), then int32 [8][max_tasks] slots, one array per shard */
  size_t off_runs;     /* int32 [max_tasks] per-task run counts (ET_DEBUG_COUNTS) */
  size_t off_trace;    /* int32 [max_tasks][4] task trace + [1024][2] workgroup times (ET_DEBUG_TRACE) */
  size_t off_aux;      /* workload intermediates (see et_layout) */
  size_t aux_bytes;
} et_plan;

/* Where to find things inside a workspace after a call (for checks and
 * debugging).  All offsets are bytes from the workspace base. */
typedef struct et_layout {
  size_t counters_bank[2];  /* int32 event counters of each bank */
  int n_events;
  size_t runs;              /* int32 run counts, indexed by task id */
  size_t trace;             /* int32 [max_tasks][4]: workgroup, start, end (100 MHz ticks,
                               low 32 bits), 1; then [1024][2] workgroup start / end */
  size_t topk_ids;          /* MoE: int32 [T, k] */
  size_t topk_w;            /* MoE: float [T, k] renormalised routing weights */
  size_t counts;            /* MoE: int32 [E] rows per expert */
  size_t tok_indptr;        /* MoE: int32 [E+1] */
  size_t perm;              /* MoE: int32 [T*k], perm[pos] = t*k + s */
  size_t inv;               /* MoE: int32 [T, k], inv[t, s] = pos */
  size_t task_indptr;       /* MoE: int32 [E+1] gate/up tasks per expert (CSR) */
  size_t h;                 /* MLP: bf16 [B, I]; MoE: bf16 [T*k, I] (grouped rows) */
  size_t y;                 /* MoE: bf16 [T*k, H] down-projection rows (grouped rows) */
} et_layout;

/* Device-side state of a workspace, read back by et_read_status(). */
typedef struct et_report {
  int status;          /* ET_OK or the sticky device fault */
  int err_info[3];     /* fault details: task id, event index, observed counter */
  int bank;            /* bank the next call will use */
  int calls;           /* completed calls on this workspace */
  int last_tasks;      /* tasks the last call ran (queue total in dynamic mode) */
  int q_head, q_push;  /* ready-queue claim and push counters, summed over the shards
                          (reset after each call) */
  int last_extent;     /* counters used by the last call */
} et_report;

/* Plans a workspace.  dims not used by a workload are ignored (pass 0).
 *   split-K: max_tokens = max rows (multiple of 32), hidden = 128.
 *   MLP:     max_tokens = max batch; hidden H, inter I (multiples of 128).
 *   MoE:     max_tokens = max tokens; hidden H, inter I (multiples of 128);
 *            n_experts E (1..1024); top_k (1..min(E, 16)).
 * Returns ET_OK, ET_EINVAL or ET_EUNSUPPORTED. */
int et_plan_workspace(int workload, int max_tokens, int hidden, int inter,
                      int n_experts, int top_k, et_plan* plan);

/* Clears the workspace state (counters, queue, fault word) on `stream`.
 * Call once after allocation, and again after a device fault. */
int et_workspace_init(void* ws, const et_plan* plan, hipStream_t stream);

/* Offsets of the workspace regions for a call with `n_tokens` tokens. */
int et_workspace_layout(const et_plan* plan, int n_tokens, et_layout* out);

/* Split-K two-stage reduction (Event Tensor notes, section "Split-K reduction 示例").
 *   A     float [rows, 128] row-major, rows a multiple of 32 (runtime, <= plan.max_tokens)
 *   Bpart float [rows, 4] out: Bpart[r, j] = sum_{c<32} A[r, 32j + c]
 *   C     float [rows]    out: C[r] = ((Bpart[r,0] + Bpart[r,1]) + Bpart[r,2]) + Bpart[r,3]
 * Stage-1 task (i, j) (rows 32i..32i+31, slice j) notifies E[i] (wait count 4, map "ij->i");
 * stage-2 task i waits on E[i] (map "i->i"). */
int et_splitk_reduce(const float* A, int rows, float* Bpart, float* C,
                     void* ws, const et_plan* plan, int sched, const et_opts* opts,
                     hipStream_t stream);

/* Dense SiLU-gated MLP chain: y = (SiLU(x Wg) * (x Wu)) Wd, bf16 inputs, fp32 accumulate.
 *   x      bf16 [B, H] row-major, B = n_tokens (runtime, <= plan.max_tokens)
 *   w_gate bf16 [I, H]  = Wg transposed (K-contiguous: row i holds Wg[:, i])
 *   w_up   bf16 [I, H]  = Wu transposed
 *   w_down bf16 [H, I]  = Wd transposed (row n holds Wd[:, n])
 *   y      float [B, H] out
 * h = SiLU(g) * u is rounded to bf16 (the MFMA input of the down projection) in the
 * workspace.  One event per 128-column tile of h gates the down-projection K-slices
 * that read it.  H and I must be multiples of 128 (else ET_EUNSUPPORTED). */
int et_mlp(const uint16_t* x, int n_tokens, const uint16_t* w_gate, const uint16_t* w_up,
           const uint16_t* w_down, float* y, void* ws, const et_plan* plan, int sched,
           const et_opts* opts, hipStream_t stream);

/* MoE layer: routing -> token grouping -> grouped gate/up GEMM -> grouped down GEMM ->
 * weighted combine (Event Tensor notes, sections "Data-dependent event update",
 * "Data-dependent task triggering" and "完整 MoE layer").
 *   logits float [T, E] router logits, T = n_tokens (runtime, <= plan.max_tokens)
 *   x      bf16 [T, H]
 *   w_gate bf16 [E, I, H]  expert e's gate weights transposed (K-contiguous)
 *   w_up   bf16 [E, I, H]
 *   w_down bf16 [E, H, I]
 *   out    float [T, H] out: out[t] = sum_s w[t,s] * MLP_{ids[t,s]}(x[t]) in slot order s
 * Routing keeps the top_k largest logits per token (ties to the lower expert index,
 * -0.0 == +0.0) and renormalises their softmax weights to sum to 1.  Grouping is a
 * stable counting sort of (t, s) by expert.  Routing tensors, counts, CSR offsets and
 * the permutation stay in the workspace (et_workspace_layout).  Grouping tasks notify
 * the events of the experts their tokens selected (data-dependent targets); in dynamic
 * mode the notify that zeroes expert e's event pushes its task range
 * tasks[task_indptr[e] : task_indptr[e+1]].  Deterministic: no float atomics. */
int et_moe_layer(const float* logits, const uint16_t* x, int n_tokens,
                 const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                 float* out, void* ws, const et_plan* plan, int sched,
                 const et_opts* opts, hipStream_t stream);

/* Waits for `stream`, then reads the workspace's device state. */
int et_read_status(const void* ws, const et_plan* plan, hipStream_t stream, et_report* out);

/* Static string for a status code. */
const char* et_status_str(int status);

/* Number of workgroups (= compute units) the persistent kernels launch on the
 * current device, or a negative et_status. */
int et_num_workers(void);

#ifdef __cplusplus
}
#endif
#endif /* ET_H_ */
