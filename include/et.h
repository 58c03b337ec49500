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
                           consumers, or consumers are queued early and wait on their event;
                           workers claim up to `fetch_batch` queue slots per atomic */
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
  ET_ESTATE = 6,        /* device: an event was over-notified or the ready queue overflowed */
  ET_ERANGE = 7         /* device: an index read from a device input is out of range (a decode
                           position outside the cache) */
};

/* Workloads (a workspace is planned for one of them). */
enum { ET_WL_SPLITK = 1, ET_WL_MLP = 2, ET_WL_MOE = 3, ET_WL_BLOCK = 4, ET_WL_DECODE = 5 };

/* Debug flags. */
enum {
  ET_DEBUG_COUNTS = 1,  /* count how many times each task ran (et_layout.runs) */
  ET_DEBUG_TRACE = 2,   /* record each task's workgroup and start / end time (et_layout.trace) */
  ET_SCRATCH_RESET = 4, /* et_moe_layer_noalloc only: clear the library-held scratch state (event
                           counters, ready queue, sticky fault word) before this call */
  ET_DEBUG_WATCHDOG_TICK = 8, /* watchdog of one 10 ns clock tick instead of timeout_ms, checked
                                 at every poll: a wait that is not satisfied at its first poll
                                 ends the call with ET_ETIMEOUT (tests of the timeout path) */
  ET_DEBUG_CLOCK = 16   /* record only each workgroup's start / end stamps (et_layout.trace's
                           workgroup part): the clock a call ran at, without per-task records */
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
  int fetch_batch;   /* dynamic mode: queue slots claimed per atomic (1..8; default 2) */
  int debug_flags;   /* ET_DEBUG_* (default 0) */
  int timeout_ms;    /* watchdog for every wait / queue spin (default 2000 ms) */
  int tile;          /* MoE / MLP tile-variant override (-1 = chosen from the token count) */
  int launch;        /* ET_LAUNCH_* (default ET_LAUNCH_ORDINARY) */
  int queue_shards;  /* dynamic mode: ready-queue shards, 1 (one central queue) or 8 (one per
                        XCD: a pushed task goes to the shard its weight tile hashes to, and a
                        worker pops only the shard of its own XCD); 0 = default (8) */
  int queue_order;   /* dynamic mode, MoE layer and chain: ET_QORDER_* (default ET_QORDER_AUTO) */
} et_opts;

/* Dynamic schedule of the MoE GEMM tasks (et_opts.queue_order).
 * READY: the scan pushes every gate/up task early (each waits on its expert's
 *   grouping event, E_exp); the notify that completes an expert's gate/up
 *   tiles (E_he) pushes its down tasks, which enter the queue ready to run.
 * STATIC: once the scan knows the row blocks, every gate/up task and then
 *   every down task becomes a queue entry in the static schedule's order, in
 *   the shard of the XCD the static schedule would run it on (the scan
 *   publishes their count; no slots are written); gate/up tasks wait on
 *   E_exp, down tasks on their row block's E_h, and these entries are claimed
 *   one at a time (a shard's consecutive entries are the row blocks sharing a
 *   weight tile, which then stream it side by side).  The early-push form of
 *   the dynamic schedule (Event Tensor notes, section on dynamic scheduling
 *   and its appendix).
 * AUTO: the scan picks, from the routing of the call: READY when one expert
 *   is chosen by at least 90% of the tokens and holds at least 4 row blocks,
 *   else STATIC. */
enum {
  ET_QORDER_AUTO = 0,
  ET_QORDER_READY = 1,
  ET_QORDER_STATIC = 2
};

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
  size_t off_trace;    /* int32 [max_tasks][4] task trace + [1024][2] workgroup start / end times
                          (100 MHz real-time counter) + [1024][2] the shader clock counter at the
                          same points (low 32 bits each; ET_DEBUG_TRACE, ET_DEBUG_CLOCK) */
  size_t off_aux;      /* workload intermediates (see et_layout) */
  size_t aux_bytes;
  int mlp_inter;       /* ET_WL_BLOCK: intermediate size of the dense MLP (else 0) */
  int n_heads;         /* ET_WL_DECODE: query heads Hq (else 0) */
  int n_kv_heads;      /* ET_WL_DECODE: key/value heads Hk (else 0) */
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
  size_t logits;            /* chain: float [T, E] router logits */
  size_t z;                 /* chain: bf16 [T, H] MoE output rounded to bf16 (the MLP's input) */
  size_t h2;                /* chain: bf16 [T, Im] dense MLP h */
  size_t q_rot;             /* decode: float [B, Hq, D] normalised and rotated queries */
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
 * the events of the experts their tokens selected (data-dependent targets); expert e's
 * gate/up tasks tasks[task_indptr[e] : task_indptr[e+1]] wait on that event.  In
 * dynamic mode the GEMM tasks are queued at the scan, in the order
 * et_opts.queue_order selects (ET_QORDER_*).  Deterministic: no float atomics.
 * H and I must be multiples of 128 (checked when the workspace is planned).  The
 * tile variant follows the token count unless et_opts.tile forces one; a forced
 * variant whose column tiles do not divide H or I (the wide variants 3 and 4 cover
 * 256 output columns per down task) returns ET_EUNSUPPORTED and enqueues nothing. */
int et_moe_layer(const float* logits, const uint16_t* x, int n_tokens,
                 const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                 float* out, void* ws, const et_plan* plan, int sched,
                 const et_opts* opts, hipStream_t stream);

/* Plans a workspace for the router GEMM -> MoE layer -> dense MLP chain
 * (et_moe_block): the MoE layer's dimensions as for et_plan_workspace(ET_WL_MOE, ...)
 * plus the dense MLP's intermediate size mlp_inter (a multiple of 128).
 * Returns ET_OK, ET_EINVAL or ET_EUNSUPPORTED. */
int et_plan_block(int max_tokens, int hidden, int inter, int n_experts, int top_k,
                  int mlp_inter, et_plan* plan);

/* Router GEMM -> MoE layer -> dense MLP in ONE persistent launch (Event Tensor
 * notes, section "端到端低 batch serving": the MoE GroupGEMM pipelined with the
 * dense MLP GEMM across stages, the next stage's weights fetched before its
 * activations arrive).
 *   x         bf16 [T, H], T = n_tokens (runtime, <= plan.max_tokens)
 *   w_router  bf16 [E, H]  = W_router [H, E] transposed (row e holds column e)
 *   w_gate, w_up bf16 [E, I, H], w_down bf16 [E, H, I]: the experts, as for et_moe_layer
 *   mlp_gate, mlp_up bf16 [Im, H], mlp_down bf16 [H, Im]: the dense MLP, as for et_mlp
 *   moe_out   float [T, H] out: z = the MoE layer on x with logits = x W_router
 *   y         float [T, H] out: y = (SiLU(z' Wg) * (z' Wu)) Wd, z' = z rounded to bf16
 * The routing task of each token chunk computes the chunk's logits (fp32
 * accumulation; kept in the workspace, et_layout.logits) before ranking them; the
 * combine writes z and its bf16 copy; a dense MLP gate/up tile of a row block waits
 * on the event of that block's combine tiles (E_z, a cross-operator event) after
 * starting its weight stream, and its down tiles wait per 128-column h tile.  All
 * four schedules; the MoE combine always runs as tiles.  Errors as for et_moe_layer. */
int et_moe_block(const uint16_t* x, int n_tokens, const uint16_t* w_router,
                 const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                 const uint16_t* mlp_gate, const uint16_t* mlp_up, const uint16_t* mlp_down,
                 float* moe_out, float* y, void* ws, const et_plan* plan, int sched,
                 const et_opts* opts, hipStream_t stream);

/* Plans a workspace for et_decode_attention: up to max_batch sequences, n_heads
 * query heads sharing n_kv_heads key/value heads (n_heads a multiple of n_kv_heads,
 * at most 16 query heads per key/value head), head_dim 128.
 * Returns ET_OK, ET_EINVAL or ET_EUNSUPPORTED. */
int et_plan_decode(int max_batch, int n_heads, int n_kv_heads, int head_dim, et_plan* plan);

/* One decode step's attention front in ONE persistent launch (Event Tensor notes,
 * section "端到端低 batch serving": the query branch's Norm + RoPE runs in parallel
 * with the key branch's Norm + RoPE + cache append).
 *   q        bf16 [B, Hq, D], k, v bf16 [B, Hk, D]: the new token of each sequence,
 *            B = n_seqs (runtime, <= plan.max_tokens), D = 128
 *   q_norm_w, k_norm_w bf16 [D]: RMSNorm weights, applied per head with `eps`
 *   pos      int32 [B] (device): position of each sequence's new token; the caches
 *            hold positions 0 .. pos[b]-1 and pos[b] < max_seq (else ET_ERANGE on
 *            the device)
 *   k_cache, v_cache bf16 [B, max_seq, Hk, D], updated in place: position pos[b]
 *            receives the rotated key (rounded to bf16) and the value row
 *   out      float [B, Hq, D] out: softmax(q' K^T / sqrt(D)) V over positions
 *            0 .. pos[b], query head j reading key/value head j / (Hq / Hk)
 * q' and k' are RMSNorm(x) * w rotated pairwise: elements (i, i + D/2) by the angle
 * pos * rope_theta^(-2i/D).  Query-branch task (b, h) and key-branch task (b, h)
 * both notify E_qk[b, h] (wait count 2), on which the attention task (b, h) waits;
 * the static and dynamic schedules run the two branches side by side.  Errors as for
 * et_moe_layer. */
int et_decode_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* q_norm_w, const uint16_t* k_norm_w, const int32_t* pos,
                        int n_seqs, float rope_theta, float eps, uint16_t* k_cache,
                        uint16_t* v_cache, int max_seq, float* out, void* ws,
                        const et_plan* plan, int sched, const et_opts* opts, hipStream_t stream);

/* Allocation-free variant of et_moe_layer, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as et_moe_layer, with the layer's
 * dimensions passed directly instead of a workspace: the workspace is a fixed
 * 64 MiB array of device memory held by the library, one copy per device for the
 * life of the process, so the call itself allocates nothing (no hipMalloc, no
 * allocating library routine).  The call lays that array out for the given
 * dimensions and a power-of-two token bound; when the dimensions change or the
 * token count outgrows the bound it re-plans and clears the array's state with a
 * kernel on `stream`.  A layer whose workspace would exceed 64 MiB returns
 * ET_EWORKSPACE and enqueues nothing (64 MiB holds e.g. 1024 tokens of a layer with
 * hidden 2048, 128 experts, top-8, intermediate 768, or 256 tokens of hidden 7168,
 * 256 experts, top-8, intermediate 2048).  Every call on one device shares its
 * array and leaves its contents (routing tensors, intermediates) behind for the
 * next: calls that can overlap in time on one device (two streams) race and must
 * not be issued.  A device fault recorded in the array is sticky, as in a
 * workspace, until a call passes ET_SCRATCH_RESET in opts->debug_flags or
 * re-plans. */
int et_moe_layer_noalloc(const float* logits, const uint16_t* x, int n_tokens, int hidden,
                         int inter, int n_experts, int top_k, const uint16_t* w_gate,
                         const uint16_t* w_up, const uint16_t* w_down, float* out, int sched,
                         const et_opts* opts, hipStream_t stream);

/* Roofline ceilings of the current device (measurement helpers; no workload uses them).
 * et_ceiling_mfma: one workgroup of four waves per compute unit, each wave issuing
 *   `iters` blocks of 32 bf16 MFMAs (v_mfma_f32_16x16x32_bf16, 16384 flops each; 8
 *   independent accumulator chains) on register operands, no memory traffic:
 *   flops = G * 4 * iters * 32 * 16384 for G = et_num_workers().  operands: NULL
 *   (small constants in every lane) or a device buffer (16-byte aligned) of
 *   G * 256 * 32 bytes -- thread t of workgroup w loads its A and B fragments
 *   (16 bytes each) from bytes 32 (256 w + t) .. +32 once.  out: float [G * 4] (one
 *   value per wave, keeps the results live).  stamps: NULL or long long [G * 4] --
 *   per workgroup the shader clock counter and the 100 MHz real-time counter before
 *   and after the loop (clock = shader-counter delta / real-time delta x 100 MHz).
 *   Timing the launch gives the sustained bf16 MFMA rate.
 * et_ceiling_stream: reads `bytes` (a multiple of 16; src 16-byte aligned) with
 *   16-byte loads in a grid-stride loop, G * wgs_per_cu workgroups (1..16 per
 *   compute unit).  out: int [G * wgs_per_cu * 4].  Timing it on a buffer far larger
 *   than the caches gives the sustained HBM read rate.
 * Both enqueue one kernel on `stream` and return ET_OK, ET_EINVAL or ET_EHIP. */
int et_ceiling_mfma(const void* operands, float* out, long long* stamps, int iters,
                    hipStream_t stream);
int et_ceiling_stream(const void* src, size_t bytes, int* out, int wgs_per_cu,
                      hipStream_t stream);

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
