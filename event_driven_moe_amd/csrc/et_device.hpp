// et_device.hpp -- device side of the Event Tensor runtime for gfx950.
//
// Event Tensors (Event Tensor notes = page "Event Tensor：用“事件张量”编译动态
// Megakernel", notes.kuangjux.top, sections "Event Tensor 抽象" and "Minimal
// runtime") lower to plain int32 arrays: notify() is an atomic decrement,
// wait() holds until the count is zero, and under dynamic scheduling the
// notify that zeroes a count pushes the event's consumers to a ready queue
// (section "动态调度").  The only mutable run-time state is the counters and
// the queue.
//
// Storage choice: a counter is stored RELATIVE to its wait count, i.e. the
// stored value is (count - wait_count).  Every event is therefore armed by the
// same value, 0, whatever its wait count, which may depend on the run-time
// token count (symbolic event shapes) or on routing results (data-dependent
// counts); the wait count is supplied by whoever waits or notifies, and an
// event has fired when its stored value equals -wait_count.  Counters live in
// two banks: a call uses one bank and, in its prologue, re-arms (zeroes) the
// part of the other bank that the previous call used; the last workgroup to
// leave flips the bank.  No host memset and no grid barrier are needed.
//
// Memory ordering: producers and consumers run on different compute units,
// often on different XCDs with separate L2 caches.  Agent-scope fences would
// write back and invalidate a whole XCD's L2 at every notify and wait, which
// destroys the L2 reuse the GEMM tasks depend on.  Instead, every access to
// data that another workgroup of the same launch produced or will consume
// (intermediates, routing results, counters, queue slots) is itself
// agent-coherent -- the sc1 loads and stores that agent-scope monotonic
// atomics lower to -- and notify() first waits until all of the workgroup's
// stores have completed (s_waitcnt vmcnt(0) in every wave, then the workgroup
// barrier) before the decrement.  A consumer that observes the fired counter
// then reads the producers' data with coherent loads.  Inputs that no task
// writes (x, weights, logits) use ordinary cached loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/et.h"
#include "et_plan.hpp"

namespace et {

// ---------------------------------------------------------------------------
// agent-coherent accesses (agent scope = the whole GPU)
// ---------------------------------------------------------------------------
__device__ __forceinline__ long long now_ticks() {
  return (long long)__builtin_amdgcn_s_memrealtime();   // constant 100 MHz clock
}
template <class T>
__device__ __forceinline__ T ld_coh(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void st_coh(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_rlx(const int* p) { return ld_coh(p); }
__device__ __forceinline__ void st_rlx(int* p, int v) { st_coh(p, v); }
__device__ __forceinline__ int add_rlx(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// per-call arguments and context
// ---------------------------------------------------------------------------
struct RunArgs {
  int* hdr;            // workspace header words (HDR_*)
  int* counters;       // bank 0; bank 1 starts n_events later
  int n_events;
  int* qctl;           // ready-queue shard control words (claimed / pushed per shard)
  int* slots;          // ready-queue slots, [kMaxShards][q_cap] (implicit initial tasks need none)
  int q_cap;
  int nq;              // ready-queue shards in use (1 or kMaxShards)
  int* runs;           // per-task run counts, or nullptr
  int* trace;          // trace records (per workgroup, and per task if trace_tasks), or nullptr
  int trace_tasks;     // record per-task trace entries
  int sched;           // ET_SCHED_*
  int fetch;           // dynamic: slots claimed per atomic
  int phase;           // per-op mode: operator this launch runs
  long long timeout;   // watchdog, 100 MHz ticks
  int init_base;       // dynamic: tasks [0, init_base) run on workgroups w, w + G, ... directly
  int n_init;          // dynamic: tasks [init_base, init_base + n_init) are in the queue from the start
  int impl_base;       // dynamic: > 0: static-order implicit tasks impl_base + p, p < HDR_QIMPL
                       // (published during the call), ahead of each shard's pushed slots
  int n_single;        // dynamic: slots below this index are claimed one at a time
  int total_hint;      // dynamic: total tasks when known at launch, else kUnknownTotal
  int extent;          // counters this call uses (a prefix of its bank)
};

// Workgroup-shared scratch for broadcasts and keyed pushes.
constexpr int kMaxFetch = 8;   // largest claim batch (fetch_batch)

struct Shared {
  int v[8];
  int bids[kMaxFetch];    // pop: the slot values of the claimed batch, read together
  int qn[kMaxShards];     // push: tasks per shard, then slots filled so far
  int qb[kMaxShards];     // push: first slot per shard
  int wq[kThreads / 64][kMaxShards];   // push: items per wave and shard in a round
};

struct Ctx {
  RunArgs a;
  int* ev;             // this call's bank
  int gen;             // this call's generation (completed calls + 1): broadcast flag value
  int wg, G;
  Shared* sh;
};

__device__ __forceinline__ void raise_fault(const RunArgs& a, int code, int x, int y, int v) {
  int expected = 0;
  if (__hip_atomic_compare_exchange_strong(&a.hdr[HDR_ERR], &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    st_rlx(&a.hdr[HDR_ERR_A], x);
    st_rlx(&a.hdr[HDR_ERR_B], y);
    st_rlx(&a.hdr[HDR_ERR_C], v);
  }
}

__device__ __forceinline__ bool faulted(const RunArgs& a) { return ld_rlx(&a.hdr[HDR_ERR]) != 0; }

// Thread 0's value to the whole workgroup (two barriers so the slot can be reused).
__device__ __forceinline__ int wg_bcast(const Ctx& c, int v, int slot = 0) {
  if (threadIdx.x == 0) c.sh->v[slot] = v;
  __syncthreads();
  int r = c.sh->v[slot];
  __syncthreads();
  return r;
}

// Spin (thread 0 only) until counter `idx` of this call's bank reaches
// -wait_count.  Returns 1, or 0 after a fault (own or another workgroup's).
__device__ __forceinline__ int spin_until(const Ctx& c, int idx, int wait_count, int task) {
  const int* p = c.ev + idx;
  const int target = -wait_count;
  int v = ld_rlx(p);
  if (v == target) return 1;
  long long t0 = now_ticks();
  for (int it = 1;; ++it) {
    if (v < target) {
      raise_fault(c.a, ET_ESTATE, task, idx, v);
      return 0;
    }
    __builtin_amdgcn_s_sleep(1);
    v = ld_rlx(p);
    if (v == target) return 1;
    if ((it & 63) == 0 || c.a.timeout <= 1) {   // one-tick watchdog: check every poll
      if (faulted(c.a)) return 0;
      if (now_ticks() - t0 > c.a.timeout) {
        raise_fault(c.a, ET_ETIMEOUT, task, idx, v);
        return 0;
      }
    }
  }
}

// wait(): the whole workgroup holds until event `idx` has received
// `wait_count` notifies.  Returns false when the call is being abandoned.
__device__ __forceinline__ bool wg_wait(const Ctx& c, int idx, int wait_count, int task) {
  int ok = 1;
  if (threadIdx.x == 0) ok = spin_until(c, idx, wait_count, task);
  return wg_bcast(c, ok, 1) != 0;
}

// Several consecutive events at once (all must fire): the lanes of wave 0
// check up to 64 counters per memory round trip.
__device__ __forceinline__ int spin_until_all(const Ctx& c, int first, int n, int wait_count,
                                           int task) {
  const int lane = threadIdx.x & 63;
  const int target = -wait_count;
  long long t0 = 0;
  for (int base = 0; base < n; base += 64) {
    const int idx = first + base + lane;
    const bool mine = base + lane < n;
    for (int it = 0;; ++it) {
      const int v = mine ? ld_rlx(c.ev + idx) : target;
      if (v < target) raise_fault(c.a, ET_ESTATE, task, idx, v);
      const unsigned long long pending = __ballot(v != target);
      if (pending == 0) break;
      if (__ballot(v < target) != 0) return 0;
      if (it == 0) t0 = now_ticks();
      __builtin_amdgcn_s_sleep(1);
      if ((it & 63) == 63 || c.a.timeout <= 1) {
        if (faulted(c.a)) return 0;
        if (now_ticks() - t0 > c.a.timeout) {
          if (lane == 0) raise_fault(c.a, ET_ETIMEOUT, task, first + base, n);
          return 0;
        }
      }
    }
  }
  return 1;
}

__device__ __forceinline__ bool wg_wait_range(const Ctx& c, int first, int n, int wait_count,
                                              int task) {
  int ok = 1;
  if (threadIdx.x < 64) ok = spin_until_all(c, first, n, wait_count, task);
  return wg_bcast(c, ok, 1) != 0;
}

// Non-blocking: have all of events [first, first + n) fired?  One memory
// round trip per 64 events (wave 0's lanes), result broadcast.
__device__ __forceinline__ bool wg_probe_range(const Ctx& c, int first, int n, int wait_count) {
  int all = 1;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (int base = 0; base < n && all; base += 64) {
      const bool mine = base + lane < n;
      const int v = mine ? ld_rlx(c.ev + first + base + lane) : -wait_count;
      all = __ballot(v != -wait_count) == 0;
    }
  }
  return wg_bcast(c, all, 1) != 0;
}

// Non-blocking: how many of events [first, first + n), counted from the
// first, have fired?  One memory round trip per 64 events (wave 0's lanes),
// result broadcast.
__device__ __forceinline__ int wg_probe_prefix(const Ctx& c, int first, int n, int wait_count) {
  int done = n;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (int base = 0; base < n; base += 64) {
      const bool mine = base + lane < n;
      const int v = mine ? ld_rlx(c.ev + first + base + lane) : -wait_count;
      const unsigned long long pending = __ballot(v != -wait_count);
      if (pending != 0) {
        done = base + __builtin_ctzll(pending);
        break;
      }
    }
  }
  return wg_bcast(c, done, 1);
}

// Complete this workgroup's stores (every wave), then synchronise the
// workgroup.  Precedes every notify and push.
__device__ __forceinline__ void wg_release() {
  wait_mem();
  __syncthreads();
}

// notify(): decrement event `idx` by n.  Must follow wg_release().  Returns
// (to every thread) whether this notify fired the event, i.e. brought it to
// its wait count; every other notifier had completed its stores before its
// own decrement, so the firing workgroup may push or run the consumers.
__device__ __forceinline__ bool wg_notify(const Ctx& c, int idx, int n, int wait_count, int task) {
  int fired = 0;
  if (threadIdx.x == 0) {
    int* p = c.ev + idx;
    int old = add_rlx(p, -n);
    int now = old - n;
    if (now < -wait_count) raise_fault(c.a, ET_ESTATE, task, idx, now);
    fired = now == -wait_count;
  }
  return wg_bcast(c, fired, 2) != 0;
}

// Thread-0-only notify (no broadcast, no returned value): fire-and-forget
// after wg_release().  Over-notification is still caught by the waiter.
__device__ __forceinline__ void t0_notify(const Ctx& c, int idx, int n, int wait_count, int task) {
  (void)wait_count;
  (void)task;
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(c.ev + idx, -n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Broadcast events.  A coarse event that many workgroups wait on (every
// routing chunk, the scan, every grouping chunk, every gate/up or down tile)
// is not polled on its counter: the notify that completes the counter writes
// this call's generation into the kBcastLines flag lines of the event's slot,
// and each waiter polls the line of its own workgroup (wg mod kBcastLines).
// With all waiters polling one counter, their loads queued at one address and
// a waiter saw the event 2-4 us after it fired.  The flags need no arming:
// a line holds the generation of the last call that fired its event, and
// the generation grows with every call (the epilogue counts the calls).  The
// counter is still decremented, so its final value is checked as for any
// other event.  Every notify of such an event must use t0_notify_bcast.
__device__ __forceinline__ int* bcast_line(const Ctx& c, int slot, int line) {
  return c.a.hdr + HDR_FLAGS + (slot * kBcastLines + line) * 32;
}

// Whole workgroup, after wg_release(): wave 0 notifies; when its decrement
// completes the event, its 64 lanes write the 64 flag lines.
__device__ __forceinline__ void t0_notify_bcast(const Ctx& c, int idx, int slot, int n,
                                                int wait_count, int task) {
  static_assert(kBcastLines == 64, "one flag line per lane of wave 0");
  if (threadIdx.x < 64) {
    int old = 0;
    if (threadIdx.x == 0) old = add_rlx(c.ev + idx, -n);
    const int now = __builtin_amdgcn_readfirstlane(old) - n;
    if (now == -wait_count)
      st_rlx(bcast_line(c, slot, threadIdx.x), c.gen);
    else if (now < -wait_count && threadIdx.x == 0)
      raise_fault(c.a, ET_ESTATE, task, idx, now);
  }
}

// Thread 0 polls its workgroup's flag line of `slot` until it holds this
// call's generation.  Returns 1, or 0 after a fault or the watchdog.
__device__ __forceinline__ int spin_flag(const Ctx& c, int idx, int slot, int task) {
  const int* p = bcast_line(c, slot, c.wg % kBcastLines);
  if (ld_rlx(p) == c.gen) return 1;
  const long long t0 = now_ticks();
  for (int it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    if (ld_rlx(p) == c.gen) return 1;
    if ((it & 63) == 0 || c.a.timeout <= 1) {   // one-tick watchdog: check every poll
      if (faulted(c.a)) return 0;
      if (now_ticks() - t0 > c.a.timeout) {
        raise_fault(c.a, ET_ETIMEOUT, task, idx, ld_rlx(c.ev + idx));
        return 0;
      }
    }
  }
}

// wait() on a broadcast event: the whole workgroup holds until it fired.
__device__ __forceinline__ bool wg_wait_bcast(const Ctx& c, int idx, int slot, int task) {
  int ok = 1;
  if (threadIdx.x == 0) ok = spin_flag(c, idx, slot, task);
  return wg_bcast(c, ok, 1) != 0;
}

__device__ __forceinline__ int* q_claimed(const RunArgs& a, int q) { return a.qctl + q * kQCtlStride; }
__device__ __forceinline__ int* q_pushed(const RunArgs& a, int q) {
  return a.qctl + q * kQCtlStride + 32;
}

// push(): append tasks id_of(0..n-1) to the ready queue; task i goes to shard
// key_of(i) mod nq, so tasks with equal keys (those that read the same weight
// tile) are claimed by workers of one XCD and share its L2.  Whole
// workgroup; must follow wg_release() (or a fired wg_notify) so the pushed
// tasks' inputs are complete before their slots are published.  One atomic
// per shard reserves the slots, then each slot is written, each shard's in
// push order; a claimer that finds a reserved slot still empty waits for the
// write.
template <class F, class K>
__device__ __forceinline__ void wg_push(const Ctx& c, int n, F id_of, K key_of) {
  if (n <= 0) return;
  const int nq = c.a.nq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kMaxShards) c.sh->qn[tid] = 0;
  __syncthreads();
  if (nq > 1)
    for (int i = tid; i < n; i += kThreads) atomicAdd(&c.sh->qn[key_of(i) & (kMaxShards - 1)], 1);
  else if (tid == 0)
    c.sh->qn[0] = n;
  __syncthreads();
  if (tid < nq) {
    const int k = c.sh->qn[tid];
    c.sh->qb[tid] = k ? add_rlx(q_pushed(c.a, tid), k) : 0;
    c.sh->qn[tid] = 0;
  }
  __syncthreads();
  // Slots in push order: item i takes its shard's next slot in index order
  // (rank among the round's earlier items of the same shard: a ballot per
  // shard within the wave, plus the counts of the waves before it).
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = 0; i0 < n; i0 += kThreads) {
    const int i = i0 + tid;
    const int q = i < n ? (nq > 1 ? (key_of(i) & (kMaxShards - 1)) : 0) : -1;
    int rank = 0;
    for (int sq = 0; sq < nq; ++sq) {
      const uint64_t m = __ballot(q == sq);
      if (q == sq) rank = __popcll(m & below);
      if (lane == 0) c.sh->wq[wave][sq] = __popcll(m);
    }
    __syncthreads();
    if (q >= 0) {
      int off = c.sh->qn[q] + rank;
      for (int w = 0; w < wave; ++w) off += c.sh->wq[w][q];
      const int sl = c.sh->qb[q] + off;
      if (sl < c.a.q_cap)
        st_rlx(&c.a.slots[(size_t)q * c.a.q_cap + sl], id_of(i) + 1);
      else
        raise_fault(c.a, ET_ESTATE, -1, sl, c.a.q_cap);
    }
    __syncthreads();
    if (tid < nq) {
      int t = 0;
      for (int w = 0; w < kThreads / 64; ++w) t += c.sh->wq[w][tid];
      c.sh->qn[tid] += t;
    }
    __syncthreads();
  }
}

// Set the total number of tasks of this call (dynamic mode), once known.
__device__ __forceinline__ void set_total(const Ctx& c, int total) {
  if (threadIdx.x == 0) st_rlx(&c.a.hdr[HDR_QTOTAL], total);
}

// Worker-side claim state (meaningful in thread 0 only).
struct PopState {
  int base = 0;
  int size = 0;
  int left = 0;
  bool ahead = false;    // claim the next batch before running this one's last task
  int pre_base = 0;      // that claim's first index (its atomic's return value)
  int pre_size = 0;      // its size; 0: none outstanding
  int pre_pushed = 0;    // the shard's push counter read beside that atomic
  int impl = -1;         // static-order implicit tasks of this worker's shard (-1: not yet known)
  int impl_all = 0;      // ... of all shards
};

// Implicit initial tasks of shard q: ids q, q + nq, ... below n_init.
__device__ __forceinline__ int shard_init(const RunArgs& a, int q) {
  return a.n_init > q ? (a.n_init - q + a.nq - 1) / a.nq : 0;
}

// Static-order implicit tasks (RunArgs.impl_base > 0): the call's n tasks
// impl_base + p, p < n, published as a count in HDR_QIMPL.  Shard q holds, in
// order, the positions its XCD runs under the static schedule: with G a
// multiple of 8, G/8 consecutive positions per XCD and round (XCD (p mod G) /
// (G/8)); otherwise positions p with (p mod G) mod 8 = q; one shard: all.
__device__ __forceinline__ int impl_count(const Ctx& c, int q, int n) {
  if (c.a.nq == 1) return n;
  const int G = c.G, R = n / G, rem = n % G;
  if (G % 8 == 0) {
    const int per = G / 8;
    return R * per + min(per, max(0, rem - q * per));
  }
  return R * ((G - q + 7) / 8) + (rem > q ? (rem - q + 7) / 8 : 0);
}
__device__ __forceinline__ int impl_task(const Ctx& c, int q, int idx) {
  if (c.a.nq == 1) return c.a.impl_base + idx;
  const int G = c.G;
  if (G % 8 == 0) {
    const int per = G / 8;
    return c.a.impl_base + (idx / per) * G + q * per + idx % per;
  }
  const int pr = (G - q + 7) / 8;
  return c.a.impl_base + (idx / pr) * G + q + 8 * (idx % pr);
}

// Thread 0: slot index idx of this worker's shard -> task id; -1 when the
// call has no more tasks for this shard, -2 on a fault.  Index space of a
// shard: its implicit tasks (n_init of them, n_all over all shards), then
// its pushed slots.  A claimed slot that is not yet written is waited for;
// it is given up once every task of the call has been pushed and the index
// lies beyond what this shard received.
__device__ __forceinline__ int resolve_slot(const Ctx& c, int q, int idx, int n_init, int n_all) {
  const RunArgs& a = c.a;
  if (idx < n_init) return a.impl_base > 0 ? impl_task(c, q, idx) : a.init_base + q + a.nq * idx;
  const int s = idx - n_init;
  int* p = &a.slots[(size_t)q * a.q_cap + s];
  long long t0 = 0;
  for (int it = 0;; ++it) {
    if (s < a.q_cap) {
      const int v = ld_rlx(p);
      if (v != 0) {
        st_rlx(p, 0);   // leave the slot empty for the next call
        return v - 1;
      }
    }
    if ((it & 7) == 7) {
      int total = ld_rlx(&a.hdr[HDR_QTOTAL]);
      if (a.total_hint < total) total = a.total_hint;
      if (total != kUnknownTotal) {
        if (a.nq == 1) {
          if (idx >= total) return -1;
        } else {
          int pushed = 0, mine = 0;
          for (int j = 0; j < a.nq; ++j) {
            const int v = ld_rlx(q_pushed(a, j));
            pushed += v;
            if (j == q) mine = v;
          }
          if (n_all + pushed >= total && s >= mine) return -1;
        }
      }
    }
    if (it == 0) t0 = now_ticks();
    __builtin_amdgcn_s_sleep(1);
    if ((it & 63) == 63 || a.timeout <= 1) {
      if (faulted(a)) return -2;
      if (now_ticks() - t0 > a.timeout) {
        raise_fault(a, ET_ETIMEOUT, -1, idx, q);
        return -2;
      }
    }
  }
}

// pop(): next task of this worker (whole workgroup), -1 when there is none
// left.  The worker takes slots of its own XCD's shard (one shard: a
// central queue), `fetch` slots per atomic (batched fetch, Weave MoE
// article section 2.2) but no more than its share of the slots already
// published beyond the claim counter, so a worker never holds published
// tasks while others idle; short leading phases are claimed one slot at a
// time.  A racy peek is enough: any claim size is correct.
//
// Latency: the slots of a batch are read in one memory round trip when it is
// claimed, and while the shard holds at least three rounds of full batches
// for every worker beyond the claim counter, the next batch's atomic is
// issued before the current batch's last task runs and its result is first
// used at the next pop -- the claim round trips then overlap that task's own
// first loads instead of sitting between tasks.  (moe_large T=8192, dynamic:
// median / 90th percentile gap between a worker's tasks 1.08 / 2.4 us
// before, 0.88 / 2.0 us after; what remains is the batch's slot read and
// the claims made while the shard holds little queued work.)  Holding the next batch early cannot deadlock: a shard is FIFO,
// a worker claims from its own shard only, and in every workload here a
// claimed task waits only on tasks queued before it (or on no queued task).
__device__ __forceinline__ int wg_pop(const Ctx& c, PopState& ps) {
  int t = -1;
  if (threadIdx.x == 0) {
    const RunArgs& a = c.a;
    const int q = c.wg % a.nq;
    bool stop = false;
    if (a.impl_base > 0 && ps.impl < 0) {
      // static-order implicit tasks: wait until the call has published their
      // count (the scan does, early in the call); a fault ends the worker
      const long long t0 = now_ticks();
      int n = ld_rlx(&a.hdr[HDR_QIMPL]);
      for (int it = 1; n == kUnknownTotal; ++it) {
        __builtin_amdgcn_s_sleep(1);
        n = ld_rlx(&a.hdr[HDR_QIMPL]);
        if (n == kUnknownTotal && ((it & 63) == 0 || a.timeout <= 1)) {
          if (faulted(a)) break;
          if (now_ticks() - t0 > a.timeout) {
            raise_fault(a, ET_ETIMEOUT, -1, HDR_QIMPL, q);
            break;
          }
        }
      }
      if (n == kUnknownTotal) {
        stop = true;
      } else {
        ps.impl = impl_count(c, q, n);
        ps.impl_all = n;
      }
    }
    if (!stop) {
      const int n_init = a.impl_base > 0 ? ps.impl : shard_init(a, q);
      const int n_all = a.impl_base > 0 ? ps.impl_all : a.n_init;
      int* head = q_claimed(a, q);
      if (ps.left == 0) {
        if (ps.pre_size > 0) {
          ps.base = ps.pre_base;
          ps.size = ps.left = ps.pre_size;
          ps.pre_size = 0;
          const int per = c.G / a.nq > 0 ? c.G / a.nq : 1;
          ps.ahead = n_init + ps.pre_pushed - (ps.base + ps.size) >= 3 * per * ps.size;
        } else {
          const int h = ld_rlx(head);
          const int avail = n_init + ld_rlx(q_pushed(a, q)) - h;
          const int per = c.G / a.nq > 0 ? c.G / a.nq : 1;
          // static-order implicit entries are claimed one at a time: a
          // shard's consecutive entries are the row blocks sharing a weight
          // tile, which should run side by side on different workers
          const int cap = a.impl_base > 0 && h < n_init ? 1 : a.fetch;
          int sz = avail / per;
          sz = h * a.nq < a.n_single ? 1 : (sz < 1 ? 1 : (sz > cap ? cap : sz));
          ps.ahead = sz == cap && avail >= 3 * per * cap;
          ps.base = add_rlx(head, sz);
          ps.size = ps.left = sz;
        }
        int v[kMaxFetch];
#pragma unroll
        for (int i = 0; i < kMaxFetch; ++i) {
          const int sl = ps.base + i - n_init;
          v[i] = (i < ps.size && sl >= 0 && sl < a.q_cap) ? ld_rlx(&a.slots[(size_t)q * a.q_cap + sl]) : 0;
        }
#pragma unroll
        for (int i = 0; i < kMaxFetch; ++i)
          if (i < ps.size) c.sh->bids[i] = v[i];
      }
      const int k = ps.size - ps.left;
      const int idx = ps.base + k;
      --ps.left;
      if (idx < n_init) {
        t = a.impl_base > 0 ? impl_task(c, q, idx) : a.init_base + q + a.nq * idx;
      } else {
        const int v = c.sh->bids[k];
        if (v != 0) {
          st_rlx(&a.slots[(size_t)q * a.q_cap + (idx - n_init)], 0);   // empty for the next call
          t = v - 1;
        } else {
          t = resolve_slot(c, q, idx, n_init, n_all);   // not yet written when read: wait for it
          if (t < 0) t = -1;
        }
      }
      if (ps.left == 0 && ps.ahead && t >= 0) {
        // (the head is at least base + size: a lower bound picks the cap)
        const int cap = a.impl_base > 0 && ps.base + ps.size < n_init ? 1 : a.fetch;
        ps.pre_base = add_rlx(head, cap);
        ps.pre_pushed = ld_rlx(q_pushed(a, q));
        ps.pre_size = cap;
      }
    }
  }
  return wg_bcast(c, t, 4);
}

__device__ __forceinline__ void count_run(const Ctx& c, int task) {
  if (c.a.runs && threadIdx.x == 0) atomicAdd(&c.a.runs[task], 1);
}

// Debug trace: task -> (workgroup, start, end) in 100 MHz ticks.
__device__ __forceinline__ long long trace_now(const Ctx& c) {
  return c.a.trace && c.a.trace_tasks ? now_ticks() : 0;
}
__device__ __forceinline__ void trace_task(const Ctx& c, int task, long long t0) {
  if (c.a.trace && c.a.trace_tasks && threadIdx.x == 0 && task >= 0 && task < c.a.q_cap) {
    int* p = c.a.trace + 4 * (size_t)task;
    p[0] = c.wg;
    p[1] = (int)t0;
    p[2] = (int)now_ticks();
    p[3] = 1;
  }
}
__device__ __forceinline__ void trace_wg(const Ctx& c, int which) {
  if (c.a.trace && threadIdx.x == 0 && c.wg < 1024) {
    c.a.trace[4 * (size_t)c.a.q_cap + 2 * c.wg + which] = (int)now_ticks();
    c.a.trace[4 * (size_t)c.a.q_cap + 2048 + 2 * c.wg + which] = (int)__builtin_amdgcn_s_memtime();
  }
}

// Prologue: pick this call's bank and re-arm the part of the other bank the
// previous call used.  Returns false when the workspace carries a fault.
__device__ __forceinline__ bool prologue(Ctx& c, const RunArgs& a, Shared* sh) {
  c.a = a;
  c.sh = sh;
  c.wg = blockIdx.x;
  c.G = gridDim.x;
  trace_wg(c, 0);
  // the four header words are requested together (one memory round trip,
  // not three dependent ones)
  const int err = ld_rlx(&a.hdr[HDR_ERR]);
  const int bank_w = ld_rlx(&a.hdr[HDR_BANK]);
  const int ext0 = ld_rlx(&a.hdr[HDR_EXT0]);
  const int ext1 = ld_rlx(&a.hdr[HDR_EXT1]);
  const int calls = ld_rlx(&a.hdr[HDR_CALLS]);
  if (err != 0) return false;
  c.gen = calls + 1;
  const int bank = bank_w & 1;
  c.ev = a.counters + (size_t)bank * a.n_events;
  if (a.sched != ET_SCHED_PER_OP) {
    int* other = a.counters + (size_t)(1 - bank) * a.n_events;
    int ext = bank ? ext0 : ext1;
    if (ext > a.n_events) ext = a.n_events;
    for (int i = c.wg * kThreads + threadIdx.x; i < ext; i += c.G * kThreads) other[i] = 0;
  }
  return true;
}

// Epilogue: the last workgroup out resets the queue, records the extent of
// the bank it used and flips the bank for the next call.
__device__ __forceinline__ void epilogue(const Ctx& c, int tasks_this_call) {
  trace_wg(c, 1);
  if (c.a.sched == ET_SCHED_PER_OP) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    int old = add_rlx(&c.a.hdr[HDR_EXIT], 1);
    if (old == c.G - 1) {
      int* h = c.a.hdr;
      int bank = ld_rlx(&h[HDR_BANK]) & 1;
      st_rlx(&h[HDR_EXIT], 0);
      st_rlx(&h[HDR_QHEAD], 0);
      for (int q = 0; q < kMaxShards; ++q) {
        st_rlx(q_claimed(c.a, q), 0);
        st_rlx(q_pushed(c.a, q), 0);
      }
      st_rlx(&h[HDR_QTOTAL], kUnknownTotal);
      st_rlx(&h[HDR_QIMPL], kUnknownTotal);
      st_rlx(&h[HDR_EXT0 + bank], c.a.extent);
      st_rlx(&h[HDR_LAST_TASKS], tasks_this_call);
      st_rlx(&h[HDR_CALLS], ld_rlx(&h[HDR_CALLS]) + 1);
      st_rlx(&h[HDR_BANK], 1 - bank);
    }
  }
}

// ---------------------------------------------------------------------------
// buffer resources (out-of-range loads return zeros) and MFMA helpers
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr uint32_t kOOB = 0x80000000u;   // offset that is always out of range

__device__ __forceinline__ Rsrc make_rsrc(const void* p, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) 32-bit data format on gfx9-family parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ i32x4 ld16(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// agent-coherent 16-byte load (sc1): data written earlier in the same launch
__device__ __forceinline__ i32x4 ld16c(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16);
}
__device__ __forceinline__ void st16c(Rsrc r, uint32_t off, i32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 16);
}
template <bool COH>
__device__ __forceinline__ i32x4 ld16x(Rsrc r, uint32_t off) {
  return COH ? ld16c(r, off) : ld16(r, off);
}

__device__ __forceinline__ f32x4 mfma16(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16, round to nearest even (gfx950's conversion instruction)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// SiLU with the hardware reciprocal (about 1 ulp in fp32): its result is
// rounded to bf16 next, so the IEEE division's extra accuracy is never seen,
// and the division's instruction sequence dominated the gate/up epilogue.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Sum over each 16-lane row, result in every lane of the row (quad
// permutes, then the half-row and row mirrors).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<0xB1>(x);    // quad [1,0,3,2]
  x += dpp_f32<0x4E>(x);    // quad [2,3,0,1]
  x += dpp_f32<0x141>(x);   // row half mirror
  x += dpp_f32<0x140>(x);   // row mirror
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts of 1, 2, 4, 8
// within each 16-lane row, then the row totals carried across rows by the
// two row broadcasts (rows 1, 3 from lanes 15, 47; rows 2, 3 from lane 31).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i32<0x111, 0xf>(x);   // row_shr:1
  x += dpp_i32<0x112, 0xf>(x);   // row_shr:2
  x += dpp_i32<0x114, 0xf>(x);   // row_shr:4
  x += dpp_i32<0x118, 0xf>(x);   // row_shr:8
  x += dpp_i32<0x142, 0xa>(x);   // row_bcast:15 into rows 1, 3
  x += dpp_i32<0x143, 0xc>(x);   // row_bcast:31 into rows 2, 3
  return x;
}

// Wave-wide unsigned max / min through DPP lane moves (no LDS round trips):
// quad permutes and row mirrors reduce each 16-lane row, two row broadcasts
// fold the rows into lane 63, which is read back as a uniform value.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x) {
  // the lanes a step leaves out (row masks) receive the operation's identity
  // (0 for max, all ones for min), so each step compiles to one DPP max/min
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  constexpr int id = MAX ? 0 : -1;
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0xB1, 0xf, 0xf, false));  // quad [1,0,3,2]
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x4E, 0xf, 0xf, false));  // quad [2,3,0,1]
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x141, 0xf, 0xf, false)); // row half mirror
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x140, 0xf, 0xf, false)); // row mirror
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xa, 0xf, false)); // row bcast 15
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xc, 0xf, false)); // row bcast 31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

}  // namespace et
