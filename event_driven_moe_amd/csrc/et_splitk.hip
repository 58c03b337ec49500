// et_splitk.hip -- the two-stage split-K reduction as one persistent kernel.
//
// Event Tensor notes, section "Split-K reduction 示例": A (n*32, 128) is
// reduced along K in four 32-wide slices.  Stage-1 task (i, j) sums rows
// 32i..32i+31 over slice j into B[:, j] and notifies E[i] (map "ij->i",
// wait count 4); stage-2 task i waits on E[i] (map "i->i") and adds the four
// partials of its rows, so it can start as soon as its own row block is done
// rather than after all of B.
#include "et_device.hpp"
#include "et_launch.hpp"

namespace et {

struct SplitKArgs {
  const float* A;
  float* B;
  float* C;
  int n;       // row blocks this call
  int n_max;   // row blocks of the plan (index of the all-stage-1 event)
};

// Stage-1 tile: 32 x 32 fp32.  Thread t reads a float4 of row t/8; the eight
// lanes of a row finish the sum with a butterfly (wavefront reduction).
__device__ __forceinline__ void splitk_stage1(const SplitKArgs& s, int i, int j) {
  const int t = threadIdx.x;
  const int r = 32 * i + (t >> 3);
  const int c = 32 * j + (t & 7) * 4;
  const float4 a = *reinterpret_cast<const float4*>(s.A + (size_t)r * 128 + c);
  float v = (a.x + a.y) + (a.z + a.w);
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  if ((t & 7) == 0) st_coh(&s.B[(size_t)r * 4 + j], v);
}

// Stage-2 tile: C[r] = ((B[r,0] + B[r,1]) + B[r,2]) + B[r,3] for 32 rows.
__device__ __forceinline__ void splitk_stage2(const SplitKArgs& s, int i) {
  const int t = threadIdx.x;
  if (t < 32) {
    const int r = 32 * i + t;
    const float* b = s.B + (size_t)r * 4;
    s.C[r] = ((ld_coh(b) + ld_coh(b + 1)) + ld_coh(b + 2)) + ld_coh(b + 3);
  }
}

__global__ __launch_bounds__(kThreads, 1) void splitk_kernel(RunArgs ra, SplitKArgs s) {
  __shared__ Shared sh;
  Ctx c;
  if (!prologue(c, ra, &sh)) return;
  const int n1 = 4 * s.n;
  const int ev_all = s.n_max;
  const int sched = ra.sched;

  auto run = [&](int task) ET_INLINE -> bool {
    if (task < n1) {
      const int i = task >> 2, j = task & 3;
      splitk_stage1(s, i, j);
      if (sched == ET_SCHED_PER_OP) return true;
      wg_release();
      if (sched == ET_SCHED_BARRIER) {
        t0_notify_bcast(c, ev_all, 0, 1, n1, task);
      } else if (sched == ET_SCHED_STATIC) {
        t0_notify(c, i, 1, 4, task);
      } else if (wg_notify(c, i, 1, 4, task)) {
        wg_push(c, 1, [&](int) { return n1 + i; }, [&](int) { return i; });   // the zeroing notifier pushes stage-2 i
      }
      return true;
    }
    const int i = task - n1;
    if (sched == ET_SCHED_STATIC) {
      if (!wg_wait(c, i, 4, task)) return false;
    } else if (sched == ET_SCHED_BARRIER) {
      if (!wg_wait_bcast(c, ev_all, 0, task)) return false;
    }
    splitk_stage2(s, i);
    return true;
  };

  const int total = 5 * s.n;
  if (sched == ET_SCHED_DYNAMIC) {
    // the first round of tasks runs on workgroup w = task id directly: a
    // claim from the queue would put a contended atomic (every workgroup of
    // a shard on one claim counter) before the first task
    bool ok = true;
    for (int t = c.wg; ok && t < ra.init_base; t += c.G) {
      const long long t0 = trace_now(c);
      ok = run(t);
      if (ok) count_run(c, t);
      if (ok) trace_task(c, t, t0);
    }
    PopState ps;
    while (ok) {
      const int t = wg_pop(c, ps);
      const long long t0 = trace_now(c);
      if (t < 0 || !run(t)) break;
      count_run(c, t);
      trace_task(c, t, t0);
    }
  } else if (sched == ET_SCHED_PER_OP) {
    const int lo = ra.phase == 0 ? 0 : n1, hi = ra.phase == 0 ? n1 : total;
    for (int t = lo + c.wg; t < hi; t += c.G) {
      const long long t0 = trace_now(c);
      run(t);
      count_run(c, t);
      trace_task(c, t, t0);
    }
  } else {
    bool ok = true;
    for (int t = c.wg; ok && t < n1; t += c.G) {
      const long long t0 = trace_now(c);
      ok = run(t);
      if (ok) count_run(c, t);
      if (ok) trace_task(c, t, t0);
    }
    for (int t = n1 + c.wg; ok && t < total; t += c.G) {
      const long long t0 = trace_now(c);
      ok = run(t);
      if (ok) count_run(c, t);
      if (ok) trace_task(c, t, t0);
    }
  }
  epilogue(c, total);
}

int launch_splitk(const LaunchCommon& lc, const float* A, int rows, float* B, float* C) {
  SplitKArgs s{A, B, C, rows / 32, lc.plan->max_tokens / 32};
  RunArgs ra = lc.run_args();
  ra.init_base = 4 * s.n < lc.G ? 4 * s.n : lc.G;   // stage-1 tiles run directly, then from the queue
  ra.n_init = 4 * s.n - ra.init_base;
  ra.total_hint = 5 * s.n - ra.init_base;          // queue tasks: the rest of stage 1 and stage 2
  ra.extent = s.n_max + 1;
  if (lc.sched == ET_SCHED_PER_OP) {
    for (int ph = 0; ph < 2; ++ph) {
      ra.phase = ph;
      int e = lc.launch(reinterpret_cast<const void*>(&splitk_kernel), &ra, &s, false);
      if (e) return e;
    }
    return ET_OK;
  }
  return lc.launch(reinterpret_cast<const void*>(&splitk_kernel), &ra, &s, true);
}

}  // namespace et
