// et_mlp.hip -- the dense SiLU-gated MLP chain as one persistent kernel.
//
// y = (SiLU(x Wg) * (x Wu)) Wd with bf16 operands and fp32 accumulation, the
// dense MLP of the served models (Event Tensor notes, sections "计算通信融合"
// and "端到端低 batch serving").  Task kinds:
//   gate/up tile (mb, n): 16 columns of h for a block of rows; stores h in
//     bf16 and notifies E_h[mb, n / 8] -- one event per 128-column tile of h;
//   down tile (mb, n2): 16 output columns over all of K = I; before reading
//     the h K-blocks of a round it waits on their E_h events, so the down
//     projection starts on the first h tiles while later ones are still being
//     produced, and its weights are fetched before the first wait.
// The event array E_h has the symbolic shape (ceil(B / rows), I / 128): one
// compiled kernel serves every batch size B (section "Shape dynamism").
#include "et_device.hpp"
#include "et_gemm.hpp"
#include "et_launch.hpp"

namespace et {

struct MlpArgs {
  const uint16_t* x;
  const uint16_t* wg;
  const uint16_t* wu;
  const uint16_t* wd;
  uint16_t* h;       // [B, I] bf16 (workspace)
  float* y;          // [B, H]
  int B, H, I;
  int ev_all;        // index of the all-gate/up-tiles event (barrier mode)
};

template <int MT> constexpr int kMlpPD = MT == 1 ? 4 : (MT == 2 ? 3 : 2);   // K-blocks in flight
template <int MT> constexpr int kMlpOcc = 1;                               // workgroups per CU

template <int MT>
__global__ __launch_bounds__(kThreads, kMlpOcc<MT>) void mlp_kernel(RunArgs ra, MlpArgs m) {
  __shared__ Shared sh;
  __shared__ uint32_t rows_off[16 * MT];
  using Tile1 = StreamTile<MT, 2, 4, kMlpPD<MT>, false>;   // reads x
  using Tile2 = StreamTile<MT, 1, 4, kMlpPD<MT>, true>;    // reads h (this launch)
  constexpr int kRed = Tile1::kRedFloats > Tile2::kRedFloats ? Tile1::kRedFloats : Tile2::kRedFloats;
  __shared__ float red[kRed];

  Ctx c;
  if (!prologue(c, ra, &sh)) return;
  const int sched = ra.sched;
  const int rows = 16 * MT;
  const int mb = cdiv(m.B, rows);
  const int ngt = m.I / 16;             // gate/up tiles per row block
  const int ndt = m.H / 16;             // down tiles per row block
  const int nht = m.I / kHTile;         // h tiles (events) per row block
  const int n_gate = mb * ngt;
  const int n_down = mb * ndt;
  const int total = n_gate + n_down;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  auto set_rows = [&](int b, int row_bytes) ET_INLINE {
    for (int i = threadIdx.x; i < rows; i += kThreads) {
      const int r = b * rows + i;
      rows_off[i] = r < m.B ? (uint32_t)r * (uint32_t)row_bytes : kOOB;
    }
    __syncthreads();
  };

  auto run = [&](int task) ET_INLINE -> bool {
    if (task < n_gate) {
      const int b = task / ngt, n = task % ngt;
      set_rows(b, m.H * 2);
      const Rsrc ra_ = make_rsrc(m.x, (uint32_t)m.B * m.H * 2);
      const uint32_t wbytes = (uint32_t)m.I * m.H * 2;
      const Rsrc rb[2] = {make_rsrc(m.wg, wbytes), make_rsrc(m.wu, wbytes)};
      const uint32_t boff = (uint32_t)(16 * n + (lane & 15)) * (uint32_t)(m.H * 2);
      const uint32_t bo[2] = {boff, boff};
      Tile1 tile;
      tile.run(ra_, rows_off, rb, bo, m.H / kKBlock, [](int) { return true; }, red);
      // epilogue: h = SiLU(g) * u in bf16; wave q stores accumulator row r == q
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r == wave) {
            const int row = b * rows + 16 * mt + 4 * (lane >> 4) + r;
            if (row < m.B) {
              const float g = tile.acc[mt][0][r], u = tile.acc[mt][1][r];
              st_coh(&m.h[(size_t)row * m.I + 16 * n + (lane & 15)], f32_to_bf16(silu(g) * u));
            }
          }
      if (sched == ET_SCHED_PER_OP) return true;
      wg_release();
      if (sched == ET_SCHED_BARRIER)
        t0_notify_bcast(c, m.ev_all, 0, 1, n_gate, task);
      else
        t0_notify(c, b * nht + n / (kHTile / 16), 1, kHTile / 16, task);
      return true;
    }
    const int t2 = task - n_gate;
    const int b = t2 / ndt, n2 = t2 % ndt;
    set_rows(b, m.I * 2);
    const Rsrc ra_ = make_rsrc(m.h, (uint32_t)m.B * m.I * 2);
    const Rsrc rb[1] = {make_rsrc(m.wd, (uint32_t)m.H * m.I * 2)};
    const uint32_t bo[1] = {(uint32_t)(16 * n2 + (lane & 15)) * (uint32_t)(m.I * 2)};
    const int nkb = m.I / kKBlock;
    // K-blocks (h tiles) known complete.  A poll inside the weight stream
    // completes only after every load its wave issued before it (loads
    // complete in order), so a round inside the known-complete prefix polls
    // nothing; the first round beyond it counts the complete h tiles from
    // there on (one round trip for all of them) and waits only if its own
    // are not among them.
    int ready_kb = sched == ET_SCHED_PER_OP ? nkb : 0;
    auto gate = [&](int round) ET_INLINE -> bool {
      if (sched == ET_SCHED_BARRIER) return round > 0 || wg_wait_bcast(c, m.ev_all, 0, task);
      const int k0 = round * 4;
      const int nk = nkb - k0 < 4 ? nkb - k0 : 4;
      if (k0 + nk <= ready_kb) return true;
      ready_kb = k0 + wg_probe_prefix(c, b * nht + k0, nht - k0, kHTile / 16);
      if (k0 + nk <= ready_kb) return true;
      if (!wg_wait_range(c, b * nht + k0, nk, kHTile / 16, task)) return false;
      ready_kb = k0 + nk;
      return true;
    };
    Tile2 tile;
    if (!tile.run(ra_, rows_off, rb, bo, nkb, gate, red)) return false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r == wave) {
          const int row = b * rows + 16 * mt + 4 * (lane >> 4) + r;
          if (row < m.B) m.y[(size_t)row * m.H + 16 * n2 + (lane & 15)] = tile.acc[mt][0][r];
        }
    return true;
  };

  if (sched == ET_SCHED_DYNAMIC) {
    // Every task is in the queue from the start, gate/up tiles first.  A
    // worker claims slots in FIFO order, so when it reaches a down tile every
    // gate/up tile has already been claimed by a running worker: the down
    // tile may wait on its h events without risk of deadlock (the "early
    // push" of Event Tensor notes, section "动态调度").
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
    const int lo = ra.phase == 0 ? 0 : n_gate, hi = ra.phase == 0 ? n_gate : total;
    for (int t = lo + c.wg; t < hi; t += c.G) {
      const long long t0 = trace_now(c);
      run(t);
      count_run(c, t);
      trace_task(c, t, t0);
    }
  } else {
    // one round-robin over all tasks (gate/up ids first): the down tiles land
    // on the workgroups with the fewest gate/up tiles, and every workgroup
    // finishes its gate/up tiles before it waits in a down tile
    bool ok = true;
    for (int t = c.wg; ok && t < total; t += c.G) {
      const long long t0 = trace_now(c);
      ok = run(t);
      if (ok) count_run(c, t);
      if (ok) trace_task(c, t, t0);
    }
  }
  epilogue(c, total);
}

int launch_mlp(const LaunchCommon& lc, const uint16_t* x, int B, const uint16_t* wg,
               const uint16_t* wu, const uint16_t* wd, float* y) {
  const et_plan* p = lc.plan;
  MlpPlan mp{p->max_tokens, p->hidden, p->inter};
  const int tv = pick_mlp_tile(B, lc.tile);
  const Tiling t = tiling_of(tv);
  MlpArgs m{x, wg, wu, wd, reinterpret_cast<uint16_t*>(lc.ws + p->off_aux), y, B,
            p->hidden, p->inter, 0};
  const int mb = mp.mb(B, t);
  m.ev_all = mp.n_events_max() - 1;
  const int n_gate = mb * (p->inter / 16), n_down = mb * (p->hidden / 16);
  RunArgs ra = lc.run_args();
  ra.init_base = n_gate + n_down < lc.G ? n_gate + n_down : lc.G;   // first round runs directly
  ra.n_init = n_gate + n_down - ra.init_base;
  ra.total_hint = n_gate + n_down - ra.init_base;
  ra.extent = mp.n_events_max();
  const void* k = tv == TV_M16   ? reinterpret_cast<const void*>(&mlp_kernel<1>)
                  : tv == TV_M32 ? reinterpret_cast<const void*>(&mlp_kernel<2>)
                                 : reinterpret_cast<const void*>(&mlp_kernel<4>);
  LaunchCommon l = lc;
  l.G = lc.G * (tv == TV_M16 ? kMlpOcc<1> : tv == TV_M32 ? kMlpOcc<2> : kMlpOcc<4>);
  if (lc.sched == ET_SCHED_PER_OP) {
    for (int ph = 0; ph < 2; ++ph) {
      ra.phase = ph;
      int e = l.launch(k, &ra, &m, false);
      if (e) return e;
    }
    return ET_OK;
  }
  return l.launch(k, &ra, &m, true);
}

}  // namespace et
