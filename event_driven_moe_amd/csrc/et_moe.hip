// et_moe.hip -- the MoE layer as one persistent kernel.
//
// The chain TopK routing -> token grouping -> grouped GEMMs of Event Tensor
// notes (section "两类动态性如何进入依赖表示", section "完整 MoE layer") with a
// weighted combine at the end:
//   routing task r   top-k of the router logits of token chunk r, renormalised
//                    weights, a per-chunk expert histogram; notifies EV_ROUTE;
//   scan task        column sums of the histograms (rows per expert), CSR
//                    offsets of rows, row blocks and tasks per expert, and the
//                    base position of every (chunk, expert); it learns the
//                    number of GEMM tasks of this call;
//   grouping task r  stable positions of chunk r's (token, slot) pairs; notifies
//                    EV_EXP[e] of the experts its tokens chose, by its number of
//                    rows for each (data-dependent targets, data-dependent wait
//                    count = rows routed to e);
//   gate/up task     (block gb, 16 columns of h): rows gathered from x by the
//                    permutation; h = SiLU(x Wg) * (x Wu) in bf16; notifies
//                    EV_H[gb];
//   down task        (block gb, 16 output columns): y = h Wd in fp32; waits on
//                    EV_H[gb] only, not on all gate/up tasks -- the event that
//                    removes the barrier between the two GroupGEMMs;
//   combine          out[t] = sum_s w[t, s] y[inv[t, s]] in slot order.
// Dynamic mode: the notify that zeroes EV_EXP[e] pushes expert e's task range
// tasks[task_indptr[e] : task_indptr[e+1]] (data-dependent fan-out), the one
// that zeroes EV_H[gb] pushes block gb's down tasks, and the one that zeroes
// EV_C[t, c] (k down rows of token t for column tile c) runs that combine
// inline.  Static mode keeps the fine-grained EV_H edge but, as the page's
// static lowering does for data-dependent edges, replaces EV_EXP by one
// coarse "all grouped" event and EV_C by one "all down tiles done" event.
#include "et_device.hpp"
#include "et_gemm.hpp"
#include "et_launch.hpp"

namespace et {

struct MoeArgs {
  const float* logits;
  const uint16_t* x;
  const uint16_t* wg;
  const uint16_t* wu;
  const uint16_t* wd;
  float* out;
  int* topk_ids;
  float* topk_w;
  int* hist;
  int* counts;
  int* tok_indptr;
  int* blk_indptr;
  int* task_indptr;
  int* blk_expert;
  int* perm;
  int* inv;
  uint16_t* h;
  float* y;
  int T, H, I, E, k, NR, tpr;
  int ev_exp, ev_h, ev_c;
};

template <int MT> constexpr int kMoePD = MT == 1 ? 4 : (MT == 2 ? 3 : 2);   // K-blocks in flight
constexpr int kMoeSmem = 16384 * 4 + 3 * 1024 * 4 + 256;   // scan histogram + scan temps

// ---------------------------------------------------------------------------
// block-wide exclusive scan of n <= 1024 ints held in LDS (in place);
// returns the total.  256 threads, 4 consecutive elements per thread.
// ---------------------------------------------------------------------------
__device__ int block_exscan(int* a, int n, int* tmp /* >= 8 ints */) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * t + i;
    v[i] = j < n ? a[j] : 0;
    s += v[i];
  }
  int inc = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += tmp[w];
  const int total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  int run = wbase + inc - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * t + i;
    if (j < n) a[j] = run;
    run += v[i];
  }
  __syncthreads();
  return total;
}

// float -> key that orders like the value (with -0.0 == +0.0), then by lower index
__device__ __forceinline__ unsigned long long route_key(float v, int e) {
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}
__device__ __forceinline__ float key_value(unsigned long long key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __builtin_bit_cast(float, u);
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, d), hi = __shfl_xor((uint32_t)(v >> 32), d);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// one output element of the combine; the same fixed-order sum serves the
// inline (dynamic) and the tiled (static) combine, so both give the same bits
__device__ __forceinline__ float combine_elem(const MoeArgs& m, int t, int col) {
  float acc = 0.f;
  for (int s = 0; s < m.k; ++s) {
    const float w = m.topk_w[t * m.k + s];
    const int pos = m.inv[t * m.k + s];
    acc = __fmaf_rn(w, m.y[(size_t)pos * m.H + col], acc);
  }
  return acc;
}

template <int MT>
__global__ __launch_bounds__(kThreads, 1) void moe_kernel(RunArgs ra, MoeArgs m) {
  __shared__ Shared sh;
  __shared__ __align__(16) unsigned char smem[kMoeSmem];
  using Tile1 = StreamTile<MT, 2, 4, kMoePD<MT>>;
  using Tile2 = StreamTile<MT, 1, 4, kMoePD<MT>>;

  Ctx c;
  if (!prologue(c, ra, &sh)) return;
  const int sched = ra.sched;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows = 16 * MT;
  const int nt1 = m.I / 16, nt2 = m.H / 16;
  const int NR = m.NR;
  const int base1 = 2 * NR + 1;
  const int wc = m.k * 1;   // EV_C wait count: k rows of a token per column tile

  // LDS carve-outs (task kinds never overlap in time inside one workgroup)
  int* s_i = reinterpret_cast<int*>(smem);
  uint32_t* rows_off = reinterpret_cast<uint32_t*>(smem);            // gemm: [16*MT]
  float* red = reinterpret_cast<float*>(smem + 1024);                 // gemm: reduction
  int* fired = reinterpret_cast<int*>(smem + 1024 - 256);             // gemm2: fired tokens

  auto meta = [&](int i) { return ld_rlx(&ra.hdr[HDR_META + i]); };

  // ------------------------------------------------------------- routing
  auto route = [&](int r) {
    int* hist_l = s_i;   // [E]
    for (int e = tid; e < m.E; e += kThreads) hist_l[e] = 0;
    __syncthreads();
    const int t0 = r * m.tpr;
    const int t1 = min(m.T, t0 + m.tpr);
    for (int t = t0 + wave; t < t1; t += 4) {
      const float* lg = m.logits + (size_t)t * m.E;
      unsigned long long keys[kMaxExperts / 64];
      const int nj = (m.E + 63) / 64;
#pragma unroll
      for (int j = 0; j < kMaxExperts / 64; ++j) {
        const int e = lane + 64 * j;
        keys[j] = (j < nj && e < m.E) ? route_key(lg[e], e) : 0ull;
      }
      int my_e = -1;
      float my_v = 0.f, v0 = 0.f;
      for (int s = 0; s < m.k; ++s) {
        unsigned long long best = 0;
#pragma unroll
        for (int j = 0; j < kMaxExperts / 64; ++j) best = keys[j] > best ? keys[j] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xffffffffu - (uint32_t)best);
        const float v = key_value(best);
        if (s == 0) v0 = v;
        if (lane == s) { my_e = e; my_v = v; }
        if ((e & 63) == lane) {
#pragma unroll
          for (int j = 0; j < kMaxExperts / 64; ++j)
            if (j == (e >> 6)) keys[j] = 0ull;
        }
      }
      // weights: softmax over the kept logits (= renormalised top-k softmax)
      float ex = lane < m.k ? expf(my_v - v0) : 0.f;
      float sum = ex;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) sum += __shfl_xor(sum, d);
      if (lane < m.k) {
        m.topk_ids[t * m.k + lane] = my_e;
        m.topk_w[t * m.k + lane] = ex / sum;
        atomicAdd(&hist_l[my_e], 1);
      }
    }
    __syncthreads();
    for (int e = tid; e < m.E; e += kThreads) m.hist[r * m.E + e] = hist_l[e];
  };

  // ------------------------------------------------------------- scan
  auto scan = [&]() {
    int* hs = s_i;                         // [n_ne][E]
    int* cnt = s_i + 16384;                // [E]
    int* blk = cnt + 1024;                 // [E] -> block offsets
    int* tmp = blk + 1024;                 // [8]
    const int n_ne = cdiv(m.T, m.tpr);
    const int tot = n_ne * m.E;
    for (int i = tid; i < tot; i += kThreads) hs[i] = m.hist[i];
    __syncthreads();
    for (int e = tid; e < m.E; e += kThreads) {
      int run = 0;
      for (int r = 0; r < n_ne; ++r) {
        const int v = hs[r * m.E + e];
        hs[r * m.E + e] = run;
        run += v;
      }
      cnt[e] = run;
      blk[e] = cdiv(run, rows);
      m.counts[e] = run;
    }
    __syncthreads();
    block_exscan(cnt, m.E, tmp);           // cnt -> tok_indptr
    const int nb = block_exscan(blk, m.E, tmp);
    for (int e = tid; e < m.E; e += kThreads) {
      m.tok_indptr[e] = cnt[e];
      m.blk_indptr[e] = blk[e];
      m.task_indptr[e] = blk[e] * nt1;
    }
    if (tid == 0) {
      m.tok_indptr[m.E] = m.T * m.k;
      m.blk_indptr[m.E] = nb;
      m.task_indptr[m.E] = nb * nt1;
    }
    for (int i = tid; i < tot; i += kThreads) m.hist[i] = hs[i] + cnt[i % m.E];
    for (int gb = tid; gb < nb; gb += kThreads) {   // block -> expert (upper bound search)
      int lo = 0, hi = m.E;                         // blk[lo] <= gb < blk[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (blk[mid] <= gb) lo = mid; else hi = mid;
      }
      m.blk_expert[gb] = lo;
    }
    if (tid == 0) {
      st_rlx(&ra.hdr[HDR_META + MD_NB], nb);
      st_rlx(&ra.hdr[HDR_META + MD_TOTAL1], nb * nt1);
      st_rlx(&ra.hdr[HDR_META + MD_TOTAL2], nb * nt2);
    }
    __syncthreads();
    return nb;
  };

  // ------------------------------------------------------------- grouping
  auto group = [&](int r) {
    int* cur = s_i;            // [E] next position per expert
    int* base = s_i + 1024;    // [E] first position of this chunk per expert
    for (int e = tid; e < m.E; e += kThreads) {
      const int b = m.hist[r * m.E + e];
      cur[e] = b;
      base[e] = b;
    }
    __syncthreads();
    const int t0 = r * m.tpr;
    const int t1 = min(m.T, t0 + m.tpr);
    if (wave == 0) {
      for (int t = t0; t < t1; ++t) {      // tokens in order: stable positions
        if (lane < m.k) {
          const int e = m.topk_ids[t * m.k + lane];
          const int pos = cur[e]++;        // a token's k experts are distinct
          m.perm[pos] = t * m.k + lane;
          m.inv[t * m.k + lane] = pos;
        }
      }
    }
    __syncthreads();
  };

  // ------------------------------------------------------------- gemm tiles
  auto gemm1 = [&](int t1g, int task) -> bool {
    const int gb = t1g / nt1, n = t1g % nt1;
    const int e = m.blk_expert[gb];
    const int pos0 = m.tok_indptr[e] + (gb - m.blk_indptr[e]) * rows;
    const int pend = min(pos0 + rows, m.tok_indptr[e + 1]);
    const size_t wofs = (size_t)e * m.I * m.H;
    const uint32_t wbytes = (uint32_t)m.I * m.H * 2;
    const Rsrc rb[2] = {make_rsrc(m.wg + wofs, wbytes), make_rsrc(m.wu + wofs, wbytes)};
    const uint32_t boff = (uint32_t)(16 * n + (lane & 15)) * (uint32_t)(m.H * 2);
    const uint32_t bo[2] = {boff, boff};
    const Rsrc rx = make_rsrc(m.x, (uint32_t)m.T * m.H * 2);
    auto gate = [&](int round) -> bool {
      if (round != 0) return true;
      if (sched == ET_SCHED_STATIC || sched == ET_SCHED_BARRIER)
        if (!wg_wait(c, EV_GROUP, NR, task)) return false;
      for (int i = tid; i < rows; i += kThreads) {
        const int pos = pos0 + i;
        rows_off[i] = pos < pend ? (uint32_t)(m.perm[pos] / m.k) * (uint32_t)(m.H * 2) : kOOB;
      }
      __syncthreads();
      return true;
    };
    Tile1 tile;
    if (!tile.run(rx, rows_off, rb, bo, m.H / kKBlock, gate, red)) return false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r == wave) {
          const int pos = pos0 + 16 * mt + 4 * (lane >> 4) + r;
          if (pos < pend) {
            const float g = tile.acc[mt][0][r], u = tile.acc[mt][1][r];
            m.h[(size_t)pos * m.I + 16 * n + (lane & 15)] = f32_to_bf16(silu(g) * u);
          }
        }
    if (sched == ET_SCHED_PER_OP) return true;
    wg_release();
    if (sched == ET_SCHED_BARRIER) {
      t0_notify(c, EV_G1ALL, 1, meta(MD_TOTAL1), task);
    } else if (sched == ET_SCHED_STATIC) {
      t0_notify(c, m.ev_h + gb, 1, nt1, task);
    } else if (wg_notify(c, m.ev_h + gb, 1, nt1, task, true)) {
      const int b2 = base1 + meta(MD_TOTAL1) + gb * nt2;
      wg_push(c, nt2, [&](int i) { return b2 + i; });
    }
    return true;
  };

  auto gemm2 = [&](int t2g, int task) -> bool {
    const int gb = t2g / nt2, n2 = t2g % nt2;
    const int e = m.blk_expert[gb];
    const int pos0 = m.tok_indptr[e] + (gb - m.blk_indptr[e]) * rows;
    const int pend = min(pos0 + rows, m.tok_indptr[e + 1]);
    const Rsrc rb[1] = {make_rsrc(m.wd + (size_t)e * m.H * m.I, (uint32_t)m.H * m.I * 2)};
    const uint32_t bo[1] = {(uint32_t)(16 * n2 + (lane & 15)) * (uint32_t)(m.I * 2)};
    const Rsrc rh = make_rsrc(m.h, (uint32_t)m.T * m.k * m.I * 2);
    auto gate = [&](int round) -> bool {
      if (round != 0) return true;
      if (sched == ET_SCHED_STATIC) {
        if (!wg_wait(c, m.ev_h + gb, nt1, task)) return false;
      } else if (sched == ET_SCHED_BARRIER) {
        if (!wg_wait(c, EV_G1ALL, meta(MD_TOTAL1), task)) return false;
      }
      for (int i = tid; i < rows; i += kThreads) {
        const int pos = pos0 + i;
        rows_off[i] = pos < pend ? (uint32_t)pos * (uint32_t)(m.I * 2) : kOOB;
      }
      __syncthreads();
      return true;
    };
    Tile2 tile;
    if (!tile.run(rh, rows_off, rb, bo, m.I / kKBlock, gate, red)) return false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r == wave) {
          const int pos = pos0 + 16 * mt + 4 * (lane >> 4) + r;
          if (pos < pend) m.y[(size_t)pos * m.H + 16 * n2 + (lane & 15)] = tile.acc[mt][0][r];
        }
    if (sched == ET_SCHED_PER_OP) return true;
    wg_release();
    if (sched != ET_SCHED_DYNAMIC) {
      t0_notify(c, EV_DOWN, 1, meta(MD_TOTAL2), task);
      return true;
    }
    // dynamic: one notify per row on EV_C[token, n2]; zeroing rows run the combine
    if (tid == 0) sh.v[5] = 0;
    __syncthreads();
    if (tid < rows) {
      const int pos = pos0 + tid;
      if (pos < pend) {
        const int t = m.perm[pos] / m.k;
        const int idx = m.ev_c + t * nt2 + n2;
        const int old = add_acqrel(c.ev + idx, -1);
        if (old - 1 == -wc) fired[atomicAdd(&sh.v[5], 1)] = t;
        else if (old - 1 < -wc) raise_fault(ra, ET_ESTATE, task, idx, old - 1);
      }
    }
    __syncthreads();
    const int nf = sh.v[5];
    if (nf > 0) {
      fence_acquire();
      for (int i = tid; i < nf * 16; i += kThreads) {
        const int t = fired[i >> 4];
        const int col = 16 * n2 + (i & 15);
        m.out[(size_t)t * m.H + col] = combine_elem(m, t, col);
      }
    }
    __syncthreads();
    return true;
  };

  auto combine_tile = [&](int t3, int task) -> bool {
    if (sched == ET_SCHED_STATIC || sched == ET_SCHED_BARRIER)
      if (!wg_wait(c, EV_DOWN, meta(MD_TOTAL2), task)) return false;
    const int ncol = cdiv(m.H, kCombCols);
    const int tc = t3 / ncol, cc = t3 % ncol;
    const int col = cc * kCombCols + tid;
    if (col < m.H) {
      const int te = min(m.T, (tc + 1) * kCombTok);
      for (int t = tc * kCombTok; t < te; ++t) m.out[(size_t)t * m.H + col] = combine_elem(m, t, col);
    }
    return true;
  };

  // ------------------------------------------------------------- dispatch
  auto run = [&](int task) -> bool {
    if (task < NR) {
      route(task);
      if (sched == ET_SCHED_PER_OP) return true;
      wg_release();
      if (sched != ET_SCHED_DYNAMIC) {
        t0_notify(c, EV_ROUTE, 1, NR, task);
      } else if (wg_notify(c, EV_ROUTE, 1, NR, task, true)) {
        wg_push(c, 1, [&](int) { return NR; });          // the scan task
      }
      return true;
    }
    if (task == NR) {
      if (sched != ET_SCHED_PER_OP && sched != ET_SCHED_DYNAMIC)
        if (!wg_wait(c, EV_ROUTE, NR, task)) return false;
      const int nb = scan();
      if (sched == ET_SCHED_PER_OP) return true;
      if (sched == ET_SCHED_DYNAMIC) {
        set_total(c, base1 + nb * (nt1 + nt2));
        wg_release();
        wg_push(c, NR, [&](int i) { return NR + 1 + i; });   // the grouping tasks
      } else {
        wg_release();
        t0_notify(c, EV_SCAN, 1, 1, task);
      }
      return true;
    }
    if (task < base1) {
      const int r = task - NR - 1;
      if (sched == ET_SCHED_STATIC || sched == ET_SCHED_BARRIER)
        if (!wg_wait(c, EV_SCAN, 1, task)) return false;
      group(r);
      if (sched == ET_SCHED_PER_OP) return true;
      wg_release();
      if (sched != ET_SCHED_DYNAMIC) {
        t0_notify(c, EV_GROUP, 1, NR, task);
        return true;
      }
      // dynamic: data-dependent notify targets -- the experts this chunk's
      // tokens chose, each decremented by this chunk's rows for it
      int* base = s_i + 1024;
      int* cur = s_i;
      int* fe = s_i + 2048;   // fired experts
      if (tid == 0) sh.v[6] = 0;
      __syncthreads();
      for (int e = tid; e < m.E; e += kThreads) {
        const int n = cur[e] - base[e];
        if (n > 0) {
          const int wcnt = m.counts[e];
          const int old = add_acqrel(c.ev + m.ev_exp + e, -n);
          if (old - n == -wcnt) fe[atomicAdd(&sh.v[6], 1)] = e;
          else if (old - n < -wcnt) raise_fault(ra, ET_ESTATE, task, m.ev_exp + e, old - n);
        }
      }
      __syncthreads();
      const int nf = sh.v[6];
      if (nf > 0) fence_acquire();
      for (int i = 0; i < nf; ++i) {
        const int e = fe[i];
        const int lo = m.task_indptr[e], hi = m.task_indptr[e + 1];
        wg_push(c, hi - lo, [&](int j) { return base1 + lo + j; });
      }
      __syncthreads();
      return true;
    }
    const int total1 = meta(MD_TOTAL1), total2 = meta(MD_TOTAL2);
    if (task < base1 + total1) return gemm1(task - base1, task);
    if (task < base1 + total1 + total2) return gemm2(task - base1 - total1, task);
    return combine_tile(task - base1 - total1 - total2, task);
  };

  const int ncomb = cdiv(m.T, kCombTok) * cdiv(m.H, kCombCols);
  int tasks_run = 0;
  if (sched == ET_SCHED_DYNAMIC) {
    PopState ps;
    for (;;) {
      const int t = wg_pop(c, ps);
      if (t < 0 || !run(t)) break;
      count_run(c, t);
    }
  } else if (sched == ET_SCHED_PER_OP) {
    const int ph = ra.phase;
    int lo = 0, hi = 0;
    if (ph == 0) { lo = 0; hi = NR; }
    else if (ph == 1) { lo = NR; hi = NR + 1; }
    else if (ph == 2) { lo = NR + 1; hi = base1; }
    else {
      const int total1 = meta(MD_TOTAL1), total2 = meta(MD_TOTAL2);
      if (ph == 3) { lo = base1; hi = base1 + total1; }
      else if (ph == 4) { lo = base1 + total1; hi = lo + total2; }
      else { lo = base1 + total1 + total2; hi = lo + ncomb; }
    }
    for (int t = lo + c.wg; t < hi; t += c.G) {
      run(t);
      count_run(c, t);
    }
  } else {
    bool ok = true;
    for (int t = c.wg; ok && t < NR; t += c.G) {
      ok = run(t);
      if (ok) count_run(c, t);
    }
    if (ok && c.wg == c.G - 1) {
      ok = run(NR);
      if (ok) count_run(c, NR);
    }
    for (int r = c.wg; ok && r < NR; r += c.G) {
      ok = run(NR + 1 + r);
      if (ok) count_run(c, NR + 1 + r);
    }
    if (ok) ok = wg_wait(c, EV_SCAN, 1, -1);
    if (ok) {
      const int total1 = meta(MD_TOTAL1), total2 = meta(MD_TOTAL2);
      const int end = base1 + total1 + total2 + ncomb;
      for (int t = base1 + c.wg; ok && t < end; t += c.G) {
        ok = run(t);
        if (ok) count_run(c, t);
      }
    }
  }
  (void)tasks_run;
  epilogue(c, 0);
}

int launch_moe(const LaunchCommon& lc, const float* logits, const uint16_t* x, int T,
               const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, float* out) {
  const et_plan* p = lc.plan;
  MoePlan mp{p->max_tokens, p->hidden, p->inter, p->n_experts, p->top_k,
             moe_n_route(p->n_experts)};
  const MoeAux ax = moe_aux_layout(mp);
  char* aux = lc.ws + p->off_aux;
  const int tv = pick_tile(T, lc.tile);
  const Tiling tl = tiling_of(tv);
  MoeArgs m;
  m.logits = logits;
  m.x = x;
  m.wg = wg;
  m.wu = wu;
  m.wd = wd;
  m.out = out;
  m.topk_ids = reinterpret_cast<int*>(aux + ax.topk_ids);
  m.topk_w = reinterpret_cast<float*>(aux + ax.topk_w);
  m.hist = reinterpret_cast<int*>(aux + ax.hist);
  m.counts = reinterpret_cast<int*>(aux + ax.counts);
  m.tok_indptr = reinterpret_cast<int*>(aux + ax.tok_indptr);
  m.blk_indptr = reinterpret_cast<int*>(aux + ax.blk_indptr);
  m.task_indptr = reinterpret_cast<int*>(aux + ax.task_indptr);
  m.blk_expert = reinterpret_cast<int*>(aux + ax.blk_expert);
  m.perm = reinterpret_cast<int*>(aux + ax.perm);
  m.inv = reinterpret_cast<int*>(aux + ax.inv);
  m.h = reinterpret_cast<uint16_t*>(aux + ax.h);
  m.y = reinterpret_cast<float*>(aux + ax.y);
  m.T = T;
  m.H = p->hidden;
  m.I = p->inter;
  m.E = p->n_experts;
  m.k = p->top_k;
  m.NR = mp.n_route;
  m.tpr = mp.tpr(T);
  m.ev_exp = mp.ev_exp();
  m.ev_h = mp.ev_h();
  m.ev_c = mp.ev_c();
  RunArgs ra = lc.run_args();
  ra.n_init = mp.n_route;
  ra.total_hint = kUnknownTotal;
  ra.extent = mp.extent(T, tl);
  const void* k = tv == TV_M16   ? reinterpret_cast<const void*>(&moe_kernel<1>)
                  : tv == TV_M32 ? reinterpret_cast<const void*>(&moe_kernel<2>)
                                 : reinterpret_cast<const void*>(&moe_kernel<4>);
  if (lc.sched == ET_SCHED_PER_OP) {
    for (int ph = 0; ph < 6; ++ph) {
      ra.phase = ph;
      int e = lc.launch(k, &ra, &m, false);
      if (e) return e;
    }
    return ET_OK;
  }
  return lc.launch(k, &ra, &m, true);
}

}  // namespace et
