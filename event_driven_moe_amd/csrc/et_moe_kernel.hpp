// et_moe_kernel.hpp -- the MoE layer as one persistent kernel (template shared by
// the MoE entry point and the router -> MoE -> dense MLP chain).
//
// The chain TopK routing -> token grouping -> grouped GEMMs of Event Tensor
// notes (section "两类动态性如何进入依赖表示", section "完整 MoE layer") with a
// weighted combine at the end:
//   routing task r   top-k of the router logits of token chunk r, renormalised
//                    weights, a per-chunk expert histogram; notifies EV_ROUTE;
//   scan             column sums of the histograms (rows per expert), CSR
//                    offsets of rows, row blocks and tasks per expert, the
//                    base position of every (chunk, expert); it learns the
//                    number of GEMM tasks of this call;
//   grouping r       stable positions of chunk r's (token, slot) pairs;
//                    dynamic: notifies EV_EXP[e] of the experts its tokens
//                    chose, by its number of rows for each (data-dependent
//                    targets, data-dependent wait count = rows routed to e);
//   gate/up task     (block gb, bn1 columns of h): rows gathered from x by the
//                    permutation; h = SiLU(x Wg) * (x Wu) in bf16; static:
//                    notifies EV_H[gb]; dynamic: EV_HE[e] (all of expert e's
//                    gate/up tiles);
//   down task        (block gb, bn2 output columns): y = h Wd (bf16 rows);
//                    waits on EV_H[gb] only, not on all gate/up tasks -- the
//                    event that removes the barrier between the two
//                    GroupGEMMs (dynamic: pushed when EV_HE[e] fires);
//   combine          out[t] = sum_s w[t, s] y[inv[t, s]] in slot order, in
//                    tiles after EV_DOWN (all down tiles), after EV_CG[group,
//                    column tile] (static, shallow down phases), or inline in
//                    the down tile completing EV_C[t, c] (a few tokens).
// Static and dynamic modes: every routing workgroup, once all histograms are
// out (EV_ROUTE), runs its own share of the scan (the totals, and the rows
// of earlier chunks for its own chunk) and groups its own chunk, so neither
// the scan nor the grouping is a task of its own or a hop through an event.
// Dynamic: the grouping that completes EV_EXP[e] pushes expert e's task range
// tasks[task_indptr[e] : task_indptr[e+1]] (data-dependent fan-out).  Static
// mode keeps the fine-grained EV_H edge but, as the page's static lowering
// does for data-dependent edges, replaces EV_EXP by one coarse "all grouped"
// event.  The barrier and per-operator baselines keep the scan and the
// grouping as tasks of their own and use one event per operator throughout.
#pragma once

#include <type_traits>

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
  int* perm;
  int* inv;
  uint16_t* h;
  uint16_t* y;       // [T*k, H] bf16 down-projection rows (workspace)
  int T, H, I, E, k, NR, tpr;
  int ccols;           // combine tile columns
  int ev_exp, ev_he, ev_h, ev_c;
  // router GEMM -> MoE -> dense MLP chain (kernels with kBlock only)
  const uint16_t* wr;  // [E, H] router weights, K-contiguous (row e = column e of W_router)
  float* logits_ws;    // [T, E] router logits the routing tasks compute (workspace)
  uint16_t* zb;        // [T, H] bf16 copy of out, the dense MLP's input (workspace)
  const uint16_t* mg;  // [Im, H] dense MLP gate weights, K-contiguous
  const uint16_t* mu;  // [Im, H]
  const uint16_t* md;  // [H, Im]
  uint16_t* h2;        // [T, Im] bf16 dense MLP intermediate (workspace)
  float* y2;           // [T, H] dense MLP output
  int Im;
  int ev_z, ev_hm;     // E_z[mb] (combine tiles of row block mb), E_hm[mb][Im / 128]
  int qall;   // dynamic: the static-order queue may be chosen (queue order auto or static)
  int qforce; // dynamic: ... and is chosen whatever the routing (queue order static)
};

// LDS: three slot arrays (the GEMM ring of the wide variants; scratch for
// the other task kinds) and a small general region.
constexpr int kScanHistBytes = kHistEntries * 4;                    // slot 0
// slot 1 during the scan: counts, blocks, 8 scan temporaries, partial sums;
// the per-chunk scan adds rows-before-chunk and their partial sums
constexpr int kScanTempBytes = (3 * kMaxExperts + 8 + 2 * kThreads) * 4;
constexpr int kGenRowsOff = 0, kGenFired = 512, kGenIdx = 1024;
// Static and dynamic schedules with at most this many tokens: the combine
// runs inline in the down tile whose notify completes a token's k rows for
// its column tile (EV_C), instead of as tiles after the last down tile
// (EV_DOWN).  It saves the wait for every down tile at T = 1 (static 33.2 ->
// 32.4 us, dynamic 47.0 -> 42.6 us); from 8 tokens on the per-row notifies
// cost as much as they save, and at 64 tokens (64-row blocks) far more
// (moe_skewed T=64 static 94 -> 115 us).
constexpr int kInlineCombineTokens = 4;
// Dynamic schedule: with at most this many gate/up tasks per workgroup, routing
// chunk 0 alone pushes them (early push); with more, every chunk pushes a share.
constexpr int kSoloPush = 4;
constexpr int kIdxCache = 2 * (kMaxExperts + 1) * 4;   // tok_indptr + blk_indptr copies
constexpr int kGenBytes = kGenIdx + kIdxCache;

// ---------------------------------------------------------------------------
// block-wide exclusive scan of n <= 1024 ints held in LDS (in place);
// returns the total.  256 threads, 4 consecutive elements per thread.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_exscan(int* a, int n, int* tmp /* >= 8 ints */) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * t + i;
    v[i] = j < n ? a[j] : 0;
    s += v[i];
  }
  const int inc = wave_incl_scan(s);
  if (lane == 63) tmp[wave] = inc;
  lds_barrier();
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
  lds_barrier();
  return total;
}

// float -> unsigned key with the same order (-0.0 and +0.0 map to one key);
// every finite value maps above 0
__device__ __forceinline__ uint32_t route_key32(float v) {
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, u);
}

// Tile variant traits: rows per block, columns per gate/up and down task,
// and the GEMM tile type of each projection.
template <int TV>
struct MoeCfg {
  static constexpr Tiling t = tiling_of(TV);
  static constexpr int MT = t.mt;
  static constexpr bool kWide = TV == TV_W64 || TV == TV_W128;
  static constexpr int NH = kWide ? 2 : 1;          // 16-column h groups per wave (gate/up)
  static constexpr int NB2 = t.bn2 == 16 ? 1 : 4;   // 16-column groups per wave (down)
  static constexpr int PD = MT == 1 ? 4 : (MT == 2 ? 3 : 2);
  static constexpr int PD2 = NB2 == 4 ? 2 : PD;     // down tiles: K-blocks in flight
  static constexpr int kOcc = 1;                    // workgroups per CU
};

template <int TV, bool COH, int NB, int PDX>
struct TileOf {
  using type = typename std::conditional<
      MoeCfg<TV>::kWide, RingTile<MoeCfg<TV>::MT, COH>,
      StreamTile<MoeCfg<TV>::MT, NB, 4, PDX, COH>>::type;
};

template <int A, int B>
constexpr int cmax() { return A > B ? A : B; }

// Static schedule position of workgroup w: workgroups are dispatched to the
// XCDs round-robin (w % 8), so positions p*32 .. p*32+31 -- consecutive task
// ids -- all run on XCD p and share its L2.
__device__ __forceinline__ int xcd_pos(int w, int G) {
  return (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w;
}

// kBlock: the router GEMM -> MoE layer -> dense MLP chain in the same launch
// (the routing task computes its tokens' logits first; the combine also
// writes its rows in bf16 and notifies E_z; the dense MLP's tasks follow).
template <int TV, bool kBlock = false>
__global__ __launch_bounds__(kThreads, MoeCfg<TV>::kOcc) void moe_kernel(RunArgs ra, MoeArgs m) {
  using Cfg = MoeCfg<TV>;
  using Tile1 = typename TileOf<TV, false, 2 * Cfg::NH, Cfg::PD>::type;   // gate/up: reads x
  using Tile2 = typename TileOf<TV, true, Cfg::NB2, Cfg::PD2>::type;      // down: reads h (this launch)
  constexpr int MT = Cfg::MT;
  constexpr bool kWide = Cfg::kWide;
  constexpr int bn1 = Cfg::t.bn1, bn2 = Cfg::t.bn2;
  constexpr int kSlot = kWide ? Tile1::kStageBytes : 0;
  __shared__ Shared sh;
  __shared__ __align__(16) unsigned char gen[kGenBytes];
  __shared__ __align__(16) unsigned char s0[cmax<cmax<kSlot, kScanHistBytes>(),
                                                 cmax<Tile1::kLdsBytes, Tile2::kLdsBytes>()>()];
  __shared__ __align__(16) unsigned char s1[cmax<kSlot, kScanTempBytes>()];
  __shared__ __align__(16) unsigned char s2[cmax<kSlot, 16>()];

  Ctx c;
  if (!prologue(c, ra, &sh)) return;
  const int sched = ra.sched;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
  const int rows = 16 * MT;
  const int nt1 = m.I / bn1, nt2 = m.H / bn2;
  const int NR = m.NR;
  const int base1 = 2 * NR + 1;
  // static / dynamic: every routing workgroup also scans and groups its own
  // chunk (no scan or grouping tasks of their own)
  const bool fused_front = sched == ET_SCHED_STATIC || sched == ET_SCHED_DYNAMIC;
  // one routing chunk (static / dynamic): the histogram and the chosen
  // experts stay in LDS, and no global round trip separates routing from
  // the scan and the grouping
  const bool solo_route = NR == 1 && fused_front;
  // With at least kBcastChunks routing chunks, the events their workgroups
  // wait on (EV_ROUTE; dynamic: EV_SCAN before pushing) are broadcast events
  // and chunk 0 alone publishes the scan results; with fewer, polling the
  // counter is not contended, every chunk publishes the same scan results,
  // and a chunk needs no second event before it pushes.
  const bool many_chunks = NR >= kBcastChunks;
  // static / dynamic: the routing workgroup keeps its chunk's expert ids in
  // LDS for its own grouping when they fit (the index cache's space, unused
  // until the gemm tasks)
  const bool keep_ids = fused_front && m.tpr * m.k <= kIdxCache / 4;
  const int wc = m.k;   // EV_C wait count: the k rows of a token, one per down column tile
  // (compiled into the 16-row variant only, the one tiny token counts use:
  // the extra path measurably slowed the other variants' down tiles)
  const bool inline_comb = !kBlock && TV == TV_M16 &&
                           (sched == ET_SCHED_STATIC || sched == ET_SCHED_DYNAMIC) &&
                           m.T <= kInlineCombineTokens;
  const int ncomb = inline_comb ? 0 : cdiv(m.T, kCombTok) * cdiv(m.H, m.ccols);   // combine tiles
  // The chain's dense MLP (kBlock): row blocks of 16 tokens while the MoE
  // runs its 16-row variants, else 64; 16-column gate/up and down tiles.
  constexpr int MTM = (TV == TV_M16 || TV == TV_M16W) ? 1 : 4;
  constexpr int PDM = MTM == 1 ? 4 : 2;
  const int rows_m = 16 * MTM;
  const int nmb = kBlock ? cdiv(m.T, rows_m) : 0;
  const int ngt_m = kBlock ? m.Im / 16 : 1, ndt_m = m.H / 16, nht_m = kBlock ? m.Im / kHTile : 0;
  const int n_mg = nmb * ngt_m, n_md = nmb * ndt_m;
  // wait count of E_z[b]: the combine tiles of block b's 16-token groups
  auto z_wait = [&](int b) ET_INLINE {
    const int g0 = b * rows_m / kCombTok, g1 = min(cdiv(m.T, kCombTok), (b + 1) * rows_m / kCombTok);
    return (g1 - g0) * cdiv(m.H, m.ccols);
  };
  // Static schedule with at least kCombGroupMin token groups and at most
  // kCombGroupRounds down tiles per workgroup: each combine tile waits on its
  // own event E_cg[token group, column tile] instead of the last down tile,
  // so combine tiles overlap the down tiles' tail.  With fewer groups each
  // group's rows reach nearly every active expert and its event fires only
  // at the end; with deeper down phases (and in the dynamic schedule, where
  // each down tile would have to push the tiles it completes) the notifies
  // cost more than the overlap saves.  Otherwise the combine waits on
  // EV_DOWN.
  auto comb_groups = [&](int total2) ET_INLINE {
    return !kBlock && sched == ET_SCHED_STATIC && !inline_comb && cdiv(m.T, kCombTok) >= kCombGroupMin &&
           total2 <= kCombGroupRounds * c.G;
  };
  // Dynamic: queue shard key of gate/up or down tile (expert e, column tile n
  // of nt).  The wide variants with 16 or more column tiles per expert key
  // groups of 4 adjacent tiles together: a shard then holds, block by block,
  // the same 4 weight tiles, so a batched claim takes one block's A rows
  // through 4 tiles and the workers beside it stream the same tiles for the
  // next blocks (moe_large T=8192 dynamic 8.78-8.82 -> 8.27-8.30 ms, T=2048
  // 4.17-4.18 -> 4.01-4.02 ms).  With fewer tiles (moe_skewed: 6 and 8) the
  // groups would leave shards short of work, so each tile keys alone.
  auto tile_key = [&](int e, int n, int nt) ET_INLINE {
    const int g = (kWide && nt >= 16) ? 4 : 1;
    return e * cdiv(nt, g) + n / g;
  };
  // wait count of E_cg[tc, cc]: k rows per token of the group, times the down
  // column tiles overlapping the combine tile's columns
  auto comb_wait = [&](int tc, int cc) ET_INLINE {
    const int ntok = min(m.T, (tc + 1) * kCombTok) - tc * kCombTok;
    const int c0 = cc * m.ccols, c1 = min(m.H, c0 + m.ccols);
    return ntok * m.k * ((c1 - 1) / bn2 - c0 / bn2 + 1);
  };

  // LDS carve-outs (task kinds never overlap in time inside one workgroup)
  int* s_i = reinterpret_cast<int*>(s0);                              // route / scan / group
  uint32_t* rows_off = reinterpret_cast<uint32_t*>(gen + kGenRowsOff);  // gemm: [16*MT]
  int* fired = reinterpret_cast<int*>(gen + kGenFired);                 // gemm2: fired tokens

  auto meta = [&](int i) ET_INLINE { return ld_rlx(&ra.hdr[HDR_META + i]); };
  // LDS copies of the per-expert row and block offsets (filled once per call
  // per workgroup, after the scan), so task decoding costs no memory trips
  int* c_tok = reinterpret_cast<int*>(gen + kGenIdx);
  int* c_blk = c_tok + kMaxExperts + 1;
  bool cached = false;
  // dynamic: this call's GEMM tasks are static-order queue entries (the scan's
  // choice; known to every task once the scan results are out)
  bool qs = false;
  auto load_cache = [&]() ET_INLINE {
    if (cached) return;
    if (m.qall) qs = ld_rlx(&ra.hdr[HDR_META + MD_QSTATIC]) != 0;
    for (int e = tid; e <= m.E; e += kThreads) {
      c_tok[e] = ld_coh(&m.tok_indptr[e]);
      c_blk[e] = ld_coh(&m.blk_indptr[e]);
    }
    __syncthreads();
    cached = true;
  };
  // task -> (expert, column tile, block): expert e owns nblk_e * nt tasks,
  // ordered column tile first, then block, so consecutive tasks share a
  // weight slice; e is the largest expert whose first task is <= t (experts
  // without rows own no tasks and share their successor's start)
  auto decode = [&](int t, int nt, int& e, int& n, int& gb) ET_INLINE {
    int lo = 0, hi = m.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (c_blk[mid] * nt <= t) lo = mid; else hi = mid;
    }
    e = lo;
    const int nblk = c_blk[e + 1] - c_blk[e];
    const int l = t - c_blk[e] * nt;
    n = l / nblk;
    gb = c_blk[e] + l % nblk;
  };
  const Rsrc ry = make_rsrc(m.y, (uint32_t)((size_t)m.T * m.k * m.H * 2));

  // Combine for ntok tokens (token of list entry i: tok_of(i)) over columns
  // [c0, c0 + ncols): out[t, col] = sum_{s<k} w[t, s] * y[inv[t, s], col],
  // accumulated in fp32 in slot order with one fused multiply-add per slot
  // (the y rows are bf16).  The (w, position) pairs are staged in LDS first;
  // each thread then owns 8 columns of one or two items and issues all their
  // 16-byte row loads before summing, so a pass costs one memory round trip.
  // The inline and tiled combines share this code and give bit-identical
  // results.
  auto combine = [&](int ntok, auto tok_of, int c0, int ncols, float* cw, int* cp) ET_INLINE {
    const int k = m.k;
    for (int i = tid; i < ntok * k; i += kThreads) {
      const int t = tok_of(i / k), s = i % k;
      cw[i] = ld_coh(&m.topk_w[t * k + s]);
      cp[i] = ld_coh(&m.inv[t * k + s]);
    }
    __syncthreads();
    const int nq = ncols / 8;              // 8 columns (16 bytes of bf16) per item
    const int nit = ntok * nq;
    const Rsrc rout = make_rsrc(m.out, (uint32_t)((size_t)m.T * m.H * 4));
    // IT items per thread per pass, all KM * IT row loads issued before any
    // sum (IT = 2 when k <= 8 keeps the loads within 64 registers); the next
    // pass's rows are requested before the current pass is summed, so the
    // tile pays about one memory round trip, not one per pass.  No memory
    // access sits in a branch: items past the tile and slots past k load and
    // store at an out-of-range offset (the hardware drops those), and the
    // pass loop issues one pass past the last.  With a load or store under a
    // branch the compiler can no longer count which loads are still in
    // flight at each wait, and it waited for all but the last two before
    // every load, serialising the pass.
    auto pass = [&](auto km_c, auto it_c) ET_INLINE {
      constexpr int KM = decltype(km_c)::value, IT = decltype(it_c)::value;
      auto issue = [&](int i0, i32x4 (&yv)[IT][KM]) ET_INLINE {
        uint32_t off[IT][KM];
#pragma unroll
        for (int u = 0; u < IT; ++u) {
          const int i = i0 + u * kThreads;
          const bool ok = i < nit;
          const int ti = ok ? i / nq : 0, col = c0 + 8 * (i % nq);
#pragma unroll
          for (int s = 0; s < KM; ++s) {
            const int pos = cp[ti * k + (s < k ? s : 0)];
            off[u][s] = ok && s < k ? (uint32_t)((pos * (size_t)m.H + col) * 2) : kOOB;
          }
        }
#pragma unroll
        for (int u = 0; u < IT; ++u)
#pragma unroll
          for (int s = 0; s < KM; ++s) yv[u][s] = ld16c(ry, off[u][s]);
      };
      auto finish = [&](int i0, const i32x4 (&yv)[IT][KM]) ET_INLINE {
#pragma unroll
        for (int u = 0; u < IT; ++u) {
          const int i = i0 + u * kThreads;
          const bool ok = i < nit;
          const int ti = ok ? i / nq : 0, col = c0 + 8 * (i % nq);
          float acc[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
          for (int s = 0; s < KM; ++s)
            if (s < k) {
              const float w = cw[ti * k + s];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint32_t two = (uint32_t)yv[u][s][q];   // two bf16: low half first
                acc[2 * q] = __fmaf_rn(w, __builtin_bit_cast(float, two << 16), acc[2 * q]);
                acc[2 * q + 1] = __fmaf_rn(w, __builtin_bit_cast(float, two & 0xffff0000u), acc[2 * q + 1]);
              }
            }
          const size_t el = (size_t)tok_of(ti) * m.H + col;
          const uint32_t oo = ok ? (uint32_t)(el * 4) : kOOB;
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(i32x4, make_float4(acc[0], acc[1], acc[2], acc[3])), rout, (int)oo, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(i32x4, make_float4(acc[4], acc[5], acc[6], acc[7])), rout,
              (int)(ok ? oo + 16u : kOOB), 0, 0);
          if constexpr (kBlock) {
            // the dense MLP's input: the same rows rounded to bf16
            i32x4 zv;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              zv[q] = (int)((uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16));
            st16c(make_rsrc(m.zb, (uint32_t)m.T * m.H * 2), ok ? (uint32_t)(el * 2) : kOOB, zv);
          }
        }
      };
      constexpr int kStep = IT * kThreads;
      const int npass = cdiv(nit, kStep);   // the same in every thread
      i32x4 ya[IT][KM], yb[IT][KM];
      issue(tid, ya);
      for (int p = 0;; p += 2) {
        issue(tid + (p + 1) * kStep, yb);
        finish(tid + p * kStep, ya);
        if (p + 1 >= npass) break;
        issue(tid + (p + 2) * kStep, ya);
        finish(tid + (p + 1) * kStep, yb);
        if (p + 2 >= npass) break;
      }
    };
    using std::integral_constant;
    if (k <= 8) pass(integral_constant<int, 8>{}, integral_constant<int, 2>{});
    else pass(integral_constant<int, kMaxTopK>{}, integral_constant<int, 1>{});
    __syncthreads();
  };
  // static / barrier: coarse events already seen fired by this workgroup
  bool seen_group = false, seen_g1 = false, seen_down = false;

  // ------------------------------------------------------------- routing
  // One wave per token.  Lane l holds the order-preserving integer keys of
  // experts l, l + 64, ...; each of the k rounds takes the wave-wide largest
  // key, then the lowest expert index holding it (ties go to the lower index;
  // -0.0 and +0.0 share a key), with two DPP reductions and no LDS traffic.

  auto route = [&](int r) ET_INLINE {
    int* hist_l = s_i;   // [E]
    int* ids_l = reinterpret_cast<int*>(gen + kGenIdx);   // [tpr * k] when keep_ids
    const int t0 = r * m.tpr;
    const int t1 = min(m.T, t0 + m.tpr);
    if constexpr (kBlock) {
      // The router GEMM of this chunk's tokens: logits[t, e] = x[t] . Wr[e]
      // (K = H, fp32 accumulation), 16 tokens x 32 experts per tile pass;
      // stored to the workspace and read back below like the input logits.
      const Rsrc rx = make_rsrc(m.x, (uint32_t)m.T * m.H * 2);
      const Rsrc rwr = make_rsrc(m.wr, (uint32_t)m.E * m.H * 2);
      for (int tg = t0; tg < t1; tg += 16) {
        for (int i = tid; i < 16; i += kThreads)
          rows_off[i] = tg + i < t1 ? (uint32_t)(tg + i) * (uint32_t)(m.H * 2) : kOOB;
        __syncthreads();
        for (int eg = 0; eg < m.E; eg += 32) {
          const Rsrc rb[2] = {rwr, rwr};
          uint32_t bo[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int e = eg + 16 * j + (lane & 15);
            bo[j] = e < m.E ? (uint32_t)e * (uint32_t)(m.H * 2) : kOOB;
          }
          StreamTile<1, 2, 4, 4, false> tile;   // waves split K, summed through LDS
          tile.run(rx, rows_off, rb, bo, m.H / kKBlock, [](int) { return true; },
                   reinterpret_cast<float*>(s0));
          // every wave holds the sums; wave q stores accumulator row q
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (q == wave) {
                const int t = tg + 4 * (lane >> 4) + q, e = eg + 16 * j + (lane & 15);
                if (t < t1 && e < m.E) st_coh(&m.logits_ws[(size_t)t * m.E + e], tile.acc[0][j][q]);
              }
        }
      }
      wg_release();   // the chunk's logits are complete before they are read
    }
    for (int e = tid; e < m.E; e += kThreads) hist_l[e] = 0;
    __syncthreads();
    const Rsrc rlog = make_rsrc(kBlock ? m.logits_ws : m.logits, (uint32_t)m.T * m.E * 4u);
    // NJ keys per lane (E <= 64 NJ); the logits of NB tokens of this wave
    // (t0 + wave, t0 + wave + 4, ...) are requested before any is ranked
    auto route_tokens = [&](auto nj_c, auto nb_c) ET_INLINE {
      constexpr int NJ = decltype(nj_c)::value, NB = decltype(nb_c)::value;
      for (int tb = t0 + wave; tb < t1; tb += 4 * NB) {
        // buffer loads without branches, all in flight together; lanes past
        // the chunk or past E read out of range and take key 0, below every
        // real key
        uint32_t kb[NB][NJ];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int t = tb + 4 * b, e = lane + 64 * j;
            const bool ok = t < t1 && e < m.E;
            kb[b][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                rlog, ok ? (t * m.E + e) * 4 : (int)kOOB, 0, kBlock ? 16 : 0);
          }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            kb[b][j] = (tb + 4 * b < t1 && lane + 64 * j < m.E)
                           ? route_key32(__builtin_bit_cast(float, kb[b][j])) : 0u;
        // the NB tokens' k rounds are interleaved: their wave reductions are
        // independent chains that the scheduler overlaps
        uint32_t taken[NB], my_key[NB], key0[NB];
        int my_e[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          taken[b] = 0;   // bit j: my expert lane + 64 j already chosen
          my_e[b] = -1;
          my_key[b] = key0[b] = 0;
        }
        for (int s = 0; s < m.k; ++s) {
          uint32_t best[NB], top[NB];
          int best_e[NB], e[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            best[b] = 0;
            best_e[b] = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              const bool ok = !((taken[b] >> j) & 1u) && lane + 64 * j < m.E;
              if (ok && kb[b][j] > best[b]) {   // strict: equal keys keep the lower expert
                best[b] = kb[b][j];
                best_e[b] = lane + 64 * j;
              }
            }
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) top[b] = wave_reduce_u32<true>(best[b]);
#pragma unroll
          for (int b = 0; b < NB; ++b)
            e[b] = (int)wave_reduce_u32<false>(best[b] == top[b] ? (uint32_t)best_e[b] : 0xffffffffu);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            if (s == 0) key0[b] = top[b];
            if (lane == s) { my_e[b] = e[b]; my_key[b] = top[b]; }
            if ((e[b] & 63) == lane) taken[b] |= 1u << (e[b] >> 6);
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int t = tb + 4 * b;
          if (t >= t1) break;
          // weights: softmax over the kept logits (= renormalised top-k
          // softmax); lanes 0..k-1 of row 0 hold them, summed within the row
          const float ex = lane < m.k ? expf(key_to_float(my_key[b]) - key_to_float(key0[b])) : 0.f;
          const float sum = row_sum16(ex);
          if (lane < m.k) {
            st_coh(&m.topk_ids[t * m.k + lane], my_e[b]);
            st_coh(&m.topk_w[t * m.k + lane], ex / sum);
            atomicAdd(&hist_l[my_e[b]], 1);
            if (keep_ids) ids_l[(t - t0) * m.k + lane] = my_e[b];
          }
        }
      }
    };
    using std::integral_constant;
    if (m.E <= 64) route_tokens(integral_constant<int, 1>{}, integral_constant<int, 4>{});
    else if (m.E <= 128) route_tokens(integral_constant<int, 2>{}, integral_constant<int, 4>{});
    else if (m.E <= 256) route_tokens(integral_constant<int, 4>{}, integral_constant<int, 4>{});
    else route_tokens(integral_constant<int, kMaxExperts / 64>{}, integral_constant<int, 1>{});
    lds_barrier();   // the histogram is complete; the id and weight stores stay in flight
    if (!solo_route)
      for (int e = tid; e < m.E; e += kThreads) st_coh(&m.hist[r * m.E + e], hist_l[e]);
  };

  // ------------------------------------------------------------- scan
  auto scan = [&]() ET_INLINE {
    int* hs = s_i;                         // [n_ne][E]
    int* cnt = reinterpret_cast<int*>(s1); // [E]
    int* blk = cnt + 1024;                 // [E] -> block offsets
    int* tmp = blk + 1024;                 // [8]
    int* part = tmp + 8;                   // [256] chunk sums
    const int n_ne = cdiv(m.T, m.tpr);
    const int tot = n_ne * m.E;
    // the histograms copied straight into LDS (coherent 16-byte copies that
    // take no registers, all in flight at once: at most 8 1 KB chunks per
    // wave); a solo routing chunk left its histogram in hs already
    const Rsrc rhist = make_rsrc(m.hist, (uint32_t)(4 * tot + 15) & ~15u);
    const int nv = tot / 4;
    static_assert(kHistEntries <= 4 * 8 * 256, "8 chunk copies per wave");
    if (!solo_route) {
      for (int ch = wave; ch < cdiv(tot, 256); ch += 4)
        dma16<true>(rhist, hs + 256 * ch, (uint32_t)(1024 * ch + 16 * lane));
      wait_mem();
    }
    __syncthreads();
    // per-expert prefix over the chunks r: P threads per expert, each summing
    // a contiguous range of about 4 or more chunks, then the P partial sums
    // in order
    int P = m.E >= kThreads ? 1 : kThreads / m.E;
    P = min(P, cdiv(n_ne, 4));
    const int span = cdiv(n_ne, P);
    for (int q = tid; q < m.E * P; q += kThreads) {
      const int e = q / P, p = q % P;
      int acc = 0;
#pragma unroll 8
      for (int r = p * span; r < min(n_ne, (p + 1) * span); ++r) acc += hs[r * m.E + e];
      part[q % kThreads] = acc;
    }
    __syncthreads();
    for (int q = tid; q < m.E * P; q += kThreads) {
      const int e = q / P, p = q % P;
      int run = 0;
      for (int pp = 0; pp < p; ++pp) run += part[(e * P + pp) % kThreads];
#pragma unroll 8
      for (int r = p * span; r < min(n_ne, (p + 1) * span); ++r) {
        const int v = hs[r * m.E + e];
        hs[r * m.E + e] = run;
        run += v;
      }
      if (p == P - 1) {
        cnt[e] = run;
        blk[e] = cdiv(run, rows);
        st_coh(&m.counts[e], run);
      }
    }
    lds_barrier();
    block_exscan(cnt, m.E, tmp);           // cnt -> tok_indptr
    const int nb = block_exscan(blk, m.E, tmp);
    for (int e = tid; e < m.E; e += kThreads) {
      st_coh(&m.tok_indptr[e], cnt[e]);
      st_coh(&m.blk_indptr[e], blk[e]);
      st_coh(&m.task_indptr[e], blk[e] * nt1);
    }
    if (tid == 0) {
      st_coh(&m.tok_indptr[m.E], m.T * m.k);
      st_coh(&m.blk_indptr[m.E], nb);
      st_coh(&m.task_indptr[m.E], nb * nt1);
    }
    // chunk bases hist[r, e] = tok_indptr[e] + rows of e in chunks before r,
    // four per 16-byte store (the four share a chunk when E % 4 == 0)
    if (m.E % 4 == 0) {
      for (int i = tid; i < nv; i += kThreads) {
        const int e = (4 * i) % m.E;
        const i32x4 h = *reinterpret_cast<const i32x4*>(hs + 4 * i);
        st16c(rhist, 16u * i, i32x4{h[0] + cnt[e], h[1] + cnt[e + 1], h[2] + cnt[e + 2], h[3] + cnt[e + 3]});
      }
    } else {
      for (int i = tid; i < tot; i += kThreads) st_coh(&m.hist[i], hs[i] + cnt[i % m.E]);
    }
    if (tid == 0) {
      st_rlx(&ra.hdr[HDR_META + MD_NB], nb);
      st_rlx(&ra.hdr[HDR_META + MD_TOTAL1], nb * nt1);
      st_rlx(&ra.hdr[HDR_META + MD_TOTAL2], nb * nt2);
    }
    lds_barrier();   // every caller releases (store-completion wait) before notifying
    return nb;
  };

  // ------------------------------------------------------------- grouping
  // Stable counting sort of the routed rows of tokens [ta, tb) (expert ids at
  // ids[(t - ta) * k + s]): row (t, s) of expert e goes to position cur[e] +
  // (rows of e among the range's earlier tokens).  The range is cut into S
  // consecutive sub-ranges, one per 16-lane group: each counts its rows per
  // expert, an exclusive prefix over the sub-ranges gives each its first
  // position per expert, and each then places its own tokens in order (a
  // token's k experts are distinct, so its lanes touch distinct cursors).
  // cur[e] ends advanced by the range's rows of e.  cnt: S * E ints of LDS.
  auto group_range = [&](int ta, int tb, const int* ids, int* cur, int* cnt, int S) ET_INLINE {
    S = min(S, max(1, cdiv(tb - ta, 4)));   // sub-ranges of >= 4 tokens: S prefix steps vs n / S placements
    const int L = cdiv(tb - ta, S);
    const int j = tid >> 4, l = tid & 15;
    const int u0 = j * L, u1 = min(tb - ta, u0 + L);
    const bool act = j < S && l < m.k;
    for (int i = tid; i < S * m.E; i += kThreads) cnt[i] = 0;
    __syncthreads();
    if (act)
      for (int u = u0; u < u1; ++u) atomicAdd(&cnt[j * m.E + ids[u * m.k + l]], 1);
    __syncthreads();
    for (int e = tid; e < m.E; e += kThreads) {
      int run = cur[e];
      for (int q = 0; q < S; ++q) {
        const int v = cnt[q * m.E + e];
        cnt[q * m.E + e] = run;
        run += v;
      }
      cur[e] = run;
    }
    __syncthreads();
    if (act)
      for (int u = u0; u < u1; ++u) {
        const int q = (ta + u) * m.k + l;
        const int pos = cnt[j * m.E + ids[u * m.k + l]]++;
        st_coh(&m.perm[pos], q);
        st_coh(&m.inv[q], pos);
      }
    __syncthreads();
  };

  // Grouping of routing chunk r with the cursors (first position of the
  // chunk's rows per expert) in s_i[0, E): the chunk's expert ids are staged
  // in LDS in passes of whole tokens (at most 2048 pairs), unless the routing
  // workgroup left them there (keep_ids).
  auto group_chunk = [&](int r) ET_INLINE {
    int* cur = s_i;            // [E]
    int* cnt = s_i + 5120;     // [S * E] <= 3072
    const int S = min(16, 3072 / m.E);
    const int t0 = r * m.tpr;
    const int t1 = min(m.T, t0 + m.tpr);
    if (keep_ids) {
      group_range(t0, t1, reinterpret_cast<const int*>(gen + kGenIdx), cur, cnt, S);
      cached = false;          // the ids sat in the index cache's space
      return;
    }
    int* ids = s_i + 3072;     // [2048]
    const int tp = 2048 / m.k;   // tokens per pass
    for (int ta = t0; ta < t1; ta += tp) {
      const int tb = min(t1, ta + tp);
      for (int q = ta * m.k + tid; q < tb * m.k; q += kThreads) ids[q - ta * m.k] = ld_coh(&m.topk_ids[q]);
      __syncthreads();
      group_range(ta, tb, ids, cur, cnt, S);
    }
  };

  // Grouping task of routing chunk r (barrier and per-op schedules): its rows
  // start at the chunk bases the scan stored in hist[r, :].
  auto group = [&](int r) ET_INLINE {
    for (int e = tid; e < m.E; e += kThreads) {
      const int b = ld_coh(&m.hist[r * m.E + e]);
      s_i[e] = b;
      s_i[1024 + e] = b;
    }
    group_chunk(r);
  };

  // ------------------------------------------------------------- chunk scan
  // Static and dynamic schedules: once every chunk's histogram is published
  // (EV_ROUTE), routing workgroup r computes what its grouping needs itself
  // instead of waiting for one scan task: per expert the rows over all
  // chunks and the rows in chunks before r, then the experts' first rows
  // (tok_indptr) and first blocks (blk_indptr).  Chunk 0 stores them and
  // the task totals for the gemm tasks and fires EV_SCAN; a workgroup that
  // pushes gemm tasks first sees EV_SCAN fired, so what the tasks read is
  // published before they can be claimed.  Leaves the cursors of chunk r in s_i[0, E) and a copy in
  // s_i[1024, 1024 + E), the exclusive tok_indptr / blk_indptr in s1[0, E) /
  // s1[1024, 1024 + E).  Returns the number of row blocks.
  auto scan_chunk = [&](int r) ET_INLINE -> int {
    int* hs = s_i;                         // [n_ne][E]
    int* cnt = reinterpret_cast<int*>(s1); // [E]
    int* blk = cnt + 1024;                 // [E]
    int* tmp = blk + 1024;                 // [8]
    int* part = tmp + 8;                   // [256]
    int* bef = part + kThreads;            // [E] rows in chunks before r
    int* partb = bef + kMaxExperts;        // [256]
    const int n_ne = cdiv(m.T, m.tpr);
    const int tot = n_ne * m.E;
    if (!solo_route) {   // a solo chunk's histogram is in hs already
      const Rsrc rhist = make_rsrc(m.hist, (uint32_t)(4 * tot + 15) & ~15u);
      for (int ch = wave; ch < cdiv(tot, 256); ch += 4)
        dma16<true>(rhist, hs + 256 * ch, (uint32_t)(1024 * ch + 16 * lane));
      wait_mem();
    }
    __syncthreads();
    // P threads per expert sum about n_ne / P chunks each (all rows, and the
    // rows of chunks before r), then the P partial sums are added
    int P = m.E >= kThreads ? 1 : kThreads / m.E;
    P = min(P, cdiv(n_ne, 4));
    const int span = cdiv(n_ne, P);
    for (int q = tid; q < m.E * P; q += kThreads) {
      const int e = q / P, p = q % P;
      int a_all = 0, a_bef = 0;
#pragma unroll 8
      for (int rr = p * span; rr < min(n_ne, (p + 1) * span); ++rr) {
        const int v = hs[rr * m.E + e];
        a_all += v;
        a_bef += rr < r ? v : 0;
      }
      if (P == 1) {
        cnt[e] = a_all;
        bef[e] = a_bef;
      } else {
        part[q] = a_all;
        partb[q] = a_bef;
      }
    }
    __syncthreads();
    if (P > 1)
      for (int e = tid; e < m.E; e += kThreads) {
        int a_all = 0, a_bef = 0;
        for (int p = 0; p < P; ++p) {
          a_all += part[e * P + p];
          a_bef += partb[e * P + p];
        }
        cnt[e] = a_all;
        bef[e] = a_bef;
      }
    __syncthreads();
    // Chunk 0 publishes the scan results (counts, the CSR offsets and the
    // task totals) and then fires EV_SCAN; the other chunks keep them in LDS
    // (dynamic, few chunks: every chunk publishes them).  When all 64 chunks
    // stored the same values, their stores to the same lines queued behind
    // each other and chunk 0 spent 6.5 us completing its own (moe_skewed
    // T=1024).
    const bool pub = r == 0 || (sched == ET_SCHED_DYNAMIC && !many_chunks);
    for (int e = tid; e < m.E; e += kThreads) {
      blk[e] = cdiv(cnt[e], rows);
      if (pub) st_coh(&m.counts[e], cnt[e]);
    }
    lds_barrier();
    block_exscan(cnt, m.E, tmp);           // cnt -> tok_indptr
    const int nb = block_exscan(blk, m.E, tmp);
    for (int e = tid; e < m.E; e += kThreads) {
      if (pub) {
        st_coh(&m.tok_indptr[e], cnt[e]);
        st_coh(&m.blk_indptr[e], blk[e]);
        st_coh(&m.task_indptr[e], blk[e] * nt1);
      }
      s_i[e] = s_i[1024 + e] = cnt[e] + bef[e];   // hs is no longer read
    }
    if (m.qall) {
      // Dynamic queue order: the static order, unless one expert is chosen
      // by at least 90% of the tokens and holds at least 4 row blocks --
      // then the many down tasks waiting on that expert's blocks would each
      // hold a worker still while ready tasks sit behind them in the shard,
      // and tasks pushed as they become ready do better (moe_skewed, every
      // token routed to one expert: T = 256 / 1024 135 / 220 us against
      // 147 / 223 us in static order; the static order wins at every other
      // size measured, by 2-10%: moe_small, moe_skewed_cal, moe_large).
      int mr = 0;
      for (int e = tid; e < m.E; e += kThreads)
        if ((e + 1 < m.E ? blk[e + 1] : nb) - blk[e] >= 4)
          mr = max(mr, (e + 1 < m.E ? cnt[e + 1] : m.T * m.k) - cnt[e]);
      mr = (int)wave_reduce_u32<true>((uint32_t)mr);
      if (lane == 0) tmp[wave] = mr;
      lds_barrier();
      mr = max(max(tmp[0], tmp[1]), max(tmp[2], tmp[3]));
      qs = m.qforce || 10 * mr < 9 * m.T;
    }
    if (pub && tid == 0) {
      st_coh(&m.tok_indptr[m.E], m.T * m.k);
      st_coh(&m.blk_indptr[m.E], nb);
      st_coh(&m.task_indptr[m.E], nb * nt1);
      st_rlx(&ra.hdr[HDR_META + MD_NB], nb);
      st_rlx(&ra.hdr[HDR_META + MD_TOTAL1], nb * nt1);
      st_rlx(&ra.hdr[HDR_META + MD_TOTAL2], nb * nt2);
      st_rlx(&ra.hdr[HDR_META + MD_QSTATIC], qs ? 1 : 0);
    }
    lds_barrier();
    return nb;
  };

  // ------------------------------------------------------------- gemm tiles
  auto block_rows = [&](int gb, int e, int& pos0, int& pend) ET_INLINE {
    pos0 = c_tok[e] + (gb - c_blk[e]) * rows;
    pend = min(pos0 + rows, c_tok[e + 1]);
  };

  auto gemm1 = [&](int t1g, int task) ET_INLINE -> bool {
    load_cache();
    int e, n, gb, pos0, pend;
    decode(t1g, nt1, e, n, gb);
    block_rows(gb, e, pos0, pend);
    const size_t wofs = (size_t)e * m.I * m.H;
    const uint32_t wbytes = (uint32_t)m.I * m.H * 2;
    const Rsrc rgate = make_rsrc(m.wg + wofs, wbytes), rup = make_rsrc(m.wu + wofs, wbytes);
    const int cw = kWide ? 16 * Cfg::NH * wave : 0;      // this wave's first h column
    // B rows (output columns) of this wave's groups: gate groups 0..NH-1,
    // then the up groups for the same h columns.  The stream tile takes each
    // lane's own row; the ring tile takes the first row of each group.
    const int lrow = kWide ? 0 : (lane & 15);
    Rsrc rb[2 * Cfg::NH];
    uint32_t bo[2 * Cfg::NH];
#pragma unroll
    for (int j = 0; j < Cfg::NH; ++j) {
      const uint32_t off = (uint32_t)(n * bn1 + cw + 16 * j + lrow) * (uint32_t)(m.H * 2);
      rb[j] = rgate;
      rb[Cfg::NH + j] = rup;
      bo[j] = off;
      bo[Cfg::NH + j] = off;
    }
    const Rsrc rx = make_rsrc(m.x, (uint32_t)m.T * m.H * 2);
    auto gate = [&](int round) ET_INLINE -> bool {
      if (round != 0) return true;
      if ((sched == ET_SCHED_STATIC || sched == ET_SCHED_BARRIER) && !seen_group) {
        if (!wg_wait_bcast(c, EV_GROUP, EV_GROUP, task)) return false;
        seen_group = true;
      } else if (sched == ET_SCHED_DYNAMIC &&
                 !wg_wait(c, m.ev_exp + e, c_tok[e + 1] - c_tok[e], task)) {
        return false;   // early-pushed: the expert's rows must be grouped
      }
      for (int i = tid; i < rows; i += kThreads) {
        const int pos = pos0 + i;
        rows_off[i] = pos < pend ? (uint32_t)(ld_coh(&m.perm[pos]) / m.k) * (uint32_t)(m.H * 2) : kOOB;
      }
      __syncthreads();
      return true;
    };
    Tile1 tile;
    bool ok;
    if constexpr (kWide)
      ok = tile.run(rx, rows_off, rb, bo, (uint32_t)(m.H * 2), m.H, gate, s0, s1, s2,
                    cdiv(pend - pos0, 16));
    else
      ok = tile.run(rx, rows_off, rb, bo, m.H / kKBlock, gate, reinterpret_cast<float*>(s0));
    if (!ok) return false;
    if constexpr (kWide) {
      // h = SiLU(g) * u staged as a bf16 tile in the (now idle) ring slot,
      // then written out with 16-byte coherent stores, 16 per 128-column row
      constexpr int kHs = bn1 + 8;                 // padded row (elements)
      uint16_t* hl = reinterpret_cast<uint16_t*>(s0);
      const int nrow = pend - pos0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (16 * mt < nrow) {
#pragma unroll
          for (int j = 0; j < Cfg::NH; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float g = tile.acc[mt][j][r], u = tile.acc[mt][Cfg::NH + j][r];
              hl[(16 * mt + 4 * (lane >> 4) + r) * kHs + cw + 16 * j + (lane & 15)] =
                  f32_to_bf16(silu(g) * u);
            }
        }
      lds_barrier();
      const Rsrc rh = make_rsrc(m.h, (uint32_t)m.T * m.k * m.I * 2);
      constexpr int kCpr = bn1 / 8;                // 16-byte chunks per row
      for (int i = tid; i < nrow * kCpr; i += kThreads) {
        const int row = i / kCpr, ch = i % kCpr;
        st16c(rh, (uint32_t)((pos0 + row) * m.I + n * bn1 + 8 * ch) * 2u,
              *reinterpret_cast<const i32x4*>(hl + row * kHs + 8 * ch));
      }
      lds_barrier();     // the ring slot is refilled by the next task; the stores stay in flight
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < Cfg::NH; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r == wave) {
              const int pos = pos0 + 16 * mt + 4 * (lane >> 4) + r;
              if (pos < pend) {
                const float g = tile.acc[mt][j][r], u = tile.acc[mt][Cfg::NH + j][r];
                st_coh(&m.h[(size_t)pos * m.I + n * bn1 + cw + 16 * j + (lane & 15)],
                       f32_to_bf16(silu(g) * u));
              }
            }
    }
    if (sched == ET_SCHED_PER_OP) return true;
    wg_release();
    if (sched == ET_SCHED_BARRIER) {
      t0_notify_bcast(c, EV_G1ALL, EV_G1ALL, 1, meta(MD_TOTAL1), task);
    } else if (sched == ET_SCHED_STATIC || qs) {
      t0_notify(c, m.ev_h + gb, 1, nt1, task);
    } else {
      // dynamic: the expert's event counts its gate/up tiles over all of its
      // blocks (a data-dependent wait count); the notify that completes it
      // pushes all of the expert's down tasks, in (column tile, block) order,
      // so the blocks sharing a weight tile are claimed together from one
      // shard and stream that tile through the XCD's L2 once.  (Pushing the
      // down tasks early instead, behind every gate/up task, was slower:
      // 257 us against 204 on moe_skewed T=1024 -- an early-pushed task takes
      // its queue slot in a fixed order and its worker waits for its block,
      // while tasks pushed on completion enter the queue ready to run.)
      const int nblk = c_blk[e + 1] - c_blk[e];
      if (wg_notify(c, m.ev_he + e, 1, nblk * nt1, task)) {
        // block-major push order: a shard holds (block 0: its tiles), (block 1:
        // its tiles), ..., so a batched claim mixes tiles of one block and the
        // claims taken beside it stream the same tiles for the next blocks
        const int b2 = base1 + meta(MD_TOTAL1) + c_blk[e] * nt2;
        wg_push(c, nblk * nt2, [&](int i) { return b2 + (i % nt2) * nblk + i / nt2; },
                [&](int i) { return tile_key(e, i % nt2, nt2); });
      }
    }
    return true;
  };

  auto gemm2 = [&](int t2g, int task, int total2) ET_INLINE -> bool {
    const bool cgrp = comb_groups(total2);
    load_cache();
    int e, n2, gb, pos0, pend;
    decode(t2g, nt2, e, n2, gb);
    block_rows(gb, e, pos0, pend);
    const Rsrc rdown = make_rsrc(m.wd + (size_t)e * m.H * m.I, (uint32_t)m.H * m.I * 2);
    const int cw = kWide ? 16 * Cfg::NB2 * wave : 0;     // this wave's first output column
    const int lrow = kWide ? 0 : (lane & 15);
    Rsrc rb[Cfg::NB2];
    uint32_t bo[Cfg::NB2];
#pragma unroll
    for (int j = 0; j < Cfg::NB2; ++j) {
      rb[j] = rdown;
      bo[j] = (uint32_t)(n2 * bn2 + cw + 16 * j + lrow) * (uint32_t)(m.I * 2);
    }
    const Rsrc rh = make_rsrc(m.h, (uint32_t)m.T * m.k * m.I * 2);
    auto gate = [&](int round) ET_INLINE -> bool {
      if (round != 0) return true;
      if (sched == ET_SCHED_STATIC || qs) {
        if (!wg_wait(c, m.ev_h + gb, nt1, task)) return false;
      } else if (sched == ET_SCHED_BARRIER && !seen_g1) {
        if (!wg_wait_bcast(c, EV_G1ALL, EV_G1ALL, task)) return false;
        seen_g1 = true;
      }
      for (int i = tid; i < rows; i += kThreads) {
        const int pos = pos0 + i;
        rows_off[i] = pos < pend ? (uint32_t)pos * (uint32_t)(m.I * 2) : kOOB;
      }
      __syncthreads();
      return true;
    };
    Tile2 tile;
    bool ok;
    if constexpr (kWide)
      ok = tile.run(rh, rows_off, rb, bo, (uint32_t)(m.I * 2), m.I, gate, s0, s1, s2,
                    cdiv(pend - pos0, 16));
    else
      ok = tile.run(rh, rows_off, rb, bo, m.I / kKBlock, gate, reinterpret_cast<float*>(s0));
    if (!ok) return false;
    // The combine-group notifies need each row's token: the block's perm
    // entries are copied into LDS now (wave 0, 16 bytes per lane, no
    // registers) and arrive while the y rows are staged and stored.  Slot s2
    // is idle after the ring tile; the stream tiles leave s1 unused.
    int* grp = reinterpret_cast<int*>(kWide ? s2 : s1);   // [rows]
    if (cgrp && wave == 0) {
      const Rsrc rperm = make_rsrc(m.perm, (uint32_t)m.T * m.k * 4u);
      dma16<true>(rperm, grp, 4 * lane < pend - pos0 ? (uint32_t)(pos0 + 4 * lane) * 4u : kOOB);
    }
    if constexpr (kWide) {
      // y staged as bf16 in the (now idle) ring slots -- rows 0..63 in s0,
      // 64..127 in s1, one pass -- then written out with 16-byte coherent
      // stores, 32 per 256-column row
      constexpr int kYs = bn2 + 8;                 // padded row (elements)
      static_assert(64 * kYs * 2 <= kSlot, "64 staged rows per ring slot");
      const int nrow = pend - pos0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (16 * mt < nrow) {
          uint16_t* yl = reinterpret_cast<uint16_t*>(mt < 4 ? s0 : s1);
#pragma unroll
          for (int j = 0; j < Cfg::NB2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              yl[(16 * (mt % 4) + 4 * (lane >> 4) + r) * kYs + cw + 16 * j + (lane & 15)] =
                  f32_to_bf16(tile.acc[mt][j][r]);
        }
      lds_barrier();
      constexpr int kCpr = bn2 / 8;                // 16-byte chunks (8 bf16) per row
      for (int i = tid; i < nrow * kCpr; i += kThreads) {
        const int row = i / kCpr, ch = i % kCpr;
        const uint16_t* yl = reinterpret_cast<const uint16_t*>(row < 64 ? s0 : s1);
        st16c(ry, (uint32_t)((pos0 + row) * m.H + n2 * bn2 + 8 * ch) * 2u,
              *reinterpret_cast<const i32x4*>(yl + (row % 64) * kYs + 8 * ch));
      }
      lds_barrier();     // the ring slots are refilled by the next task; the stores stay in flight
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < Cfg::NB2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r == wave) {
              const int pos = pos0 + 16 * mt + 4 * (lane >> 4) + r;
              if (pos < pend)
                st_coh(&m.y[(size_t)pos * m.H + n2 * bn2 + cw + 16 * j + (lane & 15)],
                       f32_to_bf16(tile.acc[mt][j][r]));
            }
    }
    if (sched == ET_SCHED_PER_OP) return true;
    wg_release();   // also completes wave 0's perm copy
    if (!cgrp && !inline_comb) {
      if (sched != ET_SCHED_DYNAMIC) {
        t0_notify_bcast(c, EV_DOWN, EV_DOWN, 1, total2, task);
      } else if (wg_notify(c, EV_DOWN, 1, total2, task)) {
        // the last down tile: push the combine tiles (the chain: then the
        // dense MLP's gate/up and down tiles, keyed by weight tile; each shard
        // holds them in this order, so a claimed MLP tile waits only on tiles
        // claimed before it)
        const int b3 = base1 + meta(MD_TOTAL1) + total2;
        wg_push(c, ncomb + (kBlock ? n_mg + n_md : 0), [&](int i) { return b3 + i; },
                [&](int i) {
                  return i < ncomb ? i : i < ncomb + n_mg ? (i - ncomb) % ngt_m
                                                          : (i - ncomb - n_mg) % ndt_m;
                });
      }
      return true;
    }
    if (cgrp) {
      // Data-dependent notify targets: the block's rows are in token order,
      // so the tokens of each combine group form one run of rows; the first
      // row of a run decrements E_cg[group, c] by the run's length for each
      // combine column tile c this tile's columns overlap.
      const int nrow = pend - pos0;
      const int g = tid < nrow ? grp[tid] / m.k / kCombTok : -1;
      if (tid < nrow && (tid == 0 || grp[tid - 1] / m.k / kCombTok != g)) {
        int len = 1;
        while (tid + len < nrow && grp[tid + len] / m.k / kCombTok == g) ++len;
        const int ncol = cdiv(m.H, m.ccols);
        const int cc1 = min(ncol - 1, ((n2 + 1) * bn2 - 1) / m.ccols);
        for (int cc = n2 * bn2 / m.ccols; cc <= cc1; ++cc)
          __hip_atomic_fetch_add(c.ev + m.ev_c + g * ncol + cc, -len, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
      return true;
    }
    if constexpr (TV != TV_M16) return true;   // inline combine: 16-row stream tiles only
    // one notify per row on EV_C[token, n2] (wait count k); the notify that
    // completes a token's k rows for this column tile runs its combine
    if (tid == 0) sh.v[5] = 0;
    __syncthreads();
    if (tid < rows) {
      const int pos = pos0 + tid;
      if (pos < pend) {
        const int t = ld_coh(&m.perm[pos]) / m.k;
        const int idx = m.ev_c + t * nt2 + n2;
        const int old = add_rlx(c.ev + idx, -1);
        if (old - 1 == -wc) fired[atomicAdd(&sh.v[5], 1)] = t;
        else if (old - 1 < -wc) raise_fault(ra, ET_ESTATE, task, idx, old - 1);
      }
    }
    __syncthreads();
    const int nf = sh.v[5];
    if (nf > 0)
      combine(nf, [&](int i) { return fired[i]; }, n2 * bn2, bn2,
              reinterpret_cast<float*>(s0), reinterpret_cast<int*>(s0) + kMaxTopK * 128);
    return true;
  };

  auto combine_tile = [&](int t3, int task, int total2) ET_INLINE -> bool {
    const int ncol = cdiv(m.H, m.ccols);
    const int tc = t3 / ncol, cc = t3 % ncol;
    if (comb_groups(total2)) {
      if (!wg_wait(c, m.ev_c + t3, comb_wait(tc, cc), task)) return false;
    } else if ((sched == ET_SCHED_STATIC || sched == ET_SCHED_BARRIER) && !seen_down) {
      if (!wg_wait_bcast(c, EV_DOWN, EV_DOWN, task)) return false;
      seen_down = true;
    }
    const int t0 = tc * kCombTok;
    const int ntok = min(m.T, t0 + kCombTok) - t0;
    const int c0 = cc * m.ccols;
    combine(ntok, [&](int i) { return t0 + i; }, c0, min(m.ccols, m.H - c0),
            reinterpret_cast<float*>(s0), reinterpret_cast<int*>(s0) + kMaxTopK * 128);
    if constexpr (kBlock) {
      // the dense MLP's row block holding these tokens may start once all
      // of its combine tiles are out (E_z, one notify per tile)
      if (sched == ET_SCHED_PER_OP) return true;
      wg_release();
      if (sched == ET_SCHED_BARRIER)
        t0_notify_bcast(c, EV_COMB, EV_COMB, 1, ncomb, task);
      else
        t0_notify(c, m.ev_z + t0 / rows_m, 1, z_wait(t0 / rows_m), task);
    }
    return true;
  };

  // ------------------------------------------------------------- dense MLP
  // The chain's last stage (kBlock): y2 = (SiLU(z Wg) * (z Wu)) Wd on the
  // bf16 MoE output z, as the dense MLP workload computes it.  Gate/up tile
  // (b, n): 16 h columns of row block b, after E_z[b] (weights streamed
  // before the wait); it notifies E_hm[b][n / 8].  Down tile (b, n2): 16
  // output columns over K = Im, each round of K-blocks after its h tiles.
  bool seen_comb = false, seen_mg = false;
  auto mlp_rows = [&](int b, int row_bytes) ET_INLINE {
    for (int i = tid; i < rows_m; i += kThreads) {
      const int r = b * rows_m + i;
      rows_off[i] = r < m.T ? (uint32_t)r * (uint32_t)row_bytes : kOOB;
    }
    __syncthreads();
  };
  auto mlp_gate = [&](int t, int task) ET_INLINE -> bool {
    const int b = t / ngt_m, n = t % ngt_m;
    const uint32_t wbytes = (uint32_t)m.Im * m.H * 2;
    const Rsrc rb[2] = {make_rsrc(m.mg, wbytes), make_rsrc(m.mu, wbytes)};
    const uint32_t boff = (uint32_t)(16 * n + (lane & 15)) * (uint32_t)(m.H * 2);
    const uint32_t bo[2] = {boff, boff};
    auto gate = [&](int round) ET_INLINE -> bool {
      if (round != 0) return true;
      if (sched == ET_SCHED_BARRIER) {
        if (!seen_comb && !wg_wait_bcast(c, EV_COMB, EV_COMB, task)) return false;
        seen_comb = true;
      } else if (sched != ET_SCHED_PER_OP && !wg_wait(c, m.ev_z + b, z_wait(b), task)) {
        return false;
      }
      mlp_rows(b, m.H * 2);
      return true;
    };
    StreamTile<MTM, 2, 4, PDM, true> tile;   // z was written in this launch
    if (!tile.run(make_rsrc(m.zb, (uint32_t)m.T * m.H * 2), rows_off, rb, bo, m.H / kKBlock, gate,
                  reinterpret_cast<float*>(s0)))
      return false;
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r == wave) {
          const int row = b * rows_m + 16 * mt + 4 * (lane >> 4) + r;
          if (row < m.T) {
            const float g = tile.acc[mt][0][r], u = tile.acc[mt][1][r];
            st_coh(&m.h2[(size_t)row * m.Im + 16 * n + (lane & 15)], f32_to_bf16(silu(g) * u));
          }
        }
    if (sched == ET_SCHED_PER_OP) return true;
    wg_release();
    if (sched == ET_SCHED_BARRIER)
      t0_notify_bcast(c, EV_MG, EV_MG, 1, n_mg, task);
    else
      t0_notify(c, m.ev_hm + b * nht_m + n / (kHTile / 16), 1, kHTile / 16, task);
    return true;
  };
  auto mlp_down = [&](int t, int task) ET_INLINE -> bool {
    const int b = t / ndt_m, n2 = t % ndt_m;
    const Rsrc rb[1] = {make_rsrc(m.md, (uint32_t)m.H * m.Im * 2)};
    const uint32_t bo[1] = {(uint32_t)(16 * n2 + (lane & 15)) * (uint32_t)(m.Im * 2)};
    const int nkb = m.Im / kKBlock;
    // h tiles known complete (as in the dense MLP kernel: a poll completes
    // only after the loads its wave issued before it, so rounds inside the
    // known-complete prefix poll nothing)
    int ready_kb = sched == ET_SCHED_PER_OP ? nkb : 0;
    auto gate = [&](int round) ET_INLINE -> bool {
      if (round == 0) mlp_rows(b, m.Im * 2);
      if (sched == ET_SCHED_BARRIER) {
        if (round == 0 && !seen_mg && !wg_wait_bcast(c, EV_MG, EV_MG, task)) return false;
        seen_mg = true;
        return true;
      }
      const int k0 = round * 4;
      const int nk = nkb - k0 < 4 ? nkb - k0 : 4;
      if (k0 + nk <= ready_kb) return true;
      ready_kb = k0 + wg_probe_prefix(c, m.ev_hm + b * nht_m + k0, nht_m - k0, kHTile / 16);
      if (k0 + nk <= ready_kb) return true;
      if (!wg_wait_range(c, m.ev_hm + b * nht_m + k0, nk, kHTile / 16, task)) return false;
      ready_kb = k0 + nk;
      return true;
    };
    StreamTile<MTM, 1, 4, PDM, true> tile;   // h2 was written in this launch
    if (!tile.run(make_rsrc(m.h2, (uint32_t)m.T * m.Im * 2), rows_off, rb, bo, nkb, gate,
                  reinterpret_cast<float*>(s0)))
      return false;
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r == wave) {
          const int row = b * rows_m + 16 * mt + 4 * (lane >> 4) + r;
          if (row < m.T) m.y2[(size_t)row * m.H + 16 * n2 + (lane & 15)] = tile.acc[mt][0][r];
        }
    return true;
  };

  // ------------------------------------------------------------- dispatch
  auto run = [&](int task) ET_INLINE -> bool {
    if (task < NR) {
      route(task);
      if (sched == ET_SCHED_PER_OP) return true;
      if (sched == ET_SCHED_BARRIER) {
        wg_release();
        t0_notify_bcast(c, EV_ROUTE, EV_ROUTE, 1, NR, task);
        return true;
      }
      // static / dynamic: once every chunk's histogram is out, this
      // workgroup scans and groups its own chunk
      if (!solo_route) {
        wg_release();
        if (many_chunks) {
          t0_notify_bcast(c, EV_ROUTE, EV_ROUTE, 1, NR, task);
          if (!wg_wait_bcast(c, EV_ROUTE, EV_ROUTE, task)) return false;
        } else {
          t0_notify(c, EV_ROUTE, 1, NR, task);
          if (!wg_wait(c, EV_ROUTE, NR, task)) return false;
        }
      } else {
        t0_notify(c, EV_ROUTE, 1, NR, task);
      }
      long long ts = trace_now(c);
      const int nb = scan_chunk(task);
      if (task == 0) {
        count_run(c, NR);
        trace_task(c, NR, ts);
        // static: task totals are out, gemm tasks may start and prefetch
        // weights; dynamic: pushes of gemm tasks may go out
        if (sched == ET_SCHED_STATIC || many_chunks) {
          wg_release();
          t0_notify_bcast(c, EV_SCAN, EV_SCAN, 1, 1, NR);
        }
        if (sched == ET_SCHED_DYNAMIC && m.qall) {
          // Static-order queue: the GEMM tasks base1 + p, p < nb (nt1 + nt2)
          // (every gate/up task, then every down task), become implicit
          // entries of the shards, each position in the shard of the XCD the
          // static schedule runs it on, in order -- a shard's consecutive
          // entries are the row blocks sharing one weight tile.  Publishing
          // their count is the push.  Every gate/up task precedes every down
          // task in each shard and a down task waits only on gate/up tasks,
          // so a worker waiting on a claimed down task holds back no task it
          // waits for.  Gate/up tasks still wait on their expert's E_exp.
          // (Ready order chosen: the count is 0 and the queue holds pushed
          // tasks only.)
          if (!many_chunks) wg_release();
          set_total(c, nb * (nt1 + nt2) + ncomb + (kBlock ? n_mg + n_md : 0));
          if (tid == 0) st_rlx(&c.a.hdr[HDR_QIMPL], qs ? nb * (nt1 + nt2) : 0);
        }
      }
      if (sched == ET_SCHED_DYNAMIC) {
        // Early push (the appendix of the dynamic schedule: consumers are
        // queued before their producers finish and wait on their event
        // before they run): once the scan knows every expert's row blocks,
        // the routing chunks together push all gate/up tasks, chunk r an
        // equal share of them, before any chunk has grouped its tokens.  A
        // gate/up task streams its weights and then waits on its expert's
        // E_exp event, so the weight stream overlaps the grouping.  The
        // pushed tasks read the offsets and totals chunk 0 publishes before
        // EV_SCAN (few chunks: this chunk published them itself).
        // Up to kSoloPush tasks per workgroup, chunk 0 pushes them all and the
        // other chunks go straight to their grouping: a chunk that pushes
        // first waits for EV_SCAN, and with a few tasks each that wait and the
        // push itself put 10 us on the front (moe_skewed T=1024: the front
        // ended at 28.9 us against the static schedule's 19.1 us).
        if (task == 0) set_total(c, nb * (nt1 + nt2) + ncomb + (kBlock ? n_mg + n_md : 0));
        const int total1 = nb * nt1;
        const bool solo_push = total1 <= kSoloPush * c.G;
        if (!qs && (!solo_push || task == 0)) {
          wg_release();
          if (task != 0 && many_chunks && !wg_wait_bcast(c, EV_SCAN, EV_SCAN, task)) return false;
          const int* blk = reinterpret_cast<const int*>(s1) + 1024;   // exclusive block offsets
          const int j0 = solo_push ? 0 : (int)((long long)task * total1 / NR);
          const int j1 = solo_push ? total1 : (int)((long long)(task + 1) * total1 / NR);
          // gate/up task j of the push order (experts ascending, block-major
          // within an expert) -> expert holding it: the largest e whose first
          // task is <= j (experts without rows share their successor's start)
          auto expert_of = [&](int j) ET_INLINE {
            int lo = 0, hi = m.E;
            while (hi - lo > 1) {
              const int mid = (lo + hi) >> 1;
              if (blk[mid] * nt1 <= j) lo = mid; else hi = mid;
            }
            return lo;
          };
          auto nblk_of = [&](int e) ET_INLINE { return (e + 1 < m.E ? blk[e + 1] : nb) - blk[e]; };
          wg_push(c, j1 - j0,
                  [&](int i) {
                    const int j = j0 + i, e = expert_of(j), l = j - blk[e] * nt1;
                    return base1 + blk[e] * nt1 + (l % nt1) * nblk_of(e) + l / nt1;
                  },
                  [&](int i) {
                    const int j = j0 + i, e = expert_of(j);
                    return tile_key(e, (j - blk[e] * nt1) % nt1, nt1);
                  });
        }
      }
      ts = trace_now(c);
      group_chunk(task);
      count_run(c, NR + 1 + task);
      trace_task(c, NR + 1 + task, ts);
      wg_release();
      if (sched == ET_SCHED_STATIC) {
        t0_notify_bcast(c, EV_GROUP, EV_GROUP, 1, NR, task);
        return true;
      }
      // dynamic: data-dependent notify targets -- the experts this chunk's
      // tokens chose, each decremented by this chunk's rows for it (wait
      // count: the rows routed to the expert); their gate/up tasks wait on it
      const int* cur = s_i;
      const int* base = s_i + 1024;
      const int* tokp = reinterpret_cast<const int*>(s1);
      for (int e = tid; e < m.E; e += kThreads) {
        const int n = cur[e] - base[e];
        if (n > 0) {
          const int wcnt = (e + 1 < m.E ? tokp[e + 1] : m.T * m.k) - tokp[e];
          const int old = add_rlx(c.ev + m.ev_exp + e, -n);
          if (old - n < -wcnt) raise_fault(ra, ET_ESTATE, task, m.ev_exp + e, old - n);
        }
      }
      return true;
    }
    if (task == NR) {   // the scan as a task of its own: barrier and per-op modes
      if (sched == ET_SCHED_BARRIER && !wg_wait_bcast(c, EV_ROUTE, EV_ROUTE, task)) return false;
      scan();
      if (sched == ET_SCHED_PER_OP) return true;
      wg_release();
      t0_notify_bcast(c, EV_SCAN, EV_SCAN, 1, 1, task);
      return true;
    }
    if (task < base1) {   // grouping tasks: barrier and per-op modes
      const int r = task - NR - 1;
      if (sched == ET_SCHED_BARRIER && !wg_wait_bcast(c, EV_SCAN, EV_SCAN, task)) return false;
      group(r);
      if (sched == ET_SCHED_PER_OP) return true;
      wg_release();
      t0_notify_bcast(c, EV_GROUP, EV_GROUP, 1, NR, task);
      return true;
    }
    const int total1 = meta(MD_TOTAL1), total2 = meta(MD_TOTAL2);
    if (task < base1 + total1) return gemm1(task - base1, task);
    if (task < base1 + total1 + total2) return gemm2(task - base1 - total1, task, total2);
    const int tc = task - base1 - total1 - total2;
    if constexpr (kBlock) {
      if (tc >= ncomb) return tc - ncomb < n_mg ? mlp_gate(tc - ncomb, task)
                                                : mlp_down(tc - ncomb - n_mg, task);
    }
    return combine_tile(tc, task, total2);
  };

  if (sched == ET_SCHED_DYNAMIC) {
    // routing chunk r runs on workgroup r, as under the static schedule:
    // claiming the chunks from the queue put a contended atomic (every
    // workgroup of a shard on one claim counter) before the front; the
    // gemm and combine tasks come from the queue
    bool ok = true;
    for (int r = c.wg; ok && r < ra.init_base; r += c.G) {
      const long long t0 = trace_now(c);
      ok = run(r);
      if (ok) count_run(c, r);
      if (ok) trace_task(c, r, t0);
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
    const int ph = ra.phase;
    int lo = 0, hi = 0;
    if (ph == 0) { lo = 0; hi = NR; }
    else if (ph == 1) { lo = NR; hi = NR + 1; }
    else if (ph == 2) { lo = NR + 1; hi = base1; }
    else {
      const int total1 = meta(MD_TOTAL1), total2 = meta(MD_TOTAL2);
      if (ph == 3) { lo = base1; hi = base1 + total1; }
      else if (ph == 4) { lo = base1 + total1; hi = lo + total2; }
      else if (ph == 5) { lo = base1 + total1 + total2; hi = lo + ncomb; }
      else if (ph == 6) { lo = base1 + total1 + total2 + ncomb; hi = lo + n_mg; }   // the chain
      else { lo = base1 + total1 + total2 + ncomb + n_mg; hi = lo + n_md; }
    }
    for (int t = lo + (ph >= 3 ? xcd_pos(c.wg, c.G) : c.wg); t < hi; t += c.G) {
      const long long t0 = trace_now(c);
      run(t);
      count_run(c, t);
      trace_task(c, t, t0);
    }
  } else {
    bool ok = true;
    for (int t = c.wg; ok && t < NR; t += c.G) {
      const long long t0 = trace_now(c);
      ok = run(t);
      if (ok) count_run(c, t);
      if (ok) trace_task(c, t, t0);
    }
    if (ok && sched == ET_SCHED_BARRIER && c.wg == c.G - 1) {
      const long long t0 = trace_now(c);
      ok = run(NR);
      if (ok) count_run(c, NR);
      if (ok) trace_task(c, NR, t0);
    }
    for (int r = c.wg; ok && sched == ET_SCHED_BARRIER && r < NR; r += c.G) {
      const long long t0 = trace_now(c);
      ok = run(NR + 1 + r);
      if (ok) count_run(c, NR + 1 + r);
      if (ok) trace_task(c, NR + 1 + r, t0);
    }
    if (ok) ok = wg_wait_bcast(c, EV_SCAN, EV_SCAN, -1);
    if (ok) {
      // the task totals and the index tables of the first gemm task are
      // requested in one memory round trip
      const int total1 = meta(MD_TOTAL1), total2 = meta(MD_TOTAL2);
      load_cache();
      const int end = base1 + total1 + total2 + ncomb + (kBlock ? n_mg + n_md : 0);
      for (int t = base1 + xcd_pos(c.wg, c.G); ok && t < end; t += c.G) {
        const long long t0 = trace_now(c);
        ok = run(t);
        if (ok) count_run(c, t);
        if (ok) trace_task(c, t, t0);
      }
    }
  }
  epilogue(c, 0);
}

// ---------------------------------------------------------------------------
// host side, shared by the MoE entry point and the chain's
// ---------------------------------------------------------------------------

// Tile variant, workspace pointers, per-call dimensions and run arguments of
// a call with T tokens (the caller fills the input and output pointers).
inline int moe_setup(const LaunchCommon& lc, const MoePlan& mp, const MoeAux& ax, char* aux, int T,
                     MoeArgs& m, RunArgs& ra, int& tv) {
  tv = pick_moe_tile(T, mp.top_k, mp.hidden, mp.inter, lc.tile);
  if (!moe_tile_fits(tv, mp.hidden, mp.inter)) return ET_EUNSUPPORTED;
  const Tiling tl = tiling_of(tv);
  m.topk_ids = reinterpret_cast<int*>(aux + ax.topk_ids);
  m.topk_w = reinterpret_cast<float*>(aux + ax.topk_w);
  m.hist = reinterpret_cast<int*>(aux + ax.hist);
  m.counts = reinterpret_cast<int*>(aux + ax.counts);
  m.tok_indptr = reinterpret_cast<int*>(aux + ax.tok_indptr);
  m.blk_indptr = reinterpret_cast<int*>(aux + ax.blk_indptr);
  m.task_indptr = reinterpret_cast<int*>(aux + ax.task_indptr);
  m.perm = reinterpret_cast<int*>(aux + ax.perm);
  m.inv = reinterpret_cast<int*>(aux + ax.inv);
  m.h = reinterpret_cast<uint16_t*>(aux + ax.h);
  m.y = reinterpret_cast<uint16_t*>(aux + ax.y);
  m.T = T;
  m.H = mp.hidden;
  m.I = mp.inter;
  m.E = mp.n_experts;
  m.k = mp.top_k;
  m.NR = mp.routes(T);
  m.tpr = mp.tpr(T);
  // combine tiles: 16 tokens x 256 columns, or x 64 columns when that leaves
  // workgroups without a tile
  m.ccols = cdiv(T, kCombTok) * cdiv(m.H, kCombColsWide) >= 4 * lc.G ? kCombColsWide
            : cdiv(T, kCombTok) * cdiv(m.H, kCombCols) >= lc.G       ? kCombCols
                                                                       : kCombColsMin;
  m.ev_exp = mp.ev_exp();
  m.ev_he = mp.ev_he();
  m.ev_h = mp.ev_h();
  m.ev_c = mp.ev_c();
  // dynamic schedule: the static-order queue may be chosen by the scan
  // (queue order auto) or is forced (static); implicit entries from the first
  // gate/up task on
  m.qall = lc.sched == ET_SCHED_DYNAMIC && lc.qorder != ET_QORDER_READY;
  m.qforce = lc.sched == ET_SCHED_DYNAMIC && lc.qorder == ET_QORDER_STATIC;
  ra = lc.run_args();
  ra.init_base = m.NR;   // dynamic: routing runs on workgroups 0..NR-1
  ra.n_init = 0;         // the queue holds pushed tasks only
  ra.n_single = 0;
  if (m.qall) ra.impl_base = 2 * m.NR + 1;   // the first gate/up task
  ra.total_hint = kUnknownTotal;
  ra.extent = mp.extent(T, tl);
  return ET_OK;
}

// One persistent launch, or one launch per operator phase (per-op baseline).
inline int moe_launch(const LaunchCommon& lc, const void* kernel, int tv, RunArgs& ra, MoeArgs& m,
                      int phases) {
  constexpr int occ[] = {MoeCfg<TV_M16>::kOcc, MoeCfg<TV_M32>::kOcc, MoeCfg<TV_M64>::kOcc,
                         MoeCfg<TV_W64>::kOcc, MoeCfg<TV_W128>::kOcc, MoeCfg<TV_M16W>::kOcc};
  static_assert(sizeof(occ) / sizeof(occ[0]) == TV_COUNT, "one occupancy per tile variant");
  LaunchCommon l = lc;
  l.G = lc.G * occ[tv];
  if (lc.sched == ET_SCHED_PER_OP) {
    for (int ph = 0; ph < phases; ++ph) {
      ra.phase = ph;
      const int e = l.launch(kernel, &ra, &m, false);
      if (e) return e;
    }
    return ET_OK;
  }
  return l.launch(kernel, &ra, &m, true);
}

}  // namespace et
