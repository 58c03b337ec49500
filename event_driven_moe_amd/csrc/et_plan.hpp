// et_plan.hpp -- workspace layout, task-space arithmetic and tiling constants
// shared by the host launcher and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

#define ET_HD __host__ __device__ __forceinline__
// lambdas inside the persistent kernels: inlined even when called from
// several places (an outlined task body costs a call frame in scratch)
#define ET_INLINE __attribute__((always_inline))

namespace et {

constexpr int kThreads = 256;      // every persistent workgroup: 4 waves of 64
constexpr int kMagic = 0x45545431;

// Workspace header: 256 int32 words.  Each word that several workgroups
// update sits on its own 128-byte line.
enum : int {
  HDR_MAGIC = 0,
  HDR_WORKLOAD = 1,
  HDR_BANK = 32,        // bank the next call uses
  HDR_CALLS = 33,       // completed calls
  HDR_EXT0 = 34,        // counters of bank 0 / 1 the last call on it used
  HDR_EXT1 = 35,
  HDR_LAST_TASKS = 36,  // tasks run by the last call
  HDR_ERR = 64,         // sticky fault code (0 = none)
  HDR_ERR_A = 65,
  HDR_ERR_B = 66,
  HDR_ERR_C = 67,
  HDR_QHEAD = 96,       // ready queue: implicit initial tasks claimed
  HDR_QIMPL = 128,      // ready queue: static-order implicit tasks of this call once known (else INT_MAX)
  HDR_QTOTAL = 160,     // ready queue: total tasks of this call once known (else INT_MAX)
  HDR_EXIT = 192,       // workgroups that finished this call
  HDR_META = 224,       // 32 words of per-call workload metadata
  HDR_FLAGS = 256,      // broadcast flags: [kBcastSlots][kBcastLines] lines of 32 words
  HDR_WORDS = 256 + 8 * 64 * 32
};
// Broadcast events (a coarse event with many waiters): the notify that
// completes one writes the call's generation into kBcastLines flag lines of
// its slot, and each waiter polls the line of its own workgroup.
constexpr int kBcastSlots = 8;
constexpr int kBcastLines = 64;
static_assert(HDR_WORDS == HDR_FLAGS + kBcastSlots * kBcastLines * 32, "flag region");
constexpr size_t kHdrBytes = HDR_WORDS * 4;

// Ready-queue shards (dynamic mode): control words of shard q at
// qctl[q * kQCtlStride] (claimed slots) and qctl[q * kQCtlStride + 32]
// (pushed slots), each on its own 128-byte line.
constexpr int kMaxShards = 8;
constexpr int kQCtlStride = 64;
constexpr size_t kQCtlBytes = (size_t)kMaxShards * kQCtlStride * 4;
constexpr int kUnknownTotal = 0x7fffffff;

ET_HD size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
ET_HD int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// GEMM tiling.  A tile variant fixes the rows per tile (16 * MT) and the
// columns per task of the gate/up (bn1, in h columns) and down (bn2)
// projections.  K is consumed in blocks of 128 elements.
// ---------------------------------------------------------------------------
constexpr int kKBlock = 128;
constexpr int kHTile = 128;        // MLP: one event per 128-column tile of h

struct Tiling {
  int mt;    // 16-row sub-tiles per tile
  int bn1;   // h columns per gate/up task
  int bn2;   // output columns per down task
};

// Variant ids (kernels are instantiated per variant).  The stream variants
// (16 / 32 / 64 rows, 16-column tasks) serve few rows per expert, where the
// weight stream from HBM is the bound and many narrow tasks keep every CU
// busy; the wide variants (64 / 128 rows, 128 h columns per gate/up task and
// 256 output columns per down task) serve many rows, where MFMA throughput
// and operand reuse matter.
// TV_M16W: 16 rows, 16-column gate/up tasks, 64-column down tasks (fewer,
// longer down tasks whose weight stream is mostly fetched before their h
// block is ready; used when there are enough row blocks to fill the CUs).
enum : int { TV_M16 = 0, TV_M32 = 1, TV_M64 = 2, TV_W64 = 3, TV_W128 = 4, TV_M16W = 5, TV_COUNT = 6 };

__host__ __device__ constexpr Tiling tiling_of(int tv) {
  return Tiling{(tv == TV_M16 || tv == TV_M16W) ? 1 : (tv == TV_M32 ? 2 : (tv == TV_W128 ? 8 : 4)),
                (tv == TV_W64 || tv == TV_W128) ? 128 : 16,
                (tv == TV_W64 || tv == TV_W128) ? 256 : (tv == TV_M16W ? 64 : 16)};
}
constexpr int kMinRows = 16;       // smallest rows per tile over all variants
constexpr int kMinCols = 16;       // smallest bn1 / bn2 over all variants

// ---------------------------------------------------------------------------
// Split-K example: rows = 32 n, 128 columns, 4 slices.
// events: E[0..n) (wait count 4), then one "all stage-1 done" event.
// tasks:  [0, 4n) stage-1 (i = id / 4, j = id % 4); [4n, 5n) stage-2.
// ---------------------------------------------------------------------------
struct SplitKPlan {
  int n_max;
  ET_HD int n_events() const { return n_max + 1; }
  ET_HD int max_tasks() const { return 5 * n_max; }
};

// ---------------------------------------------------------------------------
// Dense MLP chain.
// events: E_h[mb][I/128] (wait count 128 / bn1), then E_gate_all.
// tasks:  [0, n_gate) gate/up tiles (mb, n) with n fastest;
//         [n_gate, n_gate + n_down) down tiles (mb, n2).
// ---------------------------------------------------------------------------
struct MlpPlan {
  int b_max, hidden, inter;
  ET_HD int mb(int B, const Tiling& t) const { return cdiv(B, 16 * t.mt); }
  ET_HD int n_htiles() const { return inter / kHTile; }
  ET_HD int n_events_max() const { return cdiv(b_max, kMinRows) * n_htiles() + 1; }
  ET_HD int max_tasks() const {
    return cdiv(b_max, kMinRows) * (inter / kMinCols + hidden / kMinCols);
  }
};

// ---------------------------------------------------------------------------
// MoE layer.
// Routing / grouping use R = routes(T) <= n_route token chunks; chunk r
// covers tokens [r * tpr, min((r + 1) * tpr, T)) with tpr = ceil(T / R).
// events (prefix of a bank):
//   EV_ROUTE  all routing tasks done      (wait count n_route)
//   EV_SCAN   scan done                   (1)
//   EV_GROUP  all grouping tasks done     (n_route)
//   EV_G1ALL  all gate/up tasks done      (total1)        [barrier mode]
//   EV_DOWN   all down tasks done         (total2)        [without EV_CG]
//   EV_EXP[e] rows of expert e grouped    (counts[e])     data-dependent
//   EV_HE[e]  gate/up tiles of expert e   (blocks[e] * inter / bn1) data-dependent [dynamic]
//   EV_H[gb]  gate/up tiles of block gb   (inter / bn1)                    [static]
//   EV_C[t][c] down tiles covering token t, column tile c (top_k) [inline combine]
//   EV_CG[g][c] (same base as EV_C; combine tiles) rows of the kCombTok tokens
//             of group g times down column tiles overlapping combine column
//             tile c (top_k * tokens * tiles)  [static; groups >= kCombGroupMin,
//             down tiles <= kCombGroupRounds * G]
// tasks: [0, R) routing, R scan, [R+1, 2R+1) grouping, then total1 gate/up
//   tiles (block-major, column tile fastest), total2 down tiles, then the
//   combine tiles of kCombTok tokens x ccols columns (none when the combine
//   runs inline in the down tiles).
// ---------------------------------------------------------------------------
constexpr int kCombTok = 16;
constexpr int kCombCols = 256;      // combine tile columns (64 when 256 gives fewer tiles than CUs)
constexpr int kCombColsMin = 64;
constexpr int kCombColsWide = 1024; // ... and 1024 when that still gives 4 tiles per CU
constexpr int kCombGroupRounds = 4;   // static: E_cg when down tiles <= this many per workgroup
constexpr int kCombGroupMin = 16;     //   and at least this many token groups
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kHistEntries = 8192;    // n_route * E must fit (int32, 32 KB of LDS)
constexpr int kRouteTok = 8;          // tokens per routing chunk (fewer chunks when T is small)
constexpr int kBcastChunks = 16;      // routing chunks from which their events are broadcast

// EV_COMB / EV_MG: all combine tiles / all dense MLP gate/up tiles done (the
// router -> MoE -> dense MLP chain under the barrier schedule)
enum : int { EV_ROUTE = 0, EV_SCAN = 1, EV_GROUP = 2, EV_G1ALL = 3, EV_DOWN = 4, EV_COMB = 5,
             EV_MG = 6, EV_FIXED = 8 };

// per-call metadata words (HDR_META + i), written by the scan task
enum : int { MD_NB = 0, MD_TOTAL1 = 1, MD_TOTAL2 = 2, MD_QSTATIC = 3 };

struct MoePlan {
  int t_max, hidden, inter, n_experts, top_k, n_route;
  ET_HD int nb_max() const { return cdiv(t_max * top_k, kMinRows) + n_experts; }
  ET_HD int ev_exp() const { return EV_FIXED; }
  ET_HD int ev_he() const { return EV_FIXED + n_experts; }
  ET_HD int ev_h() const { return EV_FIXED + 2 * n_experts; }
  ET_HD int ev_c() const { return ev_h() + nb_max(); }
  ET_HD int n_events_max() const { return ev_c() + t_max * (hidden / kMinCols); }
  ET_HD int extent(int T, const Tiling& t) const {
    const int c = T * (hidden / t.bn2), g = cdiv(T, kCombTok) * cdiv(hidden, kCombColsMin);
    return ev_c() + (c > g ? c : g);
  }
  ET_HD int n_comb(int T) const { return cdiv(T, kCombTok) * cdiv(hidden, kCombColsMin); }
  ET_HD int max_tasks() const {
    return 2 * n_route + 1 + nb_max() * (inter / kMinCols + hidden / kMinCols) + n_comb(t_max);
  }
  // routing chunks of a call: about kRouteTok tokens each, at most n_route
  ET_HD int routes(int T) const {
    const int r = cdiv(T, kRouteTok);
    return r < 1 ? 1 : (r > n_route ? n_route : r);
  }
  ET_HD int tpr(int T) const { return cdiv(T, routes(T)); }
};

ET_HD int moe_n_route(int n_experts) {
  int r = kHistEntries / n_experts;
  return r > 128 ? 128 : (r < 1 ? 1 : r);
}

// ---------------------------------------------------------------------------
// Router GEMM -> MoE layer -> dense MLP chain: the MoE layer's events and
// tasks, then the dense MLP's.  The MLP runs on row blocks of mrows(T)
// tokens (16 while the MoE uses its 16-row variants, else 64).
// events (after the MoE layer's n_events_max()):
//   E_z[mb]      combine tiles covering the tokens of MLP row block mb
//                (16-token groups of the block x combine column tiles)
//   E_hm[mb][n]  dense MLP gate/up tiles of 128-column h tile n (8)
// tasks (after the MoE layer's, whose combine always runs as tiles): the
//   gate/up tiles (mb, n < Im/16), then the down tiles (mb, n2 < H/16).
// ---------------------------------------------------------------------------
struct BlockPlan {
  MoePlan moe;
  int mlp_inter;
  ET_HD int nmb_max() const { return cdiv(moe.t_max, kMinRows); }
  ET_HD int ev_z() const { return moe.n_events_max(); }
  ET_HD int ev_hm() const { return ev_z() + nmb_max(); }
  ET_HD int n_events_max() const { return ev_hm() + nmb_max() * (mlp_inter / kHTile); }
  ET_HD int max_tasks() const {
    return moe.max_tasks() + nmb_max() * (mlp_inter / kMinCols + moe.hidden / kMinCols);
  }
};

// Byte offsets of the MoE intermediates inside the aux region.
struct MoeAux {
  size_t topk_ids, topk_w, hist, counts, tok_indptr, blk_indptr, task_indptr, perm, inv, h, y,
      bytes;
};

inline MoeAux moe_aux_layout(const MoePlan& p) {
  MoeAux a;
  size_t o = 0;
  const size_t TK = (size_t)p.t_max * p.top_k;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes, 256); return r; };
  a.topk_ids = take(TK * 4);
  a.topk_w = take(TK * 4);
  a.hist = take((size_t)p.n_route * p.n_experts * 4);
  a.counts = take((size_t)p.n_experts * 4);
  a.tok_indptr = take((size_t)(p.n_experts + 1) * 4);
  a.blk_indptr = take((size_t)(p.n_experts + 1) * 4);
  a.task_indptr = take((size_t)(p.n_experts + 1) * 4);
  a.perm = take(TK * 4);
  a.inv = take(TK * 4);
  a.h = take(TK * p.inter * 2);
  a.y = take(TK * p.hidden * 2);   // bf16 down-projection rows
  a.bytes = o;
  return a;
}

// The chain's intermediates after the MoE layer's: router logits, the MoE
// output in bf16 (the dense MLP's input), the dense MLP's h.
struct BlockAux {
  MoeAux moe;
  size_t logits, zb, h2, bytes;
};

inline BlockAux block_aux_layout(const BlockPlan& p) {
  BlockAux a;
  a.moe = moe_aux_layout(p.moe);
  size_t o = a.moe.bytes;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes, 256); return r; };
  a.logits = take((size_t)p.moe.t_max * p.moe.n_experts * 4);
  a.zb = take((size_t)p.moe.t_max * p.moe.hidden * 2);
  a.h2 = take((size_t)p.moe.t_max * p.mlp_inter * 2);
  a.bytes = o;
  return a;
}

}  // namespace et
