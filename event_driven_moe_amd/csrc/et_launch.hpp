// et_launch.hpp -- host-side launch helpers shared by the workloads.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/et.h"
#include "et_plan.hpp"

namespace et {

struct RunArgs;

struct LaunchCommon {
  const et_plan* plan;
  char* ws;
  int sched;
  int fetch;
  int debug;
  int timeout_ms;
  int tile;
  int coop;            // persistent launches: cooperative (1) or ordinary (0)
  int shards;          // dynamic mode: ready-queue shards (1 or kMaxShards)
  int qorder;          // dynamic mode, MoE: ET_QORDER_*
  int G;               // workgroups of a persistent launch (one per CU)
  hipStream_t stream;

  RunArgs run_args() const;

  // Launches kernel(ra, args).  `persistent`: every workgroup must be
  // resident, since tasks spin on each other's events -- cooperative when the
  // caller asked for the guarantee, else an ordinary launch of one workgroup
  // per compute unit (one fits per unit).
  template <class A>
  int launch(const void* kernel, RunArgs* ra, A* args, bool persistent) const {
    void* kargs[] = {ra, args};
    hipError_t e;
    if (persistent && coop)
      e = hipLaunchCooperativeKernel(kernel, dim3(G), dim3(kThreads), kargs, 0, stream);
    else
      e = hipLaunchKernel(kernel, dim3(G), dim3(kThreads), kargs, 0, stream);
    return e == hipSuccess ? ET_OK : ET_EHIP;
  }
};

int launch_splitk(const LaunchCommon& lc, const float* A, int rows, float* B, float* C);
int launch_mlp(const LaunchCommon& lc, const uint16_t* x, int B, const uint16_t* wg,
               const uint16_t* wu, const uint16_t* wd, float* y);
int launch_moe(const LaunchCommon& lc, const float* logits, const uint16_t* x, int T,
               const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, float* out);
int launch_decode(const LaunchCommon& lc, const uint16_t* q, const uint16_t* k,
                  const uint16_t* v, const uint16_t* wq, const uint16_t* wk, const int* pos,
                  int B, float theta, float eps, uint16_t* kc, uint16_t* vc, int S, float* out);
int launch_block(const LaunchCommon& lc, const uint16_t* x, int T, const uint16_t* wr,
                 const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, const uint16_t* mg,
                 const uint16_t* mu, const uint16_t* md, float* moe_out, float* y);

// Dense MLP: rows per tile from the batch (stream variants only), unless forced.
inline int pick_mlp_tile(int batch, int forced) {
  if (forced >= 0 && forced <= TV_M64) return forced;
  if (batch <= 16) return TV_M16;
  if (batch <= 32) return TV_M32;
  return TV_M64;
}

// MoE: a token count bounds the rows any one expert receives (a token picks
// an expert at most once); few rows -> narrow stream tiles (their tasks are
// short, so the weights of a small expert spread over many CUs), many routed
// rows in total -> wide LDS-staged MFMA tiles (each weight byte feeds more
// rows).  `forced` (0 .. TV_COUNT-1) overrides.  The wide variants' down
// tasks cover 256 output columns, so they serve only hidden sizes that are a
// multiple of 256 (the rule falls back to the 64-row stream variant).
inline bool moe_tile_fits(int tv, int hidden, int inter) {
  const Tiling t = tiling_of(tv);
  return hidden % t.bn2 == 0 && inter % t.bn1 == 0;
}
inline int pick_moe_tile(int tokens, int top_k, int hidden, int inter, int forced) {
  if (forced >= 0 && forced < TV_COUNT) return forced;
  // 64-column down tasks once 16 or more (token, expert) pairs are routed
  // (typically 8+ row blocks, so 256+ such tasks); with fewer rows the
  // 16-column ones keep every CU busy
  if (tokens <= 32) return tokens * top_k >= 16 ? TV_M16W : TV_M16;
  const int wide = tokens <= 512 ? TV_W64 : TV_W128;
  if (tokens * top_k <= 256 || !moe_tile_fits(wide, hidden, inter)) return TV_M64;
  return wide;
}

}  // namespace et
