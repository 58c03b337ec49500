// et_moe.hip -- the MoE layer entry point: launches the persistent MoE
// kernel of et_moe_kernel.hpp (the chain of Event Tensor notes, sections
// "两类动态性如何进入依赖表示" and "完整 MoE layer").
#include "et_moe_kernel.hpp"

namespace et {

int launch_moe(const LaunchCommon& lc, const float* logits, const uint16_t* x, int T,
               const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, float* out) {
  const et_plan* p = lc.plan;
  MoePlan mp{p->max_tokens, p->hidden, p->inter, p->n_experts, p->top_k,
             moe_n_route(p->n_experts)};
  MoeArgs m{};
  RunArgs ra;
  int tv = 0;
  const int e = moe_setup(lc, mp, moe_aux_layout(mp), lc.ws + p->off_aux, T, m, ra, tv);
  if (e) return e;
  m.logits = logits;
  m.x = x;
  m.wg = wg;
  m.wu = wu;
  m.wd = wd;
  m.out = out;
  const void* const kernels[] = {
      reinterpret_cast<const void*>(&moe_kernel<TV_M16>),
      reinterpret_cast<const void*>(&moe_kernel<TV_M32>),
      reinterpret_cast<const void*>(&moe_kernel<TV_M64>),
      reinterpret_cast<const void*>(&moe_kernel<TV_W64>),
      reinterpret_cast<const void*>(&moe_kernel<TV_W128>),
      reinterpret_cast<const void*>(&moe_kernel<TV_M16W>)};
  static_assert(sizeof(kernels) / sizeof(kernels[0]) == TV_COUNT, "one kernel per tile variant");
  return moe_launch(lc, kernels[tv], tv, ra, m, 6);
}

}  // namespace et
