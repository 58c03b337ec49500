// et_block.hip -- the router GEMM -> MoE layer -> dense MLP chain as one
// persistent kernel: the MoE kernel of et_moe_kernel.hpp instantiated with
// the chain's extra stages (Event Tensor notes, section "端到端低 batch
// serving": the MoE GroupGEMM pipelined with the dense MLP GEMM across
// stages, the next stage's weights fetched before its activations arrive).
#include "et_moe_kernel.hpp"

namespace et {

int launch_block(const LaunchCommon& lc, const uint16_t* x, int T, const uint16_t* wr,
                 const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, const uint16_t* mg,
                 const uint16_t* mu, const uint16_t* md, float* moe_out, float* y) {
  const et_plan* p = lc.plan;
  const BlockPlan bp{MoePlan{p->max_tokens, p->hidden, p->inter, p->n_experts, p->top_k,
                             moe_n_route(p->n_experts)},
                     p->mlp_inter};
  const BlockAux ax = block_aux_layout(bp);
  char* aux = lc.ws + p->off_aux;
  MoeArgs m{};
  RunArgs ra;
  int tv = 0;
  const int e = moe_setup(lc, bp.moe, ax.moe, aux, T, m, ra, tv);
  if (e) return e;
  m.x = x;
  m.wg = wg;
  m.wu = wu;
  m.wd = wd;
  m.out = moe_out;
  m.wr = wr;
  m.logits_ws = reinterpret_cast<float*>(aux + ax.logits);
  m.zb = reinterpret_cast<uint16_t*>(aux + ax.zb);
  m.mg = mg;
  m.mu = mu;
  m.md = md;
  m.h2 = reinterpret_cast<uint16_t*>(aux + ax.h2);
  m.y2 = y;
  m.Im = p->mlp_inter;
  m.ev_z = bp.ev_z();
  m.ev_hm = bp.ev_hm();
  // the chain's events follow the MoE layer's: this call uses the bank's
  // prefix up to its dense-MLP h events
  const int mrows = (tv == TV_M16 || tv == TV_M16W) ? 16 : 64;
  ra.extent = bp.ev_hm() + cdiv(T, mrows) * (p->mlp_inter / kHTile);
  const void* const kernels[] = {
      reinterpret_cast<const void*>(&moe_kernel<TV_M16, true>),
      reinterpret_cast<const void*>(&moe_kernel<TV_M32, true>),
      reinterpret_cast<const void*>(&moe_kernel<TV_M64, true>),
      reinterpret_cast<const void*>(&moe_kernel<TV_W64, true>),
      reinterpret_cast<const void*>(&moe_kernel<TV_W128, true>),
      reinterpret_cast<const void*>(&moe_kernel<TV_M16W, true>)};
  static_assert(sizeof(kernels) / sizeof(kernels[0]) == TV_COUNT, "one kernel per tile variant");
  return moe_launch(lc, kernels[tv], tv, ra, m, 8);
}

}  // namespace et
