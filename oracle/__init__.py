"""CPU oracle for the Event Tensor hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library under ``event_driven_moe_amd/``) never imports, links or calls it, and
this package imports nothing from the product path: the two share no kernels,
headers, helpers, tables or pre/post-processing.  Inputs reach both sides from
the seeded generators in ``event_driven_moe_amd/synth.py``, which hold none of
the method's arithmetic.

Everything here is a plain, slow, obviously correct restatement of what the
method computes, in float64 (the pages fix no precision), using numpy only for
library primitives (sums, matmuls, a stable sort).  Each function cites the
passage it follows.  Citation keys:

* "Event Tensor notes" -- the page "Event Tensor：用“事件张量”编译动态
  Megakernel" (notes.kuangjux.top), the authority on what the method computes.
* "Weave MoE article" -- the page "MoE Kernel动态SM调度：从静态分配到任务池，
  4卡H100加速2.89×" (icman.com.cn), prior art for the dynamic MoE queue.

Parity status of each function is stated in its module header; functions that
have no pin are marked "parity unpinned" there.
"""

from . import splitk, mlp, moe, events, block, decode  # noqa: F401
