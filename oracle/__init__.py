"""Float64 CPU oracle for the Single-Pass mHC residual step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library, its
Python binding, or the timed part of ``bench.py``) may import, call or link this
package. It is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``. It shares no code, tables or constants
with the HIP path; the only module both sides use is the seeded input generator
``stream_hyper_connections_amd.workloads``, which holds none of the method's
arithmetic.

Pages cited (by title and section):

* "DeepSeek V4.1 · Stream weights for the feed-forward" (atlas page on the
  stream weights): the formula list "All 5 steps", the "Parameters" accounting
  table, the "Explanation" paragraph and the "Code" excerpts (the ``Block``
  constructor, ``hc_mixes`` / ``hc_pre`` / ``hc_post`` and the
  ``hc_split_sinkhorn`` kernel with its wrapper).
* "DeepSeek V4.1 · MoE RMSNorm" (atlas page on the feed-forward norm): the
  RMSNorm formula, its "Parameters" table and the "Code" excerpts (``RMSNorm``
  and ``Block.forward``).
* "2A · Single-Pass mHC" (openarchlab course page): §1 definition, §3 solution
  and §4 profiling (the hand-checked Sinkhorn example).

``mhc_backward`` derives the gradient of the step from these forward
definitions (the pages give no backward); its pins are finite differences of
the forward and automatic differentiation of an independent transcription.
"""

from .mhc_oracle import (  # noqa: F401
    N_STREAMS,
    n_mix,
    parameter_count,
    round_bf16,
    round_to,
    sigmoid,
    split_sinkhorn,
    sinkhorn_plain,
    mixes,
    hc_post,
    hc_pre,
    rmsnorm,
    fused_step,
    fused_step_from_xprime,
)
from .mhc_backward import (  # noqa: F401
    fused_step_backward,
    split_sinkhorn_backward,
)
