"""Plain, slow CPU oracle for MoE row movement (layout, dispatch, combine).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, the smoke check and the CPU-baseline leg of the benchmark call
it.  It shares no code with the HIP library (no kernels, headers, helpers,
tables or pre/post-processing) and never imports it.

What the oracle follows
-----------------------
The pages this work starts from are:

* "How DeepEP Utilizes TMA Instructions for Minimal SM Usage on Hopper GPUs"
  (instagit.com, DeepEP deep-dive), cited below as [DeepEP-TMA];
* the TMA study notes at mkbk-pku.cn, cited as [TMA-notes];
* "Tensor Memory Accelerator" (semiaifoundry.com atlas), cited as [TMA-atlas].

[DeepEP-TMA] section "High-Level DeepEP API Usage" shows a ``dispatch`` call
that takes hidden states, top-k expert indices, top-k weights and the number
of experts, and returns the expert-grouped output plus a handle.  The pages
never spell out what dispatch computes nor mention combine, so the oracle
fixes the plainest reading:

* ``layout``   -- per-expert counts, their exclusive prefix sum, and for every
  (token, slot) entry its row in an expert-grouped receive buffer, tokens in
  ascending order inside each expert (a stable counting sort);
* ``dispatch`` -- copy each token's row to each of its destination rows;
* ``combine``  -- per token, the gate-weighted sum of its k expert-output rows,
  accumulated in fp32 from +0.0 in slot order, rounded once to bf16 (RNE).

``pipeline`` holds the two-stage copy/compute timing model of [TMA-atlas]
sections "Science and assumptions" and "Engineering example".

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
library routines, closed forms, exact rational arithmetic and brute force.
The only piece without such a pin is the workload generators' notion of
"Zipf popularity" (it lives in ``synth``, not here).
"""

from .bf16 import bf16_to_f32, f32_to_bf16_rne
from .moe import (
    STATUS_DUPLICATE_EXPERT,
    STATUS_EXPERT_OUT_OF_RANGE,
    combine,
    dispatch,
    expert_identity,
    expert_scale,
    layout,
)
from .pipeline import pipelined_time, serial_time

__all__ = [
    "bf16_to_f32",
    "f32_to_bf16_rne",
    "layout",
    "dispatch",
    "combine",
    "expert_identity",
    "expert_scale",
    "STATUS_EXPERT_OUT_OF_RANGE",
    "STATUS_DUPLICATE_EXPERT",
    "pipelined_time",
    "serial_time",
]
