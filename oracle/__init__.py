"""CPU oracle for the MoE layer hot path. TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy code in fp64 that states what the layer computes. Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may import it; the library
path never does, and it shares no code, tables or helpers with the HIP kernels. Its inputs come
from ``synth`` (seeded draws) and nowhere else.

Sources (cited by page title and section):

* Cursor blog post "Mixture-of-Kittens: our open-source MoE megakernel for NVL72s" (the Blog):
  the notation and MoE layer equation in "Overlapping computation and communication in MoE",
  the pull-schedule table and its reuse by all four exchanges in "Scheduling".
* Paper notes "Mixture-of-Kittens: MoE Megakernel for NVL72s" on sparsenotes.com (the Notes):
  the schedule sort key in "Pull dispatch, push combine", determinism, MXFP8 and the router
  gradient identity in "The production details".
* OCP Microscaling Formats (MX) v1.0 specification, a published format, for the MXFP8 encoding
  that the Notes name but do not define.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force, closed forms,
library routines or worked examples; see each function's docstring.
"""
from .moe import (  # noqa: F401
    silu, sigmoid, route_topk, routing_weights, schedule, pull_schedule,
    swiglu_expert, moe_forward, moe_backward, d_logits_from_dg,
    experts_forward, experts_backward, shared_backward, combine,
    mx_along, experts_forward_mx, experts_backward_mx, experts_forward_mx_w, experts_backward_mx_w,
    moe_forward_mx, router_logits, router_backward,
)
from .mx import (  # noqa: F401
    e4m3_round, e4m3_encode, e4m3_decode, mx_quantize, mx_dequantize, mx_roundtrip, E4M3_MAX,
    MX_BLOCK,
)
