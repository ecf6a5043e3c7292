"""CPU oracle for the local Mixture-of-Experts forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
constants or helpers with the HIP library under ``mixture_experts_layer_28_amd``
and imports nothing from it.

What it computes follows the ruDNN user guide (RUDA docs, German edition),
sections 3 to 6 (MoE workflow, routing contract, expert weights and dispatch,
calling MoE), and the expert stage of the docs.rs page "ruDNN 0.1.25 source,
src/moe/experts.rs" (``SwiGluExperts::forward_dispatched_with_strategy``).

Every function is plain and slow on purpose: Python loops per token or per
row, numpy float64 for every product the pages leave unspecified, numpy
float32 only where the pages fix FP32 (the routing softmax).

Parity status of each function (what pins it is listed in the test files
``tests/test_oracle_*.py``):

* ``fp.round_to``             pinned (library casts, IEEE boundary cases)
* ``moe.route``               pinned (brute force, closed forms, golden cases)
* ``moe.dispatch``            pinned (invariants, brute-force scan)
* ``moe.experts``             pinned (dense-MLP reduction, scalar closed form,
                              brute-force loops)
* ``moe.combine``             pinned (k=1 identity, brute force)
* ``moe.forward``             pinned (brute force at T<=4, identical experts)
* ``moe.clipped_silu_times`` and ``experts(..., clip=...)``
                              pinned (reduces to the plain SwiGLU, torch
                              clamp/sigmoid, closed forms at the clamps)
* ``grouped.route_sigmoid_grouped``  pinned (golden cases, brute force by
                              counting, sort reduction, scipy ``expit``)
* ``grouped.forward_sigmoid_grouped`` pinned (per-token sum, identical
                              experts)

* ``router_weights.selected_router_weights`` / ``selected_router_backward``
                              pinned (torch autograd in float64, finite
                              differences, closed forms, invariants)

* ``backward.experts_forward_training``, ``combine_backward``,
  ``experts_backward``, ``dispatch_backward``
                              pinned (torch autograd in float64 through the
                              whole layer, finite differences, adjointness
                              of dispatch and combine, training forward equal
                              to the inference forward)

``grouped`` follows section 10 of the same guide (group-limited sigmoid
routing) and the experts page's ``forward_sigmoid_grouped``;
``router_weights`` follows section 12 (router weights of a fixed selection
and their logits gradient); ``backward`` follows section 12's backward chain
and the experts page's training forward and expert backward.
"""

from . import backward, fp, grouped, moe, router_weights  # noqa: F401
