"""Local Mixture-of-Experts forward for AMD Instinct MI355X (gfx950).

route (FP32 softmax + top-k, or group-limited sigmoid routing) -> compact
dispatch -> SwiGLU experts -> weighted combine, and the first-order backward
chain (combine, experts, dispatch, router weights of a fixed selection), as
hand-written HIP kernels behind the C ABI of libmoe.so (include/moe.h).  This package is the thin
torch binding: the functions below have the names of the C entry points and
only marshal arguments.
"""

from .ops import (moe_combine, moe_combine_backward, moe_dispatch,
                  moe_dispatch_backward, moe_dispatch_noalloc,
                  moe_dispatch_workspace_size,
                  moe_experts_backward, moe_experts_backward_workspace_size,
                  moe_experts_forward, moe_experts_forward_clipped,
                  moe_experts_forward_training,
                  moe_forward, moe_forward_clipped,
                  moe_forward_sigmoid_grouped,
                  moe_forward_workspace_size, moe_route,
                  moe_route_sigmoid_grouped, moe_selected_router_backward,
                  moe_selected_router_weights)

__all__ = ["moe_route", "moe_dispatch", "moe_dispatch_workspace_size",
           "moe_experts_forward", "moe_combine", "moe_forward",
           "moe_forward_workspace_size", "moe_route_sigmoid_grouped",
           "moe_forward_sigmoid_grouped", "moe_selected_router_weights",
           "moe_selected_router_backward", "moe_experts_forward_training",
           "moe_combine_backward", "moe_experts_backward_workspace_size",
           "moe_experts_backward", "moe_dispatch_backward",
           "moe_experts_forward_clipped", "moe_forward_clipped",
           "moe_dispatch_noalloc"]
