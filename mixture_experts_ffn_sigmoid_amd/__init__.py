"""MI355X-native Stable LatentMoE forward (K3 sigmoid routing, SiTU-GLU experts).

The compute path is liblatentmoe.so (hand-written gfx950 HIP kernels behind a
C ABI, include/latentmoe.h); this package is its thin ctypes binding.
"""
from ._lib import (  # noqa: F401
    ENTRY_DISPATCH, ENTRY_EXPERTS, ENTRY_FORWARD, ENTRY_ROUTE, ENTRY_ROUTED_BACKWARD, ENTRY_BACKWARD, EXPORTS, LIB_PATH, LMOE_BF16, LMOE_F32,
    GRAD_NAMES, Dims, Grads, LatentMoEError, Weights, dims_of, latentmoe_backward, latentmoe_dispatch, latentmoe_experts, latentmoe_forward,
    latentmoe_forward_check, latentmoe_forward_noalloc, latentmoe_forward_timed, latentmoe_route, latentmoe_route_softmax, latentmoe_routed_backward, latentmoe_router_losses, load,
    make_dims, router_losses_workspace_bytes, weights_struct, workspace_bytes,
    STEP_NAMES, TIMING_EVENTS,
)
