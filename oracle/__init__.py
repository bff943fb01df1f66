"""CPU oracle of the Stable LatentMoE forward and of its routed-block
backward (test infrastructure only).

Importable only from tests, the smoke check and the bench's CPU-baseline leg.
"""
from .latentmoe_oracle import (  # noqa: F401
    Dispatch, RoutedGrads, Routes, Weights, balancing_losses, dispatch, forward, padded_layout,
    rmsnorm, route, route_from_logits, route_softmax_topk, layer_backward, rmsnorm_backward, routed_backward, routed_dense,
    routed_sparse, shared_sum, sigmoid, situ, situ_hidden, situ_hidden_grad, weights_from_arrays,
)
from .config_weights import config_weights, config_x  # noqa: F401
