"""MI355X-native forward pass of one Mixture-of-Experts layer (libmoe.so + binding).

Importing the package does not load the library; the first call does, and
raises if ``libmoe.so`` has not been built (there is no CPU fallback).
"""
from . import native
from .layer import (ECBuffers, ExpertCache, MoEBuffers, MoEGrads, ec_ffn_k, moe_layer_backward,
                    moe_layer_backward_ec, moe_layer_forward, moe_layer_forward_cached, moe_layer_forward_ec)
from .native import (MoEError, moe_aux_loss, moe_combine, moe_expert_choice, moe_grouped_ffn,
                     moe_permute, moe_router_topk, moe_workspace_size)

__all__ = ["native", "MoEBuffers", "MoEGrads", "ECBuffers", "ExpertCache", "ec_ffn_k",
           "moe_layer_forward", "moe_layer_backward", "moe_layer_backward_ec",
           "moe_layer_forward_ec", "moe_layer_forward_cached", "MoEError", "moe_router_topk", "moe_permute",
           "moe_grouped_ffn", "moe_combine", "moe_aux_loss", "moe_expert_choice",
           "moe_workspace_size"]
