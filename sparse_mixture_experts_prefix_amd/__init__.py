"""MI355X (gfx950) sparse Mixture-of-Experts SwiGLU layer, forward pass.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe.so, built in-tree by ``build.build()``); this package is the thin
Python binding over it.  Importing the package does not load the library;
the first call does, and raises if it is missing.
"""
from .binding import (MOE_ERR_ALIGNMENT, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_SCRATCH,
                      MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_OK, MoEError, Shape, Weights, alloc_workspace,
                      ROUTER_BIAS_LOGITS, ROUTER_BIAS_NONE, ROUTER_BIAS_SELECT, WEIGHTS_BF16,
                      WEIGHTS_FP8_E4M3,
                      HipEvents, bias_mode, block_m, layer_shape, load_library, make_shape, moe_align, moe_block_m,
                      moe_backward, moe_backward_workspace_size, backward_workspace_size,
                      moe_forward_train, moe_train_workspace_size, train_workspace_size,
                      moe_expert_load, moe_forward, moe_forward_noalloc, moe_forward_routed, moe_forward_timed,
                      moe_route,
                      moe_strerror, moe_workspace_size, strerror, workspace_size)

__all__ = ["moe_forward", "moe_forward_noalloc", "moe_route", "moe_align", "moe_forward_routed", "moe_workspace_size",
           "moe_block_m", "moe_strerror", "moe_forward_timed", "moe_expert_load", "moe_backward",
           "moe_backward_workspace_size", "moe_forward_train", "moe_train_workspace_size",
           "HipEvents", "MoEError",
           "make_shape", "layer_shape", "alloc_workspace", "load_library", "ROUTER_BIAS_NONE",
           "ROUTER_BIAS_LOGITS", "ROUTER_BIAS_SELECT", "WEIGHTS_BF16", "WEIGHTS_FP8_E4M3"]
