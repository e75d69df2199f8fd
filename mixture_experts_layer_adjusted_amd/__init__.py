"""MI355X (gfx950) DeepSeekMoE layer forward: HIP kernels behind the C ABI of include/moe.h.

The Python surface is the ctypes binding in ``binding.py`` (same names as the
C entry points).  Importing the package fails if libmoe.so has not been built.
"""
from .binding import (MOE_DTYPE_BF16, MOE_DTYPE_F32, MOE_DTYPE_FP8_B128, MOE_FORWARD_EVENTS, MoeError, Shape,
                      WeightGrads, Weights, make_shape, make_weight_grads, make_weights, moe_backward,
                      moe_backward_saved, moe_backward_workspace_size, moe_forward, moe_forward_profiled,
                      moe_forward_train, moe_prepare_weights, moe_saved_inputs_size, moe_quantize_act,
                      moe_quantize_weights, moe_route, moe_route_balance, moe_route_grouped, moe_route_noalloc, moe_status_string,
                      moe_update_bias,
                      moe_workspace_size)

__all__ = ["MOE_DTYPE_BF16", "MOE_DTYPE_F32", "MOE_DTYPE_FP8_B128", "MOE_FORWARD_EVENTS", "MoeError", "Shape",
           "WeightGrads", "Weights", "make_shape", "make_weight_grads", "make_weights", "moe_backward",
           "moe_backward_saved", "moe_backward_workspace_size", "moe_forward", "moe_forward_profiled",
           "moe_forward_train", "moe_prepare_weights", "moe_saved_inputs_size", "moe_quantize_act",
           "moe_quantize_weights", "moe_route", "moe_route_balance", "moe_route_grouped", "moe_route_noalloc",
           "moe_status_string", "moe_update_bias",
           "moe_workspace_size"]
