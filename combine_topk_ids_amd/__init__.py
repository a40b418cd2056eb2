"""MoE expert-parallel layer on one MI355X: dispatch -> grouped SwiGLU GEMM -> combine.

The work runs in the hand-written HIP library libmoe_ep.so (C ABI in
include/moe_ep.h); this package only binds it.  Importing fails loudly if the
library has not been built.
"""
from ._lib import (EXPERT_MAJOR, FLAT, LAYOUTS, RANK_MAJOR, Handle, MoeEpError, Params,  # noqa: F401
                   moe_ep_combine, moe_ep_dispatch, moe_ep_expert_compute, moe_ep_layer_forward, moe_ep_layer_forward_fused_combine, moe_ep_layer_forward_noalloc,
                   moe_ep_layer_forward_timed,
                   moe_ep_fp8_scale_stride, moe_ep_layer_forward_fp8, moe_ep_quantize_fp8, moe_ep_query_status, moe_ep_router_topk, moe_ep_workspace_size, params, strerror)
from . import _lib  # noqa: F401
