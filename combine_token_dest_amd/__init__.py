"""MI355X (gfx950) rank-major MoE expert-parallel dispatch and combine.

The C ABI is include/moe_ep.h (libmoe_ep.so, built in-tree by
``python -m combine_token_dest_amd.build``); ``_lib`` binds it with the same
names and ``MoEEp`` gives it the flashinfer.moe_ep API shape over torch
tensors, one list entry per rank.
"""

from ._lib import (MOE_EP_ALL_RANKS, MOE_EP_BF16, MOE_EP_F16, MOE_EP_F32, MOE_EP_MAX_RANKS, MOE_EP_ORDER_AUTO,
                   MOE_EP_ORDER_DESTINATION, MOE_EP_ORDER_SOURCE_ROW, MoeEpError,
                   moe_ep_active_rank_mask, moe_ep_checkpoint_prepare, moe_ep_checkpoint_restore,
                   moe_ep_combine, moe_ep_create, moe_ep_create_vmm, moe_ep_destroy, moe_ep_dispatch,
                   moe_ep_get_combine_input_buffer, moe_ep_is_platform_supported, moe_ep_last_error,
                   moe_ep_status_string, moe_ep_workspace, moe_ep_workspace_bytes)
from .moe_ep import DispatchResult, MoEEp

__all__ = [
    "MOE_EP_ALL_RANKS", "MOE_EP_BF16", "MOE_EP_F16", "MOE_EP_F32", "MOE_EP_MAX_RANKS", "MOE_EP_ORDER_AUTO",
    "MOE_EP_ORDER_DESTINATION", "MOE_EP_ORDER_SOURCE_ROW", "MoeEpError",
    "moe_ep_active_rank_mask", "moe_ep_checkpoint_prepare", "moe_ep_checkpoint_restore",
    "moe_ep_combine", "moe_ep_create", "moe_ep_create_vmm", "moe_ep_destroy", "moe_ep_dispatch",
    "moe_ep_get_combine_input_buffer", "moe_ep_is_platform_supported", "moe_ep_last_error",
    "moe_ep_status_string", "moe_ep_workspace", "moe_ep_workspace_bytes",
    "DispatchResult", "MoEEp",
]
