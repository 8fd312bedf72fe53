"""MoE token layout, dispatch and combine for MI355X (gfx950).

The hot path is the C-ABI library ``libepget.so`` (HIP kernels under
``csrc/``, declared in ``include/ep_get.h``); this package binds it with
ctypes and offers a small helper that allocates the layout outputs with
torch.  PyTorch provides device memory and streams only.
"""
from ._binding import (  # noqa: F401
    EP_ERR_BAD_EXPERT, EP_ERR_CAPACITY, EP_ERR_HIP, EP_ERR_INVALID_ARG, EP_ERR_SCRATCH_LIMIT,
    EP_MAX_EXPERTS, EP_MAX_EXPERTS_PER_RANK, EP_MAX_HIDDEN, EP_MAX_RANKS, EP_MAX_TOPK,
    EP_NOALLOC_SCRATCH_BYTES, EP_OK, EXPORTS, LIB_PATH, BoundCall, EpError, Problem, ep_combine,
    ep_combine_hier, ep_combine_topk_weights, ep_dispatch, ep_dispatch_fp8, ep_dispatch_hier,
    ep_get_group_layout, ep_get_layout, ep_layout_dispatch, ep_layout_dispatch_fp8,
    ep_layout_dispatch_noalloc, ep_quantize_fp8, ep_rank_stride_hint, ep_read_status,
    ep_workspace_bytes, error_string, load,
)
from .buffers import LayoutBuffers, alloc_layout  # noqa: F401
