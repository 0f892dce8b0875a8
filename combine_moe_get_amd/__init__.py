"""MI355X-native MoE expert-parallel dispatch and combine.

The routing layout, the optional int8 quantization, the scatter of routed
token copies into expert-major receive rows and the weighted combine with
zero / copy / constant experts run in hand-written HIP kernels for gfx950,
behind the C ABI of include/moe_get.h (libmoe_get.so).  This package is the
thin Python binding over that ABI plus seeded input generators.
"""
from .binding import (  # noqa: F401
    DEV_STATUS_BAD_EXPERT_ID, DEV_STATUS_RANK_OVERFLOW, LIB_PATH, QUANT_DYNAMIC_INT8, QUANT_NONE, QUANT_STATIC_INT8,
    Layout, MoeGetError, PreparedCall, Shape, abi_version, alloc_layout, alloc_workspace, check_shape, combine,
    dispatch, layout, layout_dispatch, layout_dispatch_launches, layout_launches, layout_noalloc, lib, make_shape,
    noalloc_scratch_bytes, prepare_layout_dispatch, prepare_combine, prepare_dispatch, prepare_layout,
    prepare_layout_noalloc, rank_capacity, recv_capacity, status_string, workspace_size,
)
