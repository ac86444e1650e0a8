"""Routed weight-only-quantized (WNA16) MoE layer for AMD Instinct MI355X.

The layer runs in hand-written gfx950 HIP kernels behind the C ABI of
include/moe_wna16.h (libmoe_wna16.so, built in-tree by
`python -m weight_only_bit_moe_amd.build`).  This package binds that ABI;
`inputs` draws seeded synthetic layers.
"""
from .binding import (EXPORTED, LIB_PATH, SYNC_BYTES, MoeWna16Error, align, forward, load_library,
                      moe_wna16_align, moe_wna16_forward, moe_wna16_forward_profiled,
                      moe_wna16_plan, moe_wna16_quantize, quantize, moe_wna16_prepare,
                      moe_wna16_forward_prepared, moe_wna16_forward_noalloc, prepare,
                      moe_wna16_status_string, moe_wna16_workspace_f32_offset,
                      moe_wna16_workspace_layout, moe_wna16_workspace_size, workspace_f32_sum,
                      workspace_for, workspace_meta, workspace_sort)

__all__ = ["EXPORTED", "LIB_PATH", "SYNC_BYTES", "MoeWna16Error", "align", "forward", "load_library",
           "moe_wna16_align", "moe_wna16_forward", "moe_wna16_forward_profiled", "moe_wna16_plan", "moe_wna16_quantize", "quantize",
           "moe_wna16_prepare", "moe_wna16_forward_prepared", "moe_wna16_forward_noalloc", "prepare",
           "moe_wna16_status_string",
           "moe_wna16_workspace_f32_offset", "moe_wna16_workspace_layout",
           "moe_wna16_workspace_size", "workspace_f32_sum", "workspace_for", "workspace_meta",
           "workspace_sort"]
