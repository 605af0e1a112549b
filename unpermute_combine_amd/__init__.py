"""MI355X (gfx950) MoE token dispatch / unpermute-combine.

Top-k routing with a softmax over the selected logits (optionally group-limited), the expert
histogram with its running sum (group_list), the stable expert-major permute (standard,
drop-and-pad, expert-aligned, the two-stage group dispatch, an FP8 E4M3 dispatch), the weighted
unpermute-combine (optional bias) and the per-group local pre-combine, with the backward of the
combine and of the routing softmax, as hand-written HIP kernels behind a C ABI
(``include/moe_dispatch.h``, ``libmoe_dispatch.so``). This package is the torch binding.
"""
from .ops import (MoeIndex, alloc_index, build_index, build_index_noalloc, expert_capacity, group_precombine, index_rows, permute,
                  permute_grouped, permute_grouped_fp8, permute_scatter, permute_scatter_fp8, quantize_fp8, route_topk,
                  route_topk_backward, route_topk_index, unpermute_combine,
                  unpermute_combine_backward, workspace_bytes)
from ._capi import MoeError, lib

__all__ = ["MoeIndex", "MoeError", "alloc_index", "build_index", "build_index_noalloc", "expert_capacity", "group_precombine", "index_rows",
           "lib", "permute", "permute_grouped", "permute_grouped_fp8", "permute_scatter", "permute_scatter_fp8", "quantize_fp8",
           "route_topk", "route_topk_backward", "route_topk_index",
           "unpermute_combine", "unpermute_combine_backward", "workspace_bytes"]
