"""Torch-facing binding of the MoE dispatch / combine C ABI.

Argument marshalling only: tensors are checked (device, dtype, shape, contiguity), their
device pointers and the current HIP stream are handed to libmoe_dispatch.so, and every step
of the computation runs in the gfx950 kernels. Calls are asynchronous on
``torch.cuda.current_stream()``. There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _capi
from ._capi import MOE_BF16, MOE_F32, MOE_FP8_E4M3, check, lib

# hidden-row element types; uint8 / float8_e4m3fn rows are FP8 (E4M3) codes, which only the
# permutes accept (they copy bytes)
_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.uint8: MOE_FP8_E4M3,
       torch.float8_e4m3fn: MOE_FP8_E4M3}


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, dims=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the calls launch on the current device "
                         f"cuda:{torch.cuda.current_device()} (use torch.cuda.device(...))")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _hidden_dt(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"{name} must be float32, bfloat16 or FP8 codes (uint8), got {t.dtype}")
    return _DT[t.dtype]


def expert_capacity(tokens: int, top_k: int, num_experts: int, cf_num: int = 5, cf_den: int = 4) -> int:
    """ceil(tokens * top_k / num_experts * cf_num / cf_den), computed exactly on the host."""
    v = lib().moe_expert_capacity(tokens, top_k, num_experts, cf_num, cf_den)
    if v < 0:
        raise ValueError("invalid capacity arguments")
    return int(v)


def route_topk(logits: torch.Tensor, k: int, out=None, group_size: int = 0, topk_groups: int = 0):
    """Top-k experts per token (ties -> lower id) and softmax over the k selected logits.
    With group_size > 0 and topk_groups > 0: group-limited routing (the topk_groups groups
    of group_size experts with the best logit first, then top-k among their experts).

    Returns (topk_idx int32 [T, k], topk_w float32 [T, k])."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    if out is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    else:
        idx, w = out
        _need(idx, "topk_idx", torch.int32, 2)
        _need(w, "topk_w", torch.float32, 2)
        if tuple(idx.shape) != (T, k) or tuple(w.shape) != (T, k):
            raise ValueError("output shapes must be [T, k]")
    if group_size > 0 or topk_groups > 0:
        check("moe_route_topk_grouped", lib().moe_route_topk_grouped(
            _p(logits), T, E, k, group_size, topk_groups, _p(idx), _p(w), _stream()))
    else:
        check("moe_route_topk", lib().moe_route_topk(_p(logits), T, E, k, _p(idx), _p(w), _stream()))
    return idx, w


@dataclass
class MoeIndex:
    """The dispatch "handle": built once by build_index, reused by permute and combine."""
    T: int
    K: int
    E: int
    capacity: int
    group_size: int
    alignment: int
    counts: torch.Tensor
    group_list: torch.Tensor
    kept_counts: torch.Tensor
    sorted_indices: torch.Tensor
    row_of: torch.Tensor
    permuted_probs: torch.Tensor
    slot_of: Optional[torch.Tensor] = None
    gsrc: Optional[torch.Tensor] = None
    esrc: Optional[torch.Tensor] = None
    group_counts: Optional[torch.Tensor] = None
    n_slots: Optional[torch.Tensor] = None
    slot_src: Optional[torch.Tensor] = None
    workspace: Optional[torch.Tensor] = None

    @property
    def rows(self) -> int:
        """Rows of the expert-major buffers: T*K, E*capacity in drop-and-pad mode, or
        T*K + E*(alignment-1) with expert alignment (rows after the last segment are unused)."""
        return index_rows(self.T, self.K, self.E, self.capacity, self.alignment)

    @property
    def num_groups(self) -> int:
        return self.E // self.group_size if self.group_size > 0 else 0

    def struct(self) -> _capi.MoeIndexStruct:
        return _capi.MoeIndexStruct(*[None if t is None else t.data_ptr() for t in (
            self.counts, self.group_list, self.kept_counts, self.sorted_indices, self.row_of,
            self.permuted_probs, self.slot_of, self.gsrc, self.esrc, self.group_counts, self.n_slots,
            self.slot_src)])


def workspace_bytes(T: int, K: int, E: int, group_size: int = 0) -> int:
    """Workspace bytes for these sizes: enough for build_index and for route_topk_index."""
    n = ctypes.c_size_t(0)
    check("moe_build_index_workspace_size",
          lib().moe_build_index_workspace_size(T, K, E, group_size, ctypes.byref(n)))
    f = ctypes.c_size_t(0)
    check("moe_route_topk_index_workspace_size",
          lib().moe_route_topk_index_workspace_size(T, K, E, group_size, ctypes.byref(f)))
    return max(int(n.value), int(f.value))


def index_rows(T: int, K: int, E: int, capacity: int = 0, alignment: int = 0) -> int:
    """Rows of the expert-major arrays for these sizes (moe_index_rows)."""
    r = lib().moe_index_rows(T, K, E, capacity, alignment)
    if r < 0:
        raise ValueError("invalid index sizes (or capacity together with alignment)")
    return int(r)


def alloc_index(T: int, K: int, E: int, capacity: int = 0, group_size: int = 0, device="cuda",
                alignment: int = 0, workspace: bool = True) -> MoeIndex:
    """Device arrays of an index for these sizes (and the workspace build_index needs, unless
    workspace=False: build_index_noalloc uses none)."""
    i32 = dict(dtype=torch.int32, device=device)
    rows = index_rows(T, K, E, capacity, alignment)
    ix = MoeIndex(
        T=T, K=K, E=E, capacity=capacity, group_size=group_size, alignment=alignment,
        counts=torch.empty(E, **i32), group_list=torch.empty(E, **i32), kept_counts=torch.empty(E, **i32),
        sorted_indices=torch.empty(rows, **i32), row_of=torch.empty((T, K), **i32),
        permuted_probs=torch.empty(rows, dtype=torch.float32, device=device))
    if group_size > 0:
        G = E // group_size
        ix.slot_of = torch.empty((T, G), **i32)
        ix.gsrc = torch.empty(T * min(K, G), **i32)
        ix.esrc = torch.empty(rows, **i32)
        ix.group_counts = torch.empty(G, **i32)
        ix.n_slots = torch.empty(1, **i32)
        ix.slot_src = torch.empty((T, K), **i32)
    if workspace:
        ws = workspace_bytes(T, K, E, group_size)
        ix.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
    return ix


def build_index(topk_idx: torch.Tensor, topk_w: Optional[torch.Tensor], num_experts: int,
                capacity: int = 0, group_size: int = 0, out: Optional[MoeIndex] = None,
                alignment: int = 0) -> MoeIndex:
    """Expert-major index of the routing result (sorted_indices, row_of, counts, group_list, ...);
    alignment > 1 rounds every expert segment up to a multiple of it (padding rows)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    T, K = topk_idx.shape
    if topk_w is not None:
        _need(topk_w, "topk_w", torch.float32, 2)
        if tuple(topk_w.shape) != (T, K):
            raise ValueError("topk_w must have the shape of topk_idx")
    ix = out if out is not None else alloc_index(T, K, num_experts, capacity, group_size, topk_idx.device,
                                                 alignment)
    if (ix.T, ix.K, ix.E, ix.capacity, ix.group_size, ix.alignment) != (T, K, num_experts, capacity, group_size,
                                                                        alignment):
        raise ValueError("preallocated index was made for other sizes")
    if ix.counts.device != topk_idx.device:
        raise ValueError(f"preallocated index is on {ix.counts.device}, topk_idx on {topk_idx.device}")
    s = ix.struct()
    ws = ix.workspace
    if ws is None:
        raise ValueError("this index was allocated without a workspace (use build_index_noalloc)")
    check("moe_build_index", lib().moe_build_index(
        _p(topk_idx), _p(topk_w), T, K, num_experts, capacity, group_size, alignment, ctypes.byref(s),
        _p(ws), ws.numel(), _stream()))
    return ix


def route_topk_index(logits: torch.Tensor, k: int, capacity: int = 0, group_size: int = 0, alignment: int = 0,
                     route_group_size: int = 0, topk_groups: int = 0, out=None, index: Optional[MoeIndex] = None):
    """route_topk (group-limited when route_group_size > 0) followed by build_index, in one call
    (moe_route_topk_index: the same arrays, bit for bit, with one launch fewer for large inputs).
    Returns (topk_idx, topk_w, index)."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    if out is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    else:
        idx, w = out
        _need(idx, "topk_idx", torch.int32, 2)
        _need(w, "topk_w", torch.float32, 2)
        if tuple(idx.shape) != (T, k) or tuple(w.shape) != (T, k):
            raise ValueError("output shapes must be [T, k]")
    ix = index if index is not None else alloc_index(T, k, E, capacity, group_size, logits.device, alignment)
    if (ix.T, ix.K, ix.E, ix.capacity, ix.group_size, ix.alignment) != (T, k, E, capacity, group_size, alignment):
        raise ValueError("preallocated index was made for other sizes")
    if ix.counts.device != logits.device:
        raise ValueError(f"preallocated index is on {ix.counts.device}, logits on {logits.device}")
    ws = ix.workspace
    if ws is None:
        raise ValueError("this index was allocated without a workspace")
    s = ix.struct()
    check("moe_route_topk_index", lib().moe_route_topk_index(
        _p(logits), T, E, k, route_group_size, topk_groups, _p(idx), _p(w), capacity, group_size, alignment,
        ctypes.byref(s), _p(ws), ws.numel(), _stream()))
    return idx, w, ix


def build_index_noalloc(topk_idx: torch.Tensor, topk_w: Optional[torch.Tensor], num_experts: int,
                        capacity: int = 0, group_size: int = 0, out: Optional[MoeIndex] = None,
                        alignment: int = 0) -> MoeIndex:
    """build_index through moe_build_index_noalloc: the same arrays, the tile counts in the
    library's own per-GPU scratch (no workspace; the library allocates nothing). Calls that
    overlap on one GPU race on that scratch."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    T, K = topk_idx.shape
    if topk_w is not None:
        _need(topk_w, "topk_w", torch.float32, 2)
        if tuple(topk_w.shape) != (T, K):
            raise ValueError("topk_w must have the shape of topk_idx")
    ix = out if out is not None else alloc_index(T, K, num_experts, capacity, group_size, topk_idx.device,
                                                 alignment, workspace=False)
    if (ix.T, ix.K, ix.E, ix.capacity, ix.group_size, ix.alignment) != (T, K, num_experts, capacity, group_size,
                                                                        alignment):
        raise ValueError("preallocated index was made for other sizes")
    if ix.counts.device != topk_idx.device:
        raise ValueError(f"preallocated index is on {ix.counts.device}, topk_idx on {topk_idx.device}")
    s = ix.struct()
    check("moe_build_index_noalloc", lib().moe_build_index_noalloc(
        _p(topk_idx), _p(topk_w), T, K, num_experts, capacity, group_size, alignment, ctypes.byref(s), _stream()))
    return ix


def permute(src: torch.Tensor, src_row: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[i] = src[src_row[i]] bit for bit; an out-of-range src_row (e.g. -1) gives a zero row."""
    _need(src, "src", None, 2)
    dt = _hidden_dt(src, "src")
    _need(src_row, "src_row", torch.int32, 1)
    N = src_row.shape[0]
    H = src.shape[1]
    if out is None:
        out = torch.empty((N, H), dtype=src.dtype, device=src.device)
    _need(out, "out", src.dtype, 2)
    if tuple(out.shape) != (N, H):
        raise ValueError(f"out must be [{N}, {H}]")
    check("moe_permute", lib().moe_permute(_p(src), src.shape[0], H, dt, _p(src_row), N, _p(out), _stream()))
    return out


def permute_scatter(src: torch.Tensor, dst_of: torch.Tensor, num_rows: int,
                    src_row: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Source-major permute: out[dst_of[t, j]] = src[t]; rows with src_row[i] out of range are zeros.

    With dst_of = index.row_of and src_row = index.sorted_indices this equals
    permute(src, index.sorted_indices), reading every source row once."""
    _need(src, "src", None, 2)
    dt = _hidden_dt(src, "src")
    _need(dst_of, "dst_of", torch.int32, 2)
    if dst_of.shape[0] != src.shape[0]:
        raise ValueError("dst_of must have one row per source row")
    if src_row is not None:
        _need(src_row, "src_row", torch.int32, 1)
        if src_row.shape[0] != num_rows:
            raise ValueError("src_row must have num_rows entries")
    H = src.shape[1]
    if out is None:
        out = torch.empty((num_rows, H), dtype=src.dtype, device=src.device)
    _need(out, "out", src.dtype, 2)
    if tuple(out.shape) != (num_rows, H):
        raise ValueError(f"out must be [{num_rows}, {H}]")
    check("moe_permute_scatter", lib().moe_permute_scatter(
        _p(src), src.shape[0], H, dt, _p(dst_of), dst_of.shape[1], _p(src_row), num_rows, _p(out), _stream()))
    return out


def permute_grouped(src: torch.Tensor, src_row: torch.Tensor, dst_of: torch.Tensor,
                    out: Optional[torch.Tensor] = None, src_of: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The gather out[r] = src[src_row[r]] (zero rows where src_row is out of range), done in the
    groups of destination rows that dst_of [M, J] lists; a source row named by several rows of
    one group is read once. Rows with a valid src_row that dst_of never lists are not written.
    src_of [M, J], if given, names each listed row's source (= src_row[dst_of]) so that it need
    not be looked up.

    The group dispatch's receive side: permute_grouped(group_buffer, index.esrc, index.row_of,
    src_of=index.slot_src)."""
    _need(src, "src", None, 2)
    dt = _hidden_dt(src, "src")
    _need(src_row, "src_row", torch.int32, 1)
    _need(dst_of, "dst_of", torch.int32, 2)
    if src_of is not None:
        _need(src_of, "src_of", torch.int32, 2)
        if tuple(src_of.shape) != tuple(dst_of.shape):
            raise ValueError("src_of must have the shape of dst_of")
    N = src_row.shape[0]
    H = src.shape[1]
    if out is None:
        out = torch.empty((N, H), dtype=src.dtype, device=src.device)
    _need(out, "out", src.dtype, 2)
    if tuple(out.shape) != (N, H):
        raise ValueError(f"out must be [{N}, {H}]")
    check("moe_permute_grouped", lib().moe_permute_grouped(
        _p(src), src.shape[0], H, dt, _p(src_row), N, _p(dst_of), dst_of.shape[0], dst_of.shape[1], _p(src_of),
        _p(out), _stream()))
    return out


def quantize_fp8(x: torch.Tensor, block: int = 128, out=None):
    """Per-(token, block) FP8 E4M3 quantization: q [T, H] uint8 codes, scales [T, H/block] float32
    with x ~ value(q) * scale (scale = amax/448 per block)."""
    _need(x, "x", None, 2)
    dt = _hidden_dt(x, "x")
    T, H = x.shape
    if block < 1 or H % block:
        raise ValueError("block must divide H")
    q, sc = (None, None) if out is None else out
    q = torch.empty((T, H), dtype=torch.uint8, device=x.device) if q is None else q
    sc = torch.empty((T, H // block), dtype=torch.float32, device=x.device) if sc is None else sc
    _need(q, "q", torch.uint8, 2)
    _need(sc, "scales", torch.float32, 2)
    if tuple(q.shape) != (T, H) or tuple(sc.shape) != (T, H // block):
        raise ValueError(f"output shapes must be [{T}, {H}] and [{T}, {H // block}]")
    check("moe_quantize_fp8", lib().moe_quantize_fp8(_p(x), dt, T, H, block, _p(q), _p(sc), _stream()))
    return q, sc


def permute_scatter_fp8(src: torch.Tensor, dst_of: torch.Tensor, num_rows: int, block: int = 128,
                        src_row: Optional[torch.Tensor] = None, out=None):
    """FP8 dispatch: the source rows quantized once (per-block E4M3 + float32 scales) and scattered
    source-major like permute_scatter. Returns (q [num_rows, H] uint8, scales [num_rows, H/block])."""
    _need(src, "src", None, 2)
    dt = _hidden_dt(src, "src")
    _need(dst_of, "dst_of", torch.int32, 2)
    if dst_of.shape[0] != src.shape[0]:
        raise ValueError("dst_of must have one row per source row")
    H = src.shape[1]
    if block < 1 or H % block:
        raise ValueError("block must divide H")
    if src_row is not None:
        _need(src_row, "src_row", torch.int32, 1)
        if src_row.shape[0] != num_rows:
            raise ValueError("src_row must have num_rows entries")
    q, sc = (None, None) if out is None else out
    q = torch.empty((num_rows, H), dtype=torch.uint8, device=src.device) if q is None else q
    sc = torch.empty((num_rows, H // block), dtype=torch.float32, device=src.device) if sc is None else sc
    _need(q, "q", torch.uint8, 2)
    _need(sc, "scales", torch.float32, 2)
    if tuple(q.shape) != (num_rows, H) or tuple(sc.shape) != (num_rows, H // block):
        raise ValueError("output shapes must be [num_rows, H] and [num_rows, H/block]")
    check("moe_permute_scatter_fp8", lib().moe_permute_scatter_fp8(
        _p(src), dt, src.shape[0], H, block, _p(dst_of), dst_of.shape[1], _p(src_row), num_rows, _p(q), _p(sc),
        _stream()))
    return q, sc


def permute_grouped_fp8(codes: torch.Tensor, scales: torch.Tensor, src_row: torch.Tensor, dst_of: torch.Tensor,
                        out=None, src_of: Optional[torch.Tensor] = None):
    """The FP8 group receive: permute_grouped of the codes and of their scale rows in one launch,
    bit for bit the two permute_grouped calls. Returns (codes [N, H] uint8, scales [N, H/block])."""
    _need(codes, "codes", None, 2)
    if codes.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"codes must be FP8 codes (uint8), got {codes.dtype}")
    _need(scales, "scales", torch.float32, 2)
    _need(src_row, "src_row", torch.int32, 1)
    _need(dst_of, "dst_of", torch.int32, 2)
    if scales.shape[0] != codes.shape[0]:
        raise ValueError("scales must have one row per code row")
    H, nb = codes.shape[1], scales.shape[1]
    if nb < 1 or H % nb:
        raise ValueError("the scale rows must split H into equal blocks")
    if src_of is not None:
        _need(src_of, "src_of", torch.int32, 2)
        if tuple(src_of.shape) != tuple(dst_of.shape):
            raise ValueError("src_of must have the shape of dst_of")
    N = src_row.shape[0]
    q, sc = (None, None) if out is None else out
    q = torch.empty((N, H), dtype=codes.dtype, device=codes.device) if q is None else q
    sc = torch.empty((N, nb), dtype=torch.float32, device=codes.device) if sc is None else sc
    _need(q, "out codes", codes.dtype, 2)
    _need(sc, "out scales", torch.float32, 2)
    if tuple(q.shape) != (N, H) or tuple(sc.shape) != (N, nb):
        raise ValueError(f"outputs must be [{N}, {H}] and [{N}, {nb}]")
    check("moe_permute_grouped_fp8", lib().moe_permute_grouped_fp8(
        _p(codes), _p(scales), codes.shape[0], H, H // nb, _p(src_row), N, _p(dst_of), dst_of.shape[0],
        dst_of.shape[1], _p(src_of), _p(q), _p(sc), _stream()))
    return q, sc


def unpermute_combine(y: torch.Tensor, row_of: torch.Tensor, weights: Optional[torch.Tensor] = None,
                      out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                      bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = sum_k weights[t,k] * y[row_of[t,k]] (float32 FMA chain in k order) [+ bias[t],
    one float32 addition; bias has the output's shape and dtype]."""
    _need(y, "y", None, 2)
    y_dt = _hidden_dt(y, "y")
    _need(row_of, "row_of", torch.int32, 2)
    T, K = row_of.shape
    H = y.shape[1]
    if weights is not None:
        _need(weights, "weights", torch.float32, 2)
        if tuple(weights.shape) != (T, K):
            raise ValueError("weights must have the shape of row_of")
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype or y.dtype, device=y.device)
    _need(out, "out", None, 2)
    out_dt = _hidden_dt(out, "out")
    if tuple(out.shape) != (T, H):
        raise ValueError(f"out must be [{T}, {H}]")
    if bias is not None:
        _need(bias, "bias", out.dtype, 2)
        if tuple(bias.shape) != (T, H):
            raise ValueError(f"bias must be [{T}, {H}]")
    check("moe_unpermute_combine", lib().moe_unpermute_combine(
        _p(y), y_dt, y.shape[0], H, _p(row_of), _p(weights), _p(bias), T, K, _p(out), out_dt, _stream()))
    return out


def group_precombine(y: torch.Tensor, row_of: torch.Tensor, weights: Optional[torch.Tensor],
                     topk_idx: torch.Tensor, num_experts: int, group_size: int, slot_of: torch.Tensor,
                     slots_cap: Optional[int] = None, out: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Per-(token, group) weighted partial sums (a float32 chain) stored at row slot_of[t, g], as
    float32 or, with out_dtype (or out) bfloat16, rounded once to bf16."""
    _need(y, "y", None, 2)
    y_dt = _hidden_dt(y, "y")
    _need(row_of, "row_of", torch.int32, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(slot_of, "slot_of", torch.int32, 2)
    T, K = row_of.shape
    H = y.shape[1]
    if tuple(topk_idx.shape) != (T, K):
        raise ValueError("topk_idx must have the shape of row_of")
    if weights is not None:
        _need(weights, "weights", torch.float32, 2)
        if tuple(weights.shape) != (T, K):
            raise ValueError("weights must have the shape of row_of")
    if group_size < 1 or num_experts % group_size:
        raise ValueError("group_size must divide num_experts")
    if tuple(slot_of.shape) != (T, num_experts // group_size):
        raise ValueError(f"slot_of must be [{T}, {num_experts // group_size}]")
    if out is None:
        if slots_cap is None:
            raise ValueError("give slots_cap or out")
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("partials are float32 or bfloat16")
        out = torch.empty((slots_cap, H), dtype=out_dtype, device=y.device)
    _need(out, "out", None, 2)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("partials are float32 or bfloat16")
    if out.shape[1] != H:
        raise ValueError(f"out rows must have {H} elements")
    check("moe_group_precombine", lib().moe_group_precombine(
        _p(y), y_dt, y.shape[0], H, _p(row_of), _p(weights), _p(topk_idx), T, K, num_experts, group_size,
        _p(slot_of), out.shape[0], _p(out), _DT[out.dtype], _stream()))
    return out


# ---------------------------------------------------------------- backward


def unpermute_combine_backward(dout: torch.Tensor, y: Optional[torch.Tensor], row_of: torch.Tensor,
                               weights: Optional[torch.Tensor] = None, src_row: Optional[torch.Tensor] = None,
                               num_rows: Optional[int] = None, want_dw: bool = True,
                               dy_dtype: Optional[torch.dtype] = None, out=None):
    """Backward of unpermute_combine: dy[row_of[t,k]] = weights[t,k] * dout[t] (rows with
    src_row out of range are zeros), dw[t,k] = <dout[t], y[row_of[t,k]]>. Returns (dy, dw|None).

    The dispatch's backward is unpermute_combine(dxp, row_of) (unit weights)."""
    _need(dout, "dout", None, 2)
    dout_dt = _hidden_dt(dout, "dout")
    _need(row_of, "row_of", torch.int32, 2)
    T, K = row_of.shape
    H = dout.shape[1]
    if dout.shape[0] != T:
        raise ValueError("dout must have one row per token of row_of")
    if y is not None:
        _need(y, "y", None, 2)
        if y.shape[1] != H:
            raise ValueError("y and dout must have the same hidden size")
    elif want_dw:
        raise ValueError("dw needs y")
    rows = num_rows if num_rows is not None else (y.shape[0] if y is not None else None)
    if rows is None:
        raise ValueError("num_rows is needed without y")
    if y is not None and y.shape[0] != rows:
        raise ValueError("y must have num_rows rows")
    y_dt = _hidden_dt(y, "y") if y is not None else dout_dt
    if weights is not None:
        _need(weights, "weights", torch.float32, 2)
        if tuple(weights.shape) != (T, K):
            raise ValueError("weights must be [T, K]")
    if src_row is not None:
        _need(src_row, "src_row", torch.int32, 1)
        if src_row.shape[0] != rows:
            raise ValueError("src_row must have num_rows entries")
    ddt = dy_dtype or (y.dtype if y is not None else dout.dtype)
    dy, dw = (None, None) if out is None else out
    if dy is None:
        dy = torch.empty((rows, H), dtype=ddt, device=dout.device)
    _need(dy, "dy", ddt, 2)
    if tuple(dy.shape) != (rows, H):
        raise ValueError(f"dy must be [{rows}, {H}]")
    if want_dw:
        if dw is None:
            dw = torch.empty((T, K), dtype=torch.float32, device=dout.device)
        _need(dw, "dw", torch.float32, 2)
        if tuple(dw.shape) != (T, K):
            raise ValueError("dw must be [T, K]")
    else:
        dw = None
    check("moe_unpermute_combine_backward", lib().moe_unpermute_combine_backward(
        _p(dout), dout_dt, _p(y), y_dt, rows, H, _p(row_of), _p(weights), T, K, _p(src_row), _p(dy),
        _DT[ddt], _p(dw), _stream()))
    return dy, dw


def route_topk_backward(topk_idx: torch.Tensor, topk_w: torch.Tensor, d_topk_w: torch.Tensor, num_experts: int,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the router logits through the softmax over the K selected logits."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    _need(d_topk_w, "d_topk_w", torch.float32, 2)
    T, K = topk_idx.shape
    if tuple(topk_w.shape) != (T, K) or tuple(d_topk_w.shape) != (T, K):
        raise ValueError("topk_w and d_topk_w must be [T, K]")
    if out is None:
        out = torch.empty((T, num_experts), dtype=torch.float32, device=topk_idx.device)
    _need(out, "out", torch.float32, 2)
    if tuple(out.shape) != (T, num_experts):
        raise ValueError(f"out must be [{T}, {num_experts}]")
    check("moe_route_topk_backward", lib().moe_route_topk_backward(
        _p(topk_idx), _p(topk_w), _p(d_topk_w), T, num_experts, K, _p(out), _stream()))
    return out
