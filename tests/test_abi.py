"""The C-ABI library loads on a machine without a GPU and exports every symbol the header
declares; host-only entry points and argument validation (which returns before any launch)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, load_golden

HEADER = os.path.join(ROOT, "include", "moe_dispatch.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def capi():
    from unpermute_combine_amd import _capi
    return _capi


def test_header_declares_the_five_operations():
    names = declared_functions()
    for op in ("moe_route_topk", "moe_build_index", "moe_permute", "moe_unpermute_combine",
               "moe_group_precombine"):
        assert op in names


def test_library_exports_every_declared_symbol(capi):
    lib = capi.lib()
    names = declared_functions()
    assert set(names) == set(capi.SIGNATURES)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(capi):
    assert capi.status_string(0) == "ok"
    assert "invalid" in capi.status_string(1)
    assert capi.status_string(99) == "unknown status"


def test_library_capacity_matches_the_pages_example(capi):
    g = load_golden("capacity_example.json")
    lib = capi.lib()
    assert lib.moe_expert_capacity(g["tokens_per_rank"], g["top_k"], g["num_experts"], 5, 4) == g["capacity"]
    assert lib.moe_expert_capacity(8192, 8, 128, 5, 4) == 640
    assert lib.moe_expert_capacity(-1, 8, 128, 5, 4) == -1
    assert lib.moe_expert_capacity(8, 0, 128, 5, 4) == -1


def test_workspace_size_and_limits(capi):
    lib = capi.lib()
    n = ctypes.c_size_t(0)
    assert lib.moe_build_index_workspace_size(16384, 8, 256, 0, ctypes.byref(n)) == capi.MOE_OK
    assert n.value == 128 * 256 * 4  # one row of expert counts per tile, 128 tiles
    assert lib.moe_build_index_workspace_size(16384, 8, 256, 8, ctypes.byref(n)) == capi.MOE_OK
    assert n.value == 128 * 256 * 4 + 128 * 32 * 4  # and one row of group counts per tile
    assert lib.moe_build_index_workspace_size(16, 8, 4, 0, ctypes.byref(n)) == capi.MOE_ERR_INVALID  # K > E
    assert lib.moe_build_index_workspace_size(16, 2, 2048, 0, ctypes.byref(n)) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_build_index_workspace_size(16, 2, 12, 5, ctypes.byref(n)) == capi.MOE_ERR_INVALID
    assert lib.moe_build_index_workspace_size(0, 2, 8, 0, ctypes.byref(n)) == capi.MOE_OK
    assert n.value == 0  # no tokens, no tiles


def test_argument_errors_return_before_any_launch(capi):
    lib = capi.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert lib.moe_route_topk(fake, 4, 8, 9, fake, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_route_topk(fake, 4, 2048, 2, fake, fake, None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(fake, 4, 64, 33, fake, fake, None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(None, 4, 8, 2, fake, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == capi.MOE_OK  # empty: no-op
    assert lib.moe_route_topk_grouped(fake, 4, 16, 2, 3, 2, fake, fake, None) == capi.MOE_ERR_INVALID  # 3 does not divide 16
    assert lib.moe_route_topk_grouped(fake, 4, 16, 2, 4, 5, fake, fake, None) == capi.MOE_ERR_INVALID  # 5 of 4 groups
    assert lib.moe_route_topk_grouped(fake, 4, 16, 9, 4, 2, fake, fake, None) == capi.MOE_ERR_INVALID  # K > 2*4
    assert lib.moe_route_topk_grouped(fake, 4, 16, 2, 4, 0, fake, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_route_topk_grouped(fake, 4, 1024, 2, 2, 4, fake, fake, None) == capi.MOE_ERR_UNSUPPORTED  # 512 groups
    assert lib.moe_route_topk_grouped(None, 0, 16, 2, 4, 2, None, None, None) == capi.MOE_OK
    assert lib.moe_permute(fake, 4, 0, 1, fake, 4, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_permute(fake, 4, 8, 7, fake, 4, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_permute(None, 0, 8, 1, None, 0, None, None) == capi.MOE_OK
    assert lib.moe_unpermute_combine(fake, 1, 4, 8, fake, None, None, 2, 0, fake, 1, None) == capi.MOE_ERR_INVALID
    assert lib.moe_unpermute_combine(fake, 1, 4, 8, fake, None, None, 2, 2000, fake, 1, None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_unpermute_combine(fake, 1, 4, 8, None, None, None, 2, 2, fake, 1, None) == capi.MOE_ERR_INVALID
    assert lib.moe_unpermute_combine(fake, 2, 4, 8, fake, None, None, 2, 2, fake, 1, None) == \
        capi.MOE_ERR_UNSUPPORTED  # the combine does not take FP8 rows
    assert lib.moe_group_precombine(fake, 1, 4, 8, fake, None, fake, 2, 2, 8, 3, fake, 4, fake, 0, None) == \
        capi.MOE_ERR_INVALID
    assert lib.moe_group_precombine(fake, 1, 4, 8, fake, None, fake, 2, 2, 8, 2, fake, 4, fake, 7, None) == \
        capi.MOE_ERR_INVALID  # partials neither float32 nor bf16
    assert lib.moe_group_precombine(fake, 1, 4, 8, fake, None, fake, 2, 2, 8, 2, fake, 4, fake, 2, None) == \
        capi.MOE_ERR_UNSUPPORTED  # no FP8 partials
    assert lib.moe_permute_grouped(fake, 4, 8, 1, fake, 4, fake, 2, 65, None, fake, None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_permute_grouped(fake, 4, 8, 1, None, 4, fake, 2, 2, None, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_permute_grouped(fake, 4, 8, 1, fake, 4, None, 2, 2, None, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_permute_grouped(fake, 4, 8, 1, fake, 4, fake, -1, 2, None, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_permute_grouped(None, 0, 8, 1, None, 0, None, 0, 2, None, None, None) == capi.MOE_OK
    # the FP8 group receive: block must divide H, the scale buffers are needed, the rest as moe_permute_grouped
    assert lib.moe_permute_grouped_fp8(fake, fake, 4, 100, 30, fake, 4, fake, 2, 2, None, fake, fake, None) == \
        capi.MOE_ERR_INVALID
    assert lib.moe_permute_grouped_fp8(fake, fake, 4, 128, 0, fake, 4, fake, 2, 2, None, fake, fake, None) == \
        capi.MOE_ERR_INVALID
    assert lib.moe_permute_grouped_fp8(fake, None, 4, 128, 128, fake, 4, fake, 2, 2, None, fake, fake, None) == \
        capi.MOE_ERR_INVALID
    assert lib.moe_permute_grouped_fp8(fake, fake, 4, 128, 128, fake, 4, fake, 2, 2, None, fake, None, None) == \
        capi.MOE_ERR_INVALID
    assert lib.moe_permute_grouped_fp8(fake, fake, 4, 128, 128, fake, 4, fake, 2, 65, None, fake, fake, None) == \
        capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_permute_grouped_fp8(fake, fake, 4, 128, 128, None, 4, fake, 2, 2, None, fake, fake, None) == \
        capi.MOE_ERR_INVALID
    assert lib.moe_permute_grouped_fp8(None, None, 0, 128, 128, None, 0, None, 0, 2, None, None, None, None) == \
        capi.MOE_OK
    assert lib.moe_route_topk_backward(fake, fake, fake, 4, 8, 9, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_route_topk_backward(fake, fake, fake, 4, 2048, 2, fake, None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk_backward(fake, None, fake, 4, 8, 2, fake, None) == capi.MOE_ERR_INVALID
    assert lib.moe_route_topk_backward(None, None, None, 0, 8, 2, None, None) == capi.MOE_OK
    assert lib.moe_unpermute_combine_backward(fake, 1, fake, 1, 4, 8, fake, None, 2, 2000, None, fake, 1, None,
                                              None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_unpermute_combine_backward(None, 1, fake, 1, 4, 8, fake, None, 2, 2, None, fake, 1, None,
                                              None) == capi.MOE_ERR_INVALID
    assert lib.moe_unpermute_combine_backward(fake, 1, None, 1, 4, 8, fake, None, 2, 2, None, fake, 1, fake,
                                              None) == capi.MOE_ERR_INVALID  # dw needs y
    assert lib.moe_unpermute_combine_backward(fake, 7, fake, 1, 4, 8, fake, None, 2, 2, None, fake, 1, None,
                                              None) == capi.MOE_ERR_INVALID
    assert lib.moe_unpermute_combine_backward(None, 1, None, 1, 4, 8, None, None, 0, 2, None, None, 1, None,
                                              None) == capi.MOE_OK  # no tokens, no gather map: nothing to do
    assert lib.moe_quantize_fp8(fake, 1, 4, 100, 30, fake, fake, None) == capi.MOE_ERR_INVALID  # 30 does not divide 100
    assert lib.moe_quantize_fp8(fake, 2, 4, 128, 128, fake, fake, None) == capi.MOE_ERR_UNSUPPORTED  # FP8 input
    assert lib.moe_quantize_fp8(None, 1, 0, 128, 128, None, None, None) == capi.MOE_OK
    assert lib.moe_permute_scatter_fp8(fake, 1, 4, 384, 96, fake, 2, None, 8, fake, fake, None) == \
        capi.MOE_ERR_UNSUPPORTED  # block not a power of two
    assert lib.moe_permute_scatter_fp8(fake, 1, 4, 4096, 2048, fake, 2, None, 8, fake, fake, None) == \
        capi.MOE_ERR_UNSUPPORTED  # block above 1024
    assert lib.moe_permute_scatter_fp8(fake, 1, 4, 128, 128, fake, 2, None, 8, None, fake, None) == \
        capi.MOE_ERR_INVALID
    assert lib.moe_permute(fake, 4, 8, 2, None, 4, fake, None) == capi.MOE_ERR_INVALID  # FP8 rows: map needed
    # hidden rows longer than 2^31 - 1 bytes are refused (buffer resources address a row in 32 bits)
    big = 1 << 30
    assert lib.moe_permute(fake, 4, big, 1, fake, 4, fake, None) == capi.MOE_ERR_UNSUPPORTED  # bf16: 2 GiB rows
    assert lib.moe_permute(fake, 4, big // 2, 0, fake, 4, fake, None) == capi.MOE_ERR_UNSUPPORTED  # f32
    assert lib.moe_permute_scatter(fake, 4, big, 1, fake, 2, None, 8, fake, None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_permute_scatter(fake, 4, 8, 1, fake, 1025, None, 8, fake, None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_permute_scatter_fp8(fake, 1, 4, 128, 128, fake, 1025, None, 8, fake, fake, None) == \
        capi.MOE_ERR_UNSUPPORTED  # more destination columns than experts
    assert lib.moe_permute_grouped(fake, 4, big, 1, fake, 4, fake, 2, 2, None, fake, None) == capi.MOE_ERR_UNSUPPORTED
    assert lib.moe_unpermute_combine(fake, 1, 4, big // 2, fake, None, None, 2, 2, fake, 0, None) == \
        capi.MOE_ERR_UNSUPPORTED  # float32 output rows of 2 GiB
    assert lib.moe_group_precombine(fake, 1, 4, big // 2, fake, None, fake, 2, 2, 8, 2, fake, 4, fake, 0, None) == \
        capi.MOE_ERR_UNSUPPORTED  # float32 partial rows of 2 GiB
    ix = capi.MoeIndexStruct()
    assert lib.moe_build_index(fake, None, 4, 2, 8, 4, 2, 0, ctypes.byref(ix), fake, 1 << 20, None) == \
        capi.MOE_ERR_UNSUPPORTED  # drop-and-pad with groups
    assert lib.moe_build_index(fake, None, 4, 2, 8, 0, 0, 0, ctypes.byref(ix), fake, 1 << 20, None) == \
        capi.MOE_ERR_INVALID  # null outputs
    assert lib.moe_build_index(fake, None, 4, 2, 8, 0, 0, 0, None, fake, 1 << 20, None) == capi.MOE_ERR_INVALID
    assert lib.moe_build_index(fake, None, 4, 2, 8, 4, 0, 128, ctypes.byref(ix), fake, 1 << 20, None) == \
        capi.MOE_ERR_UNSUPPORTED  # drop-and-pad with alignment
    assert lib.moe_build_index(fake, None, 4, 2, 8, 0, 0, -3, ctypes.byref(ix), fake, 1 << 20, None) == \
        capi.MOE_ERR_INVALID
    # the allocation-free index build checks the same arguments before any HIP call
    assert lib.moe_build_index_noalloc(fake, None, 4, 2, 8, 4, 2, 0, ctypes.byref(ix), None) == \
        capi.MOE_ERR_UNSUPPORTED  # drop-and-pad with groups
    assert lib.moe_build_index_noalloc(fake, None, 4, 2, 8, 0, 0, 0, ctypes.byref(ix), None) == \
        capi.MOE_ERR_INVALID  # null outputs
    assert lib.moe_build_index_noalloc(fake, None, 4, 2, 8, 0, 0, 0, None, None) == capi.MOE_ERR_INVALID
    assert lib.moe_build_index_noalloc(fake, None, 4, 9, 8, 0, 0, 0, ctypes.byref(ix), None) == \
        capi.MOE_ERR_INVALID  # K > E
    assert lib.moe_build_index_noalloc(fake, None, 4, 2, 2048, 0, 0, 0, ctypes.byref(ix), None) == \
        capi.MOE_ERR_UNSUPPORTED  # more experts than the kernels take
    assert lib.moe_build_index_noalloc(fake, None, 4, 2, 12, 0, 5, 0, ctypes.byref(ix), None) == \
        capi.MOE_ERR_INVALID  # group size not dividing E
    # rows of the expert-major arrays
    assert lib.moe_index_rows(16384, 8, 256, 0, 0) == 16384 * 8
    assert lib.moe_index_rows(16384, 8, 256, 0, 128) == 16384 * 8 + 256 * 127
    assert lib.moe_index_rows(8192, 8, 128, 640, 0) == 128 * 640
    assert lib.moe_index_rows(8192, 8, 128, 640, 128) == -1
    assert lib.moe_index_rows(1 << 30, 8, 8, 0, 0) == -1


def test_route_topk_index_sizes_and_argument_errors(capi):
    """moe_route_topk_index: its workspace (the fused route's tile counts, a multiple of 64 tokens
    per tile and at most 256 tiles, where the index build counts tiles; otherwise the index build's
    own), and every argument error of either of its two calls returned before any launch."""
    lib = capi.lib()
    n = ctypes.c_size_t(0)
    assert lib.moe_route_topk_index_workspace_size(16384, 8, 256, 0, ctypes.byref(n)) == capi.MOE_OK
    assert n.value == 256 * 256 * 4  # 64-token tiles
    assert lib.moe_route_topk_index_workspace_size(8192, 8, 256, 8, ctypes.byref(n)) == capi.MOE_OK
    assert n.value == 128 * (256 + 32) * 4
    assert lib.moe_route_topk_index_workspace_size(1 << 20, 8, 256, 0, ctypes.byref(n)) == capi.MOE_OK
    assert n.value == 256 * 256 * 4  # 4096-token tiles
    small = ctypes.c_size_t(0)
    assert lib.moe_build_index_workspace_size(2048, 8, 256, 0, ctypes.byref(small)) == capi.MOE_OK
    assert lib.moe_route_topk_index_workspace_size(2048, 8, 256, 0, ctypes.byref(n)) == capi.MOE_OK
    assert n.value == small.value  # 16384 slots: the index build counts no tiles
    assert lib.moe_route_topk_index_workspace_size(16, 8, 4, 0, ctypes.byref(n)) == capi.MOE_ERR_INVALID
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    ix = capi.MoeIndexStruct()
    for name, _ in capi.MoeIndexStruct._fields_:
        setattr(ix, name, fake.value)
    ok_ws = 1 << 20

    def call(logits, T, E, K, rgs, m, cap, gs, align, ws=fake, ws_bytes=ok_ws, out=ix):
        return lib.moe_route_topk_index(logits, T, E, K, rgs, m, fake, fake, cap, gs, align,
                                        ctypes.byref(out) if out is not None else None, ws, ws_bytes, None)

    assert call(fake, 4, 8, 9, 0, 0, 0, 0, 0) == capi.MOE_ERR_INVALID  # K > E
    assert call(fake, 4, 16, 2, 3, 2, 0, 0, 0) == capi.MOE_ERR_INVALID  # route groups of 3 in 16 experts
    assert call(fake, 4, 16, 2, 4, 5, 0, 0, 0) == capi.MOE_ERR_INVALID  # 5 of 4 route groups
    assert call(fake, 4, 2048, 2, 0, 0, 0, 0, 0) == capi.MOE_ERR_UNSUPPORTED
    assert call(fake, 4, 16, 2, 0, 0, 0, 3, 0) == capi.MOE_ERR_INVALID  # index groups of 3
    assert call(fake, 4, 16, 2, 0, 0, 4, 4, 0) == capi.MOE_ERR_UNSUPPORTED  # capacity with groups
    assert call(fake, 4, 16, 2, 0, 0, 0, 0, -1) == capi.MOE_ERR_INVALID
    assert call(fake, 4, 16, 2, 0, 0, 0, 0, 0, out=None) == capi.MOE_ERR_INVALID
    assert call(None, 4, 16, 2, 0, 0, 0, 0, 0) == capi.MOE_ERR_INVALID  # no logits
    assert call(fake, 100000, 256, 8, 0, 0, 0, 0, 0, ws_bytes=16) == capi.MOE_ERR_INVALID  # workspace too small
    assert call(fake, 100000, 256, 8, 0, 0, 0, 0, 0, ws=ctypes.c_void_p(0x1004)) == capi.MOE_ERR_INVALID  # unaligned
