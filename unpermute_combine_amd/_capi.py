"""ctypes declarations of libmoe_dispatch.so (the C ABI in include/moe_dispatch.h)."""
from __future__ import annotations

import ctypes
import os

from .build import library_path

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, 1, 2, 3
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2

_P = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class MoeIndexStruct(ctypes.Structure):
    _fields_ = [(name, _P) for name in (
        "counts", "group_list", "kept_counts", "sorted_indices", "row_of", "permuted_probs",
        "slot_of", "gsrc", "esrc", "group_counts", "n_slots", "slot_src")]


# name -> (restype, argtypes); every symbol the header declares
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_expert_capacity": (_i64, [_i64, _i32, _i32, _i32, _i32]),
    "moe_route_topk": (ctypes.c_int, [_P, _i64, _i32, _i32, _P, _P, _P]),
    "moe_route_topk_grouped": (ctypes.c_int, [_P, _i64, _i32, _i32, _i32, _i32, _P, _P, _P]),
    "moe_build_index_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_build_index": (ctypes.c_int, [_P, _P, _i64, _i32, _i32, _i32, _i32, _i32,
                                       ctypes.POINTER(MoeIndexStruct), _P, ctypes.c_size_t, _P]),
    "moe_build_index_noalloc": (ctypes.c_int, [_P, _P, _i64, _i32, _i32, _i32, _i32, _i32,
                                               ctypes.POINTER(MoeIndexStruct), _P]),
    "moe_index_rows": (ctypes.c_int64, [_i64, _i32, _i32, _i32, _i32]),
    "moe_route_topk_index_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route_topk_index": (ctypes.c_int, [_P, _i64, _i32, _i32, _i32, _i32, _P, _P, _i32, _i32, _i32,
                                            ctypes.POINTER(MoeIndexStruct), _P, ctypes.c_size_t, _P]),
    "moe_permute": (ctypes.c_int, [_P, _i64, _i64, ctypes.c_int, _P, _i64, _P, _P]),
    "moe_permute_scatter": (ctypes.c_int, [_P, _i64, _i64, ctypes.c_int, _P, _i32, _P, _i64, _P, _P]),
    "moe_quantize_fp8": (ctypes.c_int, [_P, ctypes.c_int, _i64, _i64, _i32, _P, _P, _P]),
    "moe_permute_scatter_fp8": (ctypes.c_int, [_P, ctypes.c_int, _i64, _i64, _i32, _P, _i32, _P, _i64, _P, _P, _P]),
    "moe_permute_grouped": (ctypes.c_int, [_P, _i64, _i64, ctypes.c_int, _P, _i64, _P, _i64, _i32, _P, _P, _P]),
    "moe_permute_grouped_fp8": (ctypes.c_int, [_P, _P, _i64, _i64, _i32, _P, _i64, _P, _i64, _i32, _P, _P, _P, _P]),
    "moe_unpermute_combine_backward": (ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_int, _i64, _i64, _P, _P, _i64,
                                                      _i32, _P, _P, ctypes.c_int, _P, _P]),
    "moe_route_topk_backward": (ctypes.c_int, [_P, _P, _P, _i64, _i32, _i32, _P, _P]),
    "moe_unpermute_combine": (ctypes.c_int, [_P, ctypes.c_int, _i64, _i64, _P, _P, _P, _i64, _i32, _P,
                                             ctypes.c_int, _P]),
    "moe_group_precombine": (ctypes.c_int, [_P, ctypes.c_int, _i64, _i64, _P, _P, _P, _i64, _i32, _i32,
                                            _i32, _P, _i64, _P, ctypes.c_int, _P]),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {status_string(code)} (code {code})")


_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()' or python unpermute_combine_amd/build.py)")
    handle = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    _lib = handle
    return handle


def status_string(code: int) -> str:
    return lib().moe_status_string(code).decode()


def check(fn: str, code: int) -> None:
    if code != MOE_OK:
        raise MoeError(fn, code)
