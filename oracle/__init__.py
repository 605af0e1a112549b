"""CPU oracle for the MoE token dispatch / unpermute-combine path (ctypes shim over moe_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package. The HIP product path never does, and the two share
no code.

All functions take and return numpy arrays. bf16 tensors are ``uint16`` bit patterns.
Each wrapper documents the passage of the source pages it follows in ``moe_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build as _build, library_path

F32 = 0
BF16 = 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    src = os.path.join(os.path.dirname(path), "moe_oracle.c")
    if not os.path.exists(path) or os.path.getmtime(src) > os.path.getmtime(path):
        _build()
    _lib = _declare(ctypes.CDLL(path))
    return _lib


def use_library(path):
    """Test hook: route every call to the oracle library at `path` (None restores the default).
    The mutation tests use it to check that the pins catch deliberately broken oracles."""
    global _lib
    _lib = None if path is None else _declare(ctypes.CDLL(path))


def _declare(lib):
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.oracle_capacity.argtypes = [i64, i32, i32, i32, i32]
    lib.oracle_capacity.restype = i64
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_route_topk.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_route_topk.restype = ctypes.c_int
    lib.oracle_build_index.argtypes = [P, P, i64, i32, i32, i32, i32, i32] + [P] * 12
    lib.oracle_build_index.restype = ctypes.c_int
    lib.oracle_permute.argtypes = [P, i64, i64, i32, P, i64, P]
    lib.oracle_permute.restype = ctypes.c_int
    lib.oracle_unpermute_combine.argtypes = [P, i32, i64, i64, P, P, P, i64, i32, P, i32]
    lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f32.restype = ctypes.c_float
    lib.oracle_quantize_fp8.argtypes = [P, i32, i64, i64, i32, P, P]
    lib.oracle_quantize_fp8.restype = ctypes.c_int
    lib.oracle_unpermute_combine.restype = ctypes.c_int
    lib.oracle_group_precombine.argtypes = [P, i32, i64, i64, P, P, P, i64, i32, i32, i32, P, i64, P, i32]
    lib.oracle_route_topk_grouped.argtypes = [P, i64, i32, i32, i32, i32, P, P]
    lib.oracle_route_topk_grouped.restype = ctypes.c_int
    lib.oracle_combine_backward.argtypes = [P, i32, P, i32, i64, i64, P, P, i64, i32, P, i32, P]
    lib.oracle_combine_backward.restype = ctypes.c_int
    lib.oracle_route_topk_backward.argtypes = [P, P, P, i64, i32, i32, P]
    lib.oracle_route_topk_backward.restype = ctypes.c_int
    lib.oracle_group_precombine.restype = ctypes.c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def _dt_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"hidden tensors must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _poisoned(shape, dtype) -> np.ndarray:
    """Output buffer pre-filled with a NaN pattern, so that an entry the oracle forgets to write
    shows up in the pins instead of passing as a fresh page's zeros."""
    a = np.empty(shape, dtype)
    a.view(np.uint8)[...] = 0xFF
    return a


def _out(out, shape, dtype, what) -> np.ndarray:
    """The caller's output array (written in place: a C-contiguous array of exactly this shape and
    dtype, e.g. a slice of rows of a larger one), or a fresh poisoned one."""
    if out is None:
        return _poisoned(shape, dtype)
    if out.shape != tuple(shape) or out.dtype != np.dtype(dtype) or not out.flags.c_contiguous:
        raise ValueError(f"{what}: out must be a C-contiguous {np.dtype(dtype)} array of shape {tuple(shape)}")
    return out


def capacity(tokens: int, top_k: int, num_experts: int, cf_num: int, cf_den: int) -> int:
    """Expert capacity ceil(tokens*top_k/num_experts*cf), cf = cf_num/cf_den, exact."""
    v = _load().oracle_capacity(tokens, top_k, num_experts, cf_num, cf_den)
    if v < 0:
        raise ValueError("invalid capacity arguments")
    return int(v)


def f32_to_bf16(x: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(x)))


def route_topk(logits: np.ndarray, K: int):
    """Top-K experts per token (ties -> lower id) and softmax over the K selected logits."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.full((T, K), -7, np.int32)
    w = np.full((T, K), np.nan, np.float32)
    _check(_load().oracle_route_topk(_ptr(logits), T, E, K, _ptr(idx), _ptr(w)), "route_topk")
    return idx, w


def index_rows(T: int, K: int, E: int, capacity: int = 0, alignment: int = 0) -> int:
    """Rows of the expert-major buffer: E*cap with a capacity, T*K + E*(A-1) with alignment A."""
    if capacity > 0:
        return E * capacity
    return T * K + (E * (alignment - 1) if alignment > 1 else 0)


def route_topk_grouped(logits: np.ndarray, K: int, group_size: int, topk_groups: int):
    """Group-limited routing: the topk_groups groups with the best expert, then top-K inside them."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.full((T, K), -7, np.int32)
    w = np.full((T, K), np.nan, np.float32)
    _check(_load().oracle_route_topk_grouped(_ptr(logits), T, E, K, group_size, topk_groups, _ptr(idx), _ptr(w)),
           "route_topk_grouped")
    return idx, w


def build_index(topk_idx: np.ndarray, topk_w, E: int, capacity: int = 0, group_size: int = 0,
                alignment: int = 0):
    """Expert-major index (the dispatch "handle"). Returns a dict of numpy arrays."""
    topk_idx = _c(topk_idx, np.int32)
    T, K = topk_idx.shape
    w = None if topk_w is None else _c(topk_w, np.float32)
    rows = index_rows(T, K, E, capacity, alignment)
    out = dict(
        counts=np.zeros(E, np.int32),
        group_list=np.zeros(E, np.int32),
        kept_counts=np.zeros(E, np.int32),
        sorted_indices=np.full(rows, -7, np.int32),
        row_of=np.full((T, K), -7, np.int32),
        permuted_probs=np.full(rows, np.nan, np.float32),
    )
    g_arrays = [None] * 6
    if group_size > 0:
        G = E // group_size
        out.update(
            slot_of=np.full((T, G), -7, np.int32),
            gsrc=np.full(T * min(K, G), -7, np.int32),
            esrc=np.full(rows, -7, np.int32),
            group_counts=np.zeros(G, np.int32),
            n_slots=np.zeros(1, np.int32),
            slot_src=np.full((T, K), -7, np.int32),
        )
        g_arrays = [out["slot_of"], out["gsrc"], out["esrc"], out["group_counts"], out["n_slots"], out["slot_src"]]
    rc = _load().oracle_build_index(
        _ptr(topk_idx), _ptr(w), T, K, E, capacity, group_size, alignment,
        _ptr(out["counts"]), _ptr(out["group_list"]), _ptr(out["kept_counts"]),
        _ptr(out["sorted_indices"]), _ptr(out["row_of"]), _ptr(out["permuted_probs"]),
        *[_ptr(a) for a in g_arrays])
    _check(rc, "build_index")
    if group_size > 0:
        m = int(out["n_slots"][0])
        out["gsrc"] = out["gsrc"][:m]
    return out


def permute(src: np.ndarray, src_row: np.ndarray, out=None) -> np.ndarray:
    """dst[i] = src[src_row[i]] bitwise; rows outside [0, len(src)) give zeros, except -2
    (unused slack), which leaves the row as it is (here: the NaN poison, or out's contents)."""
    src = np.ascontiguousarray(src)
    if src.dtype != np.uint8:
        _dt_of(src)
    src_rows, H = src.shape
    src_row = _c(src_row, np.int32).reshape(-1)
    dst = _out(out, (src_row.shape[0], H), src.dtype, "permute")
    rc = _load().oracle_permute(_ptr(src), src_rows, H, src.dtype.itemsize, _ptr(src_row),
                                src_row.shape[0], _ptr(dst))
    _check(rc, "permute")
    return dst


def unpermute_combine(y: np.ndarray, row_of: np.ndarray, w, out_dtype, bias=None, out=None) -> np.ndarray:
    """out[t] = sum_k w[t,k] * y[row_of[t,k]] (float32 FMA chain in k order) [+ bias[t]]."""
    y = np.ascontiguousarray(y)
    y_dt = _dt_of(y)
    y_rows, H = y.shape
    row_of = _c(row_of, np.int32)
    T, K = row_of.shape
    w = None if w is None else _c(w, np.float32).reshape(T, K)
    out = _out(out, (T, H), out_dtype, "unpermute_combine")
    out_dt = _dt_of(out)
    if bias is not None:
        bias = np.ascontiguousarray(bias)
        assert bias.dtype == out.dtype and bias.shape == (T, H)
    rc = _load().oracle_unpermute_combine(_ptr(y), y_dt, y_rows, H, _ptr(row_of), _ptr(w), _ptr(bias),
                                          T, K, _ptr(out), out_dt)
    _check(rc, "unpermute_combine")
    return out


def group_precombine(y: np.ndarray, row_of, w, topk_idx, E: int, group_size: int,
                     slot_of: np.ndarray, slots_cap: int, out_dtype=np.float32, out=None) -> np.ndarray:
    """Per-(token, group) weighted partial sums (a float32 chain) stored at slot_of[t, g], as
    float32 or rounded once to bf16 (out_dtype np.uint16); rows slot_of does not name are left
    as they are (the poison, or out's contents)."""
    y = np.ascontiguousarray(y)
    y_dt = _dt_of(y)
    y_rows, H = y.shape
    row_of = _c(row_of, np.int32)
    T, K = row_of.shape
    topk_idx = _c(topk_idx, np.int32)
    w = None if w is None else _c(w, np.float32)
    slot_of = _c(slot_of, np.int32)
    partials = _out(out, (slots_cap, H), out_dtype, "group_precombine")
    rc = _load().oracle_group_precombine(_ptr(y), y_dt, y_rows, H, _ptr(row_of), _ptr(w),
                                         _ptr(topk_idx), T, K, E, group_size, _ptr(slot_of),
                                         slots_cap, _ptr(partials), _dt_of(partials))
    _check(rc, "group_precombine")
    return partials


def combine_backward(dout: np.ndarray, y: np.ndarray, row_of: np.ndarray, w, dy_dtype, want_dw: bool = True,
                     out=None):
    """Backward of the weighted combine: dy[row_of[t,k]] = w[t,k] * dout[t] (zero elsewhere),
    dw[t,k] = <dout[t], y[row_of[t,k]]> (double sum, rounded to float32). Returns (dy, dw|None);
    out = (dy, dw|None) writes into the caller's arrays."""
    dout = np.ascontiguousarray(dout)
    dout_dt = _dt_of(dout)
    y = np.ascontiguousarray(y)
    y_dt = _dt_of(y)
    y_rows, H = y.shape
    row_of = _c(row_of, np.int32)
    T, K = row_of.shape
    assert dout.shape == (T, H)
    w = None if w is None else _c(w, np.float32).reshape(T, K)
    dy = _out(None if out is None else out[0], (y_rows, H), dy_dtype, "combine_backward dy")
    dw = None
    if want_dw:
        dw = np.full((T, K), np.nan, np.float32) if out is None or out[1] is None else \
            _out(out[1], (T, K), np.float32, "combine_backward dw")
    rc = _load().oracle_combine_backward(_ptr(dout), dout_dt, _ptr(y), y_dt, y_rows, H, _ptr(row_of), _ptr(w),
                                         T, K, _ptr(dy), _dt_of(dy), _ptr(dw))
    _check(rc, "combine_backward")
    return dy, dw


def route_topk_backward(topk_idx: np.ndarray, topk_w: np.ndarray, d_topk_w: np.ndarray, E: int) -> np.ndarray:
    """Gradient of the logits through the softmax over the K selected logits (zero elsewhere)."""
    topk_idx = _c(topk_idx, np.int32)
    T, K = topk_idx.shape
    topk_w = _c(topk_w, np.float32).reshape(T, K)
    d_topk_w = _c(d_topk_w, np.float32).reshape(T, K)
    d_logits = np.full((T, E), np.nan, np.float32)
    rc = _load().oracle_route_topk_backward(_ptr(topk_idx), _ptr(topk_w), _ptr(d_topk_w), T, E, K, _ptr(d_logits))
    _check(rc, "route_topk_backward")
    return d_logits


def f32_to_e4m3(x: float) -> int:
    return int(_load().oracle_f32_to_e4m3(float(x)))


def e4m3_to_f32(c: int) -> float:
    return float(_load().oracle_e4m3_to_f32(int(c)))


def quantize_fp8(x: np.ndarray, block: int, out=None):
    """Per-(token, block) E4M3 quantization: returns (q uint8 [T, H], scales float32 [T, H/block]);
    out = (q, scales) writes into the caller's arrays."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    if out is None:
        q = np.full((T, H), 0x7F, np.uint8)
        scales = np.full((T, H // block if block > 0 else 0), np.nan, np.float32)
    else:
        q = _out(out[0], (T, H), np.uint8, "quantize_fp8 q")
        scales = _out(out[1], (T, H // block if block > 0 else 0), np.float32, "quantize_fp8 scales")
    _check(_load().oracle_quantize_fp8(_ptr(x), _dt_of(x), T, H, block, _ptr(q), _ptr(scales)), "quantize_fp8")
    return q, scales
