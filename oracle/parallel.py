"""The oracle's token- and row-independent functions run over slices on host threads.

TEST INFRASTRUCTURE: the all-cores leg of ``bench.py``'s CPU baseline, and its tests. Every call
below is one of the oracle's own functions applied to a contiguous range of tokens (routing, the
combine, the pre-combine, the backward of the routing softmax, the FP8 quantization) or of
output rows (the permute, the combine's backward), writing into disjoint slices of one output
array. The oracle computes each token's or each row's result from that token or row alone, so
the result is bit for bit that of one call over everything; only the wall-clock time changes.
The index build is not split: its scan over the routing map defines the row order.

The threads run concurrently because ctypes releases the interpreter lock for the duration of
each foreign call.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import (combine_backward, group_precombine, permute, quantize_fp8, route_topk, route_topk_backward,
               route_topk_grouped, unpermute_combine)

# worker threads at most: the share of a one-GPU machine's host CPUs that its jobs may use
MAX_THREADS = 16


def usable_cores() -> int:
    """Host CPUs this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def default_threads() -> int:
    return max(1, min(MAX_THREADS, usable_cores()))


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _ranges(n: int, pieces: int):
    """Contiguous [a, b) ranges covering [0, n), at most `pieces` of them."""
    pieces = max(1, min(pieces, n))
    step = -(-n // pieces) if n else 1
    return [(a, min(a + step, n)) for a in range(0, n, step)]


class Pool:
    """A fixed set of host threads; each method splits its work into slices (four per thread)."""

    def __init__(self, threads: int | None = None):
        self.threads = threads or default_threads()
        self._ex = ThreadPoolExecutor(self.threads)

    def close(self):
        self._ex.shutdown()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _run(self, n: int, fn):
        list(self._ex.map(lambda ab: fn(*ab), _ranges(n, 4 * self.threads)))

    def route_topk(self, logits: np.ndarray, K: int, group_size: int = 0, topk_groups: int = 0):
        logits = np.ascontiguousarray(logits, np.float32)
        T = logits.shape[0]
        idx = np.empty((T, K), np.int32)
        w = np.empty((T, K), np.float32)

        def one(a, b):
            if topk_groups:
                i, ww = route_topk_grouped(logits[a:b], K, group_size, topk_groups)
            else:
                i, ww = route_topk(logits[a:b], K)
            idx[a:b], w[a:b] = i, ww

        self._run(T, one)
        return idx, w

    def permute(self, src: np.ndarray, src_row: np.ndarray, out=None) -> np.ndarray:
        src_row = np.ascontiguousarray(src_row, np.int32).reshape(-1)
        N = src_row.shape[0]
        if out is None:
            out = np.empty((N, src.shape[1]), src.dtype)
        self._run(N, lambda a, b: permute(src, src_row[a:b], out=out[a:b]))
        return out

    def unpermute_combine(self, y: np.ndarray, row_of: np.ndarray, w, out_dtype, bias=None) -> np.ndarray:
        row_of = np.ascontiguousarray(row_of, np.int32)
        T = row_of.shape[0]
        w = None if w is None else np.ascontiguousarray(w, np.float32)
        out = np.empty((T, y.shape[1]), out_dtype)
        self._run(T, lambda a, b: unpermute_combine(y, row_of[a:b], None if w is None else w[a:b], out_dtype,
                                                    bias=None if bias is None else bias[a:b], out=out[a:b]))
        return out

    def group_precombine(self, y, row_of, w, topk_idx, E, group_size, slot_of, slots_cap,
                         out_dtype=np.float32) -> np.ndarray:
        """Token ranges write the partial rows their (token, group) slots name: disjoint rows of
        one array."""
        row_of = np.ascontiguousarray(row_of, np.int32)
        topk_idx = np.ascontiguousarray(topk_idx, np.int32)
        slot_of = np.ascontiguousarray(slot_of, np.int32)
        w = None if w is None else np.ascontiguousarray(w, np.float32)
        out = np.empty((slots_cap, y.shape[1]), out_dtype)
        self._run(row_of.shape[0], lambda a, b: group_precombine(
            y, row_of[a:b], None if w is None else w[a:b], topk_idx[a:b], E, group_size, slot_of[a:b], slots_cap,
            out_dtype=out_dtype, out=out))
        return out

    def combine_backward(self, dout, y, row_of, w, dy_dtype, want_dw: bool = True):
        """Split by rows of dy: the slice [r0, r1) sees y[r0:r1] and row_of shifted by r0, so that
        it writes (and zero-fills) exactly its own rows of dy and computes dw for the slots whose
        row lies in it; each slot's dw is taken from the slice that owns its row (the others
        report 0 for it)."""
        row_of = np.ascontiguousarray(row_of, np.int32)
        T, K = row_of.shape
        rows, H = y.shape
        dy = np.empty((rows, H), dy_dtype)
        dw = np.zeros((T, K), np.float32) if want_dw else None

        def one(r0, r1):
            local = row_of - np.int32(r0)  # rows outside [r0, r1) fall outside [0, r1 - r0): no term
            part = np.empty((T, K), np.float32) if want_dw else None
            combine_backward(dout, y[r0:r1], local, w, dy_dtype, want_dw=want_dw, out=(dy[r0:r1], part))
            if want_dw:
                own = (row_of >= r0) & (row_of < r1)
                dw[own] = part[own]

        self._run(rows, one)
        return dy, dw

    def route_topk_backward(self, topk_idx, topk_w, d_topk_w, E: int) -> np.ndarray:
        topk_idx = np.ascontiguousarray(topk_idx, np.int32)
        T = topk_idx.shape[0]
        out = np.empty((T, E), np.float32)

        def one(a, b):
            out[a:b] = route_topk_backward(topk_idx[a:b], topk_w[a:b], d_topk_w[a:b], E)

        self._run(T, one)
        return out

    def quantize_fp8(self, x: np.ndarray, block: int):
        T, H = x.shape
        q = np.empty((T, H), np.uint8)
        s = np.empty((T, H // block), np.float32)
        self._run(T, lambda a, b: quantize_fp8(x[a:b], block, out=(q[a:b], s[a:b])))
        return q, s


class Serial:
    """The same interface as Pool, every function called once over everything on this thread
    (the single-thread leg of the CPU baseline)."""

    threads = 1

    def close(self):
        pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        pass

    @staticmethod
    def route_topk(logits, K, group_size=0, topk_groups=0):
        if topk_groups:
            return route_topk_grouped(logits, K, group_size, topk_groups)
        return route_topk(logits, K)

    @staticmethod
    def permute(src, src_row, out=None):
        return permute(src, src_row, out=out)

    @staticmethod
    def unpermute_combine(y, row_of, w, out_dtype, bias=None):
        return unpermute_combine(y, row_of, w, out_dtype, bias=bias)

    @staticmethod
    def group_precombine(y, row_of, w, topk_idx, E, group_size, slot_of, slots_cap, out_dtype=np.float32):
        return group_precombine(y, row_of, w, topk_idx, E, group_size, slot_of, slots_cap, out_dtype=out_dtype)

    @staticmethod
    def combine_backward(dout, y, row_of, w, dy_dtype, want_dw=True):
        return combine_backward(dout, y, row_of, w, dy_dtype, want_dw=want_dw)

    @staticmethod
    def route_topk_backward(topk_idx, topk_w, d_topk_w, E):
        return route_topk_backward(topk_idx, topk_w, d_topk_w, E)

    @staticmethod
    def quantize_fp8(x, block):
        return quantize_fp8(x, block)
