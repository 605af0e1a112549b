"""Comparison rules of the GPU-vs-oracle parity checks (test infrastructure: used by the tests
and smoke() only).

Tolerances (the only ones used anywhere):
  * integers, indices, counts, permuted/padded rows: bit-exact;
  * router weights: relative error <= 1e-6;
  * combined outputs: float32 |a-b| <= 1e-6 * max(|b|, FLT_MIN); bf16 at most 1 unit in the last
    place (distance of the bit patterns on the ordered-integer line).
The combine and pre-combine use the same weight bits on both sides, so equality is expected
and the tolerance is slack.
"""
from __future__ import annotations

import numpy as np

FLT_MIN = np.float32(np.finfo(np.float32).tiny)


def bf16_ordered(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))


def assert_exact(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    if not np.array_equal(got.view(np.uint8) if got.dtype.kind == "f" else got,
                          want.view(np.uint8) if want.dtype.kind == "f" else want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} entries differ, first at {bad[:5].tolist()}")


def assert_rel_f32(got: np.ndarray, want: np.ndarray, what: str, rtol: float = 1e-6):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    lim = rtol * np.maximum(np.abs(want.astype(np.float64)), float(FLT_MIN))
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} values beyond rel {rtol}, first at {i}")


def assert_combined(got: np.ndarray, want: np.ndarray, what: str):
    """Combined outputs: float32 rel 1e-6, bf16 (uint16 bits) 1 ulp."""
    if want.dtype == np.uint16:
        d = bf16_ulp_distance(got, want)
        if (d > 1).any():
            raise AssertionError(f"{what}: {int((d > 1).sum())} bf16 values more than 1 ulp apart, "
                                 f"max {int(d.max())}")
    else:
        assert_rel_f32(got, want, what)


def exact_fraction(got: np.ndarray, want: np.ndarray) -> float:
    """Share of entries that are bit-identical (reported; equality is expected)."""
    g = np.asarray(got).view(np.uint8).reshape(np.asarray(got).shape + (-1,))
    w = np.asarray(want).view(np.uint8).reshape(np.asarray(want).shape + (-1,))
    return float(np.all(g == w, axis=-1).mean()) if g.size else 1.0
