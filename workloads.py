"""Seeded synthetic inputs for the MoE token dispatch / unpermute-combine path.

This module only draws random numbers. It holds no step of the method: no top-k, no
softmax, no index build, no permute and no combine. Both the CPU oracle (under
``oracle/``) and the HIP path consume exactly the arrays produced here, so that the two
sides see the same input bits.

Recipe (one rule for every tensor)
----------------------------------
* A tensor of shape ``[rows, cols]`` is generated in blocks of ``BLOCK_ROWS`` rows.
  Block ``b`` (rows ``[b*BLOCK_ROWS, (b+1)*BLOCK_ROWS)``) is drawn with
  ``numpy.random.default_rng([*key, stream, b]).standard_normal((n, cols), float32)``.
  ``key`` is ``(cfg_id,)`` for the five named workloads and ``(1000, *case)`` for the
  small test cases; ``stream`` is 0 for router logits, 1 for hidden states ``x`` and 2
  for expert outputs ``y``.
* Router logits get an optional per-expert bias ``float32(log(p_e))`` with
  ``p_e = (e+1)^-s / sum_j (j+1)^-s`` (Zipf weights, computed in float64, expert ``e``
  has Zipf rank ``e+1``), added in float32. This skews the load: low ids are hot.
* bf16 tensors are the float32 draws rounded to bf16 with round-to-nearest-even and
  returned as their raw ``uint16`` bit patterns.

The named workloads (``WORKLOADS``) are the five configurations the path is measured
and checked on; sizes derived from routing (capacity, group slots) are not computed here.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK_ROWS = 1024

STREAM_LOGITS = 0
STREAM_HIDDEN = 1
STREAM_EXPERT_OUT = 2

# Named workloads. ``cf`` is the capacity factor as a fraction (numerator, denominator);
# ``group_size`` > 0 selects the group (dedup + pre-combine) mode; ``identity_experts``
# means the expert outputs are the permuted hidden states themselves.
WORKLOADS = {
    1: dict(name="route-permute-combine T1024 H512 E8 K2 fp32 identity-experts",
            T=1024, H=512, E=8, K=2, dtype="f32", zipf_s=None, group_size=0, cf=None,
            identity_experts=True),
    2: dict(name="route-permute-combine T4096 H4096 E64 K2 bf16",
            T=4096, H=4096, E=64, K=2, dtype="bf16", zipf_s=None, group_size=0, cf=None,
            identity_experts=False),
    3: dict(name="route-permute-combine T16384 H7168 E256 K8 bf16 zipf1.2",
            T=16384, H=7168, E=256, K=8, dtype="bf16", zipf_s=1.2, group_size=0, cf=None,
            identity_experts=False),
    4: dict(name="group-dedup-precombine T8192 H7168 E256(32x8) K8 bf16 zipf1.2",
            T=8192, H=7168, E=256, K=8, dtype="bf16", zipf_s=1.2, group_size=8, cf=None,
            identity_experts=False),
    5: dict(name="drop-and-pad T8192 H4096 E128 K8 bf16 zipf1.0 cf1.25",
            T=8192, H=4096, E=128, K=8, dtype="bf16", zipf_s=1.0, group_size=0, cf=(5, 4),
            identity_experts=False),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_blocks(key: tuple, stream: int, rows: int, cols: int, convert) -> np.ndarray:
    """Draw ``[rows, cols]`` standard normals block by block and apply ``convert`` per block."""
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    first = None
    out = None

    def one(b: int):
        lo = b * BLOCK_ROWS
        n = min(BLOCK_ROWS, rows - lo)
        g = np.random.default_rng([*key, stream, b])
        return lo, convert(g.standard_normal((n, cols), dtype=np.float32))

    if nblk == 0:
        return convert(np.zeros((0, cols), np.float32))
    lo, first = one(0)
    out = np.empty((rows, cols), dtype=first.dtype)
    out[: first.shape[0]] = first
    if nblk > 1:
        def fill(b):
            lo, blk = one(b)
            out[lo: lo + blk.shape[0]] = blk
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(1, nblk)))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _as_dtype(dtype: str):
    if dtype == "f32":
        return lambda f: f
    if dtype == "bf16":
        return f32_to_bf16_bits
    raise ValueError(f"unknown dtype {dtype!r}")


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Per-expert logit bias float32(log p_e), p_e proportional to (e+1)^-s."""
    r = np.arange(1, E + 1, dtype=np.float64) ** (-float(s))
    return np.log(r / r.sum()).astype(np.float32)


def router_logits(key: tuple, T: int, E: int, zipf_s=None) -> np.ndarray:
    z = _normal_blocks(key, STREAM_LOGITS, T, E, lambda f: f)
    if zipf_s is not None:
        z = (z + zipf_bias(E, zipf_s)[None, :]).astype(np.float32)
    return np.ascontiguousarray(z)


def hidden_states(key: tuple, T: int, H: int, dtype: str) -> np.ndarray:
    return _normal_blocks(key, STREAM_HIDDEN, T, H, _as_dtype(dtype))


def expert_outputs(key: tuple, rows: int, H: int, dtype: str) -> np.ndarray:
    return _normal_blocks(key, STREAM_EXPERT_OUT, rows, H, _as_dtype(dtype))


def workload_key(cfg_id: int, seed=None) -> tuple:
    """Key of a named workload: (cfg_id,) for its fixed draw, (cfg_id, 2000 + seed) for another
    draw of the same shapes and distributions (disjoint from the fixed keys and the test cases)."""
    return (int(cfg_id),) if seed is None else (int(cfg_id), 2000 + int(seed))


def case_key(*case: int) -> tuple:
    """Key of a small ad-hoc test case; disjoint from the named workloads."""
    return (1000, *[int(c) for c in case])


def random_topk_ids(key: tuple, T: int, E: int, K: int, p_missing: float = 0.0) -> np.ndarray:
    """Distinct expert ids per token drawn uniformly, with a fraction of slots set to -1.

    Used by tests that feed the index build directly (without routing)."""
    g = np.random.default_rng([*key, 7])
    ids = np.argsort(g.random((T, E)), axis=1)[:, :K].astype(np.int32)
    if p_missing > 0:
        ids[g.random((T, K)) < p_missing] = -1
    return np.ascontiguousarray(ids)


def random_weights(key: tuple, T: int, K: int) -> np.ndarray:
    g = np.random.default_rng([*key, 8])
    return np.ascontiguousarray(g.random((T, K), dtype=np.float32))
