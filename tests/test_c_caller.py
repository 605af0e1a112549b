"""The C ABI used from plain C (tests/c/moe_c_caller.c): gcc builds it against the public header
and the library alone, with no Python or torch in the process.

- host (no GPU): the calls that launch nothing give the documented values and argument errors;
- GPU: the C program runs route -> index -> source-major permute -> combine on seeded inputs
  (T1000 H520 E64 K8 bf16, Zipf-skewed router logits) and its outputs match the oracle: indices
  and permuted rows bit for bit, weights within the float32 bound, combined rows within 1 bf16
  ulp.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle.compare import assert_combined, assert_exact, assert_rel_f32

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c"))
import build_caller  # noqa: E402


def test_c_caller_builds_and_checks_host_calls(tmp_path):
    exe = build_caller.build(str(tmp_path / "moe_c_caller"))
    r = subprocess.run([exe, "check"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"


@pytest.mark.gpu
def test_c_caller_runs_the_path_on_the_gpu(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    exe = build_caller.binary_path()
    assert os.path.exists(exe), "tests/c/moe_c_caller is missing: run __graft_entry__.build() first"
    T, H, E, K = 1000, 520, 64, 8
    key = wl.case_key(4343)
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    x = wl.hidden_states(key, T, H, "bf16")
    y = wl.expert_outputs(key, T * K, H, "bf16")
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.asarray([T, E, K, H], np.int64).tobytes())
        f.write(np.ascontiguousarray(logits, np.float32).tobytes())
        f.write(np.ascontiguousarray(x).tobytes())
        f.write(np.ascontiguousarray(y).tobytes())
    print(f"C caller T={T} H={H} E={E} K={K}", flush=True)
    r = subprocess.run([exe, "run", str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    R = T * K
    buf = open(dst, "rb").read()
    parts, off = {}, 0
    for name, dt, n in (("idx", np.int32, T * K), ("w", np.float32, T * K), ("counts", np.int32, E),
                        ("group_list", np.int32, E), ("sorted_indices", np.int32, R), ("row_of", np.int32, T * K),
                        ("permuted_probs", np.float32, R), ("xp", np.uint16, R * H), ("out", np.uint16, T * H)):
        size = np.dtype(dt).itemsize * n
        parts[name] = np.frombuffer(buf[off:off + size], dt)
        off += size
    assert off == len(buf)
    want_i, want_w = oracle.route_topk(logits, K)
    assert_exact(parts["idx"].reshape(T, K), want_i, "topk_idx")
    assert_rel_f32(parts["w"].reshape(T, K), want_w, "topk_w")
    w = parts["w"].reshape(T, K).copy()
    want = oracle.build_index(want_i, w, E)
    for name in ("counts", "group_list", "sorted_indices", "permuted_probs"):
        assert_exact(parts[name], want[name], name)
    assert_exact(parts["row_of"].reshape(T, K), want["row_of"], "row_of")
    assert_exact(parts["xp"].reshape(R, H), oracle.permute(x, want["sorted_indices"]), "permuted rows")
    assert_combined(parts["out"].reshape(T, H), oracle.unpermute_combine(y, want["row_of"], w, np.uint16), "combined")
