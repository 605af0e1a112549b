"""The all-cores leg of the CPU baseline (oracle.parallel) gives, bit for bit, what one call of
each oracle function gives: every function split over token or row ranges on several threads,
in the standard, drop-and-pad, aligned and group layouts, float32 and bf16."""
import numpy as np
import pytest

import oracle
import workloads as wl
from oracle.parallel import Pool, Serial, cpu_model, default_threads, usable_cores


def same(a, b):
    return a.shape == b.shape and np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


@pytest.fixture(scope="module", params=["pool", "serial"])
def pool(request):
    with (Pool(threads=5) if request.param == "pool" else Serial()) as p:
        yield p


@pytest.mark.parametrize("mode,dt", [("standard", "bf16"), ("drop", "bf16"), ("aligned", "f32"), ("group", "bf16"),
                                     ("group", "f32"), ("limited", "bf16")])
def test_parallel_oracle_equals_single_call(pool, mode, dt):
    T, H, E, K = 701, 136, 32, 4
    key = wl.case_key(500, len(mode), len(dt))
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    gs = 4 if mode in ("group", "limited") else 0
    rg = 3 if mode == "limited" else 0
    idx, w = oracle.route_topk_grouped(logits, K, gs, rg) if rg else oracle.route_topk(logits, K)
    pidx, pw = pool.route_topk(logits, K, group_size=gs, topk_groups=rg)
    assert same(pidx, idx) and same(pw, w)
    cap = oracle.capacity(T, K, E, 1, 2) if mode == "drop" else 0
    align = 16 if mode == "aligned" else 0
    ix = oracle.build_index(idx, w, E, capacity=cap, group_size=gs, alignment=align)
    x = wl.hidden_states(key, T, H, dt)
    rows = len(ix["sorted_indices"])
    live = ix["sorted_indices"] != -2
    out_np = np.uint16 if dt == "bf16" else np.float32
    if gs:
        n = int(ix["n_slots"][0])
        g1 = oracle.permute(x, ix["gsrc"])
        assert same(pool.permute(x, ix["gsrc"]), g1)
        assert same(pool.permute(g1, ix["esrc"])[live], oracle.permute(g1, ix["esrc"])[live])
    else:
        assert same(pool.permute(x, ix["sorted_indices"])[live], oracle.permute(x, ix["sorted_indices"])[live])
    y = wl.expert_outputs(key, rows, H, dt)
    if gs:
        for p_dt in (np.float32, np.uint16):
            p1 = oracle.group_precombine(y, ix["row_of"], w, idx, E, gs, ix["slot_of"], n, out_dtype=p_dt)
            p2 = pool.group_precombine(y, ix["row_of"], w, idx, E, gs, ix["slot_of"], n, out_dtype=p_dt)
            assert same(p2, p1)
            assert same(pool.unpermute_combine(p1, ix["slot_of"], None, out_np),
                        oracle.unpermute_combine(p1, ix["slot_of"], None, out_np))
    assert same(pool.unpermute_combine(y, ix["row_of"], w, out_np), oracle.unpermute_combine(y, ix["row_of"], w, out_np))
    dout = wl.expert_outputs((*key, 7), T, H, dt)
    dy1, dw1 = oracle.combine_backward(dout, y, ix["row_of"], w, out_np)
    dy2, dw2 = pool.combine_backward(dout, y, ix["row_of"], w, out_np)
    assert same(dy2, dy1) and same(dw2, dw1)
    assert same(pool.route_topk_backward(idx, w, dw1, E), oracle.route_topk_backward(idx, w, dw1, E))
    if H % 8 == 0:
        q1, s1 = oracle.quantize_fp8(x, 8)
        q2, s2 = pool.quantize_fp8(x, 8)
        assert same(q2, q1) and same(s2, s1)


def test_parallel_oracle_edge_sizes():
    """No tokens, fewer tokens than threads, one thread."""
    with Pool(threads=8) as p:
        for T in (0, 1, 3):
            logits = wl.router_logits(wl.case_key(501, T), T, 8)
            idx, w = oracle.route_topk(logits, 2)
            pi, pw = p.route_topk(logits, 2)
            assert same(pi, idx) and same(pw, w)
            y = wl.expert_outputs(wl.case_key(501, T), 2 * T, 16, "bf16")
            ix = oracle.build_index(idx, w, 8)
            assert same(p.unpermute_combine(y, ix["row_of"], w, np.uint16),
                        oracle.unpermute_combine(y, ix["row_of"], w, np.uint16))
    with Pool(threads=1) as p:
        logits = wl.router_logits(wl.case_key(502), 50, 8)
        assert same(p.route_topk(logits, 3)[0], oracle.route_topk(logits, 3)[0])


def test_host_description():
    assert 1 <= default_threads() <= 16
    assert usable_cores() >= 1
    assert isinstance(cpu_model(), str) and cpu_model()
