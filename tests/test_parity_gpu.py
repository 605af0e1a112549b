"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Small cases span several tiles and ragged tails; edge cases cover empty inputs, experts and
groups with no tokens, slots that route nowhere, out-of-range ids and rows, capacities below
and above the largest count; the five named workloads run at full size through the same
entry points and launch configuration that bench.py times (every mode it offers: expert
alignment, group-limited routing, the FP8 dispatch, bf16 partials, the backward), with every
index entry, every dispatched row, every partial and every combined token compared with the
oracle on the same inputs.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from oracle.compare import assert_combined, assert_exact, assert_rel_f32, exact_fraction

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import unpermute_combine_amd as mod
    mod.lib()  # the HIP library must be there: no fallback
    return mod


DEV = "cuda:0"


def dev(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def say(*args):
    print(*args, flush=True)


# ------------------------------------------------------------------ routing


def tie_logits(key, T, E):
    g = np.random.default_rng([*key, 99])
    v = (g.integers(-6, 7, size=(T, E)) * 0.25).astype(np.float32)
    v[g.random((T, E)) < 0.1] = -0.0
    return v


@pytest.mark.parametrize("T,E,K,kind", [
    (1, 1, 1, "normal"), (37, 8, 2, "normal"), (1030, 64, 2, "normal"), (999, 256, 8, "zipf"),
    (130, 33, 5, "ties"), (77, 1000, 32, "normal"), (500, 1024, 8, "ties"), (64, 64, 32, "ties"),
    (301, 65, 1, "normal"), (200, 128, 8, "ties")])
def test_route_topk(m, T, E, K, kind):
    say(f"route_topk T={T} E={E} K={K} {kind}")
    key = wl.case_key(20, T, E, K)
    if kind == "ties":
        logits = tie_logits(key, T, E)
    else:
        logits = wl.router_logits(key, T, E, zipf_s=1.2 if kind == "zipf" else None)
    want_i, want_w = oracle.route_topk(logits, K)
    gi, gw = m.route_topk(dev(logits), K)
    torch.cuda.synchronize()
    assert_exact(host(gi), want_i, "topk_idx")
    assert_rel_f32(host(gw), want_w, "topk_w")


@pytest.mark.parametrize("T,E,K,gs,M", [(1000, 256, 8, 8, 4), (777, 64, 6, 8, 2), (500, 256, 8, 32, 1),
                                        (300, 16, 4, 4, 4), (2000, 1024, 8, 16, 8), (400, 12, 3, 3, 2),
                                        (64, 8, 8, 1, 8), (10, 256, 1, 8, 1), (333, 256, 32, 8, 4)])
@pytest.mark.parametrize("ties", [False, True])
def test_route_topk_grouped(m, T, E, K, gs, M, ties):
    say(f"route_topk grouped T={T} E={E} K={K} gs={gs} M={M} ties={ties}")
    key = wl.case_key(38, T, E, K, gs, M)
    logits = tie_logits(key, T, E) if ties else wl.router_logits(key, T, E, zipf_s=1.2)
    want_i, want_w = oracle.route_topk_grouped(logits, K, gs, M)
    gi, gw = m.route_topk(dev(logits), K, group_size=gs, topk_groups=M)
    torch.cuda.synchronize()
    assert_exact(host(gi), want_i, "topk_idx")
    assert_rel_f32(host(gw), want_w, "topk_w")


def test_route_topk_empty(m):
    gi, gw = m.route_topk(torch.empty((0, 8), dtype=torch.float32, device=DEV), 2)
    torch.cuda.synchronize()
    assert gi.shape == (0, 2) and gw.shape == (0, 2)


# ------------------------------------------------------------------ index build


def ids_case(key, T, E, K, p_missing=0.1, junk=False):
    ids = wl.random_topk_ids(key, T, E, K, p_missing=p_missing)
    if junk and T > 3:
        ids[1, 0] = E + 5  # out of range: routes nowhere on both sides
        ids[2, -1] = -7
    return ids


def check_index(m, ids, w, E, cap=0, gs=0, align=0):
    want = oracle.build_index(ids, w, E, capacity=cap, group_size=gs, alignment=align)
    ix = m.build_index(dev(ids), None if w is None else dev(w), E, capacity=cap, group_size=gs, alignment=align)
    torch.cuda.synchronize()
    for name in ("counts", "group_list", "kept_counts", "sorted_indices", "row_of", "permuted_probs"):
        assert_exact(host(getattr(ix, name)), want[name], name)
    if gs > 0:
        n = int(host(ix.n_slots)[0])
        assert n == int(want["n_slots"][0])
        assert_exact(host(ix.gsrc)[:n], want["gsrc"], "gsrc")
        for name in ("slot_of", "esrc", "group_counts", "slot_src"):
            assert_exact(host(getattr(ix, name)), want[name], name)
    return ix, want


@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (5, 3, 2), (300, 8, 2), (512, 64, 8), (4097, 16, 1), (4099, 64, 8),
                                   (1024, 64, 8), (8193, 16, 1), (256, 1024, 32), (2000, 256, 8), (1500, 1024, 32),
                                   (700, 40, 7), (9000, 128, 4), (50000, 64, 8), (33333, 130, 6),
                                   (2048, 64, 8), (16385, 16, 1)])
@pytest.mark.parametrize("weighted", [True, False])
def test_build_index_standard(m, T, E, K, weighted):
    say(f"build_index standard T={T} E={E} K={K} weighted={weighted}")
    key = wl.case_key(21, T, E, K)
    ids = ids_case(key, T, E, K, junk=True)
    w = wl.random_weights(key, T, K) if weighted else None
    check_index(m, ids, w, E)


@pytest.mark.parametrize("mode", ["standard", "drop", "group", "aligned"])
def test_build_index_repeated_experts(m, mode):
    """Rows that name an expert more than once (drawn with replacement, some slots -1): one row
    per slot in slot order, as the oracle's (expert, token, slot) order gives -- across tiles
    and internal batches (T = 5000, K = 8, E = 16)."""
    T, E, K = 5000, 16, 8
    g = np.random.default_rng([41, len(mode)])
    ids = g.integers(-1, E, size=(T, K)).astype(np.int32)  # with replacement: repeats are common
    ids[:, 1] = ids[:, 0]  # and every row repeats its first slot's expert
    w = wl.random_weights(wl.case_key(41, len(mode)), T, K)
    say(f"build_index repeated experts {mode}")
    cap = 2000 if mode == "drop" else 0
    gs = 4 if mode == "group" else 0
    align = 128 if mode == "aligned" else 0
    check_index(m, ids, w, E, cap=cap, gs=gs, align=align)


def test_build_index_skewed_with_empty_experts(m):
    T, E, K = 3000, 256, 8
    logits = wl.router_logits(wl.case_key(22), T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    ix, want = check_index(m, idx, w, E)
    assert (want["counts"] == 0).any()


def test_route_and_index_at_a_million_tokens(m):
    """Large sizes: T = 1 048 576 tokens, E = 256, K = 8 (8.4M slots, 8192 tokens per tile):
    routing and the full index (standard, and aligned to 128) against the oracle."""
    T, E, K = 1 << 20, 256, 8
    say(f"route + index T={T} E={E} K={K}")
    logits = wl.router_logits(wl.case_key(80), T, E, zipf_s=1.2)
    want_i, want_w = oracle.route_topk(logits, K)
    gi, gw = m.route_topk(dev(logits), K)
    assert_exact(host(gi), want_i, "topk_idx")
    assert_rel_f32(host(gw), want_w, "topk_w")
    w_np = host(gw)
    for align in (0, 128):
        want = oracle.build_index(want_i, w_np, E, alignment=align)
        ix = m.build_index(gi, gw, E, alignment=align)
        torch.cuda.synchronize()
        for name in ("counts", "group_list", "sorted_indices", "row_of", "permuted_probs"):
            assert_exact(host(getattr(ix, name)), want[name], f"{name} (align {align})")
        del ix
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,E,K,cap", [(300, 8, 2, 3), (4099, 64, 8, 40), (2000, 128, 8, 200),
                                       (1000, 16, 4, 1000), (50, 1024, 8, 1), (1, 4, 2, 5), (40000, 96, 8, 2000)])
def test_build_index_drop_and_pad(m, T, E, K, cap):
    say(f"build_index drop T={T} E={E} K={K} cap={cap}")
    key = wl.case_key(23, T, E, K)
    logits = wl.router_logits(key, T, E, zipf_s=1.0)
    idx, w = oracle.route_topk(logits, K)
    idx[0, -1] = -1
    check_index(m, idx, w, E, cap=cap)


@pytest.mark.parametrize("T,E,K,gs", [(300, 8, 2, 2), (4099, 64, 8, 8), (2000, 256, 8, 8), (500, 32, 8, 32),
                                      (700, 96, 6, 1), (1000, 1024, 8, 32), (3, 4, 2, 2), (50000, 64, 6, 8),
                                      (20000, 36, 5, 3), (3000, 1024, 8, 1), (1000, 64, 32, 4),
                                      (777, 128, 16, 16), (900, 16, 1, 4), (1200, 48, 4, 6), (512, 64, 8, 8),
                                      (4097, 16, 1, 2), (1365, 30, 3, 5), (2730, 60, 6, 6), (2048, 64, 8, 8)])
def test_build_index_groups(m, T, E, K, gs):
    say(f"build_index group T={T} E={E} K={K} gs={gs}")
    key = wl.case_key(24, T, E, K)
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    idx[min(1, T - 1), 0] = -1
    check_index(m, idx, w, E, gs=gs)


@pytest.mark.parametrize("cap,gs,align", [(0, 0, 0), (4, 0, 0), (0, 2, 0), (0, 0, 128), (0, 2, 4)])
def test_build_index_no_tokens(m, cap, gs, align):
    ids = np.zeros((0, 2), np.int32)
    check_index(m, ids, None, 8, cap=cap, gs=gs, align=align)


@pytest.mark.parametrize("T,E,K,align,gs", [(300, 8, 2, 128, 0), (4099, 64, 8, 128, 0), (2000, 256, 8, 128, 0),
                                            (700, 40, 7, 3, 0), (50000, 64, 8, 16, 0), (1, 4, 2, 8, 0),
                                            (2000, 256, 8, 128, 8), (500, 32, 8, 5, 4), (1500, 1024, 32, 2, 0)])
def test_build_index_aligned(m, T, E, K, align, gs):
    """Expert alignment: segments rounded up to a multiple of the alignment, padding rows -1,
    the slack after the last segment -2, with skewed routing (empty experts) and holes."""
    say(f"build_index aligned T={T} E={E} K={K} align={align} gs={gs}")
    key = wl.case_key(36, T, E, K, align)
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    idx[::7, -1] = -1
    ix, want = check_index(m, idx, w, E, gs=gs, align=align)
    gl = np.concatenate([[0], want["group_list"]])
    assert (gl % align == 0).all()


INDEX_FIELDS = ("counts", "group_list", "kept_counts", "sorted_indices", "row_of", "permuted_probs")
GROUP_FIELDS = ("slot_of", "esrc", "group_counts", "slot_src")


@pytest.mark.parametrize("T,E,K,cap,gs,align,rgs,M,ties", [
    (16384, 256, 8, 0, 0, 0, 0, 0, False),     # 64-token tiles, 256 of them
    (8192, 256, 8, 0, 8, 0, 0, 0, False),      # index groups
    (8192, 128, 8, 640, 0, 0, 0, 0, False),    # drop-and-pad
    (16384, 256, 8, 0, 0, 128, 0, 0, False),   # expert alignment
    (8192, 256, 8, 0, 8, 0, 8, 4, False),      # group-limited routing and index groups
    (5000, 64, 8, 0, 0, 0, 0, 0, True),        # a partial last tile, tie-heavy logits
    (3001, 96, 6, 0, 8, 0, 0, 0, False),       # K not a power of two: the separate esrc launch
    (2049, 1024, 32, 0, 32, 4, 32, 8, False),  # the largest E and K
    (300000, 64, 8, 0, 0, 0, 0, 0, False),     # 1216-token tiles: 19 passes per workgroup
    (1000, 64, 8, 0, 8, 0, 0, 0, False),       # 8000 slots: route, then the index build alone
    (0, 64, 8, 0, 0, 0, 0, 0, False),
])
def test_route_topk_index(m, T, E, K, cap, gs, align, rgs, M, ties):
    """moe_route_topk_index against the oracle (routing, then the index of the oracle's routing
    with the GPU's weights) and bit for bit against moe_route_topk(_grouped) + moe_build_index."""
    say(f"route_topk_index T={T} E={E} K={K} cap={cap} gs={gs} align={align} route groups {rgs}/{M}")
    key = wl.case_key(42, T, E, K, gs, rgs)
    logits = tie_logits(key, T, E) if ties else wl.router_logits(key, T, E, zipf_s=1.2)
    dl = dev(logits)
    gi, gw, ix = m.route_topk_index(dl, K, capacity=cap, group_size=gs, alignment=align, route_group_size=rgs,
                                    topk_groups=M)
    si, sw = m.route_topk(dl, K, group_size=rgs, topk_groups=M)
    six = m.build_index(si, sw, E, capacity=cap, group_size=gs, alignment=align)
    torch.cuda.synchronize()
    assert_exact(host(gi), host(si), "topk_idx against the separate route")
    assert_exact(host(gw).view(np.int32), host(sw).view(np.int32), "topk_w against the separate route")
    for name in INDEX_FIELDS + (GROUP_FIELDS if gs else ()):
        assert_exact(host(getattr(ix, name)), host(getattr(six, name)), f"{name} against the separate calls")
    want_i, want_w = oracle.route_topk_grouped(logits, K, rgs, M) if rgs else oracle.route_topk(logits, K)
    assert_exact(host(gi), want_i, "topk_idx")
    assert_rel_f32(host(gw), want_w, "topk_w")
    want = oracle.build_index(want_i, host(gw), E, capacity=cap, group_size=gs, alignment=align)
    for name in INDEX_FIELDS:
        assert_exact(host(getattr(ix, name)), want[name], name)
    if gs:
        n = int(host(ix.n_slots)[0])
        assert n == int(want["n_slots"][0])
        assert_exact(host(ix.gsrc)[:n], want["gsrc"], "gsrc")
        assert_exact(host(six.gsrc)[:n], want["gsrc"], "gsrc (separate calls)")
        for name in GROUP_FIELDS:
            assert_exact(host(getattr(ix, name)), want[name], name)


# ------------------------------------------------------------------ permute


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H", [1, 3, 8, 64, 1000, 7168, 4095, 65536])
def test_permute(m, dtype, H):
    say(f"permute {dtype} H={H}")
    key = wl.case_key(25, H)
    src_rows = 301
    x = wl.hidden_states(key, src_rows, H, dtype)
    g = np.random.default_rng([*key, 1])
    src_row = g.integers(-3, src_rows + 3, size=1234).astype(np.int32)  # includes -1.. and >= rows
    src_row[:4] = [0, src_rows - 1, -1, src_rows]
    src_row[4] = -2  # unused slack: left untouched
    want = oracle.permute(x, src_row)
    out = dev(np.full((len(src_row), H), 0x7F81 if dtype == "bf16" else 0x7F800001,
                      np.uint16 if dtype == "bf16" else np.uint32).view(np.uint16 if dtype == "bf16" else np.float32))
    got = host(m.permute(dev(x), dev(src_row), out=out))
    live = src_row != -2
    assert_exact(got[live], want[live], "permuted rows")
    assert (got[~live].view(np.uint16 if dtype == "bf16" else np.uint32) ==
            (0x7F81 if dtype == "bf16" else 0x7F800001)).all(), "unused rows must be left untouched"


def test_permute_empty_source_gives_zero_rows(m):
    x = np.zeros((0, 16), np.uint16)
    src_row = np.asarray([-1, 0, 3], np.int32)
    got = host(m.permute(dev(x), dev(src_row)))
    assert (got == 0).all() and got.shape == (3, 16)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,T,E,K,mode", [(7168, 600, 64, 8, "standard"), (1000, 300, 16, 4, "drop"),
                                          (3, 257, 8, 2, "standard"), (4096, 513, 32, 8, "drop"),
                                          (64, 100, 8, 2, "missing"), (24, 90, 12, 6, "group"),
                                          (65536, 40, 8, 4, "standard")])
def test_permute_scatter_matches_gather(m, dtype, H, T, E, K, mode):
    """Source-major permute with the index's inverse maps equals the pages' gather, bit for bit."""
    say(f"permute_scatter {dtype} H={H} T={T} E={E} K={K} {mode}")
    key = wl.case_key(28, H, T, E, K)
    logits = wl.router_logits(key, T, E, zipf_s=1.0)
    idx, w = oracle.route_topk(logits, K)
    if mode == "missing":
        idx[::3, -1] = -1
    cap = oracle.capacity(T, K, E, 1, 2) if mode == "drop" else 0
    gs = 3 if mode == "group" else 0
    ix = oracle.build_index(idx, w, E, capacity=cap, group_size=gs)
    x = wl.hidden_states(key, T, H, dtype)
    want = oracle.permute(x, ix["sorted_indices"])
    xd = dev(x)
    got = host(m.permute_scatter(xd, dev(ix["row_of"]), len(ix["sorted_indices"]), src_row=dev(ix["sorted_indices"])))
    live = ix["sorted_indices"] != -2  # unused slack is not written
    assert_exact(got[live], want[live], "scatter rows")
    if mode == "group":  # stage 1 of the group dispatch: one copy per (token, group)
        n = int(ix["n_slots"][0])
        got1 = host(m.permute_scatter(xd, dev(ix["slot_of"]), n))
        assert_exact(got1, oracle.permute(x, ix["gsrc"]), "group slots")


def test_permute_scatter_leaves_unnamed_rows(m):
    x = wl.hidden_states(wl.case_key(29), 10, 16, "bf16")
    dst_of = np.full((10, 2), -1, np.int32)
    dst_of[3, 1] = 5
    dst_of[7, 0] = 0
    out = dev(np.full((8, 16), 0x1234, np.uint16))
    m.permute_scatter(dev(x), dev(dst_of), 8, out=out)
    got = host(out)
    assert np.array_equal(got[5], x[3]) and np.array_equal(got[0], x[7])
    assert (got[[1, 2, 3, 4, 6, 7]] == 0x1234).all()
    src_row = np.asarray([7, -1, 99, -1, -1, 3, -1, -1], np.int32)
    m.permute_scatter(dev(x), dev(dst_of), 8, src_row=dev(src_row), out=out)
    got = host(out)
    assert (got[[1, 2, 3, 4, 6, 7]] == 0).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,T,E,K,gs", [(7168, 300, 64, 8, 8), (1000, 513, 32, 8, 4), (3, 200, 16, 4, 4),
                                        (4096, 257, 256, 8, 32), (24, 90, 12, 6, 3), (520, 128, 8, 8, 8)])
def test_permute_grouped_group_receive(m, dtype, H, T, E, K, gs):
    """Receive side of the group dispatch: group slots to expert-major rows, one group per token;
    bit for bit the pages' gather (oracle permute of the group buffer by esrc) and the flat permute."""
    say(f"permute_grouped {dtype} H={H} T={T} E={E} K={K} gs={gs}")
    key = wl.case_key(30, H, T, E, K, gs)
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    idx[::5, -1] = -1  # some slots route nowhere: unused tail rows are zero
    ix = oracle.build_index(idx, w, E, group_size=gs)
    x = wl.hidden_states(key, T, H, dtype)
    gbuf = oracle.permute(x, ix["gsrc"])
    want = oracle.permute(gbuf, ix["esrc"])
    live = ix["esrc"] != -2  # unused slack is not written
    assert np.array_equal(want[live], oracle.permute(x, ix["sorted_indices"])[live])
    got = host(m.permute_grouped(dev(gbuf), dev(ix["esrc"]), dev(ix["row_of"])))
    assert_exact(got[live], want[live], "expert-major rows")
    # the same with each destination's source given beside it (the per-slot group slots)
    got2 = host(m.permute_grouped(dev(gbuf), dev(ix["esrc"]), dev(ix["row_of"]), src_of=dev(ix["slot_src"])))
    assert_exact(got2[live], want[live], "expert-major rows (src_of)")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,J", [(1, 1), (8, 3), (1000, 8), (7168, 16), (4095, 64), (64, 64)])
def test_permute_grouped_random_maps(m, dtype, H, J):
    """Arbitrary groups: shared sources inside a group, repeated rows, out-of-range entries;
    listed rows and zero rows as the oracle's gather, unlisted rows untouched."""
    say(f"permute_grouped random {dtype} H={H} J={J}")
    key = wl.case_key(31, H, J)
    g = np.random.default_rng([*key, 3])
    src_rows, N = 97, 700
    x = wl.hidden_states(key, src_rows, H, dtype)
    src_row = g.integers(0, src_rows, size=N).astype(np.int32)
    src_row[g.random(N) < 0.1] = -1
    src_row[:3] = [src_rows, -5, src_rows - 1]
    rows = g.permutation(N + 40)  # entries >= N are outside [0, N): ignored
    M = (len(rows) * 3 // 4 + J - 1) // J
    dst_of = np.full(M * J, -1, np.int64)
    dst_of[: len(rows) * 3 // 4] = rows[: len(rows) * 3 // 4]
    dst_of = dst_of.reshape(M, J)
    dst_of[g.random((M, J)) < 0.05] = -3
    if J > 1:
        dst_of[0, 1] = dst_of[0, 0]  # a row listed twice
    for i in range(0, M, 7):  # rows of one group naming one source
        live = dst_of[i][(dst_of[i] >= 0) & (dst_of[i] < N)]
        src_row[live] = src_row[live[0]] if len(live) else 0
    dst_of = dst_of.astype(np.int32)
    listed = np.zeros(N, bool)
    listed[dst_of[(dst_of >= 0) & (dst_of < N)]] = True
    zero = (src_row < 0) | (src_row >= src_rows)
    want = oracle.permute(x, src_row)
    poison = np.full((N, H), 0x3F01 if dtype == "bf16" else 0x7FC00001, np.uint16 if dtype == "bf16" else np.uint32)
    # src_of: each listed entry's source; entries outside [0, N) carry junk, which must be ignored
    src_of = np.where((dst_of >= 0) & (dst_of < N), src_row[np.clip(dst_of, 0, N - 1)], 12345).astype(np.int32)
    for so in (None, src_of):
        out = dev(poison.view(np.float32) if dtype == "f32" else poison)
        m.permute_grouped(dev(x), dev(src_row), dev(dst_of), out=out, src_of=None if so is None else dev(so))
        got = host(out)
        if dtype == "f32":
            got, want_b = got.view(np.uint32), want.view(np.uint32)
        else:
            want_b = want
        sel = listed | zero
        assert_exact(got[sel], want_b[sel], "listed and zero rows")
        assert np.array_equal(got[~sel], poison[~sel]), "rows never listed must be left untouched"


@pytest.mark.parametrize("H,block,J", [(16, 8, 8), (7168, 128, 8), (1024, 8, 3), (24, 8, 64), (8192, 8, 16),
                                       (4096, 4096, 1), (448, 64, 5)])
def test_permute_grouped_fp8_random_maps(m, H, block, J):
    """The FP8 group receive moves codes and scale rows together: listed rows get their source's
    codes and scales, zero rows zero codes and zero scales, unlisted rows stay untouched -- the
    oracle's gather of both, as two moe_permute_grouped calls give it (scale rows of 1 to 1024
    floats; H = 24 takes the element-wise path)."""
    say(f"permute_grouped_fp8 random H={H} block={block} J={J}")
    key = wl.case_key(36, H, block, J)
    g = np.random.default_rng([*key, 3])
    src_rows, N, nb = 83, 500, H // block
    q = g.integers(0, 256, size=(src_rows, H), dtype=np.uint8)
    sc = g.standard_normal((src_rows, nb), dtype=np.float32)
    src_row = g.integers(0, src_rows, size=N).astype(np.int32)
    src_row[g.random(N) < 0.1] = -1
    src_row[:4] = [src_rows, -5, src_rows - 1, -2]  # out of range, padding, last row, unused
    rows = g.permutation(N + 30)  # entries >= N are ignored
    M = (len(rows) * 3 // 4 + J - 1) // J
    dst_of = np.full(M * J, -1, np.int64)
    dst_of[: len(rows) * 3 // 4] = rows[: len(rows) * 3 // 4]
    dst_of = dst_of.reshape(M, J)
    if J > 1:
        dst_of[0, 1] = dst_of[0, 0]  # a row listed twice
    for i in range(0, M, 5):  # rows of one group naming one source
        live = dst_of[i][(dst_of[i] >= 0) & (dst_of[i] < N)]
        src_row[live] = src_row[live[0]] if len(live) else 0
    dst_of = dst_of.astype(np.int32)
    listed = np.zeros(N, bool)
    listed[dst_of[(dst_of >= 0) & (dst_of < N)]] = True
    zero = ((src_row < 0) | (src_row >= src_rows)) & (src_row != -2)
    want_q, want_s = oracle.permute(q, src_row), oracle.permute(sc, src_row)
    src_of = np.where((dst_of >= 0) & (dst_of < N), src_row[np.clip(dst_of, 0, N - 1)], 777).astype(np.int32)
    sel = (listed | zero) & (src_row != -2)  # unused rows are never written, listed or not
    for so in (None, src_of):
        oq = dev(np.full((N, H), 0xA5, np.uint8))
        os_ = dev(np.full((N, nb), np.float32(-7.25)))
        rq, rs = m.permute_grouped_fp8(dev(q), dev(sc), dev(src_row), dev(dst_of), out=(oq, os_),
                                       src_of=None if so is None else dev(so))
        gq, gs_ = host(rq), host(rs)
        assert_exact(gq[sel], want_q[sel], "codes of listed and zero rows")
        assert_exact(gs_[sel].view(np.uint32), want_s[sel].view(np.uint32), "scales of listed and zero rows")
        assert (gq[~sel] == 0xA5).all() and (gs_[~sel] == np.float32(-7.25)).all(), "unlisted rows untouched"
        # the same as the two separate grouped gathers
        tq = host(m.permute_grouped(dev(q), dev(src_row), dev(dst_of), out=dev(np.full((N, H), 0xA5, np.uint8)),
                                    src_of=None if so is None else dev(so)))
        ts = host(m.permute_grouped(dev(sc), dev(src_row), dev(dst_of),
                                    out=dev(np.full((N, nb), np.float32(-7.25))), src_of=None if so is None else dev(so)))
        assert np.array_equal(gq, tq) and np.array_equal(gs_.view(np.uint32), ts.view(np.uint32))


@pytest.mark.parametrize("H,block", [(128, 16), (24, 8)])
def test_permute_grouped_fp8_without_groups_writes_zero_rows(m, H, block):
    """No groups at all: only the zero rows are written, codes and scales alike (the 16-byte and
    the element-wise paths); other rows keep their contents."""
    nb = H // block
    q = np.random.default_rng(5).integers(0, 256, size=(4, H), dtype=np.uint8)
    sc = np.random.default_rng(6).standard_normal((4, nb), dtype=np.float32)
    src_row = np.asarray([-1, 2, 9, -2, -1], np.int32)
    oq = dev(np.full((5, H), 0x77, np.uint8))
    os_ = dev(np.full((5, nb), np.float32(3.5)))
    m.permute_grouped_fp8(dev(q), dev(sc), dev(src_row), dev(np.zeros((0, 4), np.int32)), out=(oq, os_))
    gq, gs_ = host(oq), host(os_)
    assert (gq[[0, 2, 4]] == 0).all() and (gs_[[0, 2, 4]] == 0).all()
    assert (gq[[1, 3]] == 0x77).all() and (gs_[[1, 3]] == np.float32(3.5)).all()


def test_permute_grouped_without_groups_writes_zero_rows(m):
    x = wl.hidden_states(wl.case_key(32), 4, 16, "bf16")
    src_row = np.asarray([-1, 2, 9, -1], np.int32)
    out = dev(np.full((4, 16), 0x1234, np.uint16))
    m.permute_grouped(dev(x), dev(src_row), dev(np.zeros((0, 4), np.int32)), out=out)
    got = host(out)
    assert (got[[0, 2, 3]] == 0).all() and (got[1] == 0x1234).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,T,E,K,align", [(7168, 600, 64, 8, 128), (1000, 300, 16, 4, 8), (3, 257, 8, 2, 4),
                                           (520, 200, 32, 8, 16)])
def test_permute_aligned(m, dtype, H, T, E, K, align):
    """Aligned expert buffer: tokens bit for bit, padding rows zero, the slack after the last
    segment untouched; the combine over the aligned rows equals the oracle's."""
    say(f"permute aligned {dtype} H={H} T={T} E={E} K={K} align={align}")
    key = wl.case_key(37, H, T, E, K, align)
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    idx[::9, 0] = -1
    ix = oracle.build_index(idx, w, E, alignment=align)
    si = ix["sorted_indices"]
    x = wl.hidden_states(key, T, H, dtype)
    want = oracle.permute(x, si)
    pat = 0x7F81 if dtype == "bf16" else 0x7F800001
    u = np.uint16 if dtype == "bf16" else np.uint32
    out = dev(np.full((len(si), H), pat, u).view(np.uint16 if dtype == "bf16" else np.float32))
    got = host(m.permute_scatter(dev(x), dev(ix["row_of"]), len(si), src_row=dev(si), out=out))
    live = si != -2
    assert_exact(got[live], want[live], "aligned rows")
    assert (got[si == -1].view(u) == 0).all()
    assert (got[~live].view(u) == pat).all(), "slack rows must be left untouched"
    y = wl.expert_outputs(key, len(si), H, dtype)
    out_np = np.uint16 if dtype == "bf16" else np.float32
    assert_exact(host(m.unpermute_combine(dev(y), dev(ix["row_of"]), dev(w))),
                 oracle.unpermute_combine(y, ix["row_of"], w, out_np), "combine over aligned rows")


# ------------------------------------------------------------------ FP8 dispatch


def fp8_inputs(key, T, H, dtype):
    x = wl.hidden_states(key, T, H, dtype)
    x[min(1, T - 1)] = 0  # an all-zero token: scale 1, zero codes
    if T > 3:
        f = wl.bf16_bits_to_f32(x[2]) if dtype == "bf16" else x[2]
        f = (f * 1e-30 if dtype == "f32" else f * 1e-20).astype(np.float32)  # tiny blocks: subnormal quotients
        x[2] = wl.f32_to_bf16_bits(f) if dtype == "bf16" else f
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,H,block", [(100, 7168, 128), (77, 512, 32), (50, 1024, 512), (30, 7168, 7168),
                                       (40, 384, 96), (3, 8, 8), (60, 4096, 64), (5, 21, 7)])
def test_quantize_fp8(m, dtype, T, H, block):
    say(f"quantize_fp8 {dtype} T={T} H={H} block={block}")
    x = fp8_inputs(wl.case_key(70, T, H, block), T, H, dtype)
    want_q, want_s = oracle.quantize_fp8(x, block)
    q, sc = m.quantize_fp8(dev(x), block)
    assert_exact(host(q), want_q, "codes")
    assert_exact(host(sc), want_s, "scales")


def _bf16_rounding_rows():
    """float32 values whose bf16 rounding is a boundary case: exact ties with an even and with an
    odd kept mantissa, one float32 step either side of a tie, carries into the next binade,
    float32 subnormals (ties among them too), values rounding up past the largest bf16 to
    infinity, infinities, zeros, and the negatives of all of them; 256 per row."""
    rng = np.random.default_rng(20260)
    hi = rng.integers(0, 0x7f7f, size=600, dtype=np.uint32) << 16      # finite bf16 patterns
    tie = hi | 0x8000
    bits = np.concatenate([tie, tie + 1, tie - 1, hi | 0x7fff, hi | 0xffff, hi | 0x0001,
                           rng.integers(1, 0x800000, size=200, dtype=np.uint32),     # subnormals
                           (rng.integers(0, 0x80, size=100, dtype=np.uint32) << 16) | 0x8000,
                           np.asarray([0x7f7f8000, 0x7f7fffff, 0x7f7f7fff, 0x7f800000, 0, 0x00008000,
                                       0x00018000, 0x3f808000, 0x3f818000], np.uint32)])
    bits = np.concatenate([bits, bits | 0x80000000]).astype(np.uint32)
    n = -(-len(bits) // 256) * 256
    bits = np.concatenate([bits, np.zeros(n - len(bits), np.uint32)])
    return bits.view(np.float32).reshape(-1, 256)


def test_bf16_output_rounding_at_boundaries(m):
    """float32 rows combined with unit weights into bf16: every output is the round-to-nearest-
    even of one float32 value, at ties, around ties, in the subnormal range and at overflow --
    against the oracle, bit for bit; then bf16 rows through the batched combine (an FMA with
    weight 1 from +0 reproduces each row)."""
    say("bf16 output rounding at boundaries")
    y = _bf16_rounding_rows()
    R = y.shape[0]
    row_of = np.arange(R, dtype=np.int32).reshape(R, 1)
    want = oracle.unpermute_combine(y, row_of, None, np.uint16)
    got = host(m.unpermute_combine(dev(y), dev(row_of), None, out_dtype=torch.bfloat16))
    assert_exact(got, want, "bf16 outputs")
    # the same float32 values reach the batched combine as bf16 rows (8 slots per token, one
    # valid): 16384 tokens, row t % R each
    yb = want
    T = 16384
    rows8 = np.full((T, 8), -1, np.int32)
    rows8[:, 0] = np.arange(T) % R
    w8 = np.ones((T, 8), np.float32)
    want8 = oracle.unpermute_combine(yb, rows8, w8, np.uint16)
    got8 = host(m.unpermute_combine(dev(yb), dev(rows8), dev(w8), out_dtype=torch.bfloat16))
    assert_exact(got8, want8, "bf16 batched outputs")


def _e4m3_boundary_rows():
    """float32 rows of 8 whose first element is 448 (so the block's scale is exactly 1 and every
    code is the E4M3 rounding of the value itself), the other 7 taken in turn from: every finite
    E4M3 value, every midpoint between neighbouring values (the round-to-nearest-even ties), the
    float32 neighbours of each midpoint, and the negatives of all of them."""
    vals = sorted({oracle.e4m3_to_f32(c) for c in range(0x7F)})
    mids = [np.float32((a + b) / 2) for a, b in zip(vals[:-1], vals[1:])]
    pool = [np.float32(v) for v in vals] + mids
    pool += [np.nextafter(m, np.float32(np.inf)) for m in mids] + [np.nextafter(m, np.float32(-np.inf)) for m in mids]
    pool += [np.float32(2.0 ** -10), np.float32(2.0 ** -11), np.float32(3 * 2.0 ** -11), np.float32(1e-30)]
    pool = np.asarray(pool, np.float32)
    pool = np.concatenate([pool, -pool])
    n = -(-len(pool) // 7)
    rows = np.zeros((n, 8), np.float32)
    rows[:, 0] = 448.0
    rows[:, 1:].flat[:len(pool)] = pool
    return rows


def test_fp8_codes_at_rounding_boundaries(m):
    """E4M3 codes of every finite value, every tie and the float32 neighbours of every tie,
    with a scale of exactly 1: the quantizer and the fused dispatch against the oracle, bit for bit."""
    say("fp8 codes at rounding boundaries")
    x = _e4m3_boundary_rows()
    want_q, want_s = oracle.quantize_fp8(x, 8)
    assert (want_s == 1.0).all()
    q, sc = m.quantize_fp8(dev(x), 8)
    assert_exact(host(q), want_q, "codes")
    assert_exact(host(sc), want_s, "scales")
    T = x.shape[0]
    ident = np.arange(T, dtype=np.int32).reshape(T, 1)
    q2, sc2 = m.permute_scatter_fp8(dev(x), dev(ident), T, 8)
    assert_exact(host(q2), want_q, "dispatched codes")
    assert_exact(host(sc2), want_s, "dispatched scales")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,T,E,K,mode,block", [(7168, 300, 64, 8, "standard", 128), (1024, 200, 16, 4, "drop", 64),
                                                (4096, 257, 32, 8, "aligned", 128), (512, 100, 8, 2, "holes", 512),
                                                (64, 90, 12, 6, "standard", 8), (2048, 128, 64, 8, "group", 128),
                                                (520, 64, 8, 2, "drop", 8), (3072, 50, 16, 4, "standard", 1024),
                                                (1040, 70, 8, 4, "holes", 16)])
def test_permute_scatter_fp8(m, dtype, H, T, E, K, mode, block):
    """Fused FP8 dispatch = the oracle's quantization followed by the oracle's row gather of the
    codes and of the scales, bit for bit; padding rows zero, unused slack untouched."""
    say(f"permute_scatter_fp8 {dtype} H={H} T={T} E={E} K={K} {mode} block={block}")
    key = wl.case_key(71, H, T, E, K)
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    if mode == "holes":
        idx[::4, -1] = -1
    cap = oracle.capacity(T, K, E, 1, 2) if mode == "drop" else 0
    ix = oracle.build_index(idx, w, E, capacity=cap, alignment=128 if mode == "aligned" else 0,
                            group_size=8 if mode == "group" else 0)
    x = fp8_inputs(key, T, H, dtype)
    qs, ss = oracle.quantize_fp8(x, block)
    if mode == "group":  # the send stage: one copy per (token, group)
        n = int(ix["n_slots"][0])
        q, sc = m.permute_scatter_fp8(dev(x), dev(ix["slot_of"]), n, block)
        assert_exact(host(q), oracle.permute(qs, ix["gsrc"]), "slot codes")
        assert_exact(host(sc), oracle.permute(ss, ix["gsrc"]), "slot scales")
        # the receive stage moves FP8 rows and scale rows like any rows
        rq = m.permute_grouped(q, dev(ix["esrc"]), dev(ix["row_of"]))
        live = ix["esrc"] != -2
        assert_exact(host(rq)[live], oracle.permute(qs, ix["sorted_indices"])[live], "received codes")
        return
    si = ix["sorted_indices"]
    N = len(si)
    nb = H // block
    out = (dev(np.full((N, H), 0xA5, np.uint8)), dev(np.full((N, nb), np.float32(-7.0))))
    q, sc = m.permute_scatter_fp8(dev(x), dev(ix["row_of"]), N, block, src_row=dev(si), out=out)
    live = si != -2
    assert_exact(host(q)[live], oracle.permute(qs, si)[live], "codes")
    assert_exact(host(sc)[live], oracle.permute(ss, si)[live], "scales")
    assert (host(q)[~live] == 0xA5).all() and (host(sc)[~live] == -7.0).all(), "slack rows must be untouched"
    # the same bytes as quantizing, then moving codes and scales with the plain permutes
    q2 = m.permute(dev(qs), dev(si))
    assert_exact(host(q2)[live], host(q)[live], "byte permute of the codes")


@pytest.mark.parametrize("J", [65, 200, 1024])
@pytest.mark.parametrize("H,dtype", [(7168, "bf16"), (1000, "f32"), (13, "bf16")])
def test_permute_scatter_wide_maps(m, J, H, dtype):
    """Destination maps wider than a wavefront (e.g. slot_of with more than 64 expert groups):
    each source row names a few destinations spread over J mostly empty columns, some rows name
    none; the scatter (and, for 16-byte rows, the fused FP8 scatter) equals the oracle's gather
    through the inverse map, zero rows included."""
    say(f"permute_scatter wide J={J} H={H} {dtype}")
    g = np.random.default_rng([72, J, H])
    src_rows, N = 50, 300
    dst_of = np.full((src_rows, J), -1, np.int32)
    cells = g.choice(src_rows * J, size=N - 20, replace=False)  # 20 destination rows stay unnamed
    rows = g.permutation(N)[: N - 20]
    dst_of.reshape(-1)[cells] = rows
    src_row = np.full(N, -1, np.int32)
    src_row[rows] = (cells // J).astype(np.int32)
    x = wl.hidden_states(wl.case_key(72, J, H), src_rows, H, dtype)
    got = host(m.permute_scatter(dev(x), dev(dst_of), N, src_row=dev(src_row)))
    assert_exact(got, oracle.permute(x, src_row), "rows")
    if (H * (2 if dtype == "bf16" else 4)) % 16 == 0 and H % 8 == 0:
        block = 8 if H % 16 else 8 * (H // 8 & -(H // 8))  # a power of two dividing H
        block = min(block, 1024)
        qs, ss = oracle.quantize_fp8(x, block)
        q, sc = m.permute_scatter_fp8(dev(x), dev(dst_of), N, block, src_row=dev(src_row))
        assert_exact(host(q), oracle.permute(qs, src_row), "codes")
        assert_exact(host(sc), oracle.permute(ss, src_row), "scales")


@pytest.mark.parametrize("J,holes", [(5, 0.0), (8, 0.0), (8, 0.3), (8, 0.9), (9, 0.2), (64, 0.5), (65, 0.0),
                                     (200, 0.4), (1024, 0.97)])
@pytest.mark.parametrize("H,dtype", [(7168, "bf16"), (1000, "f32"), (8, "bf16")])
def test_permute_scatter_dense_maps(m, J, holes, H, dtype):
    """Maps with one output row per entry (N = rows * J, the standard dispatch's shape), whose
    destinations the scatter shares among two waves per slice by their rank among a row's valid
    entries: holes (-1 entries) shift the ranks, maps wider than a wavefront count them across
    64-entry chunks; every listed row equals the oracle's gather, the unnamed rows are untouched."""
    say(f"permute_scatter dense J={J} holes={holes} H={H} {dtype}")
    g = np.random.default_rng([74, J, int(holes * 100), H])
    src_rows = max(3, 3000 // J)
    N = src_rows * J
    dst = g.permutation(N).astype(np.int32)
    dst_of = dst.reshape(src_rows, J).copy()
    dst_of[g.random((src_rows, J)) < holes] = -1
    dst_of[0] = -1  # a row with no destination
    if J > 5:
        dst_of[1, :5] = -1  # valid entries only past the first wave's share
    src_row = np.full(N, -3, np.int32)
    live = dst_of >= 0
    src_row[dst_of[live]] = np.nonzero(live)[0].astype(np.int32)
    x = wl.hidden_states(wl.case_key(74, J, H), src_rows, H, dtype)
    u = np.uint16 if dtype == "bf16" else np.uint32
    out = dev(np.full((N, H), 0x7F81 if dtype == "bf16" else 0x7F800001, u).view(
        np.uint16 if dtype == "bf16" else np.float32))
    got = host(m.permute_scatter(dev(x), dev(dst_of), N, out=out))
    named = src_row >= 0
    assert_exact(got[named], oracle.permute(x, src_row)[named], "named rows")
    assert (got[~named].view(u) == (0x7F81 if dtype == "bf16" else 0x7F800001)).all(), "unnamed rows untouched"


@pytest.mark.parametrize("ydt,odt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("H,K,T", [(7168, 8, 60), (1000, 2, 50), (5, 3, 20), (512, 8, 40), (64, 1, 30), (24, 40, 16)])
def test_unpermute_combine_bias(m, ydt, odt, H, K, T):
    """The combine's final bias: one float32 addition after the slot-order sum, in every path
    (many and few terms per token, float32 split rows, element-wise rows)."""
    say(f"combine bias y={ydt} out={odt} H={H} K={K} T={T}")
    key = wl.case_key(72, H, K, T)
    y_rows = T * K + 3
    y = wl.expert_outputs(key, y_rows, H, ydt)
    g = np.random.default_rng([*key, 1])
    row_of = g.permutation(y_rows)[: T * K].astype(np.int32).reshape(T, K)
    row_of[g.random((T, K)) < 0.3] = -1
    row_of[0] = -1  # no term: the output is the bias
    w = wl.random_weights(key, T, K)
    bias = wl.expert_outputs((*key, 2), T, H, odt)
    out_np = np.uint16 if odt == "bf16" else np.float32
    want = oracle.unpermute_combine(y, row_of, w, out_np, bias=bias)
    got = host(m.unpermute_combine(dev(y), dev(row_of), dev(w), bias=dev(bias),
                                   out_dtype=torch.bfloat16 if odt == "bf16" else torch.float32))
    assert_exact(got, want, "combined with bias")


# ------------------------------------------------------------------ combine


@pytest.mark.parametrize("ydt,odt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("H,K,T", [(1, 1, 10), (5, 2, 33), (512, 2, 1024), (7168, 8, 130), (1000, 8, 77),
                                   (64, 32, 200), (24, 256, 40), (16, 1024, 6),
                                   (65536, 8, 24), (32776, 3, 20)])  # long rows: > 1024 threads' worth
@pytest.mark.parametrize("weighted", [True, False])
def test_unpermute_combine(m, ydt, odt, H, K, T, weighted):
    say(f"combine y={ydt} out={odt} H={H} K={K} T={T} weighted={weighted}")
    key = wl.case_key(26, H, K, T)
    y_rows = T * K + 5
    y = wl.expert_outputs(key, y_rows, H, ydt)
    g = np.random.default_rng([*key, 2])
    row_of = g.permutation(y_rows)[: T * K].astype(np.int32).reshape(T, K)
    row_of[g.random((T, K)) < 0.15] = -1
    row_of[0, 0] = y_rows + 2  # out of range: no term
    w = wl.random_weights(key, T, K) if weighted else None
    out_np = np.uint16 if odt == "bf16" else np.float32
    want = oracle.unpermute_combine(y, row_of, w, out_np)
    got = host(m.unpermute_combine(dev(y), dev(row_of), None if w is None else dev(w),
                                   out_dtype=torch.bfloat16 if odt == "bf16" else torch.float32))
    assert_combined(got, want, "combined")
    assert exact_fraction(got, want) == 1.0


@pytest.mark.parametrize("H,K", [(64, 8), (1000, 5), (7168, 8)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_unpermute_combine_batched_path(m, H, K, with_bias):
    """Many tokens with 5..8 slots in bf16: the combine that stages 8 tokens' rows in LDS and
    writes them in one burst; T = 16 389 leaves a ragged last batch. Every token against the oracle."""
    T = 16389 if H < 7168 else 16392
    say(f"combine batched H={H} K={K} T={T} bias={with_bias}")
    key = wl.case_key(73, H, K)
    y_rows = T * K + 7
    y = wl.expert_outputs(key, y_rows, H, "bf16")
    g = np.random.default_rng([*key, 1])
    row_of = g.permutation(y_rows)[: T * K].astype(np.int32).reshape(T, K)
    row_of[g.random((T, K)) < 0.1] = -1
    row_of[5] = -1
    w = wl.random_weights(key, T, K)
    bias = wl.expert_outputs((*key, 2), T, H, "bf16") if with_bias else None
    want = oracle.unpermute_combine(y, row_of, w, np.uint16, bias=bias)
    got = host(m.unpermute_combine(dev(y), dev(row_of), dev(w), bias=None if bias is None else dev(bias)))
    assert_exact(got, want, "combined")


def test_combine_no_tokens(m):
    out = m.unpermute_combine(torch.zeros((4, 8), dtype=torch.bfloat16, device=DEV),
                              torch.zeros((0, 2), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert out.shape == (0, 8)


# ------------------------------------------------------------------ group pre-combine


@pytest.mark.parametrize("T,E,K,gs,H,ydt,holes", [
    (300, 8, 2, 2, 64, "bf16", False), (513, 64, 8, 8, 1000, "bf16", False),
    (200, 256, 8, 8, 7168, "bf16", False), (100, 32, 4, 4, 5, "f32", False),
    (150, 16, 8, 16, 24, "bf16", False),
    (200, 64, 16, 8, 1000, "bf16", False),   # K > 8: member rows loaded per (group, slot)
    (64, 64, 32, 4, 520, "f32", False),      # K = 32, float32 rows, a ragged 512-element unit
    (90, 64, 8, 8, 7168, "f32", False),
    (400, 64, 8, 8, 1000, "bf16", True),     # some slots route nowhere (id -1)
    (150, 64, 16, 4, 1000, "bf16", True)])
@pytest.mark.parametrize("layout", ["compact", "dense"])
@pytest.mark.parametrize("pdt", ["f32", "bf16"])
def test_group_precombine_and_final_sum(m, T, E, K, gs, H, ydt, holes, layout, pdt):
    say(f"precombine T={T} E={E} K={K} gs={gs} H={H} {ydt} holes={holes} {layout} partials={pdt}")
    key = wl.case_key(27, T, E, K, gs, H)
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    if holes:
        idx[np.random.default_rng([*key, 9]).random((T, K)) < 0.2] = -1
    want_ix = oracle.build_index(idx, w, E, group_size=gs)
    G = E // gs
    if layout == "compact":
        slot_of = want_ix["slot_of"]
        cap = int(want_ix["n_slots"][0])
    else:
        slot_of = np.arange(T * G, dtype=np.int32).reshape(T, G)
        cap = T * G
    y = wl.expert_outputs(key, T * K, H, ydt)
    want_p = oracle.group_precombine(y, want_ix["row_of"], w, idx, E, gs, slot_of, cap,
                                     out_dtype=np.uint16 if pdt == "bf16" else np.float32)
    got_p = host(m.group_precombine(dev(y), dev(want_ix["row_of"]), dev(w), dev(idx), E, gs, dev(slot_of),
                                    slots_cap=cap, out_dtype=torch.bfloat16 if pdt == "bf16" else torch.float32))
    assert_combined(got_p, want_p, "partials")
    assert exact_fraction(got_p, want_p) == 1.0
    want_o = oracle.unpermute_combine(want_p, slot_of, None, np.uint16)
    got_o = host(m.unpermute_combine(dev(want_p), dev(slot_of), None, out_dtype=torch.bfloat16))
    assert_combined(got_o, want_o, "final sum")


# ------------------------------------------------------------------ the five workloads at full size
# Every row and every token of the bench's launch configuration is compared with the oracle on the
# same inputs; device tensors are brought to the host in row chunks so that host memory stays bounded.

ROW_CHUNK = 8192


def assert_rows_exact(got, want: np.ndarray, what: str, live=None):
    """Device tensor `got` [N, H] against the oracle's host array `want`, bit for bit, every row
    (rows with live[i] False -- the unused slack that no call writes -- are skipped)."""
    assert tuple(got.shape) == want.shape, f"{what}: shape {tuple(got.shape)} != {want.shape}"
    for a in range(0, want.shape[0], ROW_CHUNK):
        b = min(a + ROW_CHUNK, want.shape[0])
        g, w_ = host(got[a:b]), want[a:b]
        if live is not None:
            g, w_ = g[live[a:b]], w_[live[a:b]]
        if not np.array_equal(g.view(np.uint8), w_.view(np.uint8)):
            bad = np.flatnonzero((g.view(np.uint8) != w_.view(np.uint8)).reshape(len(g), -1).any(axis=1))
            rows = (np.flatnonzero(live[a:b]) if live is not None else np.arange(b - a))[bad] + a
            raise AssertionError(f"{what}: {len(bad)} rows differ in rows {a}..{b - 1}, first {rows[:5].tolist()}")


def assert_combined_all(got, want: np.ndarray, what: str):
    """Every combined value within the parity tolerance, and (the same weight bits on both sides)
    every one bit-identical."""
    g = host(got)
    assert_combined(g, want, what)
    share = exact_fraction(g, want)
    assert share == 1.0, f"{what}: bit-identical share {share}"


def check_route_and_index(m, c, logits, route_groups, cap, align):
    """Routing and the index on the GPU against the oracle, every entry; returns the GPU's
    outputs and the oracle's index built on the GPU's weight bits."""
    T, E, K, gs = c["T"], c["E"], c["K"], c["group_size"]
    if route_groups:
        want_i, want_w = oracle.route_topk_grouped(logits, K, gs, route_groups)
    else:
        want_i, want_w = oracle.route_topk(logits, K)
    # routing and index in one call, as bench.py launches them
    gi, gw, ix = m.route_topk_index(dev(logits), K, capacity=cap, group_size=gs, alignment=align,
                                    route_group_size=gs if route_groups else 0, topk_groups=route_groups)
    assert_exact(host(gi), want_i, "topk_idx")
    assert_rel_f32(host(gw), want_w, "topk_w")
    w_np = host(gw)  # the same weight bits on both sides from here on
    want = oracle.build_index(want_i, w_np, E, capacity=cap, group_size=gs, alignment=align)
    for name in ("counts", "group_list", "kept_counts", "sorted_indices", "row_of", "permuted_probs"):
        assert_exact(host(getattr(ix, name)), want[name], name)
    if gs > 0:
        n = int(host(ix.n_slots)[0])
        assert n == int(want["n_slots"][0])
        assert_exact(host(ix.gsrc)[:n], want["gsrc"], "gsrc")
        for name in ("slot_of", "esrc", "group_counts", "slot_src"):
            assert_exact(host(getattr(ix, name)), want[name], name)
    return gi, gw, ix, want_i, w_np, want


FP8_BLOCK = 128  # one float32 scale per 128 elements, as bench.py --fp8


def run_workload(m, cfg_id, align=0, route_groups=0, fp8=False, bf16_partials=False):
    """Runs route -> index -> dispatch -> (pre-)combine on the GPU in bench.py's launch
    configuration and checks every stage against the oracle in full: every index entry, every
    dispatched row (the group dispatch against the oracle's two-stage gather x -> group slots ->
    expert rows; FP8 codes and scales against the oracle's quantization moved by its gather),
    every partial and every combined token. align > 1: the expert-aligned layout; route_groups >
    0: group-limited routing over the workload's expert groups, that many groups per token.
    Returns the combined output (device)."""
    c = wl.WORKLOADS[cfg_id]
    T, H, E, K, dt = c["T"], c["H"], c["E"], c["K"], c["dtype"]
    key = wl.workload_key(cfg_id)
    say(f"workload {cfg_id}: {c['name']} align={align} route_groups={route_groups} fp8={fp8} "
        f"bf16_partials={bf16_partials}")
    logits = wl.router_logits(key, T, E, zipf_s=c["zipf_s"])
    x = wl.hidden_states(key, T, H, dt)
    cap = oracle.capacity(T, K, E, *c["cf"]) if c["cf"] else 0
    assert cap == (m.expert_capacity(T, K, E, *c["cf"]) if c["cf"] else 0)
    gs = c["group_size"]
    G = E // gs if gs else 0
    slots = T * min(K, G) if gs else 0  # group buffers sized by the bound, as bench.py does
    gi, gw, ix, want_i, w_np, want = check_route_and_index(m, c, logits, route_groups, cap, align)
    rows = ix.rows
    si = want["sorted_indices"]
    live = si != -2  # the unused slack after the last segment is never written
    n = int(want["n_slots"][0]) if gs else 0
    xd = dev(x)

    # ---- dispatch
    if fp8:
        qs, ss = oracle.quantize_fp8(x, FP8_BLOCK)
        if gs:
            gq, gsc = m.permute_scatter_fp8(xd, ix.slot_of, slots, FP8_BLOCK)
            want_gq, want_gs = oracle.permute(qs, want["gsrc"]), oracle.permute(ss, want["gsrc"])
            assert_rows_exact(gq[:n], want_gq, "FP8 group-slot codes")
            assert_rows_exact(gsc[:n], want_gs, "FP8 group-slot scales")
            xq, xs = m.permute_grouped_fp8(gq, gsc, ix.esrc, ix.row_of, src_of=ix.slot_src)
            want_xq, want_xs = oracle.permute(want_gq, want["esrc"]), oracle.permute(want_gs, want["esrc"])
            del gq, gsc, want_gq, want_gs
        else:
            xq, xs = m.permute_scatter_fp8(xd, ix.row_of, rows, FP8_BLOCK, src_row=ix.sorted_indices)
            want_xq, want_xs = oracle.permute(qs, si), oracle.permute(ss, si)
        assert_rows_exact(xq, want_xq, "FP8 expert-major codes", live)
        assert_rows_exact(xs, want_xs, "FP8 expert-major scales", live)
        del xq, xs, want_xq, want_xs, qs, ss
        xp = want_xp = None
    else:
        if gs:
            gbuf = m.permute_scatter(xd, ix.slot_of, slots)
            want_g = oracle.permute(x, want["gsrc"])
            assert_rows_exact(gbuf[:n], want_g, "group slots (send)")
            xp = m.permute_grouped(gbuf, ix.esrc, ix.row_of, src_of=ix.slot_src)
            want_xp = oracle.permute(want_g, want["esrc"])
            del gbuf, want_g
        else:
            xp = m.permute_scatter(xd, ix.row_of, rows, src_row=ix.sorted_indices)
            want_xp = oracle.permute(x, si)
        assert_rows_exact(xp, want_xp, "expert-major rows", live)
    del xd

    # ---- combine
    if c["identity_experts"]:
        y_np, yd = want_xp, xp  # identity experts: y is the permuted x (checked bit for bit above)
    else:
        del xp, want_xp
        y_np = wl.expert_outputs(key, rows, H, dt)
        yd = dev(y_np)
    out_np = np.uint16 if dt == "bf16" else np.float32
    out_t = torch.bfloat16 if dt == "bf16" else torch.float32
    if gs:
        p_np = np.uint16 if bf16_partials else np.float32
        part = m.group_precombine(yd, ix.row_of, gw, gi, E, gs, ix.slot_of, slots_cap=slots,
                                  out_dtype=torch.bfloat16 if bf16_partials else torch.float32)
        want_p = oracle.group_precombine(y_np, want["row_of"], w_np, want_i, E, gs, want["slot_of"], n,
                                         out_dtype=p_np)
        assert_combined_all(part[:n], want_p, "partials")
        out = m.unpermute_combine(part, ix.slot_of, None, out_dtype=out_t)
        want_o = oracle.unpermute_combine(want_p, want["slot_of"], None, out_np)
        del part, want_p
    else:
        out = m.unpermute_combine(yd, ix.row_of, gw, out_dtype=out_t)
        want_o = oracle.unpermute_combine(y_np, want["row_of"], w_np, out_np)
    assert_combined_all(out, want_o, "combined")
    if c["identity_experts"]:
        rel = np.abs(host(out).astype(np.float64) - x) / np.maximum(np.abs(x), np.finfo(np.float32).tiny)
        assert rel.max() <= 1e-6
    return out


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_workload_full_size(m, cfg_id):
    run_workload(m, cfg_id)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg_id", [2, 3, 4, 5])
def test_workload_fp8_dispatch(m, cfg_id):
    """The FP8 dispatch as bench.py --fp8 launches it (workloads with expert outputs)."""
    run_workload(m, cfg_id, fp8=True)
    torch.cuda.empty_cache()


def test_workload_bf16_partials(m):
    """Workload 4 with the per-group partials rounded to bf16 (the BF16 exchange), as bench.py
    --bf16-partials launches it."""
    run_workload(m, 4, bf16_partials=True)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bf16_partials", [False, True])
def test_workload_group_limited_routing(m, bf16_partials):
    """Workload 4 with every token limited to 4 of its 32 expert groups, as bench.py
    --route-groups 4 launches it."""
    run_workload(m, 4, route_groups=4, bf16_partials=bf16_partials)
    torch.cuda.empty_cache()


def test_workload_fp8_group_limited_bf16_partials(m):
    """Workload 4 with every option bench.py combines: group-limited routing, the FP8 dispatch and
    bf16 partials."""
    run_workload(m, 4, route_groups=4, fp8=True, bf16_partials=True)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg_id,align", [(3, 128), (2, 128), (4, 128), (1, 128)])
def test_workload_aligned(m, cfg_id, align):
    """The named workloads with every expert segment aligned to 128 rows, as bench.py --alignment
    128 launches them."""
    run_workload(m, cfg_id, align=align)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg_id,mode", [(2, "standard"), (5, "drop"), (4, "group"), (2, "aligned"),
                                         (4, "route_groups"), (2, "fp8"), (4, "fp8"), (2, "backward"),
                                         (4, "backward"), (4, "bf16_partials")])
def test_step_replays_from_a_hip_graph(m, cfg_id, mode):
    """A whole step (route, index, permute, combine; or its backward) captured once in a HIP
    graph and replayed three times, with eager work (the outputs cleared by a fill kernel) and
    synchronizations between the replays: every replay matches the eager step bit for bit.
    Nothing in the step allocates, waits on the host or records a memset."""
    c = wl.WORKLOADS[cfg_id]
    T, H, E, K, dt = c["T"], c["H"], c["E"], c["K"], c["dtype"]
    say(f"graph replay workload {cfg_id} ({mode})")
    key = wl.workload_key(cfg_id)
    cap = oracle.capacity(T, K, E, *c["cf"]) if c["cf"] else 0
    gs = c["group_size"]
    align = 128 if mode == "aligned" else 0
    rg = 4 if mode == "route_groups" else 0
    logits = dev(wl.router_logits(key, T, E, zipf_s=c["zipf_s"]))
    x = dev(wl.hidden_states(key, T, H, dt))
    rows = m.index_rows(T, K, E, cap, align)
    y = dev(wl.expert_outputs(key, rows, H, dt))
    tdt = x.dtype
    gi = torch.empty((T, K), dtype=torch.int32, device=DEV)
    gw = torch.empty((T, K), dtype=torch.float32, device=DEV)
    ix = m.alloc_index(T, K, E, cap, gs, alignment=align)
    G = E // gs if gs else 0
    slots = T * min(K, G) if gs else 0
    outs = {"out": torch.empty((T, H), dtype=tdt, device=DEV)}
    block = 128
    if mode == "fp8":
        outs["xp"] = torch.empty((rows, H), dtype=torch.uint8, device=DEV)
        outs["xs"] = torch.empty((rows, H // block), dtype=torch.float32, device=DEV)
        gq = torch.empty((slots, H), dtype=torch.uint8, device=DEV) if gs else None
        gsc = torch.empty((slots, H // block), dtype=torch.float32, device=DEV) if gs else None
    else:
        outs["xp"] = torch.empty((rows, H), dtype=tdt, device=DEV)
    gbuf = torch.empty((slots, H), dtype=tdt, device=DEV) if gs else None
    part = torch.empty((slots, H), dtype=torch.bfloat16 if mode == "bf16_partials" else torch.float32,
                       device=DEV) if gs else None
    if mode == "backward":
        dout = dev(wl.expert_outputs((*key, 7), T, H, dt))
        dxp = dev(wl.expert_outputs((*key, 8), rows, H, dt))
        outs["dy"] = torch.empty((rows, H), dtype=tdt, device=DEV)
        outs["dw"] = torch.empty((T, K), dtype=torch.float32, device=DEV)
        outs["dx"] = torch.empty((T, H), dtype=tdt, device=DEV)
        outs["dlog"] = torch.empty((T, E), dtype=torch.float32, device=DEV)

    def step():
        m.route_topk_index(logits, K, capacity=cap, group_size=gs, alignment=align, route_group_size=gs if rg else 0,
                           topk_groups=rg, out=(gi, gw), index=ix)
        if mode == "fp8" and gs:
            m.permute_scatter_fp8(x, ix.slot_of, slots, block, out=(gq, gsc))
            m.permute_grouped_fp8(gq, gsc, ix.esrc, ix.row_of, out=(outs["xp"], outs["xs"]), src_of=ix.slot_src)
        elif mode == "fp8":
            m.permute_scatter_fp8(x, ix.row_of, rows, block, src_row=ix.sorted_indices,
                                  out=(outs["xp"], outs["xs"]))
        elif gs:
            m.permute_scatter(x, ix.slot_of, slots, out=gbuf)
            m.permute_grouped(gbuf, ix.esrc, ix.row_of, out=outs["xp"], src_of=ix.slot_src)
        else:
            m.permute_scatter(x, ix.row_of, rows, src_row=ix.sorted_indices, out=outs["xp"])
        if gs:
            m.group_precombine(y, ix.row_of, gw, gi, E, gs, ix.slot_of, out=part)
            m.unpermute_combine(part, ix.slot_of, None, out=outs["out"])
        else:
            m.unpermute_combine(y, ix.row_of, gw, out=outs["out"])
        if mode == "backward":
            m.unpermute_combine_backward(dout, y, ix.row_of, gw, src_row=ix.sorted_indices,
                                         out=(outs["dy"], outs["dw"]))
            if gs:
                m.group_precombine(dxp, ix.row_of, None, gi, E, gs, ix.slot_of, out=part)
                m.unpermute_combine(part, ix.slot_of, None, out=outs["dx"])
            else:
                m.unpermute_combine(dxp, ix.row_of, None, out=outs["dx"])
            m.route_topk_backward(gi, gw, outs["dw"], E, out=outs["dlog"])

    def results():
        live = host(ix.sorted_indices) >= 0  # rows that hold a token (pads and slack are not compared)
        r = {k: host(v).copy() for k, v in outs.items()}
        for k in ("xp", "xs", "dy"):
            if k in r:
                r[k] = r[k][live[: len(r[k])]]
        r.update(row_of=host(ix.row_of).copy(), gi=host(gi).copy(), gw=host(gw).copy(), live=live)
        return r

    step()
    torch.cuda.synchronize()
    want = results()
    assert want["live"].sum() > 0
    step()  # warm the allocator and the launch paths outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (*outs.values(), gi, gw, ix.row_of, ix.sorted_indices):
            t.zero_()  # eager fill kernels between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = results()
        for k, v in want.items():
            assert np.array_equal(got[k], v), f"replay {rep}: {k}"
    del g


def _random_config(i):
    g = np.random.default_rng([91, i])
    mode = ["standard", "drop", "group", "aligned"][i % 4]
    E = int(g.integers(1, 300))
    K = int(g.integers(1, min(E, 32) + 1))
    H = int(8 * g.integers(1, 1100)) if g.random() < 0.7 else int(g.integers(1, 600))
    T = int(g.integers(1, max(2, min(2500, 3_000_000 // (K * H)))))
    dtype = "bf16" if g.random() < 0.6 else "f32"
    cap = gs = align = M = 0
    if mode == "drop":
        cap = int(g.integers(1, max(2, 2 * T * K // E)))
    if mode == "group":
        divisors = [d for d in range(1, E + 1) if E % d == 0 and E // d <= 1024]
        gs = int(g.choice(divisors))
        G = E // gs
        if g.random() < 0.5 and G > 1:
            M = int(g.integers(1, G + 1))
            if K > M * gs:
                M = 0
        align = int(g.choice([0, 4])) if g.random() < 0.3 else 0
    if mode == "aligned":
        align = int(g.choice([2, 8, 16, 128]))
    ties = g.random() < 0.3
    zipf = 1.2 if g.random() < 0.5 else None
    pdt = "bf16" if mode == "group" and i % 8 == 6 else "f32"  # partials of the group pre-combine
    return dict(mode=mode, T=T, E=E, K=K, H=H, dtype=dtype, cap=cap, gs=gs, align=align, M=M, ties=ties, zipf=zipf,
                pdt=pdt)


@pytest.mark.parametrize("i", range(40))
def test_random_configuration(m, i):
    """Seeded random sizes and modes (standard, drop-and-pad, group with and without limited
    routing and alignment, aligned; float32 and bf16; hidden sizes with and without a 16-byte
    multiple; tie-heavy and skewed logits): the whole path against the oracle."""
    c = _random_config(i)
    T, E, K, H, dt, cap, gs, align, M = (c[k] for k in ("T", "E", "K", "H", "dtype", "cap", "gs", "align", "M"))
    say(f"random config {i}: {c}")
    key = wl.case_key(92, i)
    logits = tie_logits(key, T, E) if c["ties"] else wl.router_logits(key, T, E, zipf_s=c["zipf"])
    want_i, want_w = oracle.route_topk_grouped(logits, K, gs, M) if M else oracle.route_topk(logits, K)
    gi, gw = m.route_topk(dev(logits), K, group_size=gs if M else 0, topk_groups=M)
    assert_exact(host(gi), want_i, "topk_idx")
    assert_rel_f32(host(gw), want_w, "topk_w")
    w = host(gw)  # downstream, both sides use the same weight bits
    want = oracle.build_index(want_i, w, E, capacity=cap, group_size=gs, alignment=align)
    ix = m.build_index(gi, gw, E, capacity=cap, group_size=gs, alignment=align)
    for name in ("counts", "group_list", "kept_counts", "sorted_indices", "row_of", "permuted_probs"):
        assert_exact(host(getattr(ix, name)), want[name], name)
    rows = ix.rows
    x = wl.hidden_states(key, T, H, dt)
    y = wl.expert_outputs(key, rows, H, dt)
    out_dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    live = want["sorted_indices"] != -2
    if gs:
        n = int(host(ix.n_slots)[0])
        assert n == int(want["n_slots"][0])
        assert_exact(host(ix.gsrc)[:n], want["gsrc"], "gsrc")
        for name in ("slot_of", "esrc", "group_counts", "slot_src"):
            assert_exact(host(getattr(ix, name)), want[name], name)
        slots = T * min(K, E // gs)
        gbuf = m.permute_scatter(dev(x), ix.slot_of, slots)
        xp = m.permute_grouped(gbuf, ix.esrc, ix.row_of, src_of=ix.slot_src if i % 2 else None)
        p16 = c["pdt"] == "bf16"
        part = m.group_precombine(dev(y), ix.row_of, gw, gi, E, gs, ix.slot_of, slots_cap=slots,
                                  out_dtype=torch.bfloat16 if p16 else torch.float32)
        out = m.unpermute_combine(part, ix.slot_of, None, out_dtype=out_dtype)
        want_p = oracle.group_precombine(y, want["row_of"], w, want_i, E, gs, want["slot_of"], slots,
                                         out_dtype=np.uint16 if p16 else np.float32)
        want_o = oracle.unpermute_combine(want_p[:n], want["slot_of"], None, np.uint16 if dt == "bf16" else np.float32)
        assert_combined(host(part)[:n], want_p[:n], "partials")
    else:
        xp = m.permute_scatter(dev(x), ix.row_of, rows, src_row=ix.sorted_indices)
        out = m.unpermute_combine(dev(y), ix.row_of, gw)
        want_o = oracle.unpermute_combine(y, want["row_of"], w, np.uint16 if dt == "bf16" else np.float32)
    assert_exact(host(xp)[live], oracle.permute(x, want["sorted_indices"])[live], "permuted rows")
    assert_combined(host(out), want_o, "combined")


def test_binding_rejects_wrong_shapes_before_launch(m):
    """Output or side-input tensors whose shapes do not match the call raise ValueError in the
    binding (the kernels index them by the call's sizes), and nothing is written."""
    T, H, E, K, gs = 6, 64, 8, 2, 4
    G = E // gs
    i32 = dict(dtype=torch.int32, device=DEV)
    x = torch.ones((T, H), dtype=torch.bfloat16, device=DEV)
    row_of = torch.zeros((T, K), **i32)
    idx = torch.zeros((T, K), **i32)
    w = torch.ones((T, K), dtype=torch.float32, device=DEV)
    slot_of = torch.zeros((T, G), **i32)
    q_bad = torch.full((T, H - 8), 7, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        m.quantize_fp8(x, 32, out=(q_bad, torch.empty((T, H // 32), dtype=torch.float32, device=DEV)))
    with pytest.raises(ValueError):
        m.quantize_fp8(x, 32, out=(torch.empty((T, H), dtype=torch.uint8, device=DEV),
                                   torch.empty((T, 1), dtype=torch.float32, device=DEV)))
    part = torch.empty((T * G, H), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):  # weights not [T, K]
        m.group_precombine(x, row_of, w[:, :1].contiguous(), idx, E, gs, slot_of, out=part)
    with pytest.raises(ValueError):  # topk_idx not [T, K]
        m.group_precombine(x, row_of, w, idx[:3].contiguous(), E, gs, slot_of, out=part)
    with pytest.raises(ValueError):  # slot_of not [T, G]
        m.group_precombine(x, row_of, w, idx, E, gs, torch.zeros((T, G + 1), **i32), out=part)
    with pytest.raises(ValueError):  # partial rows of another length
        m.group_precombine(x, row_of, w, idx, E, gs, slot_of, out=torch.empty((T * G, H // 2), dtype=torch.float32,
                                                                              device=DEV))
    with pytest.raises(ValueError):  # group size not dividing E
        m.group_precombine(x, row_of, w, idx, E, 3, slot_of, out=part)
    with pytest.raises(ValueError):  # preallocated index for other sizes
        m.build_index(idx, w, E, out=m.alloc_index(T + 1, K, E))
    torch.cuda.synchronize()
    assert (q_bad == 7).all()


# ------------------------------------------------------------------ backward


def _dw_bound(dout, y, row_of, H, chunk=512):
    """Error bound of the kernel's fixed-order float32 dot: at most ceil(H/64) + 30 roundings
    along any product's path (per-lane chain, wavefront butterfly, wavefronts), each at most
    2^-24 of the sum of |products|; plus the oracle's own rounding to float32. Computed in token
    chunks so that full-size workloads fit in host memory."""
    T, K = row_of.shape
    mag = np.zeros((T, K), np.float64)
    for a in range(0, T, chunk):
        b = min(a + chunk, T)
        d = np.abs(wl.bf16_bits_to_f32(dout[a:b]) if dout.dtype == np.uint16 else dout[a:b]).astype(np.float64)
        r = row_of[a:b]
        ok = (r >= 0) & (r < len(y))
        yc = y[np.where(ok, r, 0)]
        yy = np.abs(wl.bf16_bits_to_f32(yc) if y.dtype == np.uint16 else yc).astype(np.float64)
        mag[a:b] = np.where(ok, np.einsum("th,tkh->tk", d, yy), 0.0)
    return (-(-H // 64) + 30) * 2.0 ** -24 * mag + 2.0 ** -130


def _check_dw(got, want, bound):
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert (diff <= bound + 2.0 ** -24 * np.abs(want.astype(np.float64))).all(), float((diff - bound).max())


@pytest.mark.parametrize("dts", [("bf16", "bf16", "bf16"), ("f32", "f32", "f32"), ("bf16", "bf16", "f32"),
                                 ("f32", "bf16", "bf16")])
@pytest.mark.parametrize("H,T,E,K,mode", [(7168, 130, 64, 8, "standard"), (1000, 200, 16, 4, "drop"),
                                          (5, 90, 8, 2, "holes"), (520, 150, 32, 8, "holes"), (8, 300, 8, 2, "drop"),
                                          (4096, 64, 128, 16, "standard"), (8, 1000, 16, 8, "standard"),
                                          (1000, 300, 16, 5, "standard"), (264, 70, 64, 32, "standard")])
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_backward(m, dts, H, T, E, K, mode, weighted):
    ddt, ydt, dydt = dts
    say(f"combine_backward dout={ddt} y={ydt} dy={dydt} H={H} T={T} E={E} K={K} {mode} weighted={weighted}")
    key = wl.case_key(33, H, T, E, K)
    logits = wl.router_logits(key, T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    if mode == "holes":
        idx[np.random.default_rng([*key, 4]).random((T, K)) < 0.2] = -1
    cap = oracle.capacity(T, K, E, 1, 2) if mode == "drop" else 0
    ix = oracle.build_index(idx, w, E, capacity=cap)
    rows = len(ix["sorted_indices"])
    y = wl.expert_outputs(key, rows, H, ydt)
    dout = wl.expert_outputs((*key, 1), T, H, ddt)
    ww = w if weighted else None
    dy_np = np.uint16 if dydt == "bf16" else np.float32
    want_dy, want_dw = oracle.combine_backward(dout, y, ix["row_of"], ww, dy_np)
    dy, dw = m.unpermute_combine_backward(dev(dout), dev(y), dev(ix["row_of"]), None if ww is None else dev(ww),
                                          src_row=dev(ix["sorted_indices"]),
                                          dy_dtype=torch.bfloat16 if dydt == "bf16" else torch.float32)
    live = ix["sorted_indices"] != -2  # unused slack is not written
    assert_exact(host(dy)[live], want_dy[live], "dy")
    _check_dw(host(dw), want_dw, _dw_bound(dout, y, ix["row_of"], H))
    assert (host(dw)[ix["row_of"] < 0] == 0).all()


def test_combine_backward_without_dw_and_without_zero_rows(m):
    key = wl.case_key(34)
    T, K, H, rows = 50, 2, 64, 130
    row_of = np.random.default_rng(1).permutation(rows)[: T * K].astype(np.int32).reshape(T, K)
    dout = wl.expert_outputs(key, T, H, "bf16")
    want_dy, _ = oracle.combine_backward(dout, np.zeros((rows, H), np.uint16), row_of, None, np.uint16, want_dw=False)
    out = dev(np.full((rows, H), 0x1234, np.uint16))
    dy, dw = m.unpermute_combine_backward(dev(dout), None, dev(row_of), num_rows=rows, want_dw=False,
                                          out=(out, None))
    assert dw is None
    got = host(dy)
    named = np.zeros(rows, bool)
    named[row_of.reshape(-1)] = True
    assert_exact(got[named], want_dy[named], "named rows")
    assert (got[~named] == 0x1234).all()  # no gather map: other rows untouched


@pytest.mark.parametrize("T,E,K,holes", [(1, 8, 1, False), (333, 64, 8, False), (1000, 256, 8, True),
                                         (77, 1000, 32, False), (50, 5, 5, True), (513, 128, 2, False)])
def test_route_topk_backward(m, T, E, K, holes):
    say(f"route_backward T={T} E={E} K={K} holes={holes}")
    key = wl.case_key(35, T, E, K)
    logits = wl.router_logits(key, T, E, zipf_s=1.0)
    idx, w = oracle.route_topk(logits, K)
    if holes:
        idx[np.random.default_rng([*key, 2]).random((T, K)) < 0.2] = -1
    g = wl.random_weights((*key, 3), T, K) - 0.5
    want = oracle.route_topk_backward(idx, w, g, E)
    got = host(m.route_topk_backward(dev(idx), dev(w), dev(g), E))
    assert_exact(got, want, "d_logits")


@pytest.mark.parametrize("i", range(24))
def test_random_configuration_backward(m, i):
    """The backward over seeded random configurations (the sizes and modes of the forward sweep;
    dout, dy and y dtypes drawn independently): combine backward (dy bit for bit, dw within the
    dot-product bound), dispatch backward (the unit-weight combine, or pre-combine + final sum in
    group mode) and the router backward, all against the oracle."""
    c = _random_config(100 + i)
    T, E, K, H, cap, gs, align = (c[k] for k in ("T", "E", "K", "H", "cap", "gs", "align"))
    g = np.random.default_rng([93, i])
    ddt, ydt, dydt = (("bf16", "f32")[int(g.random() < 0.4)] for _ in range(3))
    say(f"random backward {i}: {c} dout={ddt} y={ydt} dy={dydt}")
    key = wl.case_key(94, i)
    logits = tie_logits(key, T, E) if c["ties"] else wl.router_logits(key, T, E, zipf_s=c["zipf"])
    gi, gw = m.route_topk(dev(logits), K)
    w = host(gw)
    idx = host(gi)
    ix = m.build_index(gi, gw, E, capacity=cap, group_size=gs, alignment=align)
    want = oracle.build_index(idx, w, E, capacity=cap, group_size=gs, alignment=align)
    rows = ix.rows
    y = wl.expert_outputs(key, rows, H, ydt)
    dout = wl.expert_outputs((*key, 1), T, H, ddt)
    dxp = wl.expert_outputs((*key, 2), rows, H, ydt)
    dy_np = np.uint16 if dydt == "bf16" else np.float32
    want_dy, want_dw = oracle.combine_backward(dout, y, want["row_of"], w, dy_np)
    dy, dw = m.unpermute_combine_backward(dev(dout), dev(y), ix.row_of, gw, src_row=ix.sorted_indices,
                                          dy_dtype=torch.bfloat16 if dydt == "bf16" else torch.float32)
    live = want["sorted_indices"] != -2
    assert_exact(host(dy)[live], want_dy[live], "dy")
    got_dw = host(dw)
    _check_dw(got_dw, want_dw, _dw_bound(dout, y, want["row_of"], H))
    # the dispatch's backward: expert-row gradients back to token order with unit weights
    out_np = np.uint16 if ydt == "bf16" else np.float32
    if gs:
        n = int(want["n_slots"][0])
        slots = T * min(K, E // gs)
        part = m.group_precombine(dev(dxp), ix.row_of, None, gi, E, gs, ix.slot_of, slots_cap=slots)
        dx = m.unpermute_combine(part, ix.slot_of, None, out_dtype=torch.bfloat16 if ydt == "bf16" else torch.float32)
        want_p = oracle.group_precombine(dxp, want["row_of"], None, idx, E, gs, want["slot_of"], slots)
        want_dx = oracle.unpermute_combine(want_p[:n], want["slot_of"], None, out_np)
    else:
        dx = m.unpermute_combine(dev(dxp), ix.row_of, None)
        want_dx = oracle.unpermute_combine(dxp, want["row_of"], None, out_np)
    assert_combined(host(dx), want_dx, "dx")
    # the router's backward, fed the kernel's own dw (the same bits on both sides)
    assert_exact(host(m.route_topk_backward(gi, gw, dw, E)), oracle.route_topk_backward(idx, w, got_dw, E),
                 "d_logits")


@pytest.mark.parametrize("i", range(16))
def test_random_configuration_fp8(m, i):
    """The fused FP8 dispatch over seeded random configurations whose hidden size allows it
    (a multiple of 8, 16-byte rows): codes and scales equal the oracle's quantization moved by
    the oracle's gather, in standard, drop-and-pad, aligned and group (send + receive) modes."""
    j = 200 + i
    c = _random_config(j)
    while c["H"] % 8:
        j += 1000
        c = _random_config(j)
    T, E, K, H, dt, cap, gs, align = (c[k] for k in ("T", "E", "K", "H", "dtype", "cap", "gs", "align"))
    blocks = [b for b in (8, 16, 32, 64, 128, 256, 512, 1024) if H % b == 0]
    block = blocks[i % len(blocks)]
    say(f"random fp8 {i}: {c} block={block}")
    key = wl.case_key(95, i)
    logits = wl.router_logits(key, T, E, zipf_s=c["zipf"])
    gi, gw = m.route_topk(dev(logits), K)
    idx, w = host(gi), host(gw)
    ix = m.build_index(gi, gw, E, capacity=cap, group_size=gs, alignment=align)
    want = oracle.build_index(idx, w, E, capacity=cap, group_size=gs, alignment=align)
    x = fp8_inputs(key, T, H, dt)
    qs, ss = oracle.quantize_fp8(x, block)
    si = want["sorted_indices"]
    live = si != -2
    if gs:
        n = int(want["n_slots"][0])
        slots = T * min(K, E // gs)
        q, sc = m.permute_scatter_fp8(dev(x), ix.slot_of, slots, block)
        assert_exact(host(q)[:n], oracle.permute(qs, want["gsrc"]), "slot codes")
        assert_exact(host(sc)[:n], oracle.permute(ss, want["gsrc"]), "slot scales")
        if i % 2:  # the fused receive, or the codes and scales moved one after the other
            rq, rs = (host(a) for a in m.permute_grouped_fp8(q, sc, ix.esrc, ix.row_of))
        else:
            rq = host(m.permute_grouped(q, ix.esrc, ix.row_of))
            rs = host(m.permute_grouped(sc, ix.esrc, ix.row_of))
    else:
        q, sc = m.permute_scatter_fp8(dev(x), ix.row_of, ix.rows, block, src_row=ix.sorted_indices)
        rq, rs = host(q), host(sc)
    assert_exact(rq[live], oracle.permute(qs, si)[live], "codes")
    assert_exact(rs[live], oracle.permute(ss, si)[live], "scales")


def test_backward_no_tokens(m):
    d = m.route_topk_backward(torch.zeros((0, 2), dtype=torch.int32, device=DEV),
                              torch.zeros((0, 2), dtype=torch.float32, device=DEV),
                              torch.zeros((0, 2), dtype=torch.float32, device=DEV), 8)
    torch.cuda.synchronize()
    assert d.shape == (0, 8)
    # no tokens but a gather map: every row of dy fed nothing and is zero
    dy, dw = m.unpermute_combine_backward(torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV),
                                          torch.ones((5, 16), dtype=torch.bfloat16, device=DEV),
                                          torch.zeros((0, 2), dtype=torch.int32, device=DEV),
                                          src_row=torch.full((5,), -1, dtype=torch.int32, device=DEV),
                                          out=(torch.ones((5, 16), dtype=torch.bfloat16, device=DEV), None))
    assert (host(dy) == 0).all() and dw.shape == (0, 2)


@pytest.mark.parametrize("cfg_id,bf16_partials", [(2, False), (3, False), (4, False), (4, True), (5, False)])
def test_backward_workload(m, cfg_id, bf16_partials):
    """Backward at the named workloads' full size, in the launch configuration bench.py --backward
    times, every output against the oracle: every dy row bit for bit (padding rows zero), every dw
    within the dot-product bound, the dispatch backward (the unit-weight combine; in group mode the
    unit-weight pre-combine and the final sum, float32 or bf16 partials) and the router gradient
    bit for bit."""
    c = wl.WORKLOADS[cfg_id]
    T, H, E, K, dt, gs = c["T"], c["H"], c["E"], c["K"], c["dtype"], c["group_size"]
    say(f"backward workload {cfg_id}: {c['name']} bf16_partials={bf16_partials}")
    key = wl.workload_key(cfg_id)
    cap = oracle.capacity(T, K, E, *c["cf"]) if c["cf"] else 0
    logits = wl.router_logits(key, T, E, zipf_s=c["zipf_s"])
    gi, gw, ix, idx_np, w_np, want = check_route_and_index(m, c, logits, 0, cap, 0)
    rows = ix.rows
    live = want["sorted_indices"] != -2
    out_np = np.uint16 if dt == "bf16" else np.float32
    y = wl.expert_outputs(key, rows, H, dt)
    dout = wl.expert_outputs((*key, 7), T, H, dt)
    dy, dw = m.unpermute_combine_backward(dev(dout), dev(y), ix.row_of, gw, src_row=ix.sorted_indices)
    want_dy, want_dw = oracle.combine_backward(dout, y, want["row_of"], w_np, out_np)
    assert_rows_exact(dy, want_dy, "dy", live)
    del dy, want_dy
    dw_np = host(dw)
    _check_dw(dw_np, want_dw, _dw_bound(dout, y, want["row_of"], H))
    assert (dw_np[want["row_of"] < 0] == 0).all()
    del y
    dxp = wl.expert_outputs((*key, 8), rows, H, dt)
    if gs:
        n = int(want["n_slots"][0])
        slots = T * min(K, E // gs)
        p_np = np.uint16 if bf16_partials else np.float32
        part = m.group_precombine(dev(dxp), ix.row_of, None, gi, E, gs, ix.slot_of, slots_cap=slots,
                                  out_dtype=torch.bfloat16 if bf16_partials else torch.float32)
        want_p = oracle.group_precombine(dxp, want["row_of"], None, idx_np, E, gs, want["slot_of"], n, out_dtype=p_np)
        assert_combined_all(part[:n], want_p, "dispatch backward partials")
        dx = m.unpermute_combine(part, ix.slot_of, None, out_dtype=torch.bfloat16 if dt == "bf16" else torch.float32)
        want_dx = oracle.unpermute_combine(want_p, want["slot_of"], None, out_np)
    else:
        dx = m.unpermute_combine(dev(dxp), ix.row_of, None)
        want_dx = oracle.unpermute_combine(dxp, want["row_of"], None, out_np)
    assert_combined_all(dx, want_dx, "dispatch backward")
    dlog = m.route_topk_backward(gi, gw, dw, E)
    assert_exact(host(dlog), oracle.route_topk_backward(idx_np, w_np, dw_np, E), "router gradient")
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ determinism


def _bits(t):
    """Bit pattern of a device tensor (so that -0.0 and +0.0, or two NaNs, are told apart)."""
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t


def _poison_like(t):
    """A tensor of t's shape and dtype filled with 0xFF bytes: entries a run fails to write differ."""
    p = torch.empty_like(t)
    p.view(torch.uint8).fill_(0xFF)
    return p


def _same_bits(a, b, what, live=None):
    if live is not None:
        a, b = a[live], b[live]
    assert torch.equal(_bits(a), _bits(b)), f"{what}: two runs differ"


@pytest.mark.parametrize("case", ["workload3", "workload4_group", "workload3_backward", "workload5_drop"])
def test_pipeline_is_deterministic(m, case):
    """No atomics decide positions or sums: the same step run twice -- the second time into
    output buffers filled with 0xFF bytes -- gives identical bits in every index array, every
    dispatched row, every partial and every output (workload 3 forward; workload 4 group mode with
    its partials and final sum; workload 3 backward with dy, dw and the router gradient; workload
    5 drop-and-pad)."""
    cfg_id = {"workload3": 3, "workload4_group": 4, "workload3_backward": 3, "workload5_drop": 5}[case]
    backward = case.endswith("backward")
    c = wl.WORKLOADS[cfg_id]
    T, H, E, K, dt, gs = c["T"], c["H"], c["E"], c["K"], c["dtype"], c["group_size"]
    say(f"determinism {case}")
    key = wl.workload_key(cfg_id)
    cap = m.expert_capacity(T, K, E, *c["cf"]) if c["cf"] else 0
    rows = m.index_rows(T, K, E, cap, 0)
    logits = dev(wl.router_logits(key, T, E, zipf_s=c["zipf_s"]))
    x = dev(wl.hidden_states(key, T, H, dt))
    y = dev(wl.expert_outputs(key, rows, H, dt))
    G = E // gs if gs else 0
    slots = T * min(K, G) if gs else 0
    dout = dev(wl.expert_outputs((*key, 7), T, H, dt)) if backward else None

    def run(prev=None):
        P = (lambda t: _poison_like(t)) if prev is not None else (lambda t: torch.empty_like(t))
        r = {}
        ix = m.alloc_index(T, K, E, cap, gs)
        for f in ("counts", "group_list", "kept_counts", "sorted_indices", "row_of", "permuted_probs", "slot_of",
                  "gsrc", "esrc", "group_counts", "n_slots", "slot_src"):
            t = getattr(ix, f)
            if t is not None and prev is not None:
                t.view(torch.uint8).fill_(0xFF)
        gi, gw, _ = m.route_topk_index(logits, K, capacity=cap, group_size=gs,
                                       out=(P(torch.empty((T, K), dtype=torch.int32, device=DEV)),
                                            P(torch.empty((T, K), dtype=torch.float32, device=DEV))), index=ix)
        r.update(gi=gi, gw=gw, **{f: getattr(ix, f) for f in ("counts", "group_list", "kept_counts", "sorted_indices",
                                                              "row_of", "permuted_probs")})
        if gs:
            n = int(ix.n_slots.item())
            r.update(slot_of=ix.slot_of, esrc=ix.esrc, group_counts=ix.group_counts, n_slots=ix.n_slots,
                     gsrc=ix.gsrc[:n], slot_src=ix.slot_src)
            gbuf = m.permute_scatter(x, ix.slot_of, slots, out=P(torch.empty((slots, H), dtype=x.dtype, device=DEV)))
            r["gbuf"] = gbuf[:n]
            r["xp"] = m.permute_grouped(gbuf, ix.esrc, ix.row_of, src_of=ix.slot_src, out=P(torch.empty((rows, H), dtype=x.dtype,
                                                                                  device=DEV)))
            part = m.group_precombine(y, ix.row_of, gw, gi, E, gs, ix.slot_of,
                                      out=P(torch.empty((slots, H), dtype=torch.float32, device=DEV)))
            r["partials"] = part[:n]
            r["out"] = m.unpermute_combine(part, ix.slot_of, None, out=P(torch.empty((T, H), dtype=x.dtype,
                                                                                     device=DEV)))
        else:
            r["xp"] = m.permute_scatter(x, ix.row_of, rows, src_row=ix.sorted_indices,
                                        out=P(torch.empty((rows, H), dtype=x.dtype, device=DEV)))
            r["out"] = m.unpermute_combine(y, ix.row_of, gw, out=P(torch.empty((T, H), dtype=x.dtype, device=DEV)))
        if backward:
            dy, dw = m.unpermute_combine_backward(dout, y, ix.row_of, gw, src_row=ix.sorted_indices,
                                                  out=(P(torch.empty((rows, H), dtype=x.dtype, device=DEV)),
                                                       P(torch.empty((T, K), dtype=torch.float32, device=DEV))))
            r.update(dy=dy, dw=dw, dlog=m.route_topk_backward(
                gi, gw, dw, E, out=P(torch.empty((T, E), dtype=torch.float32, device=DEV))))
        torch.cuda.synchronize()
        return r

    a = run()
    b = run(prev=a)
    live = a["sorted_indices"] != -2
    assert bool(live.all()), "these layouts have no unused slack"
    for k in a:
        _same_bits(a[k], b[k], k)
    del a, b
    torch.cuda.empty_cache()
