"""The allocation-free index build (moe_build_index_noalloc, called through the C ABI) against
moe_build_index: every output array bit for bit, in every index mode, on two calls in a row --
the second with a smaller input, so that it runs on scratch the first call left behind -- and at
the largest plan (128 tiles of 1024 expert and 1024 group counts: the whole scratch)."""
import pytest

import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FIELDS = ("counts", "group_list", "kept_counts", "sorted_indices", "row_of", "permuted_probs")
GROUP_FIELDS = ("slot_of", "esrc", "group_counts", "n_slots")


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import unpermute_combine_amd as mod
    mod.lib()
    return mod


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _check_same(m, ids, w, E, cap, gs, align, what):
    ref = m.build_index(ids, w, E, capacity=cap, group_size=gs, alignment=align)
    got = m.build_index_noalloc(ids, w, E, capacity=cap, group_size=gs, alignment=align)
    torch.cuda.synchronize()
    for f in FIELDS + (GROUP_FIELDS if gs else ()):
        assert torch.equal(_bits(getattr(got, f)), _bits(getattr(ref, f))), f"{what}: {f}"
    if gs:
        n = int(ref.n_slots.item())
        assert torch.equal(got.gsrc[:n], ref.gsrc[:n]), f"{what}: gsrc"
    assert got.workspace is None


@pytest.mark.parametrize("mode", ["standard", "drop", "group", "aligned", "single_tile"])
def test_noalloc_index_equals_index_on_two_calls(m, mode):
    E, K = 256, 8
    cap = 300 if mode == "drop" else 0
    gs = 8 if mode == "group" else 0
    align = 128 if mode == "aligned" else 0
    sizes = (400, 100) if mode == "single_tile" else (20000, 3001)  # the second call smaller
    for call, T in enumerate(sizes):
        print(f"noalloc {mode} call {call} T={T}", flush=True)
        key = wl.case_key(600, call, T)
        ids = wl.random_topk_ids(key, T, E, K, p_missing=0.05)
        w = wl.random_weights(key, T, K)
        _check_same(m, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), E, cap, gs, align,
                    f"{mode} call {call}")


def test_noalloc_index_at_the_largest_plan(m):
    """E = 1024 experts in 1024 groups of one, enough tokens for 128 tiles: the plan fills the
    whole scratch; then a small call after it."""
    E, K = 1024, 8
    for call, T in enumerate((70000, 5000)):
        print(f"noalloc largest plan call {call} T={T}", flush=True)
        logits = wl.router_logits(wl.case_key(601, call), T, E, zipf_s=1.2)
        gi, gw = m.route_topk(torch.from_numpy(logits).to(DEV), K)
        ws = m.workspace_bytes(T, K, E, 1)
        if call == 0:
            assert ws == 128 * (1024 + 1024) * 4
        _check_same(m, gi, gw, E, 0, 1, 0, f"largest plan call {call}")


def test_noalloc_index_no_tokens(m):
    ids = torch.zeros((0, 2), dtype=torch.int32, device=DEV)
    _check_same(m, ids, None, 8, 0, 2, 0, "no tokens")


def test_noalloc_index_from_a_hip_graph(m):
    """Captured in a HIP graph (the callers it is for) and replayed three times with eager work
    between the replays: every replay equals the eager build with a workspace."""
    T, E, K, gs = 8192, 256, 8, 8
    key = wl.case_key(602)
    ids = torch.from_numpy(wl.random_topk_ids(key, T, E, K)).to(DEV)
    w = torch.from_numpy(wl.random_weights(key, T, K)).to(DEV)
    ref = m.build_index(ids, w, E, group_size=gs)
    ix = m.alloc_index(T, K, E, 0, gs, workspace=False)
    m.build_index_noalloc(ids, w, E, group_size=gs, out=ix)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            m.build_index_noalloc(ids, w, E, group_size=gs, out=ix)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for f in FIELDS + GROUP_FIELDS + ("gsrc",):
            getattr(ix, f).zero_()
        # other work between the replays, on the same scratch: a smaller eager allocation-free build
        m.build_index_noalloc(ids[: T // 2].contiguous(), w[: T // 2].contiguous(), E, group_size=gs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for f in FIELDS + GROUP_FIELDS:
            assert torch.equal(_bits(getattr(ix, f)), _bits(getattr(ref, f))), f"replay {rep}: {f}"
    del g
