"""Pins of the CPU oracle against values the pages print (tests/golden) and closed forms.

Every expected value here is either printed on the pages (loaded from tests/golden with its
citation) or follows from mathematics independent of the oracle's code (closed forms,
exact rational arithmetic).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl
from conftest import load_golden


def ids_from_routing_map(rmap):
    """Convert a [T, E] 0/1 routing map into [T, K] expert ids padded with -1."""
    rmap = np.asarray(rmap)
    K = int(rmap.sum(axis=1).max())
    ids = np.full((rmap.shape[0], K), -1, np.int32)
    for t in range(rmap.shape[0]):
        es = np.nonzero(rmap[t])[0]
        ids[t, : len(es)] = es
    return ids


def letter_rows(letters, H=8):
    """Distinct float32 rows standing for the pages' letters A, B, ... (A' etc. too)."""
    rows = []
    for name in letters:
        base = (ord(name[0]) - ord("A") + 1) * 16 + (0.5 if name.endswith("'") else 0.0)
        rows.append(np.arange(H, dtype=np.float32) / 64.0 + np.float32(base))
    return np.asarray(rows, np.float32)


def test_megatron_routing_map_example():
    g = load_golden("megatron_permute_example.json")
    ids = ids_from_routing_map(g["routing_map"])
    E = len(g["routing_map"][0])
    ix = oracle.build_index(ids, None, E)
    R = len(g["sorted_indices"])
    assert ix["sorted_indices"][:R].tolist() == g["sorted_indices"]
    assert ix["sorted_indices"][R:].tolist() == [-2] * (ids.size - R)  # unused slack after the last segment
    assert ix["counts"].tolist() == [len(r) for r in g["expert_receives"]]
    # every routed (token, expert) pair finds its own token at its row
    for t in range(ids.shape[0]):
        for k in range(ids.shape[1]):
            r = ix["row_of"][t, k]
            if ids[t, k] < 0:
                assert r == -1
            else:
                assert ix["sorted_indices"][r] == t
    tokens = letter_rows("ABCD")
    out = oracle.permute(tokens, ix["sorted_indices"][:R])
    assert np.array_equal(out, tokens[g["permuted_input_rows"]])


def test_group_list_example():
    g = load_golden("group_list_example.json")
    experts = np.repeat(np.arange(len(g["counts"])), g["counts"]).astype(np.int32)[:, None]
    ix = oracle.build_index(experts, None, len(g["counts"]))
    assert ix["counts"].tolist() == g["counts"]
    assert ix["group_list"].tolist() == g["group_list"]
    starts = (ix["group_list"] - ix["counts"]).tolist()
    assert [[s, e] for s, e in zip(starts, ix["group_list"].tolist())] == g["ranges"]


def test_rank_major_to_expert_major_example():
    g = load_golden("rank_major_example.json")
    ids = np.asarray(g["rank_major_experts"], np.int32)[:, None]
    ix = oracle.build_index(ids, None, 2)
    assert ix["sorted_indices"].tolist() == g["permute_indices"]
    assert ix["counts"].tolist() == g["counts"]
    assert ix["group_list"].tolist() == g["group_list"]
    rows = letter_rows(g["rank_major"])
    out = oracle.permute(rows, ix["sorted_indices"])
    assert np.array_equal(out, letter_rows(g["expert_major"]))


def test_stable_permute_example():
    g = load_golden("stable_permute_example.json")
    ids = np.asarray(g["experts"], np.int32)[:, None]
    ix = oracle.build_index(ids, None, 2)
    out = oracle.permute(letter_rows(g["tokens"]), ix["sorted_indices"])
    assert np.array_equal(out, letter_rows(g["permuted"]))


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_unpermute_example_is_exact(dtype):
    """K = 1 and unit weights: the combine is the unpermute restored[perm] = y, bit for bit."""
    g = load_golden("unpermute_example.json")
    rank_major_experts = load_golden("rank_major_example.json")["rank_major_experts"]
    ids = np.asarray(rank_major_experts, np.int32)[:, None]
    ix = oracle.build_index(ids, None, 2)
    assert ix["sorted_indices"].tolist() == g["permute_indices"]
    y = letter_rows(g["expert_output"])
    want = letter_rows(g["restored"])
    if dtype == np.uint16:
        y, want = wl.f32_to_bf16_bits(y), wl.f32_to_bf16_bits(want)
    out = oracle.unpermute_combine(y, ix["row_of"], None, dtype)
    assert np.array_equal(out.view(np.uint8), want.view(np.uint8))


def test_weighted_merge_example():
    g = load_golden("weighted_merge_example.json")
    w = np.asarray([[float(v) for v in g["weights"]]], np.float32)
    out_1 = np.float32(1.75) * np.arange(1, 9, dtype=np.float32)
    out_3 = np.float32(-3.5) + np.arange(8, dtype=np.float32)
    y = np.stack([out_1, out_3])
    row_of = np.asarray([[0, 1]], np.int32)
    got = oracle.unpermute_combine(y, row_of, w, np.float32)[0]
    for h in range(8):
        exact = Fraction(g["weights"][0]) * Fraction(float(out_1[h])) + \
            Fraction(g["weights"][1]) * Fraction(float(out_3[h]))
        mag = abs(Fraction(g["weights"][0]) * Fraction(float(out_1[h]))) + \
            abs(Fraction(g["weights"][1]) * Fraction(float(out_3[h])))
        # two weight roundings to float32 plus two fused roundings
        assert abs(Fraction(float(got[h])) - exact) <= 4 * Fraction(1, 2 ** 24) * mag


def test_capacity_example():
    g = load_golden("capacity_example.json")
    cf = Fraction(g["capacity_factor"])
    T, K, E = g["tokens_per_rank"], g["top_k"], g["num_experts"]
    assert T * K // E == g["mean_per_expert"]
    assert oracle.capacity(T, K, E, cf.numerator, cf.denominator) == g["capacity"]


def test_capacity_rounds_up():
    assert oracle.capacity(8192, 8, 128, 5, 4) == 640
    assert oracle.capacity(10, 1, 3, 1, 1) == 4
    assert oracle.capacity(9, 1, 3, 1, 1) == 3
    assert oracle.capacity(0, 2, 8, 5, 4) == 0


def test_routed_token_count():
    g = load_golden("routed_tokens_example.json")
    T, K = g["T"], g["K"]
    ids = wl.random_topk_ids(wl.case_key(1), T, 8, K)
    ix = oracle.build_index(ids, None, 8)
    assert int(ix["counts"].sum()) == g["routed"]
    assert ix["group_list"][-1] == g["routed"]


def test_zero_token_expert():
    g = load_golden("zero_token_expert_example.json")
    cnt = g["tokens_per_expert"]
    ids = np.repeat(np.arange(len(cnt)), cnt).astype(np.int32)
    ids = np.random.default_rng(5).permutation(ids)[:, None]
    ix = oracle.build_index(ids, None, len(cnt))
    assert ix["counts"].tolist() == cnt
    gl = ix["group_list"].tolist()
    assert gl[1] == gl[0]  # the empty expert owns an empty range
    assert all(b >= a for a, b in zip(gl, gl[1:]))


# ------------------------------------------------------------------ routing closed forms


@pytest.mark.parametrize("E,K", [(8, 2), (64, 8), (256, 8), (5, 5), (3, 1)])
def test_route_equal_logits(E, K):
    """All logits equal: ties go to the lower ids and every weight is exactly float32(1/K)."""
    logits = np.full((3, E), 0.375, np.float32)
    logits[1] = -0.0
    logits[2, :] = 0.0
    logits[2, ::2] = -0.0  # +0 and -0 tie
    idx, w = oracle.route_topk(logits, K)
    assert (idx == np.arange(K)).all()
    assert (w == np.float32(1.0 / K)).all()


def test_route_k1_weight_is_one():
    logits = wl.router_logits(wl.case_key(2), 50, 16)
    idx, w = oracle.route_topk(logits, 1)
    assert (w == 1.0).all()
    assert (idx[:, 0] == np.argmax(logits, axis=1)).all()


def test_route_two_experts_is_logistic():
    """K = 2: w_0 = 1/(1 + exp(s_1 - s_0)), the logistic function of the score gap."""
    logits = wl.router_logits(wl.case_key(3), 200, 16)
    idx, w = oracle.route_topk(logits, 2)
    s0 = logits[np.arange(200), idx[:, 0]].astype(np.float64)
    s1 = logits[np.arange(200), idx[:, 1]].astype(np.float64)
    want0 = 1.0 / (1.0 + np.exp(s1 - s0))
    assert np.allclose(w[:, 0], want0, rtol=2 ** -23, atol=0)
    assert np.allclose(w[:, 1], 1.0 - want0, rtol=2 ** -22, atol=0)


def test_route_shift_invariance():
    """Adding the same constant to a token's logits changes neither selection nor weights."""
    g = np.random.default_rng(11)
    logits = (g.integers(-40, 40, size=(64, 32)) / 8.0).astype(np.float32)  # exact under +4
    i0, w0 = oracle.route_topk(logits, 4)
    i1, w1 = oracle.route_topk(logits + np.float32(4.0), 4)
    assert np.array_equal(i0, i1)
    assert np.allclose(w0, w1, rtol=2 ** -23, atol=0)


def test_route_weights_form_distribution():
    logits = wl.router_logits(wl.case_key(4), 300, 64, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, 8)
    assert np.allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=8 * 2 ** -24)
    assert (np.diff(w, axis=1) <= 0).all()  # descending score gives non-increasing weight
    s = np.take_along_axis(logits, idx, axis=1).astype(np.float64)
    ratio = w[:, 1:].astype(np.float64) / w[:, :1]
    assert np.allclose(ratio, np.exp(s[:, 1:] - s[:, :1]), rtol=3e-7)


def test_bf16_rounding_of_oracle():
    """Round to nearest even at the bf16 boundary (1 + 2^-8 is a tie)."""
    assert oracle.f32_to_bf16(1.0) == 0x3F80
    assert oracle.f32_to_bf16(1.0 + 2 ** -8) == 0x3F80  # tie -> even
    assert oracle.f32_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82  # tie -> even (up)
    assert oracle.f32_to_bf16(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81
    assert oracle.f32_to_bf16(-2.0) == 0xC000
    assert oracle.f32_to_bf16(float("inf")) == 0x7F80
    assert oracle.f32_to_bf16(3.3895313892515355e38) == 0x7F7F  # bf16 max stays finite
