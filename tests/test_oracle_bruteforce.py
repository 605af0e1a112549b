"""Brute force and invariants for the CPU oracle on tiny inputs.

The brute-force side uses formulations other than the oracle's: a full sort of
(expert, token, slot) tuples instead of a masked scan, a full sort of experts by
(-score, id) instead of repeated selection, exact rational sums instead of float FMA chains.
"""
from fractions import Fraction
from itertools import accumulate

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
import workloads as wl


def brute_index(ids, E, cap=0, gs=0, w=None, align=0):
    """The index by sorting (expert, token, slot) tuples and laying the segments out directly:
    drop-and-pad rows e*cap + p; otherwise segments back to back, each rounded up to a multiple
    of `align` (padding rows -1), rows after the last segment -2 (unused slack)."""
    T, K = ids.shape
    slots = sorted((int(ids[t, k]), t, k) for t in range(T) for k in range(K)
                   if 0 <= ids[t, k] < E)
    counts = [0] * E
    for e, _, _ in slots:
        counts[e] += 1
    A = align if align > 1 else 1
    row_of = -np.ones((T, K), np.int64)
    if cap > 0:
        gl = list(accumulate(counts))
        sorted_idx = -np.ones(E * cap, np.int64)
        pos = [0] * E
        for e, t, k in slots:
            if pos[e] < cap:
                sorted_idx[e * cap + pos[e]] = t
                row_of[t, k] = e * cap + pos[e]
            pos[e] += 1
        total = E * cap
    else:
        seglen = [-(-c // A) * A for c in counts]
        gl = list(accumulate(seglen))
        starts = [g - n for g, n in zip(gl, seglen)]
        total = gl[-1] if E else 0
        sorted_idx = np.full(T * K + E * (A - 1), -2, np.int64)
        sorted_idx[:total] = -1
        pos = [0] * E
        for e, t, k in slots:
            sorted_idx[starts[e] + pos[e]] = t
            row_of[t, k] = starts[e] + pos[e]
            pos[e] += 1
    probs = np.zeros(len(sorted_idx), np.float32)
    for e, t, k in slots:
        if row_of[t, k] >= 0:
            probs[row_of[t, k]] = 1.0 if w is None else w[t, k]
    out = dict(counts=counts, group_list=gl, sorted_indices=sorted_idx.tolist(),
               row_of=row_of.tolist(), permuted_probs=probs)
    if gs > 0:
        G = E // gs
        pairs = sorted({(e // gs, t) for e, t, _ in slots})
        slot_of = -np.ones((T, G), np.int64)
        for m, (g, t) in enumerate(pairs):
            slot_of[t, g] = m
        esrc = np.where(np.arange(len(sorted_idx)) < total, -1, -2)
        slot_src = -np.ones((T, K), np.int64)
        for e, t, k in slots:
            esrc[row_of[t, k]] = slot_of[t, e // gs]
            slot_src[t, k] = slot_of[t, e // gs]
        out.update(gsrc=[t for _, t in pairs], slot_of=slot_of.tolist(),
                   esrc=esrc.tolist(), slot_src=slot_src.tolist(), n_slots=len(pairs),
                   group_counts=[sum(1 for g, _ in pairs if g == gg) for gg in range(G)])
    return out


@st.composite
def routing(draw, max_t=12, max_e=9, max_k=4, allow_missing=True):
    E = draw(st.integers(1, max_e))
    K = draw(st.integers(1, min(max_k, E)))
    T = draw(st.integers(0, max_t))
    ids = np.full((T, K), -1, np.int32)
    for t in range(T):
        perm = draw(st.permutations(list(range(E))))
        ids[t] = perm[:K]
        if allow_missing:
            for k in range(K):
                if draw(st.integers(0, 5)) == 0:
                    ids[t, k] = -1
    return ids, E


@settings(max_examples=300, deadline=None)
@given(routing(), st.booleans())
def test_index_matches_tuple_sort(case, weighted):
    ids, E = case
    w = np.random.default_rng(ids.size).random(ids.shape).astype(np.float32) if weighted else None
    ix = oracle.build_index(ids, w, E)
    bf = brute_index(ids, E, w=w)
    assert ix["counts"].tolist() == bf["counts"]
    assert ix["group_list"].tolist() == bf["group_list"]
    assert ix["sorted_indices"].tolist() == bf["sorted_indices"]
    assert ix["row_of"].tolist() == bf["row_of"]
    assert np.array_equal(ix["permuted_probs"], bf["permuted_probs"])


@st.composite
def repeated_routing(draw, max_t=10, max_e=6, max_k=5):
    """Rows whose expert ids may repeat (drawn with replacement) or be missing."""
    E = draw(st.integers(1, max_e))
    K = draw(st.integers(1, min(max_k, E)))  # K <= E, as the calls require; ids may still repeat
    T = draw(st.integers(0, max_t))
    ids = np.asarray([[draw(st.integers(-1, E - 1)) for _ in range(K)] for _ in range(T)], np.int32).reshape(T, K)
    return ids, E


@settings(max_examples=300, deadline=None)
@given(repeated_routing(), st.sampled_from([0, 1, 2, 3]), st.sampled_from([0, 2, 4]), st.sampled_from([0, 1, 2]))
def test_repeated_experts_are_ordered_by_slot(case, cap, align, gs):
    """An expert named twice in one row (outside the pages' routing map, which cannot say it)
    gets one row per slot, in slot order: the index equals the sort of (expert, token, slot)."""
    ids, E = case
    if gs and E % gs:
        gs = 1
    if cap:
        align = gs = 0
    w = np.random.default_rng(ids.size + 7).random(ids.shape).astype(np.float32)
    ix = oracle.build_index(ids, w, E, capacity=cap, group_size=gs, alignment=align)
    bf = brute_index(ids, E, cap=cap, gs=gs, w=w, align=align)
    assert ix["counts"].tolist() == bf["counts"]
    assert ix["sorted_indices"].tolist() == bf["sorted_indices"]
    assert ix["row_of"].tolist() == bf["row_of"]
    assert np.array_equal(ix["permuted_probs"], bf["permuted_probs"])
    if gs:
        assert ix["gsrc"].tolist() == bf["gsrc"] and ix["slot_of"].tolist() == bf["slot_of"]
        assert ix["esrc"].tolist() == bf["esrc"]
        assert ix["slot_src"].tolist() == bf["slot_src"]


@settings(max_examples=200, deadline=None)
@given(routing(), st.integers(1, 5))
def test_drop_and_pad_matches_tuple_sort(case, cap):
    ids, E = case
    w = np.random.default_rng(ids.size + 1).random(ids.shape).astype(np.float32)
    ix = oracle.build_index(ids, w, E, capacity=cap)
    bf = brute_index(ids, E, cap=cap, w=w)
    assert np.array_equal(ix["permuted_probs"], bf["permuted_probs"])
    assert ix["counts"].tolist() == bf["counts"]
    assert ix["sorted_indices"].tolist() == bf["sorted_indices"]
    assert ix["row_of"].tolist() == bf["row_of"]
    assert ix["kept_counts"].tolist() == [min(c, cap) for c in bf["counts"]]
    pp = ix["permuted_probs"]
    assert (pp[np.asarray(bf["sorted_indices"]) < 0] == 0).all()


@settings(max_examples=200, deadline=None)
@given(routing(max_e=12), st.sampled_from([1, 2, 3, 4, 6, 12]))
def test_group_mode_matches_pair_sort(case, gs):
    ids, E = case
    if E % gs:
        gs = 1
    ix = oracle.build_index(ids, None, E, group_size=gs)
    bf = brute_index(ids, E, gs=gs)
    assert ix["gsrc"].tolist() == bf["gsrc"]
    assert ix["slot_of"].tolist() == bf["slot_of"]
    assert ix["esrc"].tolist() == bf["esrc"]
    assert ix["slot_src"].tolist() == bf["slot_src"]
    assert int(ix["n_slots"][0]) == bf["n_slots"]
    assert ix["group_counts"].tolist() == bf["group_counts"]


@settings(max_examples=200, deadline=None)
@given(routing(max_e=8), st.sampled_from([2, 3, 4, 8, 128]), st.sampled_from([0, 1, 2, 4]))
def test_aligned_index_matches_tuple_sort(case, align, gs):
    ids, E = case
    if gs and E % gs:
        gs = 1
    w = np.random.default_rng(ids.size + 2).random(ids.shape).astype(np.float32)
    ix = oracle.build_index(ids, w, E, group_size=gs, alignment=align)
    bf = brute_index(ids, E, gs=gs, w=w, align=align)
    assert ix["counts"].tolist() == bf["counts"]
    assert ix["group_list"].tolist() == bf["group_list"]
    assert ix["sorted_indices"].tolist() == bf["sorted_indices"]
    assert ix["row_of"].tolist() == bf["row_of"]
    assert np.array_equal(ix["permuted_probs"], bf["permuted_probs"])
    if gs:
        assert ix["esrc"].tolist() == bf["esrc"]
        assert ix["gsrc"].tolist() == bf["gsrc"]
        assert ix["slot_src"].tolist() == bf["slot_src"]
    gl = np.concatenate([[0], ix["group_list"]])
    assert (gl % align == 0).all()  # every segment starts (and ends) at a multiple of the alignment
    assert (np.diff(gl) - ix["counts"] >= 0).all() and (np.diff(gl) - ix["counts"] < align).all()


def test_aligned_hand_example():
    """[Scratch] §7's counts [3,2,4] laid out with alignment 4 (derived by hand): segments of 4,
    4 and 4 rows, padding rows -1, the slack after the last segment -2."""
    ids = np.array([[0], [0], [1], [0], [1], [2], [2], [2], [2]], np.int32)
    ix = oracle.build_index(ids, None, 3, alignment=4)
    assert ix["counts"].tolist() == [3, 2, 4]
    assert ix["group_list"].tolist() == [4, 8, 12]
    assert ix["sorted_indices"].tolist() == [0, 1, 3, -1, 2, 4, -1, -1, 5, 6, 7, 8] + [-2] * 6
    assert ix["row_of"].reshape(-1).tolist() == [0, 1, 4, 2, 5, 8, 9, 10, 11]
    x = np.arange(9 * 2, dtype=np.float32).reshape(9, 2) + 1
    xp = oracle.permute(x, ix["sorted_indices"])
    assert (xp[[3, 6, 7]] == 0).all() and np.isnan(xp[12:]).all()  # padding zero, slack untouched


def test_group_mode_hand_example():
    """Four tokens, four experts in two groups of two (worked by hand from the definition)."""
    ids = np.array([[0, 1], [1, 2], [3, 0], [2, 3]], np.int32)
    ix = oracle.build_index(ids, None, 4, group_size=2)
    assert ix["gsrc"].tolist() == [0, 1, 2, 1, 2, 3]
    assert ix["slot_of"].tolist() == [[0, -1], [1, 3], [2, 4], [-1, 5]]
    assert ix["sorted_indices"].tolist() == [0, 2, 0, 1, 1, 3, 2, 3]
    assert ix["esrc"].tolist() == [0, 2, 0, 1, 3, 5, 4, 5]
    # each routing slot's group slot: token 2's experts 3 and 0 sit in groups 1 and 0
    assert ix["slot_src"].tolist() == [[0, 0], [1, 3], [4, 2], [5, 5]]


def test_index_invariants_at_workload_scale():
    """Skewed routing at the T16384/E256/K8 shape: counts sum to T*K, segments ascending,
    row_of is a bijection onto the rows and points back at its own token."""
    T, E, K = 16384, 256, 8
    logits = wl.router_logits(wl.workload_key(3), T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    ix = oracle.build_index(idx, w, E)
    assert int(ix["counts"].sum()) == T * K
    assert (ix["counts"] == 0).any() and ix["counts"].max() > 10 * T * K // E
    si, ro = ix["sorted_indices"], ix["row_of"]
    assert sorted(ro.reshape(-1).tolist()) == list(range(T * K))
    assert (si[ro] == np.arange(T)[:, None]).all()
    assert (ix["permuted_probs"][ro] == w).all()
    starts = ix["group_list"] - ix["counts"]
    for e in range(E):
        seg = si[starts[e]: ix["group_list"][e]]
        assert (np.diff(seg) > 0).all()


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 10), st.integers(1, 12), st.data())
def test_route_matches_full_sort(T, E, data):
    K = data.draw(st.integers(1, E))
    vals = data.draw(st.lists(st.sampled_from([-1.5, -0.0, 0.0, 0.25, 1.0, 2.0, 7.5]),
                              min_size=T * E, max_size=T * E))
    logits = np.asarray(vals, np.float32).reshape(T, E)
    idx, w = oracle.route_topk(logits, K)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:K]
        assert idx[t].tolist() == order
    assert np.allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=K * 2 ** -24)


def exact_combine(y, row_of, w):
    T, K = row_of.shape
    H = y.shape[1]
    out = [[Fraction(0)] * H for _ in range(T)]
    mag = [[Fraction(0)] * H for _ in range(T)]
    for t in range(T):
        for k in range(K):
            r = row_of[t, k]
            if r < 0 or r >= y.shape[0]:
                continue
            wk = Fraction(1) if w is None else Fraction(float(w[t, k]))
            for h in range(H):
                term = wk * Fraction(float(y[r, h]))
                out[t][h] += term
                mag[t][h] += abs(term)
    return out, mag


@settings(max_examples=150, deadline=None)
@given(st.integers(1, 6), st.integers(1, 6), st.integers(1, 5), st.booleans(), st.data())
def test_combine_within_exact_error_bound(T, K, H, weighted, data):
    rows = T * K + 2
    y = np.asarray(data.draw(st.lists(st.floats(-4, 4, width=32), min_size=rows * H,
                                      max_size=rows * H)), np.float32).reshape(rows, H)
    perm = np.asarray(data.draw(st.permutations(list(range(rows)))), np.int32)
    row_of = perm[: T * K].reshape(T, K).copy()
    row_of[0, 0] = -1 if data.draw(st.booleans()) else row_of[0, 0]
    w = None
    if weighted:
        w = np.asarray(data.draw(st.lists(st.floats(0, 1, width=32), min_size=T * K,
                                          max_size=T * K)), np.float32).reshape(T, K)
    got = oracle.unpermute_combine(y, row_of, w, np.float32)
    exact, mag = exact_combine(y, row_of, w)
    u = Fraction(1, 2 ** 24)
    eta = Fraction(1, 2 ** 150)  # half the smallest float32 subnormal: underflow per rounding
    for t in range(T):
        for h in range(H):
            assert abs(Fraction(float(got[t, h])) - exact[t][h]) <= K * (u * mag[t][h] + eta)
    got16 = oracle.unpermute_combine(y, row_of, w, np.uint16)
    back = wl.bf16_bits_to_f32(got16)
    for t in range(T):
        for h in range(H):
            # float32 chain error plus one bf16 rounding (half an ulp: 2^-9 relative)
            bound = K * (u * mag[t][h] + eta) + Fraction(1, 2 ** 8) * abs(Fraction(float(got[t, h]))) \
                + Fraction(1, 2 ** 134)
            assert abs(Fraction(float(back[t, h])) - exact[t][h]) <= bound


def test_identity_experts_reproduce_x():
    """Identity experts and weights summing to one: combine(permute(x)) returns x."""
    T, H, E, K = 1024, 512, 8, 2
    x = wl.hidden_states(wl.workload_key(1), T, H, "f32")
    logits = wl.router_logits(wl.workload_key(1), T, E)
    idx, w = oracle.route_topk(logits, K)
    ix = oracle.build_index(idx, w, E)
    y = oracle.permute(x, ix["sorted_indices"])
    out = oracle.unpermute_combine(y, ix["row_of"], w, np.float32)
    rel = np.abs(out - x) / np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    assert rel.max() <= 1e-6


def test_k1_unit_weight_combine_is_bitwise_unpermute():
    T, H, E = 300, 24, 16
    ids = wl.random_topk_ids(wl.case_key(9), T, E, 1)
    ix = oracle.build_index(ids, None, E)
    x = wl.hidden_states(wl.case_key(9), T, H, "bf16")
    y = oracle.permute(x, ix["sorted_indices"])
    back = oracle.unpermute_combine(y, ix["row_of"], None, np.uint16)
    assert np.array_equal(back, x)


def test_permute_zero_rows_and_bitwise_copy():
    x = wl.hidden_states(wl.case_key(10), 20, 9, "bf16")
    src_row = np.asarray([3, -1, 19, 0, 20, 3, -5], np.int32)
    out = oracle.permute(x, src_row)
    for i, s in enumerate(src_row):
        if 0 <= s < 20:
            assert np.array_equal(out[i], x[s])
        else:
            assert (out[i] == 0).all()


def test_two_stage_group_permute_equals_flat():
    """x -> one copy per (token, group) -> per-expert rows equals the flat permute bitwise."""
    T, H, E, K, gs = 500, 16, 32, 6, 4
    logits = wl.router_logits(wl.case_key(11), T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    ix = oracle.build_index(idx, w, E, group_size=gs)
    x = wl.hidden_states(wl.case_key(11), T, H, "bf16")
    flat = oracle.permute(x, ix["sorted_indices"])
    gbuf = oracle.permute(x, ix["gsrc"])
    two = oracle.permute(gbuf, ix["esrc"])
    assert np.array_equal(flat, two)
    assert int(ix["n_slots"][0]) < T * K


def test_precombine_single_group_equals_flat_combine():
    T, H, E, K = 200, 12, 16, 4
    logits = wl.router_logits(wl.case_key(12), T, E)
    idx, w = oracle.route_topk(logits, K)
    ix = oracle.build_index(idx, w, E, group_size=E)
    y = wl.expert_outputs(wl.case_key(12), T * K, H, "bf16")
    m = int(ix["n_slots"][0])
    P = oracle.group_precombine(y, ix["row_of"], w, idx, E, E, ix["slot_of"], m)
    flat = oracle.unpermute_combine(y, ix["row_of"], w, np.float32)
    assert np.array_equal(P[ix["slot_of"][:, 0]], flat)
    final = oracle.unpermute_combine(P, ix["slot_of"], None, np.uint16)
    assert np.array_equal(final, oracle.unpermute_combine(y, ix["row_of"], w, np.uint16))


def test_bf16_partials_are_the_float32_partials_rounded_once():
    """The bf16 partials (the pre-combine's output in a BF16 exchange) are the float32 chain's
    results rounded to nearest even, element by element -- nothing else changes; ties and values
    near powers of two are covered by scaling the expert rows with odd multiples."""
    T, H, E, K, gs = 300, 40, 32, 8, 8
    logits = wl.router_logits(wl.case_key(13), T, E, zipf_s=1.2)
    idx, w = oracle.route_topk(logits, K)
    ix = oracle.build_index(idx, w, E, group_size=gs)
    y = wl.expert_outputs(wl.case_key(13), T * K, H, "f32")
    y[::3] *= np.float32(3.0)
    m = int(ix["n_slots"][0])
    p32 = oracle.group_precombine(y, ix["row_of"], w, idx, E, gs, ix["slot_of"], m)
    p16 = oracle.group_precombine(y, ix["row_of"], w, idx, E, gs, ix["slot_of"], m, out_dtype=np.uint16)
    assert p16.dtype == np.uint16
    assert np.array_equal(p16, wl.f32_to_bf16_bits(p32))


@settings(max_examples=80, deadline=None)
@given(routing(max_t=6, max_e=8, max_k=4), st.sampled_from([1, 2, 4, 8]), st.integers(1, 4),
       st.data())
def test_precombine_and_final_sum_exact_bound(case, gs, H, data):
    ids, E = case
    if E % gs:
        gs = 1
    T, K = ids.shape
    ix = oracle.build_index(ids, None, E, group_size=gs)
    G = E // gs
    rows = T * K
    y = np.asarray(data.draw(st.lists(st.floats(-4, 4, width=32), min_size=rows * H,
                                      max_size=rows * H)), np.float32).reshape(rows, H)
    w = np.asarray(data.draw(st.lists(st.floats(0, 1, width=32), min_size=T * K,
                                      max_size=T * K)), np.float32).reshape(T, K)
    m = int(ix["n_slots"][0])
    P = oracle.group_precombine(y, ix["row_of"], w, ids, E, gs, ix["slot_of"], m)
    u = Fraction(1, 2 ** 24)
    eta = Fraction(1, 2 ** 150)
    for t in range(T):
        for g in range(G):
            s = ix["slot_of"][t, g]
            if s < 0:
                continue
            for h in range(H):
                ex, mag = Fraction(0), Fraction(0)
                for k in range(K):
                    e = ids[t, k]
                    if 0 <= e < E and e // gs == g:
                        term = Fraction(float(w[t, k])) * Fraction(float(y[ix["row_of"][t, k], h]))
                        ex += term
                        mag += abs(term)
                assert abs(Fraction(float(P[s, h])) - ex) <= K * (u * mag + eta)
    final = oracle.unpermute_combine(P, ix["slot_of"], None, np.float32)
    exact, mag = exact_combine(y, np.asarray(ix["row_of"]), w)
    for t in range(T):
        for h in range(H):
            assert abs(Fraction(float(final[t, h])) - exact[t][h]) <= 2 * (K + G) * (u * mag[t][h] + eta)
