"""Pins of the oracle's group-limited routing ([Scratch] §21) against things other than itself.

- with every group allowed, or with one-expert groups and at least K of them allowed, it is
  plain top-k routing (the oracle's route_topk, itself pinned elsewhere), bit for bit;
- K = 1 picks the global argmax (ties to the lower id) with weight 1;
- on small cases an exhaustive search over all sets of topk_groups groups finds the one set in
  which every member beats every non-member (score = best logit of the group, ties to the lower
  group id); the chosen experts must lie in it and beat every other expert of it.
"""
import itertools

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
import workloads as wl


def _beats(a_val, a_id, b_val, b_id):
    return a_val > b_val or (a_val == b_val and a_id < b_id)


def _tie_logits(seed, T, E):
    g = np.random.default_rng(seed)
    v = (g.integers(-4, 5, size=(T, E)) * 0.5).astype(np.float32)
    v[g.random((T, E)) < 0.1] = -0.0
    return v


def test_all_groups_allowed_is_plain_routing():
    for seed, (T, E, K, gs) in enumerate([(50, 16, 4, 4), (40, 64, 8, 8), (30, 12, 5, 3), (20, 8, 8, 2)]):
        for logits in (wl.router_logits(wl.case_key(50, seed), T, E, zipf_s=1.0), _tie_logits(seed, T, E)):
            gi, gw = oracle.route_topk_grouped(logits, K, gs, E // gs)
            pi, pw = oracle.route_topk(logits, K)
            assert np.array_equal(gi, pi) and np.array_equal(gw, pw)


def test_single_expert_groups_is_plain_routing():
    logits = _tie_logits(7, 40, 10)
    for K, M in ((3, 3), (3, 7), (1, 1), (5, 10)):
        gi, gw = oracle.route_topk_grouped(logits, K, 1, M)
        pi, pw = oracle.route_topk(logits, K)
        assert np.array_equal(gi, pi) and np.array_equal(gw, pw)


def test_k1_is_the_argmax():
    for logits in (_tie_logits(8, 60, 12), wl.router_logits(wl.case_key(51), 60, 12, zipf_s=0.0)):
        for gs, M in ((3, 1), (4, 2), (2, 5)):
            gi, gw = oracle.route_topk_grouped(logits, 1, gs, M)
            assert gi[:, 0].tolist() == np.argmax(logits, axis=1).tolist()
            assert (gw == 1.0).all()


@st.composite
def grouped_case(draw):
    G = draw(st.integers(1, 6))
    gs = draw(st.integers(1, 4))
    E = G * gs
    M = draw(st.integers(1, G))
    K = draw(st.integers(1, min(E, M * gs)))
    vals = draw(st.lists(st.sampled_from([-1.5, -0.5, -0.0, 0.0, 0.5, 2.0, 3.25]), min_size=E, max_size=E))
    return np.asarray([vals], np.float32), K, gs, M


@settings(max_examples=300, deadline=None)
@given(grouped_case())
def test_selection_is_the_optimal_one(case):
    check_optimal(*case)


def test_selection_is_the_optimal_one_fixed_cases():
    g = np.random.default_rng(52)
    vals = np.asarray([-1.5, -0.5, -0.0, 0.0, 0.5, 2.0, 3.25], np.float32)
    for _ in range(300):
        G, gs = int(g.integers(1, 7)), int(g.integers(1, 5))
        M = int(g.integers(1, G + 1))
        K = int(g.integers(1, min(G * gs, M * gs) + 1))
        check_optimal(g.choice(vals, size=(1, G * gs)), K, gs, M)


def check_optimal(logits, K, gs, M):
    E = logits.shape[1]
    G = E // gs
    s = logits[0].astype(np.float64)
    score = [max(s[g * gs:(g + 1) * gs]) for g in range(G)]
    dominant = [A for A in itertools.combinations(range(G), M)
                if all(_beats(score[a], a, score[b], b) for a in A for b in range(G) if b not in A)]
    assert len(dominant) == 1
    A = set(dominant[0])
    idx, w = oracle.route_topk_grouped(logits, K, gs, M)
    chosen = idx[0].tolist()
    assert len(set(chosen)) == K
    assert all(e // gs in A for e in chosen)
    others = [e for e in range(E) if e // gs in A and e not in chosen]
    assert all(_beats(s[c], c, s[o], o) for c in chosen for o in others)
    assert all(_beats(s[chosen[i]], chosen[i], s[chosen[i + 1]], chosen[i + 1]) for i in range(K - 1))
    assert abs(float(w.astype(np.float64).sum()) - 1.0) <= K * 2.0 ** -24
    assert all(w[0, i] >= w[0, i + 1] for i in range(K - 1))


def test_limited_routing_uses_at_most_m_groups_at_workload_scale():
    """T8192 E256 in 32 groups of 8, 4 groups per token, K = 8: every token's experts sit in
    at most 4 groups, and the group-mode index has at most 4 slots per token."""
    T, E, K, gs, M = 8192, 256, 8, 8, 4
    logits = wl.router_logits(wl.workload_key(4), T, E, zipf_s=1.2)
    idx, w = oracle.route_topk_grouped(logits, K, gs, M)
    ngroups = np.asarray([len(set((r // gs).tolist())) for r in idx])
    assert ngroups.max() <= M
    ix = oracle.build_index(idx, w, E, group_size=gs)
    assert int(ix["n_slots"][0]) == int(ngroups.sum()) <= M * T
