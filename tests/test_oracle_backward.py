"""Pins of the oracle's backward functions against things other than the oracle itself.

- torch autograd (CPU, float64) of the forward definitions written with plain tensor indexing:
  the weighted combine out[t] = sum_k w[t,k] * y[row_of[t,k]], the permute xp = x[src_row] and
  the softmax over the K selected logits;
- the transposition of [Combine] §4.1 (the backward of the dispatch is the combine): the oracle's
  unit-weight combine of a gradient equals autograd's transpose of the gather map;
- central finite differences of the selected softmax in float64, with the top-k selection
  recomputed at every point;
- closed forms: K = 1 gives no router gradient; unselected logits get exactly 0.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")

U = 2.0 ** -24


def _f64(a):
    if a.dtype == np.uint16:
        return wl.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _case(seed, T, E, K, H, y_dt, cap=0, holes=0.0):
    key = wl.case_key(40, seed, T, E, K, H)
    logits = wl.router_logits(key, T, E, zipf_s=1.0)
    idx, w = oracle.route_topk(logits, K)
    if holes:
        idx[np.random.default_rng([*key, 5]).random((T, K)) < holes] = -1
    ix = oracle.build_index(idx, w, E, capacity=cap)
    rows = len(ix["sorted_indices"])
    y = wl.expert_outputs(key, rows, H, y_dt)
    dout = wl.expert_outputs((*key, 1), T, H, y_dt)
    return idx, w, ix, y, dout


def _autograd_combine(dout, y, row_of, w):
    yt = torch.tensor(_f64(y), requires_grad=True)
    wt = None if w is None else torch.tensor(w.astype(np.float64), requires_grad=True)
    T, K = row_of.shape
    out = torch.zeros((T, y.shape[1]), dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            r = int(row_of[t, k])
            if 0 <= r < y.shape[0]:
                out[t] = out[t] + (1.0 if wt is None else wt[t, k]) * yt[r]
    (out * torch.tensor(_f64(dout))).sum().backward()
    gw = None if wt is None else wt.grad.numpy()
    return yt.grad.numpy(), gw


def _ulp_bf16_ok(got_bits, want_f64):
    """got (bf16 bits) is one of the two bf16 neighbours of the exact value."""
    got = wl.bf16_bits_to_f32(got_bits).astype(np.float64)
    ref = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(want_f64.astype(np.float32))).astype(np.float64)
    spacing = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
    return np.abs(got - want_f64) <= spacing


@pytest.mark.parametrize("y_dt,dy_dt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("mode", ["standard", "drop", "holes"])
def test_combine_backward_matches_autograd(y_dt, dy_dt, weighted, mode):
    T, E, K, H = 37, 8, 3, 5
    cap = 9 if mode == "drop" else 0
    idx, w, ix, y, dout = _case(1, T, E, K, H, y_dt, cap=cap, holes=0.2 if mode == "holes" else 0.0)
    ww = w if weighted else None
    dy, dw = oracle.combine_backward(dout, y, ix["row_of"], ww, np.uint16 if dy_dt == "bf16" else np.float32)
    gy, gw = _autograd_combine(dout, y, ix["row_of"], ww)
    if dy_dt == "f32":
        # each named row gets one product of two float32 values: its float32 rounding is the
        # float32 multiply, so the oracle matches the exact gradient bit for bit
        assert np.array_equal(dy, gy.astype(np.float32))
    else:
        assert _ulp_bf16_ok(dy, gy).all()
        assert np.array_equal(dy[gy == 0], np.zeros_like(dy[gy == 0]))
    if weighted:
        terms = np.abs(_f64(dout))[:, None, :] * np.abs(_f64(y))[np.maximum(ix["row_of"], 0)]
        bound = U * np.abs(gw) + H * 2.0 ** -52 * terms.sum(axis=2) + 2.0 ** -140
        assert (np.abs(dw.astype(np.float64) - gw) <= bound).all()
        assert (dw[ix["row_of"] < 0] == 0).all()
    else:
        assert dw is not None and (dw[ix["row_of"] < 0] == 0).all()


def test_dispatch_backward_is_the_unit_weight_combine():
    """[Combine] §4.1: the transpose of the gather x -> xp is the gather-and-sum back to tokens."""
    for T, E, K, H, cap in ((29, 6, 2, 4, 0), (40, 8, 4, 3, 11), (25, 5, 5, 2, 0)):
        idx, w, ix, _, _ = _case(2, T, E, K, H, "f32", cap=cap, holes=0.1)
        x = wl.hidden_states(wl.case_key(41, T, H), T, H, "f32")
        src = ix["sorted_indices"]
        dxp = wl.expert_outputs(wl.case_key(42, T, H), len(src), H, "f32")
        xt = torch.tensor(x.astype(np.float64), requires_grad=True)
        valid = torch.tensor((src >= 0) & (src < T))
        xp = torch.where(valid[:, None], xt[torch.tensor(np.clip(src, 0, T - 1)).long()], torch.zeros(()))
        (xp * torch.tensor(dxp.astype(np.float64))).sum().backward()
        exact = xt.grad.numpy()
        got = oracle.unpermute_combine(dxp, ix["row_of"], None, np.float32).astype(np.float64)
        terms = np.zeros_like(exact)
        for r, t in enumerate(src):
            if 0 <= t < T:
                terms[t] += np.abs(dxp[r])
        assert (np.abs(got - exact) <= K * U * terms + 2.0 ** -140).all()


def _selected_softmax_objective(logits64, g, K):
    """f(l) = sum_k g[t,k] * softmax(top-K of l[t])_k, the selection (ties to the lower id)
    recomputed from l."""
    f = 0.0
    for t in range(logits64.shape[0]):
        order = sorted(range(logits64.shape[1]), key=lambda e: (-logits64[t, e], e))[:K]
        s = logits64[t, order]
        p = np.exp(s - s.max())
        p /= p.sum()
        f += float((g[t] * p).sum())
    return f


def test_route_backward_matches_autograd_and_finite_differences():
    g_ = np.random.default_rng(43)
    for T, E, K in ((6, 9, 3), (4, 16, 8), (5, 5, 5), (7, 12, 1)):
        logits = (g_.standard_normal((T, E)) * 3).astype(np.float32)
        idx, w = oracle.route_topk(logits, K)
        g = g_.standard_normal((T, K)).astype(np.float32)
        d = oracle.route_topk_backward(idx, w, g, E)
        # autograd of the float64 selected softmax
        lt = torch.tensor(logits.astype(np.float64), requires_grad=True)
        p = torch.softmax(lt.gather(1, torch.tensor(idx).long()), dim=1)
        (p * torch.tensor(g.astype(np.float64))).sum().backward()
        ag = lt.grad.numpy()
        pg = np.abs(p.detach().numpy() * g).sum(axis=1, keepdims=True)
        sel = np.zeros((T, E), bool)
        np.put_along_axis(sel, idx.astype(np.int64), True, axis=1)
        scale = np.zeros((T, E))
        np.put_along_axis(scale, idx.astype(np.int64), p.detach().numpy() * (np.abs(g) + pg), axis=1)
        assert (np.abs(d - ag) <= 6 * U * scale + 1e-30).all()
        assert (d[~sel] == 0).all()
        # central differences, selection recomputed at each point (no near-ties in these draws)
        l64 = logits.astype(np.float64)
        for t in range(T):
            srt = np.sort(l64[t])[::-1]
            if K < E and srt[K - 1] - srt[K] < 1e-3:
                continue
            for e in range(E):
                h = 1e-6
                lp, lm = l64.copy(), l64.copy()
                lp[t, e] += h
                lm[t, e] -= h
                fd = (_selected_softmax_objective(lp[t:t + 1], g[t:t + 1], K) -
                      _selected_softmax_objective(lm[t:t + 1], g[t:t + 1], K)) / (2 * h)
                assert abs(fd - d[t, e]) <= 1e-6 * (1 + abs(g[t]).sum()), (t, e, fd, d[t, e])


def test_route_backward_closed_forms():
    # K = 1: the single weight is exactly 1, so its gradient through the softmax is exactly 0
    logits = wl.router_logits(wl.case_key(44), 9, 7, zipf_s=0.0)
    idx, w = oracle.route_topk(logits, 1)
    d = oracle.route_topk_backward(idx, w, np.random.default_rng(44).standard_normal((9, 1)).astype(np.float32), 7)
    assert (d == 0).all()
    # equal logits: w = 1/K, the gradient is (g_k - mean(g)) / K on slots 0..K-1
    K, E = 4, 6
    idx, w = oracle.route_topk(np.zeros((1, E), np.float32), K)
    g = np.asarray([[1.0, -2.0, 0.5, 4.0]], np.float32)
    d = oracle.route_topk_backward(idx, w, g, E)
    want = (g[0].astype(np.float64) - g[0].astype(np.float64).mean()) / K
    assert np.allclose(d[0, :K], want, rtol=4 * U, atol=0) and (d[0, K:] == 0).all()
