"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/moe_oracle.c (a flipped tie rule, a dropped
term, a wrong sign or index, a transposed operand, an off-by-one bound, a truncating rounding),
builds it with gcc, routes the oracle wrapper to it, and requires that at least one pin fails.
The planted mistakes live only in temporary copies; the oracle itself is untouched.
"""
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.build import SRC
import test_oracle_backward as bw
import test_oracle_bruteforce as bf
import test_oracle_fp8 as f8
import test_oracle_grouped_route as gr
import test_oracle_pins as pins

MUTANTS = [
    ("ties go to the higher id", "if (best < 0 || s[e] > s[best])", "if (best < 0 || s[e] >= s[best])"),
    ("softmax normalised over the wrong slot", "w[k] = (float)(ex[k] / z);", "w[k] = (float)(ex[0] / z);"),
    ("softmax sum skips the first slot", "        z += ex[k];", "        if (k > 0) z += ex[k];"),
    ("softmax sign flipped", "ex[k] = exp((double)s[idx[k]] - m);", "ex[k] = exp(m - (double)s[idx[k]]);"),
    ("group_list exclusive instead of inclusive",
     "        run += capacity > 0 ? counts[e] : (counts[e] + A - 1) / A * A;\n        group_list[e] = (int32_t)run;",
     "        group_list[e] = (int32_t)run;\n        run += capacity > 0 ? counts[e] : (counts[e] + A - 1) / A * A;"),
    ("group_list ignores the alignment", "        run += capacity > 0 ? counts[e] : (counts[e] + A - 1) / A * A;",
     "        run += counts[e];"),
    ("aligned segments get no padding rows", "for (int64_t end = start + (p + A - 1) / A * A; r < end; ++r)",
     "for (int64_t end = start + p; r < end; ++r)"),
    ("unused slack marked as padding", "            sorted_indices[q] = -2;", "            sorted_indices[q] = -1;"),
    ("tokens scanned in descending order", "        for (int64_t t = 0; t < T; ++t) {\n            for (int32_t k = 0; k < K; ++k) {\n                if (topk_idx[t * K + k] != e)",
     "        for (int64_t t = T - 1; t >= 0; --t) {\n            for (int32_t k = 0; k < K; ++k) {\n                if (topk_idx[t * K + k] != e)"),
    ("row_of stored transposed", "                    row_of[t * K + k] = (int32_t)r;", "                    row_of[k * T + t] = (int32_t)r;"),
    ("permuted_probs from the wrong slot", "permuted_probs[r] = topk_w ? topk_w[t * K + k] : 1.0f;",
     "permuted_probs[r] = topk_w ? topk_w[t * K] : 1.0f;"),
    ("capacity bound off by one", "                    if (p < capacity) {", "                    if (p <= capacity) {"),
    ("drop keeps the last tokens", "                        int64_t row = (int64_t)e * capacity + p;\n                        sorted_indices[row] = (int32_t)t;",
     "                        int64_t row = (int64_t)e * capacity + (capacity - 1 - p);\n                        sorted_indices[row] = (int32_t)t;"),
    ("padding probabilities not cleared", "                if (permuted_probs)\n                    permuted_probs[row] = 0.0f;",
     "                if (permuted_probs)\n                    permuted_probs[row] = 1.0f;"),
    ("group of an expert by modulo", "if (e >= 0 && e < E && e / group_size == g)\n                        uses = 1;",
     "if (e >= 0 && e < E && e % (E / group_size) == g)\n                        uses = 1;"),
    ("esrc uses the expert instead of its group", "esrc[row] = slot_of[t * G + e / group_size];",
     "esrc[row] = slot_of[t * G + e % G];"),
    ("slot_src uses the expert instead of its group", "-1 : slot_of[t * G + e / group_size];",
     "-1 : slot_of[t * G + e % G];"),
    ("permute copies the next row", "memcpy(d, (const unsigned char *)src + (size_t)s * row_bytes, row_bytes);",
     "memcpy(d, (const unsigned char *)src + (size_t)(s + 1 < src_rows ? s + 1 : s) * row_bytes, row_bytes);"),
    ("permute leaves padding rows unwritten", "        else if (s != -2)\n            memset(d, 0, row_bytes);",
     "        else\n            (void)0;"),
    ("combine drops the accumulator", "acc = fmaf(wk, load_elem(y, y_dt, (int64_t)r * H + h), acc);\n            }\n            if (bias)",
     "acc = fmaf(wk, load_elem(y, y_dt, (int64_t)r * H + h), 0.0f);\n            }\n            if (bias)"),
    ("combine skips slot 0", "            for (int32_t k = 0; k < K; ++k) {\n                int32_t r = row_of[t * K + k];\n                if (r < 0 || r >= y_rows)\n                    continue;\n                float wk",
     "            for (int32_t k = 1; k < K; ++k) {\n                int32_t r = row_of[t * K + k];\n                if (r < 0 || r >= y_rows)\n                    continue;\n                float wk"),
    ("combine weights transposed", "                float wk = w ? w[t * K + k] : 1.0f;\n                acc = fmaf(wk, load_elem(y, y_dt, (int64_t)r * H + h), acc);\n            }\n            if (bias)",
     "                float wk = w ? w[k * T + t] : 1.0f;\n                acc = fmaf(wk, load_elem(y, y_dt, (int64_t)r * H + h), acc);\n            }\n            if (bias)"),
    ("combine subtracts", "acc = fmaf(wk, load_elem(y, y_dt, (int64_t)r * H + h), acc);\n            }\n            if (bias)",
     "acc = fmaf(-wk, load_elem(y, y_dt, (int64_t)r * H + h), acc);\n            }\n            if (bias)"),
    ("bf16 rounding truncates", "    uint32_t lsb = (u >> 16) & 1u;\n    u += 0x7fffu + lsb;", "    uint32_t lsb = 0u;\n    (void)lsb;"),
    ("bf16 ties round up", "    u += 0x7fffu + lsb;", "    u += 0x8000u + 0u * lsb;"),
    ("pre-combine mixes groups", "if (e < 0 || e >= E || e / group_size != g || r < 0 || r >= y_rows)",
     "if (e < 0 || e >= E || r < 0 || r >= y_rows)"),
    ("capacity rounds down", "    return (num + den - 1) / den;", "    return num / den;"),
    ("group score from the group's first expert", "                if (s[e] > s[top])\n                    top = e;",
     "                if (0 && s[e] > s[top])\n                    top = e;"),
    ("group ties go to the higher id", "if (bg < 0 || score[g] > score[bg])", "if (bg < 0 || score[g] >= score[bg])"),
    ("experts outside the chosen groups allowed", "taken[e] = chosen[e / group_size] ? 0 : 1;", "taken[e] = 0;"),
    ("e4m3 ties away from zero", "double mant = nearbyint((a / ldexp(1.0, E) - 1.0) * 8.0);",
     "double mant = round((a / ldexp(1.0, E) - 1.0) * 8.0);"),
    ("e4m3 subnormals truncate", "double m = nearbyint(a * 512.0);", "double m = floor(a * 512.0);"),
    ("e4m3 without saturation", "    if (a > 448.0)", "    if (a > 1e30)"),
    ("scale for the wrong FP8 maximum", "amax / 448.0f", "amax / 240.0f"),
    ("combine bias ignored", "acc = acc + load_elem(bias, out_dt, t * H + h);", "acc = acc + 0.0f;"),
    ("combine bias from the wrong token", "acc = acc + load_elem(bias, out_dt, t * H + h);",
     "acc = acc + load_elem(bias, out_dt, h);"),
    ("combine backward ignores the weight",
     "store_elem(dy, dy_dt, (int64_t)r * H + h, wk * load_elem(dout, dout_dt, t * H + h));",
     "store_elem(dy, dy_dt, (int64_t)r * H + h, load_elem(dout, dout_dt, t * H + h));"),
    ("combine backward leaves unnamed rows unwritten",
     "    for (int64_t r = 0; r < y_rows; ++r)\n        for (int64_t h = 0; h < H; ++h)\n            store_elem(dy, dy_dt, r * H + h, 0.0f);",
     "    (void)0;"),
    ("weight gradient dots with the next row",
     "* (double)load_elem(y, y_dt, (int64_t)r * H + h);",
     "* (double)load_elem(y, y_dt, (int64_t)((r + 1) % y_rows) * H + h);"),
    ("router gradient drops the mean term", "((double)d_topk_w[t * K + k] - s)", "((double)d_topk_w[t * K + k])"),
    ("router gradient sign flipped", "((double)d_topk_w[t * K + k] - s)", "(s - (double)d_topk_w[t * K + k])"),
    ("router gradient uses slot 0's weight", "acc[e] += (double)topk_w[t * K + k] *", "acc[e] += (double)topk_w[t * K] *"),
    ("bf16 partials stored without rounding", "store_elem(partials, p_dt, (int64_t)s * H + h, acc);",
     "store_elem(partials, p_dt, (int64_t)s * H + h, p_dt ? truncf(acc * 256.0f) / 256.0f : acc);"),
    ("repeated experts take the later slot first",
     "        for (int64_t t = 0; t < T; ++t) {\n            for (int32_t k = 0; k < K; ++k) {\n                if (topk_idx[t * K + k] != e)",
     "        for (int64_t t = 0; t < T; ++t) {\n            for (int32_t k = K - 1; k >= 0; --k) {\n                if (topk_idx[t * K + k] != e)"),
]


def _pins():
    """Every check the mutants must fail one of (deterministic: no hypothesis)."""
    checks = [
        pins.test_megatron_routing_map_example,
        pins.test_group_list_example,
        pins.test_rank_major_to_expert_major_example,
        pins.test_stable_permute_example,
        lambda: pins.test_unpermute_example_is_exact(np.float32),
        lambda: pins.test_unpermute_example_is_exact(np.uint16),
        pins.test_weighted_merge_example,
        pins.test_capacity_example,
        pins.test_capacity_rounds_up,
        pins.test_zero_token_expert,
        lambda: pins.test_route_equal_logits(64, 8),
        pins.test_route_k1_weight_is_one,
        pins.test_route_two_experts_is_logistic,
        pins.test_route_weights_form_distribution,
        pins.test_bf16_rounding_of_oracle,
        bf.test_group_mode_hand_example,
        bf.test_aligned_hand_example,
        bf.test_identity_experts_reproduce_x,
        bf.test_k1_unit_weight_combine_is_bitwise_unpermute,
        bf.test_permute_zero_rows_and_bitwise_copy,
        bf.test_two_stage_group_permute_equals_flat,
        bf.test_precombine_single_group_equals_flat_combine,
        _index_brute_force,
        _combine_exact_bound,
        _precombine_exact_bound,
        _route_brute_force,
        lambda: bw.test_combine_backward_matches_autograd("f32", "f32", True, "drop"),
        lambda: bw.test_combine_backward_matches_autograd("bf16", "bf16", True, "holes"),
        lambda: bw.test_combine_backward_matches_autograd("f32", "f32", False, "standard"),
        bw.test_dispatch_backward_is_the_unit_weight_combine,
        bw.test_route_backward_matches_autograd_and_finite_differences,
        bw.test_route_backward_closed_forms,
        gr.test_all_groups_allowed_is_plain_routing,
        gr.test_single_expert_groups_is_plain_routing,
        gr.test_k1_is_the_argmax,
        gr.test_selection_is_the_optimal_one_fixed_cases,
        f8.test_every_code_decodes_like_the_library,
        f8.test_encoding_matches_the_library_within_range,
        f8.test_saturation_and_nan,
        lambda: f8.test_quantize_bounds("f32", 128),
        lambda: f8.test_quantize_bounds("bf16", 32),
        f8.test_quantize_blocks_are_independent_and_bf16_is_its_widening,
        f8.test_combine_bias_is_one_final_addition,
        bf.test_bf16_partials_are_the_float32_partials_rounded_once,
        _repeated_experts,
    ]
    return checks


def _precombine_exact_bound():
    g = np.random.default_rng(8)
    u = Fraction(1, 2 ** 24)
    for trial in range(20):
        E, gs = 8, int(g.choice([1, 2, 4]))
        K, T, H = int(g.integers(2, 5)), int(g.integers(1, 6)), 2
        ids = np.argsort(g.random((T, E)), axis=1)[:, :K].astype(np.int32)
        ix = oracle.build_index(ids, None, E, group_size=gs)
        y = g.standard_normal((T * K, H)).astype(np.float32)
        w = g.random((T, K)).astype(np.float32)
        m = int(ix["n_slots"][0])
        P = oracle.group_precombine(y, ix["row_of"], w, ids, E, gs, ix["slot_of"], m)
        for t in range(T):
            for grp in range(E // gs):
                s_ = ix["slot_of"][t, grp]
                if s_ < 0:
                    continue
                for h in range(H):
                    terms = [Fraction(float(w[t, k])) * Fraction(float(y[ix["row_of"][t, k], h]))
                             for k in range(K) if ids[t, k] // gs == grp]
                    assert abs(Fraction(float(P[s_, h])) - sum(terms)) <= K * u * sum(abs(x) for x in terms) \
                        + Fraction(1, 2 ** 140)


def _index_brute_force():
    g = np.random.default_rng(5)
    for trial in range(40):
        E = int(g.integers(2, 9))
        K = int(g.integers(1, min(4, E) + 1))
        T = int(g.integers(1, 12))
        ids = np.argsort(g.random((T, E)), axis=1)[:, :K].astype(np.int32)
        ids[g.random((T, K)) < 0.15] = -1
        w = g.random((T, K)).astype(np.float32)
        divisor = [d for d in range(1, E + 1) if E % d == 0][-2 if E > 1 else 0]
        for cap, gs, al in ((0, 0, 0), (int(g.integers(1, 4)), 0, 0), (0, divisor, 0), (0, 0, 4), (0, divisor, 3)):
            ix = oracle.build_index(ids, w, E, capacity=cap, group_size=gs, alignment=al)
            want = bf.brute_index(ids, E, cap=cap, gs=gs, w=w, align=al)
            assert np.array_equal(ix["permuted_probs"], want["permuted_probs"])
            assert ix["counts"].tolist() == want["counts"]
            assert ix["group_list"].tolist() == want["group_list"]
            assert ix["sorted_indices"].tolist() == want["sorted_indices"]
            assert ix["row_of"].tolist() == want["row_of"]
            if cap > 0:
                assert (ix["permuted_probs"][np.asarray(want["sorted_indices"]) < 0] == 0).all()
            if gs > 0:
                assert ix["gsrc"].tolist() == want["gsrc"]
                assert ix["slot_of"].tolist() == want["slot_of"]
                assert ix["esrc"].tolist() == want["esrc"]
                assert ix["slot_src"].tolist() == want["slot_src"]


def _repeated_experts():
    """Rows naming an expert twice (fixed cases): the index equals the (expert, token, slot) sort."""
    g = np.random.default_rng(17)
    for T, E, K in ((9, 4, 3), (12, 3, 3), (7, 5, 4)):
        ids = g.integers(-1, E, size=(T, K)).astype(np.int32)
        ids[:, 1] = ids[:, 0]
        w = g.random((T, K)).astype(np.float32)
        ix = oracle.build_index(ids, w, E)
        b = bf.brute_index(ids, E, w=w)
        assert ix["sorted_indices"].tolist() == b["sorted_indices"] and ix["row_of"].tolist() == b["row_of"]
        assert np.array_equal(ix["permuted_probs"], b["permuted_probs"])


def _combine_exact_bound():
    g = np.random.default_rng(6)
    u = Fraction(1, 2 ** 24)
    for trial in range(20):
        T, K, H = int(g.integers(1, 5)), int(g.integers(1, 5)), int(g.integers(1, 4))
        rows = T * K + 1
        y = g.standard_normal((rows, H)).astype(np.float32)
        row_of = g.permutation(rows)[: T * K].astype(np.int32).reshape(T, K)
        w = g.random((T, K)).astype(np.float32)
        got = oracle.unpermute_combine(y, row_of, w, np.float32)
        exact, mag = bf.exact_combine(y, row_of, w)
        for t in range(T):
            for h in range(H):
                assert abs(Fraction(float(got[t, h])) - exact[t][h]) <= K * u * mag[t][h] + Fraction(1, 2 ** 140)


def _route_brute_force():
    g = np.random.default_rng(7)
    for trial in range(30):
        T, E = int(g.integers(1, 8)), int(g.integers(2, 12))
        K = int(g.integers(1, E + 1))
        logits = g.choice(np.asarray([-1.5, -0.0, 0.0, 0.25, 1.0, 7.5], np.float32), size=(T, E))
        idx, w = oracle.route_topk(logits, K)
        for t in range(T):
            assert idx[t].tolist() == sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:K]
        assert np.allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=K * 2 ** -24)


def test_pins_pass_on_the_real_oracle():
    for check in _pins():
        check()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    str(mutant), "-o", str(so), "-lm"], check=True, capture_output=True)
    oracle.use_library(str(so))
    caught = []
    try:
        for check in _pins():
            try:
                check()
            except (AssertionError, ValueError, IndexError):
                caught.append(getattr(check, "__name__", "lambda"))
    finally:
        oracle.use_library(None)
    assert caught, f"no pin catches the planted mistake: {name}"
