"""The seeded input recipe: deterministic, block-structured, bf16 rounding to nearest even."""
import numpy as np

import workloads as wl


def test_blocks_follow_the_recipe():
    a = wl.hidden_states(wl.case_key(1), 2500, 16, "f32")
    for b in range(3):
        lo = b * wl.BLOCK_ROWS
        n = min(wl.BLOCK_ROWS, 2500 - lo)
        g = np.random.default_rng([*wl.case_key(1), wl.STREAM_HIDDEN, b])
        assert np.array_equal(a[lo: lo + n], g.standard_normal((n, 16), dtype=np.float32))


def test_deterministic_and_streams_differ():
    a = wl.expert_outputs(wl.case_key(2), 3000, 8, "bf16")
    b = wl.expert_outputs(wl.case_key(2), 3000, 8, "bf16")
    c = wl.hidden_states(wl.case_key(2), 3000, 8, "bf16")
    assert a.dtype == np.uint16 and np.array_equal(a, b) and not np.array_equal(a, c)


def test_bf16_round_to_nearest_even():
    f = np.asarray([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.0,
                    np.inf, np.nan], np.float32)
    h = wl.f32_to_bf16_bits(f)
    assert h[:6].tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0x7F80]
    assert (h[6] & 0x7F80) == 0x7F80 and (h[6] & 0x7F) != 0
    assert np.array_equal(wl.bf16_bits_to_f32(h[:5]), np.asarray([1, 1, 1 + 2 ** -6, 1 + 2 ** -7, -2], np.float32))


def test_zipf_bias_skews_low_ids():
    b = wl.zipf_bias(256, 1.2)
    assert b.dtype == np.float32 and (np.diff(b) < 0).all()
    assert np.isclose(np.exp(b.astype(np.float64)).sum(), 1.0, rtol=1e-6)


def test_seeded_workload_keys_are_distinct():
    """--seed draws other inputs of the same shapes: keys differ from the fixed draw, from each
    other and from the test-case keys."""
    import workloads as wl
    assert wl.workload_key(3) == (3,)
    ks = {wl.workload_key(3, s) for s in range(5)}
    assert len(ks) == 5 and (3,) not in ks and all(k[0] == 3 for k in ks)
    assert all(k[0] != 1000 for k in ks)  # test cases use (1000, ...)
    a = wl.router_logits(wl.workload_key(1, 0), 64, 8)
    b = wl.router_logits(wl.workload_key(1), 64, 8)
    assert a.shape == b.shape and not (a == b).all()
