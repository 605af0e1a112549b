"""Pins of the oracle's FP8 (E4M3) quantization for the dispatch, and of the combine's bias.

- the E4M3 code <-> value maps against torch's float8_e4m3fn (a library implementation of the
  same OCP format, run on the CPU): all 256 codes decode alike, and values within +-448 (ties,
  subnormals, boundaries, random) encode alike; values past 448 saturate to 448;
- quantization: per block the element of largest magnitude becomes +-448 exactly, every element
  is within half an E4M3 step of x / scale, blocks are independent, bf16 input equals its
  float32 widening;
- the combine's bias is one float32 addition after the sum: combine(y, bias) equals
  fp32(combine(y) + bias) exactly; with no term the output is the bias.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")


def _torch_encode(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_every_code_decodes_like_the_library():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = np.asarray([oracle.e4m3_to_f32(int(c)) for c in codes], np.float32)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2  # 0x7f and 0xff
    assert np.array_equal(ours[~nan].view(np.uint32), lib[~nan].view(np.uint32))  # signs of zero too
    assert oracle.e4m3_to_f32(0x7E) == 448.0 and oracle.e4m3_to_f32(0x08) == 2.0 ** -6
    assert oracle.e4m3_to_f32(0x01) == 2.0 ** -9 and oracle.e4m3_to_f32(0x38) == 1.0


def test_encoding_matches_the_library_within_range():
    g = np.random.default_rng(60)
    vals = [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6, 0.9375 * 2.0 ** -6,
            1.0, 1.0625, 1.1875, 1.125, 239.9, 240.0, 248.0, 440.0, 447.9]
    # every midpoint between neighbouring finite codes (ties) and a hair to each side
    finite = sorted({oracle.e4m3_to_f32(c) for c in range(0x7F)})
    for a, b in zip(finite, finite[1:]):
        mid = (a + b) / 2
        vals += [mid, -mid, np.nextafter(np.float32(mid), np.float32(0)), np.nextafter(np.float32(mid), np.float32(1e9))]
    vals += list(g.uniform(-448, 448, 3000)) + list(g.standard_normal(2000) * 0.01)
    v = np.asarray(vals, np.float32)
    v = v[np.abs(v) <= 448]
    ours = np.asarray([oracle.f32_to_e4m3(float(x)) for x in v], np.uint8)
    assert np.array_equal(ours, _torch_encode(v))


def test_saturation_and_nan():
    for x in (448.5, 463.9, 464.0, 500.0, 1e30, float("inf")):
        assert oracle.f32_to_e4m3(x) == 0x7E and oracle.f32_to_e4m3(-x) == 0xFE
    assert oracle.f32_to_e4m3(float("nan")) & 0x7F == 0x7F


def _decode(q):
    lut = np.asarray([oracle.e4m3_to_f32(c) for c in range(256)], np.float64)
    return lut[q]


@pytest.mark.parametrize("dtype,block", [("f32", 128), ("bf16", 128), ("f32", 32), ("bf16", 512), ("f32", 64)])
def test_quantize_bounds(dtype, block):
    T, H = 40, 512
    x = wl.hidden_states(wl.case_key(61, block), T, H, dtype)
    x[3] = 0  # an all-zero token
    if dtype == "f32":
        x[5, :block] *= 1e-30  # subnormal-range quotients
    q, scales = oracle.quantize_fp8(x, block)
    xf = (wl.bf16_bits_to_f32(x) if dtype == "bf16" else x).astype(np.float64)
    nb = H // block
    assert scales.shape == (T, nb)
    xb = xf.reshape(T, nb, block)
    amax = np.abs(xb).max(axis=2)
    assert np.array_equal(scales, np.where(amax > 0, (amax.astype(np.float32) / np.float32(448.0)), 1.0).astype(np.float32))
    v = _decode(q).reshape(T, nb, block)
    # the block's largest element lands on +-448 exactly
    top = np.abs(xb).argmax(axis=2)
    vt = np.take_along_axis(v, top[..., None], axis=2)[..., 0]
    assert (np.abs(vt)[amax > 0] == 448.0).all()
    # every code is within half an E4M3 step of x / scale (step 2^(e-3) for normals, 2^-9 below)
    r = xb / scales[..., None].astype(np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -6)))
    step = np.where(np.abs(r) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))
    assert (np.abs(v - r) <= step / 2 * (1 + 1e-6) + 1e-300).all()
    assert (q[3] & 0x7F == 0).all() and (scales[3] == 1).all()


def test_quantize_blocks_are_independent_and_bf16_is_its_widening():
    x = wl.hidden_states(wl.case_key(62), 8, 256, "bf16")
    q, s = oracle.quantize_fp8(x, 64)
    q32, s32 = oracle.quantize_fp8(wl.bf16_bits_to_f32(x), 64)
    assert np.array_equal(q, q32) and np.array_equal(s, s32)
    y = x.copy()
    y[:, 64:128] = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(y[:, 64:128]) * 1000)
    q2, s2 = oracle.quantize_fp8(y, 64)
    keep = np.r_[0:64, 128:256]
    assert np.array_equal(q2[:, keep], q[:, keep]) and np.array_equal(s2[:, [0, 2, 3]], s[:, [0, 2, 3]])


def test_combine_bias_is_one_final_addition():
    g = np.random.default_rng(63)
    T, K, H, rows = 30, 4, 24, 130
    y = wl.expert_outputs(wl.case_key(63), rows, H, "f32")
    row_of = g.permutation(rows)[: T * K].astype(np.int32).reshape(T, K)
    row_of[g.random((T, K)) < 0.2] = -1
    row_of[0] = -1  # a token with no term: the output is the bias
    w = g.random((T, K)).astype(np.float32)
    bias = (g.standard_normal((T, H)) * 3).astype(np.float32)
    plain = oracle.unpermute_combine(y, row_of, w, np.float32)
    with_bias = oracle.unpermute_combine(y, row_of, w, np.float32, bias=bias)
    assert np.array_equal(with_bias, (plain + bias).astype(np.float32))
    assert np.array_equal(with_bias[0], bias[0] + np.float32(0.0))
    b16 = wl.f32_to_bf16_bits(bias)
    out16 = oracle.unpermute_combine(y, row_of, w, np.uint16, bias=b16)
    assert np.array_equal(out16, wl.f32_to_bf16_bits((plain + wl.bf16_bits_to_f32(b16)).astype(np.float32)))
