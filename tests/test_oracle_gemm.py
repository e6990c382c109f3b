"""Pins for the oracle's exact int32 contraction and the fp32 epilogue."""

import numpy as np
import pytest

import oracle as O


@pytest.mark.parametrize("seed", range(4))
def test_gemm_exact_brute_force_python_ints(seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, (4, 32)).astype(np.int8)
    b = rng.integers(-128, 128, (5, 32)).astype(np.int8)
    got = O.gemm_exact(a, b)
    for m in range(4):
        for n in range(5):
            assert got[m, n] == sum(int(a[m, k]) * int(b[n, k]) for k in range(32))


def test_gemm_exact_at_the_int32_bound_matches_int64():
    k = 4096 * 3
    a = np.full((3, k), -127, np.int8)
    a[1] = 127
    a[2, ::2] = 127
    b = np.full((4, k), -128, np.int8)
    b[1] = 127
    b[3, 1::3] = 100
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(O.gemm_exact(a, b), ref)
    assert ref.max() == 127 * 128 * k


def test_gemm_uniform_codebook_is_textbook_int8_gemm():
    # codebook code-8 with unit scales decodes to signed int4, so the layer's integer
    # core reduces to a plain integer matrix product
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 16, (12, 512))
    w8 = O.decode_w4(O.pack_codes(codes), np.full((12, 32), 0x38, np.uint8), O.uniform_codebook())
    x = rng.integers(-127, 128, (3, 512)).astype(np.int8)
    assert np.array_equal(O.gemm_exact(x, w8), x.astype(np.int64) @ (codes - 8).T)


def test_epilogue_closed_forms():
    acc = np.array([[0, 3, -5, 1 << 24]], np.int64)
    xs = np.array([0.5], np.float32)
    ws = np.array([0.25, 0.25, 2.0, 1.0], np.float32)
    y = O.epilogue(acc, xs, ws, out="f32")
    assert y.tolist() == [[0.0, 0.375, -5.0, float(1 << 23)]]
    assert not np.signbit(y[0, 0])
    yb = O.bf16_bits_to_f32(O.epilogue(acc, xs, ws, out="bf16"))
    assert yb.tolist() == [[0.0, 0.375, -5.0, float(1 << 23)]]
    bias = np.array([1.0, -0.375, 0.0, 0.0], np.float32)
    assert O.epilogue(acc, xs, ws, bias, out="f32").tolist() == [[1.0, 0.0, -5.0, float(1 << 23)]]
    assert O.epilogue(acc, xs, ws, out="i32").dtype == np.int32


def test_epilogue_int_to_float_rounds_to_nearest_even():
    # 2^24 + 1 is not representable in fp32: it rounds to 2^24 (even); 2^24 + 3 -> 2^24 + 4
    acc = np.array([[(1 << 24) + 1, (1 << 24) + 3]], np.int64)
    y = O.epilogue(acc, np.ones(1, np.float32), np.ones(2, np.float32), out="f32")
    assert y.tolist() == [[float(1 << 24), float((1 << 24) + 4)]]


def test_epilogue_within_one_rounding_of_exact_product():
    rng = np.random.default_rng(9)
    acc = rng.integers(-(1 << 26), 1 << 26, (16, 32))
    xs = rng.uniform(1e-3, 1, 16).astype(np.float32)
    ws = rng.uniform(1e-5, 1e-3, 32).astype(np.float32)
    y = O.epilogue(acc, xs, ws, out="f32").astype(np.float64)
    exact = acc * xs[:, None].astype(np.float64) * ws[None, :].astype(np.float64)
    # three fp32 roundings (int->fp32, xs*ws, product): relative error below 2^-22
    assert np.all(np.abs(y - exact) <= np.abs(exact) * 2.0 ** -22)
