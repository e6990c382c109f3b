"""Pins for the oracle's training-path and variant functions: stochastic grid
assignment, code-only requantisation, fake quantisation, the fp32 dequantisation,
the straight-through backward's bf16 weight and product, row interleaving, SwiGLU
and the LoRA delta.  Each is checked against something other than itself: extreme
draws with a closed-form outcome, unbiasedness over many draws, the bracketing
property, hand-worked bf16 roundings, the Hadamard digit rule, plain loops, a
library sigmoid, and agreement with the quantiser's own final step."""

import numpy as np
import pytest
from scipy.special import expit

import oracle as O

F32 = np.float32


def _levels(rows):
    """[1, G, 16] non-decreasing fp32 levels from a list of 16-value rows."""
    return np.asarray(rows, dtype=F32)[None]


# ---------------------------------------------------------------- stochastic grid

def test_stochastic_extreme_draws_round_up_or_down():
    lv = _levels([np.arange(-8, 8) * 10.0])                   # levels -80, -70, ..., 70
    t = np.array([[[-75.0, -41.0, 3.0, 69.5]]], F32)          # strictly inside brackets
    up = O.assign_grid_stochastic(t, lv, np.zeros_like(t))    # thr = lower level: always up
    assert up.tolist() == [[[1, 4, 9, 15]]]           # level 0 is index 8
    u1 = np.full_like(t, np.nextafter(F32(1), F32(0)))         # thr just below the upper level
    down = O.assign_grid_stochastic(t, lv, u1)
    assert down.tolist() == [[[0, 3, 8, 14]]]


def test_stochastic_outside_the_grid_and_on_levels():
    lv = _levels([np.arange(-8, 8) * 10.0])
    rng = np.random.default_rng(1)
    t = np.array([[[-1000.0, -80.0, 70.0, 500.0, 20.0]]], F32)
    for _ in range(20):
        u = rng.random(t.shape, dtype=F32)
        c = O.assign_grid_stochastic(t, lv, u)
        # below the lowest level: 0; above the highest: 15; exactly on a level: that level
        assert c[0, 0, 0] == 0 and c[0, 0, 3] == 15
        assert c[0, 0, 1] == 0 and c[0, 0, 2] == 15 and c[0, 0, 4] == 10


def test_stochastic_equal_levels_have_zero_width():
    lv = _levels([[-5.0] * 4 + [0.0] * 8 + [5.0] * 4])
    t = np.array([[[-5.0, -1.0, 0.0, 2.0, 7.0]]], F32)
    u = np.full_like(t, 0.3)
    # left insertion point p, lo = clamp(p - 1, 0, 14), thr = 0.3 * (lv[lo+1] - lv[lo]) + lv[lo]:
    #   -5: p 0, lo 0, width 0, thr -5, not above -> 0
    #   -1: p 4, lo 3, thr -3.5 -> 4;   0: p 4 (left of the run of zeros) -> 4
    #    2: p 12, lo 11, thr 1.5 -> 12;  7: p 16, lo 14, width 0, thr 5 -> 15
    assert O.assign_grid_stochastic(t, lv, u).tolist() == [[[0, 4, 4, 12, 15]]]


def test_stochastic_choice_brackets_the_target_and_is_unbiased():
    rng = np.random.default_rng(7)
    lv = _levels([np.sort(rng.integers(-127, 128, 16)).astype(np.float64)])
    lv[0, 0, 8] = lv[0, 0, 7]                                # a zero-width bracket too
    lv = np.sort(lv, axis=-1)
    t = rng.uniform(lv.min(), lv.max(), (1, 1, 64)).astype(F32)
    n_draws = 20000
    acc = np.zeros(t.shape, np.float64)
    for _ in range(n_draws // 1000):
        u = rng.random((1000,) + t.shape[1:], dtype=F32).reshape(1000, 1, 64)
        tt = np.broadcast_to(t, u.shape).reshape(1, 1000, 64)
        uu = u.reshape(1, 1000, 64)
        lvv = np.broadcast_to(lv, (1, 1000, 16))
        c = O.assign_grid_stochastic(tt, lvv, uu)
        chosen = np.take_along_axis(lvv, c, axis=2)
        below = np.array([lv[0, 0][lv[0, 0] <= x].max() for x in t[0, 0]])
        above = np.array([lv[0, 0][lv[0, 0] >= x].min() for x in t[0, 0]])
        assert np.all((chosen == below) | (chosen == above))
        acc += chosen.sum(axis=1, keepdims=True)
    mean = acc / n_draws
    width = above - below
    # the mean of the chosen levels is the target; the standard error of a mean of
    # Bernoulli bracket choices is at most width / (2 sqrt(n))
    tol = 5 * np.maximum(width, 1e-9) / (2 * np.sqrt(n_draws)) + 1e-6
    assert np.all(np.abs(mean[0, 0] - t[0, 0].astype(np.float64)) <= tol)


# ---------------------------------------------------------------- requantize / fake quant

def _layer(n=6, k=512, seed=3):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.02, (n, k)).astype(F32)
    packed, srel, sch, cb = O.quantize_w4(w)
    return w, packed, srel, sch, cb


def test_requantize_on_own_scales_reproduces_the_quantiser():
    w, packed, srel, sch, cb = _layer()
    assert np.array_equal(O.requantize_codes(w, srel, sch, cb), packed)
    w_rot = O.rotate_to_f32(w)
    assert np.array_equal(O.requantize_codes(w_rot, srel, sch, cb, rotated=True), packed)


def test_requantize_picks_the_nearest_grid_level_brute_force():
    w, packed, srel, sch, cb = _layer(n=3, k=256, seed=11)
    w2 = w + np.random.default_rng(12).normal(0, 0.01, w.shape).astype(F32)   # a trained step
    codes = O.unpack_codes(O.requantize_codes(w2, srel, sch, cb))
    target = O.rotate(w2).astype(F32) / sch[:, None]
    levels = O.grid_levels(cb, srel)                                          # [N, G, 16]
    for n in range(w.shape[0]):
        for kk in range(w.shape[1]):
            lv = levels[n, kk // 16].astype(np.float64)
            d = np.abs(lv - np.float64(target[n, kk]))
            chosen = d[codes[n, kk]]
            assert chosen <= d.min() + 1e-5 * max(1.0, abs(float(target[n, kk]))), (n, kk)


def test_requantize_stochastic_is_unbiased_on_the_grid():
    w, packed, srel, sch, cb = _layer(n=2, k=256, seed=21)
    w2 = w * F32(1.03)
    rng = np.random.default_rng(22)
    levels = O.grid_levels(cb, srel)
    target = (O.rotate_to_f32(w2).reshape(2, 16, 16) / sch[:, None, None]).astype(np.float64)
    inside = (target > levels.min(axis=-1, keepdims=True)) & (target < levels.max(axis=-1, keepdims=True))
    total = np.zeros(target.shape)
    n_draws = 3000
    for _ in range(n_draws):
        u = rng.random((2, 256), dtype=F32)
        c = O.unpack_codes(O.requantize_codes(w2, srel, sch, cb, u=u)).reshape(2, 16, 16)
        total += np.take_along_axis(levels, c, axis=2)
    mean = total / n_draws
    width = levels.max() - levels.min()
    assert np.all(np.abs(mean - target)[inside] < 5 * 254 / (2 * np.sqrt(n_draws)))
    assert np.abs(mean - target)[inside].mean() < 0.2   # far below one grid step
    assert width > 0


def test_fake_quant_is_a_projection_onto_the_grid():
    w, packed, srel, sch, cb = _layer(seed=31)
    w_rot = O.rotate_to_f32(w * F32(0.9))
    fq = O.fake_quant_rotated(w_rot, srel, sch, cb)
    assert np.array_equal(O.fake_quant_rotated(fq, srel, sch, cb), fq)        # idempotent
    # with every level inside [-127, 127] (scale bytes up to 0x70 = 128 with this
    # codebook), it equals decoding the requantised codes times the channel scale
    assert srel.max() <= 0x70
    codes = O.requantize_codes(w_rot, srel, sch, cb, rotated=True)
    assert np.array_equal(fq, O.dequantize_f32(codes, srel, sch, cb, rotate_back=False))


# ---------------------------------------------------------------- dequantize

def _digit_sign(i, j):
    s = 0
    for _ in range(4):
        s += (i % 4) + (j % 4) == 3
        i //= 4
        j //= 4
    return -1.0 if s % 2 else 1.0


def test_dequantize_constant_and_one_hot_rows():
    cb = O.uniform_codebook()                      # code c decodes to c - 8 at scale 1.0
    srel = np.full((2, 256 // 16), 0x38, np.uint8)  # e4m3 0x38 = 1.0
    codes = np.full((2, 256), 8, np.uint8)
    codes[0, :] = 11                              # constant 3: rotation keeps it constant
    codes[1, 77] = 13                             # one-hot 5 at column 77
    sch = np.array([0.5, 0.25], F32)
    w = O.dequantize_f32(O.pack_codes(codes), srel, sch, cb)
    assert np.all(w[0] == F32(1.5))
    expect = np.array([5 * 0.25 / 16 * _digit_sign(77, j) for j in range(256)], F32)
    assert np.array_equal(w[1], expect)
    w_rot = O.dequantize_f32(O.pack_codes(codes), srel, sch, cb, rotate_back=False)
    assert w_rot[1, 77] == F32(1.25) and np.count_nonzero(w_rot[1]) == 1


def test_dequantize_f32_is_the_exact_block_product_rounded_once():
    # exact rational arithmetic on two blocks of one row: the page's fp32 products
    # w8 * s_channel, multiplied by +-1/16 (digit rule) and summed exactly, then rounded
    # once to fp32; the fp64 sum of these terms is exact, so the oracle must agree bit
    # for bit
    from fractions import Fraction
    w, packed, srel, sch, cb = _layer(n=2, k=512, seed=41)
    got = O.dequantize_f32(packed, srel, sch, cb)
    prod = (O.decode_w4(packed, srel, cb).astype(F32) * sch[:, None]).astype(F32)
    row = 1
    for blk in range(2):
        terms = [Fraction(float(v)) for v in prod[row, 256 * blk:256 * blk + 256]]
        for i in range(0, 256, 17):
            exact = sum(t * int(_digit_sign(j, i)) for j, t in enumerate(terms)) / 16   # stays a Fraction
            assert float(exact) == exact                      # representable in fp64
            assert got[row, 256 * blk + i] == np.float32(float(exact)), (blk, i)


# ---------------------------------------------------------------- straight-through backward

def test_ste_weight_bf16_hand_roundings():
    cb = O.uniform_codebook()
    srel = np.full((4, 16), 0x38, np.uint8)                      # decoded levels c - 8
    codes = np.full((4, 256), 8, np.uint8)
    codes[:, 0] = [15, 0, 11, 15]                                # w8 = 7, -8, 3, 7
    # scale 0x78 = 256 gives w8 = rint(level * 256) clamped: use e4m3 16.0 (0x58) for
    # row 0 so that w8 = 7 * 16 = 112, saturating nothing
    srel[0, 0] = 0x58
    srel[1, 0] = 0x58                                            # -8 * 16 = -128
    sch = np.array([1.5, 0.75, 1.00390625, 0.1], F32)
    w = O.ste_weight_bf16(O.pack_codes(codes), srel, sch, cb)
    assert w[0, 0] == 168.0                  # 112 * 1.5 exact in bf16 (8 significant bits)
    assert w[1, 0] == -96.0                  # -128 * 0.75 = -96 exact
    assert w[2, 0] == 3.0                    # 1 + 2^-8 rounds to 1.0 in bf16 (tie to even)
    # bf16(0.1) = 1.1001101b * 2^-4 = 0.10009765625; times 7 = 1.0110011011b * 2^-1, whose
    # 8-bit rounding drops 011 (below half): 1.0110011b * 2^-1 = 0.69921875
    assert w[3, 0] == 0.69921875


def test_ste_weight_tie_rounds_to_even():
    cb = O.uniform_codebook().copy()
    cb[9] = F32(127.0 / 256.0)                                   # decodes to 127 at scale 256
    srel = np.full((1, 16), 0x78, np.uint8)                      # e4m3 0x78 = 256
    codes = np.full((1, 256), 8, np.uint8)                       # level 0 everywhere ...
    codes[0, 2] = 9                                              # ... but w8 = 127 here
    w = O.ste_weight_bf16(O.pack_codes(codes), srel, np.array([0.75], F32), cb)
    # 127 * 0.75 = 95.25 = 1011111.01b: nine significant bits, exactly half way between
    # 95.0 and 95.5 -> the even one, 95.0
    assert w[0, 2] == 95.0 and np.count_nonzero(w) == 1


def test_grad_input_matches_plain_loops_and_selects_rows():
    rng = np.random.default_rng(51)
    m, n, k = 3, 5, 7
    g = O.bf16_bits_to_f32(O.f32_to_bf16_bits(rng.normal(0, 1, (m, n)).astype(F32)))
    w = O.bf16_bits_to_f32(O.f32_to_bf16_bits(rng.normal(0, 1, (n, k)).astype(F32)))
    got = O.grad_input_exact(g, w)
    for i in range(m):
        for j in range(k):
            s = 0.0
            for t in range(n):
                s += float(g[i, t]) * float(w[t, j])
            assert abs(got[i, j] - s) <= 1e-12 * max(1.0, abs(s))
    onehot = np.zeros((1, n), F32)
    onehot[0, 3] = 1.0
    assert np.array_equal(O.grad_input_exact(onehot, w)[0], w[3].astype(np.float64))


# ---------------------------------------------------------------- variants

def test_interleave_rows_hand_example():
    t = np.arange(6)[:, None] * np.ones((1, 2), int)
    assert O.interleave_rows(t)[:, 0].tolist() == [0, 3, 1, 4, 2, 5]
    with pytest.raises(ValueError):
        O.interleave_rows(np.zeros((3, 2)))


def test_swiglu_against_library_sigmoid_and_special_values():
    rng = np.random.default_rng(61)
    y = rng.normal(0, 3, (4, 10))
    got = O.swiglu_interleaved(y)
    g, u = y[:, 0::2], y[:, 1::2]
    assert np.allclose(got, g * expit(g) * u, rtol=1e-14, atol=0)
    z = O.swiglu_interleaved(np.array([0.0, 5.0, 2.0, 0.0, 60.0, 2.0, -60.0, 2.0]))
    assert z[0] == 0.0 and z[1] == 0.0 and abs(z[2] - 120.0) < 1e-9 and abs(z[3]) < 1e-20


def test_lora_delta_exact_small_integers_and_scale():
    a = np.array([[1, 2, 3], [0, -1, 4]], F32)          # r = 2, K = 3
    b = np.array([[2, 0], [1, 1], [-3, 5]], F32)        # N = 3
    d = O.lora_delta(a, b, 0.5)
    assert np.array_equal(d, np.array([[1, 2, 3], [0.5, 0.5, 3.5], [-1.5, -5.5, 5.5]], F32))
    rng = np.random.default_rng(71)
    a = rng.normal(0, 1, (16, 256)).astype(F32)
    b = rng.normal(0, 1, (64, 16)).astype(F32)
    ref = (b.astype(np.float64) @ a.astype(np.float64)) * np.float64(F32(0.3))
    assert np.max(np.abs(O.lora_delta(a, b, 0.3) - ref)) <= 2 ** -23 * np.max(np.abs(ref))


def test_lora_merge_zero_adapter_is_the_dequantised_weight():
    w, packed, srel, sch, cb = _layer(n=4, k=256, seed=81)
    a = np.zeros((4, 256), F32)
    b = np.zeros((4, 4), F32)
    assert np.array_equal(O.lora_merge_weight(packed, srel, sch, cb, a, b, 1.0),
                          O.dequantize_f32(packed, srel, sch, cb))
