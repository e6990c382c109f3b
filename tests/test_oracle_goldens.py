"""Hand-worked pins of the oracle's weight quantiser, grid levels and epilogue
(tests/golden/, each file citing the passage it follows), and exact-arithmetic
checks of the scale steps and of the exact block rotation.

Each is chosen so that a plausible slip fails it: the number of ALS passes, the
channel-scale divisor, the scale floor, the e4m3 rounding of the relative scale,
the grid clamp at -127 and its ties-to-even rounding, and the epilogue's product
order."""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _f32(hexword):
    return np.array([int(hexword, 16)], np.uint32).view(np.float32)[0]


def _trace_golden():
    return {r[0]: r[1:] for r in _read("quantizer_trace.txt")}


def test_quantizer_trace_hand_worked():
    g = _trace_golden()
    k = np.array([int(v) for v in g["k"]], np.float64)
    row = np.concatenate([k / 16, k / 16 * 2.0 ** -22]).astype(np.float32).reshape(1, 32)
    t = O.quantize_trace(row)
    ints = lambda key: [int(v) for v in g[key]]
    for p in range(O.ALS_ITERS + 1):
        assert t[f"codes{p}"][0, 0].tolist() == ints(f"codes{p}"), p
        # group B: the same codes, scales exactly 2^-22 times group A's
        assert t[f"codes{p}"][0, 1].tolist() == ints(f"codes{p}"), p
        assert t[f"scale{p}"][0, 1] == t[f"scale{p}"][0, 0] * np.float32(2.0 ** -22), p
    assert t["scale0"][0, 0] == 1.0 and t["scale0"][0, 1] == np.float32(2.0 ** -22)
    assert O.ALS_ITERS == 2
    assert t["scale1"][0, 0] == _f32(g["scale1"][0])
    assert t["scale2"][0, 0] == _f32(g["scale2"][0])
    assert t["row_top"][0] == _f32(g["row_top"][0])
    assert t["s_channel"][0] == _f32(g["s_channel"][0])
    assert t["srel"][0].tolist() == [int(v, 16) for v in g["srel"]]
    assert t["final_codes"][0, 0].tolist() == ints("final_a")
    assert t["final_codes"][0, 1].tolist() == ints("final_b")
    assert t["packed"][0, :8].tolist() == [int(v, 16) for v in g["packed_a"]]
    # the public entry returns the same storage
    packed, srel, sch, _ = O.quantize_w4_rotated(row)
    assert np.array_equal(packed, t["packed"]) and np.array_equal(srel, t["srel"])
    assert sch.view(np.uint32)[0] == t["s_channel"].view(np.uint32)[0]


def test_grid_levels_hand_worked():
    for cbname, sb, *levels in _read("grid_levels_hand.txt"):
        cb = O.FIXED_CODEBOOK if cbname == "fixed" else O.uniform_codebook()
        got = O.grid_levels(cb, np.array([[int(sb, 16)]], np.uint8))[0, 0]
        assert got.tolist() == [float(v) for v in levels], (cbname, sb)


def test_epilogue_hand_worked():
    for acc, xs, ws, bias, y32, y16 in _read("epilogue_hand.txt"):
        a = np.array([[int(acc)]], np.int64)
        xs_, ws_ = np.array([_f32(xs)]), np.array([_f32(ws)])
        b = None if bias == "-" else np.array([_f32(bias)])
        y = O.epilogue(a, xs_, ws_, b, out="f32")
        assert y.view(np.uint32)[0, 0] == int(y32, 16)
        assert O.epilogue(a, xs_, ws_, b, out="bf16")[0, 0] == int(y16, 16)


# ---------------------------------------------------------------- scale steps, exactly

def _ulp32(v):
    v = np.float32(v)
    return Fraction(float(np.nextafter(v, np.float32(np.inf)))) - Fraction(float(v))


@pytest.mark.parametrize("seed", range(3))
def test_channel_scale_is_row_top_over_127(seed):
    # s_channel is the fp32 value nearest to row_top / 127: within half an ulp of it, with
    # exact rational arithmetic (a divisor of 128 would be ~0.8% off)
    rng = np.random.default_rng(40 + seed)
    w = (rng.standard_normal((24, 256)) * 0.02).astype(np.float32)
    t = O.quantize_trace(w)
    cb = O.FIXED_CODEBOOK
    scale = t[f"scale{O.ALS_ITERS}"]
    for r in range(w.shape[0]):
        # row_top: the largest fp32 product |level * scale| over the row, formed exactly here
        prods = [abs(Fraction(float(np.float32(Fraction(float(cb[c])) * Fraction(float(s))))))
                 for cs, s in zip(t[f"codes{O.ALS_ITERS}"][r], scale[r]) for c in cs]
        top = max(prods)
        assert Fraction(float(t["row_top"][r])) == top
        sch = t["s_channel"][r]
        assert abs(Fraction(float(sch)) - top / 127) <= _ulp32(sch) / 2


def _e4m3_values():
    vals = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        vals.append((v, b))
    return vals


@pytest.mark.parametrize("seed", range(3))
def test_relative_scale_byte_is_the_nearest_e4m3(seed):
    # brute force over the 127 non-negative finite e4m3 values: the stored byte is the one
    # nearest to fp32(scale / s_channel), a tie going to the even mantissa
    rng = np.random.default_rng(60 + seed)
    w = (rng.standard_normal((16, 512)) * np.exp(rng.uniform(-3, 3, (16, 1))) * 0.02).astype(np.float32)
    t = O.quantize_trace(w)
    scale = t[f"scale{O.ALS_ITERS}"]
    vals = _e4m3_values()
    for r in range(w.shape[0]):
        for g in range(scale.shape[1]):
            ratio = Fraction(float(np.float32(scale[r, g] / t["s_channel"][r])))
            best = min(vals, key=lambda vb: (abs(vb[0] - ratio), vb[1] & 1))
            assert t["srel"][r, g] == best[1], (r, g, float(ratio))


# ---------------------------------------------------------------- exact rotation

def _is_nearest_f32(r, exact):
    """r is the fp32 value nearest to the rational `exact` (ties to an even significand)."""
    r = np.float32(r)
    d = abs(Fraction(float(r)) - exact)
    for nb in (np.nextafter(r, np.float32(-np.inf)), np.nextafter(r, np.float32(np.inf))):
        dn = abs(Fraction(float(nb)) - exact)
        if dn < d or (dn == d and int(np.array([r]).view(np.uint32)[0]) & 1):
            return False
    return True


def _exact_block(x):
    h = np.sign(O.hadamard(256)).astype(int)
    xs = [Fraction(float(v)) for v in x]
    return [sum(h[i, j] * xs[j] for j in range(256)) / 16 for i in range(256)]


def test_round_dyadic_matches_the_ieee_cast():
    # for numbers that fp64 holds exactly, one rounding to fp32 is numpy's cast
    rng = np.random.default_rng(70)
    cases = [(0, 0), (1, 0), (-3, -200), ((1 << 24) + 1, -1), ((1 << 25) + 2, 5), ((1 << 25) + 6, 5),
             ((1 << 24) - 1, 104), ((1 << 24) - 1, 105), (1, -149), (1, -150), (3, -151), (1, 127), (1, 128)]
    for _ in range(3000):
        m = int(rng.integers(1, 1 << 53)) * (1 if rng.random() < 0.5 else -1)
        cases.append((m, int(rng.integers(-210, 80))))
    with np.errstate(over="ignore"):
        for m, e in cases:
            want = np.float32(np.float64(m) * np.float64(2.0) ** e)
            got = O.round_dyadic_to_f32(m, e)
            assert got.view(np.uint32) == want.view(np.uint32) or (got == 0 and want == 0), (m, e, got, want)


@pytest.mark.parametrize("spread", [44, 45, 60, 120])
def test_rotation_is_the_exact_product_rounded_once(spread):
    # blocks whose inputs span `spread` binades between the top exponent and the lowest set
    # bit: at 44 the fp64 product is exact, beyond it the oracle sums integers; either way
    # every output must be the fp32 value nearest to the exact block product
    rng = np.random.default_rng(spread)
    x = np.zeros((2, 256), np.float32)
    x[:, :] = (rng.standard_normal((2, 256)) * 0.25).astype(np.float32)
    # bf16-valued inputs (8 significant bits), the largest with exponent 0 and one input with
    # its lowest set bit at 2^-spread
    bits = x.view(np.uint32) & np.uint32(0xFFFF0000)
    x = bits.view(np.float32)
    x[:, 0] = 1.9921875
    x[:, 1] = np.float32(255.0 * 2.0 ** (-spread))
    x[:, 2] = -np.float32(129.0 * 2.0 ** (-spread))
    assert np.abs(x).max() < 2.0
    got = O.rotate_to_f32(x)
    for b in range(2):
        ex = _exact_block(x[b])
        for i in range(256):
            assert _is_nearest_f32(got[b, i], ex[i]), (spread, b, i)


def test_rotation_overflow_and_non_finite_blocks():
    h0 = np.sign(O.hadamard(256)[0]).astype(np.float32)   # the sign pattern of row 0 of H
    x = np.zeros((4, 512), np.float32)
    # the largest bf16 times row 0's signs: output 0 is 16 times it (overflow to +inf), the
    # other outputs are 0 (the rows of H are orthogonal)
    x[0, :256] = h0 * np.float32(3.3895313892515355e38)
    x[1, 7] = np.inf
    x[2, 300] = np.nan
    x[3, :] = 1.0
    r = O.rotate_to_f32(x)
    assert np.isposinf(r[0, 0]) and np.all(r[0, 1:256] == 0)
    assert np.all(np.isnan(r[1, :256])) and np.all(r[1, 256:] == 0)
    assert np.all(np.isnan(r[2, 256:])) and np.all(r[2, :256] == 0)
    assert np.all(r[3] == 1.0)          # every row and column of H sums to 16


def test_quant_act_rows_with_non_finite_values():
    # reading for a row without a finite maximum: scale NaN, every code 0; other rows as usual
    v = np.ones((4, 256), np.float32)
    v[1, 5] = np.inf
    v[2, 9] = -np.nan
    v[3, :] = 2.0
    q, s = O.quant_act(v)
    assert np.isnan(s[1]) and np.isnan(s[2]) and np.all(q[1:3] == 0)
    assert s[0] == np.float32(1.0) / np.float32(127.0) and np.all(q[0] == 127)
    assert s[3] == np.float32(2.0) / np.float32(127.0) and np.all(q[3] == 127)
    # through the rotation: an overflowing block poisons its row only
    x = np.ones((2, 512), np.float32)
    x[0, :256] = np.sign(O.hadamard(256)[0]).astype(np.float32) * np.float32(3.3895313892515355e38)
    q, s = O.rotate_quant_act(x)
    assert np.isnan(s[0]) and np.all(q[0] == 0)
    assert s[1] == np.float32(1.0) / np.float32(127.0) and np.all(q[1] == 127)


def test_als_sums_are_exact_then_rounded_once():
    g = _trace_golden()
    row = np.array([_f32(g["c_w0"][0])] + [_f32(g["c_wrest"][0])] * 15, np.float32).reshape(1, 16)
    t = O.quantize_trace(row)
    assert t["codes0"][0, 0].tolist() == [int(v) for v in g["c_codes0"]]
    assert t["scale1"][0, 0] == _f32(g["c_scale1"][0])
