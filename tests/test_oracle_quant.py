"""Pins for the oracle's activation quantiser, nibble packing, int8-grid decode
and weight quantiser: hand-worked values (tests/golden/), special cases that
reduce to textbook rules, brute force over all levels, and the least-squares
property of the group-scale refinement."""

import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- activation quant

def test_quant_act_ties_hand_example():
    # amax 127 -> scale exactly 1; v/scale exact; half-way values round to even
    v = np.zeros((1, 256), np.float32)
    v[0, :6] = [127, 0.5, 1.5, 2.5, -0.5, -2.5]
    q, s = O.quant_act(v)
    assert s.tolist() == [1.0]
    assert q[0, :6].tolist() == [127, 0, 2, 2, 0, -2]
    assert np.all(q[0, 6:] == 0)


def test_quant_act_zero_row_and_ones_row():
    q, s = O.quant_act(np.zeros((1, 512), np.float32))
    assert s.tolist() == [1.0] and np.all(q == 0)
    q, s = O.quant_act(np.ones((1, 512), np.float32))
    assert s[0] == np.float32(1.0) / np.float32(127.0)
    assert np.all(q == 127)


def test_rotate_quant_act_ones_and_one_hot():
    # rotate(ones) = ones exactly, so the row quantises to all 127
    q, s = O.rotate_quant_act(np.ones((1, 256), np.float32))
    assert np.all(q == 127)
    # a one-hot row rotates to +-1/16 (sign by the digit rule): |q| = 127 everywhere
    e = np.zeros((1, 256), np.float32)
    e[0, 0] = 1
    q, s = O.rotate_quant_act(e)
    assert np.all(np.abs(q) == 127)
    assert s[0] == np.float32(1 / 16) / np.float32(127)
    signs = [(-1) ** sum(1 for d in range(4) if (j >> (2 * d)) & 3 == 3) for j in range(256)]
    assert np.array_equal(np.sign(q[0]), signs)


def test_quant_act_bounds_and_scale_property():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((64, 1024)) * np.exp(rng.uniform(-5, 5, (64, 1)))).astype(np.float32)
    q, s = O.quant_act(v)
    assert np.all(np.abs(q.astype(int)) <= 127)
    # the element of largest magnitude lands on +-127; every |v - q*s| is at most s/2 (+1 ulp)
    assert np.all(np.abs(q).max(axis=1) == 127)
    err = np.abs(v.astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 1e-6))


# ---------------------------------------------------------------- pack / unpack

def test_pack_hand_bytes_and_roundtrip():
    assert O.pack_codes(np.array([[3, 12]])).tolist() == [[0xC3]]
    assert O.unpack_codes(np.array([[0x1F]], np.uint8)).tolist() == [[15, 1]]
    rng = np.random.default_rng(0)
    c = rng.integers(0, 16, (7, 64))
    assert np.array_equal(O.unpack_codes(O.pack_codes(c)), c)
    b = rng.integers(0, 256, (5, 40), dtype=np.uint8)
    assert np.array_equal(O.pack_codes(O.unpack_codes(b)), b)


# ---------------------------------------------------------------- decode

def _golden_decodes():
    rows = []
    with open(os.path.join(GOLDEN, "decode_hand.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                cbname, sb, code, want = line.split()
                rows.append((cbname, int(sb, 16), int(code), int(want)))
    return rows


def test_decode_hand_worked_values():
    rows = _golden_decodes()
    assert len(rows) > 40
    for cbname, sb, code, want in rows:
        cb = O.FIXED_CODEBOOK if cbname == "fixed" else O.uniform_codebook()
        codes = np.zeros((1, 16), np.int64)
        codes[0, 0] = code
        got = O.decode_w4(O.pack_codes(codes), np.array([[sb]], np.uint8), cb)[0, 0]
        assert got == want, (cbname, hex(sb), code, got, want)


def test_decode_uniform_codebook_unit_scale_is_signed_int4():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, (8, 256))
    srel = np.full((8, 16), 0x38, np.uint8)
    w8 = O.decode_w4(O.pack_codes(codes), srel, O.uniform_codebook())
    assert np.array_equal(w8, codes - 8)


def test_decode_group_scale_applies_per_16_columns():
    codes = np.full((1, 64), 15)
    srel = np.array([[0x38, 0x70, 0x78, 0x01]], np.uint8)
    w8 = O.decode_w4(O.pack_codes(codes), srel, O.FIXED_CODEBOOK)[0]
    assert w8[:16].tolist() == [1] * 16 and w8[16:32].tolist() == [126] * 16
    assert w8[32:48].tolist() == [127] * 16 and w8[48:].tolist() == [0] * 16


def test_decode_exhaustive_table_properties():
    # every (scale byte, code) pair: result in [-128, 127], NaN scale -> 0, monotone in the
    # code for a positive scale, and equal to the rounded product where it is in range
    sb = np.repeat(np.arange(256, dtype=np.uint8), 16).reshape(256, 16)[:, :1]
    codes = np.tile(np.arange(16), (256, 1))
    w8 = O.decode_w4(O.pack_codes(codes), sb.reshape(256, 1), O.FIXED_CODEBOOK).astype(int)
    s = O.e4m3fn_to_f32(np.arange(256, dtype=np.uint8)).astype(np.float64)
    for b in range(256):
        if np.isnan(s[b]):
            assert np.all(w8[b] == 0)
            continue
        exact = O.FIXED_CODEBOOK.astype(np.float64) * s[b]
        inrange = np.abs(exact) < 127
        assert np.all(np.abs(w8[b][inrange] - exact[inrange]) <= 0.5 + 1e-5)
        assert np.all(w8[b][exact >= 127.5] == 127) and np.all(w8[b][exact <= -128.5] == -128)
        d = np.diff(w8[b])
        assert np.all(d >= 0) if s[b] > 0 else np.all(d <= 0)


# ---------------------------------------------------------------- weight quantiser

def test_assign_codes_brute_force_nearest_lowest_on_tie():
    rng = np.random.default_rng(8)
    cb = O.FIXED_CODEBOOK
    x = np.concatenate([rng.uniform(-1.2, 1.2, 5000),
                        ((cb[1:].astype(np.float64) + cb[:-1]) / 2)]).astype(np.float32)
    got = O.assign_codes(x, cb)
    d = np.abs((x[:, None] - cb[None, :]).astype(np.float32))
    best = d.min(axis=1, keepdims=True)
    lowest = np.argmax(d == best, axis=1)
    assert np.array_equal(got, lowest)


def test_assign_grid_duplicates_follow_left_insertion_rule():
    # levels with runs of equal values, as a small scale produces:
    lv = np.array([-1] * 4 + [0] * 8 + [1] * 4, np.float32).reshape(1, 1, 16)
    t = np.array([0.3, -0.3, 0.0, 0.5, -0.5, 2.0, -2.0, 1.0], np.float32).reshape(1, 1, 8)
    # 0.3: insertion point 12 (first level >= 0.3), 0 at index 11 is closer -> 11
    # -0.3: insertion point 4, level 0 at index 4 closer than -1 -> 4
    # 0.0: insertion point 4, distance 0 to index 4 -> 4
    # 0.5 / -0.5: equal distances -> the lower candidate (11 / 3)
    # 2.0: insertion point 16 -> both candidates clamp to 15; -2.0: 0
    # 1.0: insertion point 12, distance 0 -> 12
    assert O.assign_grid(t, lv).reshape(-1).tolist() == [11, 4, 4, 11, 3, 15, 0, 12]


def test_quantizer_all_zero_row():
    packed, srel, sch, _ = O.quantize_w4_rotated(np.zeros((2, 256), np.float32))
    assert np.all(packed == 0x44)
    assert np.all(srel == 0x38)
    assert np.all(sch == np.float32(1e-8))


def _small_rotated(n=4, k=32, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, k)) * 0.02).astype(np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_quantizer_brute_force_small_tiles(seed):
    w = _small_rotated(seed=seed)
    if seed == 5:
        w[1, 3] *= 40          # an outlier weight
        w[2, 16:] = 0          # a zero group
    info = O.quantize_trace(w)
    packed, srel, sch = info["packed"], info["srel"], info["s_channel"]
    codes = O.unpack_codes(packed)
    assert codes.min() >= 0 and codes.max() <= 15
    assert np.all(O.e4m3fn_to_f32(srel) >= 0) and np.all(sch > 0)
    # final codes: the chosen level value is the nearest of all 16 to w / s_channel
    lv = O.grid_levels(O.FIXED_CODEBOOK, srel).astype(np.float64)            # [n, G, 16]
    t = (w.reshape(4, 2, 16) / sch[:, None, None]).astype(np.float32).astype(np.float64)
    dist = np.abs(t[..., None] - lv[:, :, None, :])                          # [n, G, 16, 16]
    chosen = np.take_along_axis(lv, codes.reshape(4, 2, 16), axis=2)
    assert np.all(np.abs(t - chosen) <= dist.min(axis=-1) + 1e-6)
    # the decoded grid is within [-127, 127] (grid clamp) and reconstructs w to within
    # half a grid step plus the clamp
    w8 = O.decode_w4(packed, srel, O.FIXED_CODEBOOK)
    assert np.abs(w8.astype(int)).max() <= 127
    # every pass's codes are the nearest codebook indices of w / gs
    gw = info["groups"]
    for it in range(O.ALS_ITERS + 1):
        q, gs = info[f"codes{it}"], info[f"scale{it}"][..., None]
        x = (gw / gs).astype(np.float32)
        d = np.abs((x[..., None] - O.FIXED_CODEBOOK).astype(np.float32))
        assert np.array_equal(q, np.argmax(d == d.min(axis=-1, keepdims=True), axis=-1))


@pytest.mark.parametrize("seed", range(4))
def test_als_step_solves_least_squares(seed):
    # for the codes it used, each refined group scale minimises sum (w - gs*cb[q])^2:
    # the normal equation sum cb[q]*(w - gs*cb[q]) = 0 holds to fp32 rounding
    w = _small_rotated(n=8, k=64, seed=seed)
    info = O.quantize_trace(w)
    gw = info["groups"].astype(np.float64)
    for it in range(1, O.ALS_ITERS + 1):
        lv = O.FIXED_CODEBOOK[info[f"codes{it - 1}"]].astype(np.float64)
        gs = info[f"scale{it}"].astype(np.float64)[..., None]
        resid = (lv * (gw - gs * lv)).sum(axis=-1)
        scale = (lv * lv).sum(axis=-1) * gs[..., 0]
        assert np.all(np.abs(resid) <= 1e-6 * scale + 1e-12)
        # and gs moved from the group absmax: it is a least-squares fit, not the max
        assert not np.array_equal(info[f"scale{it}"], info["scale0"])


@pytest.mark.parametrize("seed", range(3))
def test_als_passes_never_increase_the_group_error(seed):
    # the quality gain of the refinement: a least-squares scale for fixed codes, then the
    # nearest codes for that scale, so the group's squared error can only fall from the
    # absmax fit (pass 0) through each pass (up to fp32 rounding of gs), and it does fall
    w = _small_rotated(n=32, k=256, seed=100 + seed)
    info = O.quantize_trace(w)
    gw = info["groups"].astype(np.float64)
    err = []
    for it in range(O.ALS_ITERS + 1):
        lv = O.FIXED_CODEBOOK[info[f"codes{it}"]].astype(np.float64)
        err.append(((gw - info[f"scale{it}"].astype(np.float64)[..., None] * lv) ** 2).sum(axis=-1))
    for it in range(O.ALS_ITERS):
        assert np.all(err[it + 1] <= err[it] * (1 + 1e-5) + 1e-30)
    assert err[-1].mean() < 0.95 * err[0].mean()


def test_channel_scale_maps_largest_level_to_127():
    # s_channel = max |cb[q]*gs| / 127, so the largest |cb[q]| * srel per row is 127
    # up to the fp8 rounding of srel (3 mantissa bits: within 1/16 relative)
    w = _small_rotated(n=16, k=256, seed=3)
    info = O.quantize_trace(w)
    srel = info["srel"]
    s = O.e4m3fn_to_f32(srel).astype(np.float64)
    big = (np.abs(O.FIXED_CODEBOOK[info[f"codes{O.ALS_ITERS}"]]).max(axis=-1) * s).max(axis=1)
    assert np.all(np.abs(big - 127) <= 127 / 16)


def test_quantize_rejects_bad_k():
    with pytest.raises(ValueError):
        O.quantize_w4_rotated(np.zeros((2, 40), np.float32))


def test_quantize_dequantize_quality_gaussian():
    # a 4-bit Lloyd-Max grid on rotated Gaussian weights reconstructs them to about
    # 10% relative RMS error; a wrong rotation, sign or scale breaks this by far
    from bit_codebook_quantized_amd.synth import gaussian_weight
    w = gaussian_weight(64, 1024, seed=12)
    packed, srel, sch, cb = O.quantize_w4(w)
    wh = O.dequantize(packed, srel, sch, cb)
    rel = np.linalg.norm(wh - w) / np.linalg.norm(w)
    assert 0.03 < rel < 0.15, rel


def test_rows_are_quantised_independently():
    # a row's storage depends on that row alone: quantising a slice of rows gives the
    # same bytes and scales as the same rows of the whole matrix
    from bit_codebook_quantized_amd.synth import gaussian_weight
    w = O.rotate_to_f32(gaussian_weight(24, 512, seed=21))
    a = O.quantize_w4_rotated(w)
    b = O.quantize_w4_rotated(w[5:13])
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x[5:13], y)
