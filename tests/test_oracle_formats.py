"""Pins for the oracle's number formats (fp8 E4M3FN, bf16) against torch's own
conversions -- an independent library implementation of the same formats."""

import numpy as np
import pytest
import torch

import oracle as O


def test_e4m3_decode_all_256_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_to_f32(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e4m3_decode_hand_values():
    # 0x38 = exponent field 7 (bias 7) mantissa 0 -> 1.0; 0x7E -> 1.75 * 2^8
    vals = O.e4m3fn_to_f32(np.array([0x38, 0x30, 0x6C, 0x70, 0x78, 0x7E, 0x01, 0x08, 0x80], np.uint8))
    assert vals.tolist() == [1.0, 0.5, 96.0, 128.0, 256.0, 448.0, 2.0 ** -9, 2.0 ** -6, 0.0]
    assert np.signbit(vals[-1])


def _finite_e4m3_values():
    b = np.arange(256, dtype=np.uint8)
    v = O.e4m3fn_to_f32(b)
    return np.unique(v[~np.isnan(v)])


def test_e4m3_encode_matches_torch_on_values_ties_and_random():
    vals = _finite_e4m3_values()
    pos = vals[vals > 0]
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)    # exact ties
    rng = np.random.default_rng(7)
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(470.0), 20000)).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    edge = np.array([0.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6 - 2.0 ** -10, 448, 460, 464,
                     464.0001, 479, 480, 1e6], np.float32)
    x = np.concatenate([vals, mids, near, rand, edge])
    x = np.concatenate([x, -x])
    ours = O.f32_to_e4m3fn(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_roundtrip_of_representable_values():
    vals = _finite_e4m3_values()
    assert np.array_equal(O.e4m3fn_to_f32(O.f32_to_e4m3fn(vals)), vals)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-30, 30, 50000))).astype(np.float32)
    u = x.view(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)          # exact half-way cases
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1.0, 3.0e38, -3.0e38, 1e-40], np.float32)])
    ours = O.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_hand_ties():
    # 1 + 2^-8 lies half-way between bf16 1.0 and 1 + 2^-7: ties to the even mantissa (1.0)
    # 1 + 3*2^-8 lies half-way between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8], np.float32)
    assert O.bf16_bits_to_f32(O.f32_to_bf16_bits(x)).tolist() == [1.0, 1 + 2.0 ** -6]


def test_bf16_nan_stays_nan():
    assert np.isnan(O.bf16_bits_to_f32(O.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
