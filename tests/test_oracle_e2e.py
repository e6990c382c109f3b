"""End-to-end sanity of the oracle layer against the unquantised product (a
quality figure, not parity), and the synthetic input recipe."""

import numpy as np

import oracle as O
from bit_codebook_quantized_amd import synth


def test_linear_close_to_unquantised_product():
    w = synth.gaussian_weight(128, 1024, seed=synth.seed_for(0, 0, 0))
    x = synth.activations(16, 1024, seed=synth.seed_for(0, 0, 1))
    packed, srel, sch, cb = O.quantize_w4(w)
    y, xq, xs, w8 = O.linear(x, packed, srel, sch, cb, out="f32")
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.15, rel
    # bf16 output is the fp32 output rounded once
    yb, *_ = O.linear(x, packed, srel, sch, cb, out="bf16")
    assert np.array_equal(yb, O.f32_to_bf16_bits(y))


def test_synth_recipe():
    a = synth.activations(8, 4096, seed=5, kind="outliers", outlier_seed=6)
    b = synth.activations(8, 4096, seed=5, kind="outliers", outlier_seed=6)
    assert np.array_equal(a, b)
    base = synth.activations(8, 4096, seed=5, kind="normal")
    ratio = np.abs(a).mean(axis=0) / np.maximum(np.abs(base).mean(axis=0), 1e-9)
    assert int((ratio > 10).sum()) == 41          # round(0.01 * 4096) outlier columns
    # bf16-representable values
    assert np.all((a.view(np.uint32) & 0xFFFF) == 0)
    t = synth.activations(4, 3072, seed=1, kind="student_t")
    assert np.abs(t).max() > 8                     # heavy tails
    p, s, c = synth.random_layer_bytes(16, 512, seed=3)
    assert p.shape == (16, 256) and s.shape == (16, 32) and c.shape == (16,)
