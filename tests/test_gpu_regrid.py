"""GPU parity of the training-path weight kernels (requantize_codes_w4, fake_quant_w4,
dequantize_w4 through the C ABI binding) against the CPU oracle on the same seeded
inputs.

Bar: bit-exact packed codes and bit-identical fp32 outputs.  Shapes cover one to four
4096-column chunks per row (ragged last chunk included), the rotated and plain-basis
entries, nearest and stochastic assignment (uniform draws passed in), NaN scale bytes,
and a full-size layer on sampled rows."""

import numpy as np
import pytest
import torch

import oracle as O
from bit_codebook_quantized_amd import synth
from bit_codebook_quantized_amd import w4a8 as B

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPES = [(1, 256), (37, 768), (64, 4096), (9, 8192), (5, 13056)]


def say(*a):
    print("[case]", *a, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def trained_pair(n, k, seed):
    """A weight quantised by the oracle, and the weight after a small training step."""
    w = synth.gaussian_weight(n, k, seed=seed)
    packed, srel, sch, cb = O.quantize_w4(w)
    step = synth.rng(seed + 1).normal(0, 0.004, (n, k)).astype(np.float32)
    return w, (w + step).astype(np.float32), packed, srel, sch, cb


def layer_of(packed, srel, sch, cb):
    return B.W4A8Layer.from_host(packed, srel, cb, sch, None, device=DEV)


@pytest.mark.parametrize("n,k", SHAPES)
def test_requantize_nearest_and_stochastic(n, k):
    w, w2, packed, srel, sch, cb = trained_pair(n, k, synth.seed_for(13, n, k % 1000))
    layer = layer_of(packed, srel, sch, cb)
    say("requantize nearest", n, k)
    got = B.requantize_codes(dev(w2), layer).cpu().numpy()
    assert np.array_equal(got, O.requantize_codes(w2, srel, sch, cb))
    say("requantize on the layer's own weight gives its codes", n, k)
    assert np.array_equal(B.requantize_codes(dev(w), layer).cpu().numpy(), packed)
    u = synth.rng(synth.seed_for(13, n, 7)).random((n, k), dtype=np.float32)
    say("requantize stochastic", n, k)
    got = B.requantize_codes(dev(w2), layer, u=dev(u)).cpu().numpy()
    assert np.array_equal(got, O.requantize_codes(w2, srel, sch, cb, u=u))


def test_requantize_rotated_input_and_extreme_draws():
    n, k = 24, 2048
    w, w2, packed, srel, sch, cb = trained_pair(n, k, synth.seed_for(13, 1, 1))
    layer = layer_of(packed, srel, sch, cb)
    w_rot = O.rotate_to_f32(w2)
    for u in (None, np.zeros((n, k), np.float32), np.full((n, k), np.nextafter(np.float32(1), np.float32(0)))):
        say("requantize rotated, draws", None if u is None else float(u.flat[0]))
        got = B.requantize_codes(dev(w_rot), layer, rotated=True, u=None if u is None else dev(u)).cpu().numpy()
        assert np.array_equal(got, O.requantize_codes(w_rot, srel, sch, cb, rotated=True, u=u))


def test_requantize_nan_and_extreme_scale_bytes():
    n, k = 8, 1024
    g = synth.rng(synth.seed_for(13, 2, 2))
    w = g.normal(0, 1, (n, k)).astype(np.float32)
    srel = g.integers(0, 256, (n, k // 16)).astype(np.uint8)     # includes 0x7F / 0xFF (NaN) and 0
    srel[0, :4] = [0x7F, 0xFF, 0x00, 0x80]
    sch = np.abs(g.normal(0, 0.02, n)).astype(np.float32) + np.float32(1e-3)
    cb = O.FIXED_CODEBOOK
    packed = np.zeros((n, k // 2), np.uint8)
    layer = layer_of(packed, srel, sch, cb)
    u = g.random((n, k), dtype=np.float32)
    for uu in (None, u):
        say("requantize with NaN scale bytes, stochastic =", uu is not None)
        got = B.requantize_codes(dev(w), layer, u=None if uu is None else dev(uu)).cpu().numpy()
        assert np.array_equal(got, O.requantize_codes(w, srel, sch, cb, u=uu))


@pytest.mark.parametrize("n,k", SHAPES)
def test_fake_quant(n, k):
    w, w2, packed, srel, sch, cb = trained_pair(n, k, synth.seed_for(14, n, k % 1000))
    w_rot = O.rotate_to_f32(w2 * np.float32(1.1))
    say("fake quant", n, k)
    got = B.fake_quant(dev(w_rot), layer_of(packed, srel, sch, cb)).cpu().numpy()
    ref = O.fake_quant_rotated(w_rot, srel, sch, cb)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n,k", SHAPES)
def test_dequantize(n, k):
    packed, srel, sch = synth.random_layer_bytes(n, k, seed=synth.seed_for(15, n, k % 1000), srel_lo=0x00,
                                                 srel_hi=0xFF)
    cb = O.FIXED_CODEBOOK
    layer = layer_of(packed, srel, sch, cb)
    for back in (True, False):
        say("dequantize", n, k, "rotate back" if back else "rotated basis")
        got = B.dequantize(layer, rotate_back=back).cpu().numpy()
        ref = O.dequantize_f32(packed, srel, sch, cb, rotate_back=back)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_full_size_layer_sampled_rows():
    # 4096 x 4096: quantised on the GPU, one training step, requantised (nearest and
    # stochastic), fake-quantised and dequantised on the GPU; 128 seeded rows checked
    n = k = 4096
    w = synth.gaussian_weight_device(n, k, seed=synth.seed_for(16, 0, synth.ROLE_WEIGHT), device=DEV)
    layer = B.quantize_w4(w)
    w2 = w + torch.randn(n, k, device=DEV, generator=torch.Generator(DEV).manual_seed(5)) * 0.004
    u = torch.rand(n, k, device=DEV, generator=torch.Generator(DEV).manual_seed(6))
    say("full size requantize / fake quant / dequantize")
    q_near = B.requantize_codes(w2, layer).cpu().numpy()
    q_sto = B.requantize_codes(w2, layer, u=u).cpu().numpy()
    deq = B.dequantize(layer).cpu().numpy()
    w_rot_np = O.rotate_to_f32(w2.cpu().numpy())
    fq = B.fake_quant(torch.from_numpy(w_rot_np).to(DEV), layer).cpu().numpy()
    rows = np.sort(synth.rng(synth.seed_for(16, 0, 9)).choice(n, 128, replace=False))
    packed, srel, sch = layer.qpacked.cpu().numpy(), layer.srel.cpu().numpy(), layer.s_channel.cpu().numpy()
    cb = O.FIXED_CODEBOOK
    w2n, un = w2.cpu().numpy()[rows], u.cpu().numpy()[rows]
    assert np.array_equal(q_near[rows], O.requantize_codes(w2n, srel[rows], sch[rows], cb))
    assert np.array_equal(q_sto[rows], O.requantize_codes(w2n, srel[rows], sch[rows], cb, u=un))
    ref = O.dequantize_f32(packed[rows], srel[rows], sch[rows], cb)
    assert np.array_equal(deq[rows].view(np.uint32), ref.view(np.uint32))
    ref = O.fake_quant_rotated(w_rot_np[rows], srel[rows], sch[rows], cb)
    assert np.array_equal(fq[rows].view(np.uint32), ref.view(np.uint32))


def test_nearest_level_ties_exact_levels_and_duplicates():
    # Targets placed exactly on grid levels, exactly half-way between neighbouring levels
    # (the rule keeps the lower candidate on a tie), a quarter off a level, beyond both
    # ends, and NaN; scale bytes of every kind: positive (non-decreasing levels), negative
    # (non-increasing), zero and saturating (runs of equal levels), NaN.  The channel
    # scale is a power of two, so w_rot / s_channel reproduces each target exactly.
    n, k = 16, 1024
    g = synth.rng(synth.seed_for(13, 3, 3))
    cb = O.FIXED_CODEBOOK
    srel = g.integers(0, 256, (n, k // 16)).astype(np.uint8)
    srel[0, :6] = [0x7F, 0xFF, 0x00, 0x80, 0x7E, 0xFE]      # NaN, NaN, +0, -0, largest +-
    srel[1, :] = g.integers(0x40, 0x58, k // 16)              # moderate positive scales
    levels = O.grid_levels(cb, srel)                          # [n, G, 16]
    sch = np.full(n, 2.0 ** -6, np.float32)
    t = np.empty((n, k // 16, 16), np.float32)
    for r in range(n):
        for gi in range(k // 16):
            lv = levels[r, gi]
            picks = list(lv[g.integers(0, 16, 6)])                      # on a level
            a, b = np.sort(lv[g.integers(0, 16, 2)])
            picks += [(a + b) / 2, (a + b) / 2 + 0.25, a - 0.25, b + 0.25]   # ties and near-ties
            picks += [lv.min() - 3, lv.max() + 3, 127.5, -127.5, 0.0, np.nan]
            t[r, gi] = np.asarray(picks, np.float32)
    w_rot = (t.reshape(n, k) * sch[:, None]).astype(np.float32)
    assert np.array_equal((w_rot.reshape(n, k // 16, 16) / sch[:, None, None]).astype(np.float32), t,
                          equal_nan=True)
    layer = layer_of(np.zeros((n, k // 2), np.uint8), srel, sch, cb)
    say("nearest level: ties, exact levels, duplicate levels")
    got = B.requantize_codes(dev(w_rot), layer, rotated=True).cpu().numpy()
    assert np.array_equal(got, O.requantize_codes(w_rot, srel, sch, cb, rotated=True))
    got = B.fake_quant(dev(w_rot), layer).cpu().numpy()
    ref = O.fake_quant_rotated(w_rot, srel, sch, cb)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
