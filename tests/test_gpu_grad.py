"""GPU parity of the straight-through backward (w4a8_grad_input, through the C ABI
binding) against the oracle's bf16 weight and exact product.

Bar.  The weight w = bf16(w8 * bf16(s_channel)) is formed exactly as the oracle forms
it, so the only differences are the fp32 accumulation and the final bf16 rounding:
    |gpu - ref| <= 2^-8 |ref| + 1.01 * N * 2^-24 * sum_n |grad[m, n] * w[n, k]|
(half an ulp of bf16 relative, plus the worst-case error of N fp32 additions).  One-hot
gradient rows must reproduce rows of w bit for bit (a single product is exact).  Shapes
cover ragged M, N not a multiple of the 64-deep step, one and many output tiles, and
the full training shape on sampled rows."""

import numpy as np
import pytest
import torch

import oracle as O
from bit_codebook_quantized_amd import synth
from bit_codebook_quantized_amd import w4a8 as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def bf16_dev(a):
    return torch.from_numpy(O.f32_to_bf16_bits(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_f32(t):
    return O.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))


def check_against_oracle(grad_f32, w_bf, got, label):
    ref = O.grad_input_exact(grad_f32, w_bf)
    s = np.abs(grad_f32.astype(np.float64)) @ np.abs(w_bf.astype(np.float64))
    n = grad_f32.shape[1]
    tol = 2.0 ** -8 * np.abs(ref) + 1.01 * n * 2.0 ** -24 * s
    err = np.abs(got.astype(np.float64) - ref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{label}: {len(bad)} outside the bound, first {bad[:3].tolist()}"
    rel = err / np.maximum(np.abs(ref), 1e-30)
    assert np.median(rel) <= 2.0 ** -9, f"{label}: median relative error {np.median(rel)}"


def layer_np(n, k, seed):
    packed, srel, sch = synth.random_layer_bytes(n, k, seed=seed, srel_lo=0x40, srel_hi=0x78)
    return packed, srel, sch, O.FIXED_CODEBOOK


@pytest.mark.parametrize("m,n,k", [(1, 8, 256), (37, 64, 256), (130, 1000, 768), (3, 72, 512), (200, 4096, 4096)])
def test_grad_input_against_oracle(m, n, k):
    packed, srel, sch, cb = layer_np(n, k, synth.seed_for(17, n, k % 1000))
    layer = B.W4A8Layer.from_host(packed, srel, cb, sch, None, device=DEV)
    g = synth.rng(synth.seed_for(17, m, 1)).normal(0, 1, (m, n)).astype(np.float32)
    g = O.bf16_bits_to_f32(O.f32_to_bf16_bits(g))
    say("grad_input", m, n, k)
    got = to_f32(B.grad_input(bf16_dev(g), layer))
    w_bf = O.ste_weight_bf16(packed, srel, sch, cb)
    check_against_oracle(g, w_bf, got, f"{m}x{n}x{k}")


def test_grad_input_one_hot_rows_select_weight_rows_exactly():
    n, k = 200, 1024
    packed, srel, sch, cb = layer_np(n, k, synth.seed_for(17, 1, 2))
    layer = B.W4A8Layer.from_host(packed, srel, cb, sch, None, device=DEV)
    picks = [0, 1, 63, 64, 127, 128, 199]
    g = np.zeros((len(picks), n), np.float32)
    for i, p in enumerate(picks):
        g[i, p] = 1.0
    say("grad_input one-hot rows")
    got = B.grad_input(bf16_dev(g), layer).view(torch.int16).cpu().numpy().view(np.uint16)
    w_bits = O.f32_to_bf16_bits(O.ste_weight_bf16(packed, srel, sch, cb))
    assert np.array_equal(got, w_bits[picks])


def test_grad_input_training_shape_sampled_rows():
    # M = 2048 tokens, N = K = 4096, a weight quantised on the GPU from Gaussian weights
    m, n, k = 2048, 4096, 4096
    w = synth.gaussian_weight_device(n, k, seed=synth.seed_for(18, 0, synth.ROLE_WEIGHT), device=DEV)
    layer = B.quantize_w4(w)
    del w
    g = torch.randn(m, n, device=DEV, generator=torch.Generator(DEV).manual_seed(8)).to(torch.bfloat16)
    say("grad_input 2048x4096x4096")
    got = to_f32(B.grad_input(g, layer))
    rows = np.sort(synth.rng(synth.seed_for(18, 0, 3)).choice(m, 48, replace=False))
    packed, srel, sch = layer.qpacked.cpu().numpy(), layer.srel.cpu().numpy(), layer.s_channel.cpu().numpy()
    w_bf = O.ste_weight_bf16(packed, srel, sch, O.FIXED_CODEBOOK)
    check_against_oracle(to_f32(g)[rows], w_bf, got[rows], "2048x4096x4096 sampled")


def test_grad_input_empty_and_rejected():
    packed, srel, sch, cb = layer_np(64, 256, 5)
    layer = B.W4A8Layer.from_host(packed, srel, cb, sch, None, device=DEV)
    assert B.grad_input(torch.empty(0, 64, dtype=torch.bfloat16, device=DEV), layer).shape == (0, 256)
    packed, srel, sch, cb = layer_np(60, 256, 6)
    layer = B.W4A8Layer.from_host(packed, srel, cb, sch, None, device=DEV)
    with pytest.raises(B.W4A8ArgumentError):
        B.grad_input(torch.zeros(2, 60, dtype=torch.bfloat16, device=DEV), layer)
