"""GPU parity of the one-launch decode GEMV on bf16 activations (w4a8_gemv_act,
through the C ABI binding).

Bar: the output is bit-identical to rotate_quant_act followed by w4a8_gemv (both
pinned to the oracle by the other GPU tests), and its optional prepared-activation
outputs are bit-identical to rotate_quant_act's.  The full-size decode shapes are
also compared with the oracle's whole layer directly.  Covers M = 1..8, ragged N,
K from one rotation block to the largest on-chip size per M, three output types,
bias, zero and outlier rows, and the unsupported sizes."""

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


def layer_from_bytes(n, k, seed, with_bias):
    packed, srel, sch = synth.random_layer_bytes(n, k, seed=seed, srel_lo=0x40, srel_hi=0x78)
    bias = synth.rng(seed + 1).normal(0, 1, n).astype(np.float32) if with_bias else None
    return B.W4A8Layer.from_host(packed, srel, O.FIXED_CODEBOOK, sch, bias, device=DEV)


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def two_call(x, layer, out_dtype):
    xq, xs = B.rotate_quant_act(x)
    return B.w4a8_gemv(xq, xs, layer, out_dtype), xq, xs


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
# K = 768, 3072, 9216: 3 groups per lane and batch (768: lanes past the row); the others 4
@pytest.mark.parametrize("n,k", [(37, 256), (257, 768), (1000, 3072), (4096, 4096), (130, 8192), (200, 9216),
                                 (300, 16384), (64, 32768)])
def test_gemv_act_equals_rotate_quant_then_gemv(m, n, k):
    if k > B.gemv_act_max_k(m):
        pytest.skip(f"K={k} is above the on-chip size for M={m}")
    seed = synth.seed_for(12, m * 100 + n % 97, k // 256)
    layer = layer_from_bytes(n, k, seed, with_bias=(n % 2 == 0))
    x = torch.from_numpy(synth.activations(m, k, seed=seed + 7, kind="outliers",
                                           outlier_seed=seed + 8)).to(torch.bfloat16).to(DEV)
    for out_dtype in (torch.bfloat16, torch.float32, torch.int32):
        say("gemv_act", m, n, k, out_dtype)
        xq_o = torch.empty(m, k, dtype=torch.int8, device=DEV)
        xs_o = torch.empty(m, dtype=torch.float32, device=DEV)
        got = B.w4a8_gemv_act(x, layer, out_dtype, xq_out=xq_o, xs_out=xs_o)
        ref, xq, xs = two_call(x, layer, out_dtype)
        assert np.array_equal(bits(got), bits(ref)), f"output {m}x{n}x{k} {out_dtype}"
        assert torch.equal(xq_o, xq) and torch.equal(xs_o.view(torch.int32), xs.view(torch.int32))
        got2 = B.w4a8_gemv_act(x, layer, out_dtype)          # without the prepared outputs
        assert np.array_equal(bits(got2), bits(ref))


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_gemv_act_full_size_against_oracle(m):
    # the N = K = 4096 decode layer quantised on the GPU from Gaussian weights, against
    # the oracle's whole layer (rotation, activation quantisation, decode, contraction,
    # epilogue) on the same bf16 inputs
    n = k = 4096
    w = synth.gaussian_weight_device(n, k, seed=synth.seed_for(12, 0, synth.ROLE_WEIGHT), device=DEV)
    layer = B.quantize_w4(w)
    del w
    x = synth.activations(m, k, seed=synth.seed_for(12, m, synth.ROLE_ACT))
    say("gemv_act vs oracle", m)
    y = B.w4a8_gemv_act(torch.from_numpy(x).to(torch.bfloat16).to(DEV), layer)
    packed, srel, sch = layer.qpacked.cpu().numpy(), layer.srel.cpu().numpy(), layer.s_channel.cpu().numpy()
    ref, _, _, _ = O.linear(x, packed, srel, sch, O.FIXED_CODEBOOK, out="bf16")
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_gemv_act_zero_and_constant_rows_and_qmax():
    n, k = 200, 1024
    layer = layer_from_bytes(n, k, seed=31, with_bias=True)
    x = np.zeros((4, k), np.float32)
    x[1] = 0.5                                   # constant: the regular Hadamard keeps it constant
    x[2, ::7] = -3.0
    x[3] = synth.activations(1, k, seed=32)[0]
    xt = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    for qmax in (127, 100, 1):
        say("gemv_act zero/constant rows, qmax", qmax)
        xq_o = torch.empty(4, k, dtype=torch.int8, device=DEV)
        xs_o = torch.empty(4, dtype=torch.float32, device=DEV)
        got = B.w4a8_gemv_act(xt, layer, torch.float32, qmax=qmax, xq_out=xq_o, xs_out=xs_o)
        xq, xs = B.rotate_quant_act(xt, qmax)
        ref = B.w4a8_gemv(xq, xs, layer, torch.float32)
        assert np.array_equal(bits(got), bits(ref))
        assert torch.equal(xq_o, xq) and torch.equal(xs_o, xs)
        assert xs_o[0].item() == 1.0 and not xq_o[0].any()


def test_gemv_act_empty_and_unsupported():
    layer = layer_from_bytes(64, 8192, seed=41, with_bias=False)
    x0 = torch.empty(0, 8192, dtype=torch.bfloat16, device=DEV)
    assert B.w4a8_gemv_act(x0, layer).shape == (0, 64)
    x5 = torch.zeros(5, 8192, dtype=torch.bfloat16, device=DEV)   # 5 rows of 8192 do not fit on chip
    with pytest.raises(B.W4A8ArgumentError):
        B.w4a8_gemv_act(x5, layer)
    x9 = torch.zeros(9, 8192, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.W4A8ArgumentError):
        B.w4a8_gemv_act(x9, layer)
    # the layer entry point takes the two-launch path for such shapes
    y = B.linear(x5, layer)
    assert y.shape == (5, 64) and not y.float().any()


def test_gemv_act_prepared_call():
    layer = layer_from_bytes(500, 2048, seed=51, with_bias=True)
    x = torch.from_numpy(synth.activations(3, 2048, seed=52)).to(torch.bfloat16).to(DEV)
    out = torch.empty(3, 500, dtype=torch.bfloat16, device=DEV)
    run = B.prepared_gemv_act(x, layer, out)
    out.zero_()
    run()
    ref, _, _ = two_call(x, layer, torch.bfloat16)
    assert np.array_equal(bits(out), bits(ref))
