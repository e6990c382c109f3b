"""GPU parity of the grouped decode GEMV (w4a8_gemv_grouped, through the C ABI
binding): every layer's output must be bit-identical to w4a8_gemv on that layer,
which the single-layer tests pin to the oracle; one layer of each decode-set shape
is also checked against the oracle directly.  Covers mixed shapes, more layers
than one launch holds (64), M = 1..8, bias / no bias, and the three output types."""

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


def acts(m, k, seed):
    x = torch.from_numpy(synth.activations(m, k, seed=seed)).to(torch.bfloat16).to(DEV)
    return B.rotate_quant_act(x)


def as_bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32, torch.int32])
def test_grouped_equals_single_gemv(m, out_dtype):
    # 3 groups per lane and batch for K = 3072, 768 and (M <= 2) 9216, 4 for the others
    shapes = [(37, 256), (1000, 3072), (130, 12288), (4096, 4096), (257, 768), (300, 9216)]
    items = []
    for i in range(70):                                  # 70 layers: two launches
        n, k = shapes[i % len(shapes)]
        layer = layer_from_bytes(n, k, seed=synth.seed_for(11, i, synth.ROLE_BYTES), with_bias=i % 3 == 0)
        xq, xs = acts(m, k, synth.seed_for(11, i, synth.ROLE_ACT))
        items.append((xq, xs, layer, None))
    say("grouped gemv", m, out_dtype, len(items), "layers")
    outs = B.w4a8_gemv_grouped(items, out_dtype)
    for i, (xq, xs, layer, _) in enumerate(items):
        ref = B.w4a8_gemv(xq, xs, layer, out_dtype)
        assert np.array_equal(as_bits(outs[i]), as_bits(ref)), f"layer {i} ({layer.out_features}x{layer.in_features})"


def test_grouped_decode_set_against_oracle():
    # the 64-layer decode set (16 of each shape), quantised on the GPU; one layer of each
    # shape against the oracle, all 64 against the single-layer GEMV
    shapes = [(3072, 3072), (9216, 3072), (12288, 3072), (3072, 12288)]
    items = []
    for i in range(64):
        n, k = shapes[i // 16]
        w = synth.gaussian_weight_device(n, k, seed=synth.seed_for(4, i, synth.ROLE_WEIGHT), device=DEV)
        layer = B.quantize_w4(w)
        del w
        x = synth.activations(1, k, seed=synth.seed_for(4, i, synth.ROLE_ACT))
        xq, xs = B.rotate_quant_act(torch.from_numpy(x).to(torch.bfloat16).to(DEV))
        items.append((xq, xs, layer, None, x))
    say("grouped decode set, 64 layers")
    outs = B.w4a8_gemv_grouped([it[:4] for it in items])
    for i, (xq, xs, layer, _, x) in enumerate(items):
        ref = B.w4a8_gemv(xq, xs, layer)
        assert np.array_equal(as_bits(outs[i]), as_bits(ref)), f"layer {i}"
        if i % 16 == 0:
            say("oracle check of layer", i)
            packed, srel, sch = (layer.qpacked.cpu().numpy(), layer.srel.cpu().numpy(),
                                 layer.s_channel.cpu().numpy())
            y, *_ = O.linear(x, packed, srel, sch, O.FIXED_CODEBOOK, out="bf16")
            assert np.array_equal(outs[i].view(torch.int16).cpu().numpy().view(np.uint16), y), f"oracle {i}"


def test_grouped_prepared_call_and_empty():
    layer = layer_from_bytes(300, 512, seed=5, with_bias=False)
    xq, xs = acts(2, 512, 6)
    out = torch.empty(2, 300, dtype=torch.bfloat16, device=DEV)
    run = B.prepared_gemv_grouped([(xq, xs, layer, out)])
    out.zero_()
    run()
    ref = B.w4a8_gemv(xq, xs, layer)
    assert np.array_equal(as_bits(out), as_bits(ref))
    assert B.w4a8_gemv_grouped([]) == []


def test_grouped_prepared_call_allocates_missing_outputs_once():
    # outputs given as None are allocated by prepared_gemv_grouped and kept with the
    # callable, which writes them on every call and returns them
    items = []
    for i, (n, k) in enumerate([(300, 512), (1000, 3072), (37, 256)]):
        layer = layer_from_bytes(n, k, seed=40 + i, with_bias=i == 1)
        xq, xs = acts(3, k, 50 + i)
        items.append((xq, xs, layer, None))
    say("prepared grouped gemv with outputs allocated by the binding")
    run = B.prepared_gemv_grouped(items)
    outs = run()
    assert outs is run.outs and len(outs) == 3
    ptrs = [o.data_ptr() for o in outs]
    for o in outs:
        o.zero_()
    torch.cuda.synchronize()
    # other allocations in between must not take over the bound outputs
    scratch = [torch.full((3, 4096), 7, dtype=torch.bfloat16, device=DEV) for _ in range(8)]
    assert run() is outs and [o.data_ptr() for o in outs] == ptrs
    for (xq, xs, layer, _), o in zip(items, outs):
        assert np.array_equal(as_bits(o), as_bits(B.w4a8_gemv(xq, xs, layer)))
    del scratch
