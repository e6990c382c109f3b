"""GPU parity of the fused SwiGLU epilogue (out type W4A8_OUT_SWIGLU_BF16) on
gate/up-interleaved layers, through the GEMM, the GEMV, the grouped GEMV and the
one-launch GEMV.

Reference.  The fp32 epilogue values y are the oracle's (exact contraction of the
prepared activations with the oracle's decoded grid, then the fp32 epilogue; both
bit-exact with the kernels by the other tests), so only the SwiGLU itself is
approximate: the oracle evaluates silu(g) * u in fp64 from the same y, the kernels in
fp32 (exp to about an ulp, then a division and a product) and round to bf16:
    |gpu - ref| <= 2^-8 |ref| + 2^-20 |ref| + 2^-126
(half a bf16 ulp relative, a few fp32 ulps, and the smallest normal for results that
underflow).  The GEMV and GEMM paths must also agree with each other bit for bit."""

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


_QUANTISED = {}


def gate_up_layer(f, k, seed, with_bias):
    """A gate/up projection (2F x K) quantised by the oracle after interleaving its rows."""
    if (f, k, seed) not in _QUANTISED:
        wg = synth.gaussian_weight(f, k, seed=seed)
        wu = synth.gaussian_weight(f, k, seed=seed + 1)
        _QUANTISED[(f, k, seed)] = O.quantize_w4(O.interleave_rows(np.concatenate([wg, wu])))
    packed, srel, sch, cb = _QUANTISED[(f, k, seed)]
    bias = synth.rng(seed + 2).normal(0, 0.5, 2 * f).astype(np.float32) if with_bias else None
    layer = B.W4A8Layer.from_host(packed, srel, cb, sch, bias, device=DEV)
    return layer, (packed, srel, sch, cb, bias)


def reference(xq, xs, host, rows=None):
    packed, srel, sch, cb, bias = host
    xq = xq.cpu().numpy() if rows is None else xq.cpu().numpy()[rows]
    xs = xs.cpu().numpy() if rows is None else xs.cpu().numpy()[rows]
    y = O.epilogue(O.gemm_exact(xq, O.decode_w4(packed, srel, cb)), xs, sch, bias, out="f32")
    return O.swiglu_interleaved(y)


def check(got_bf16, ref, label):
    got = O.bf16_bits_to_f32(got_bf16.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    tol = (2.0 ** -8 + 2.0 ** -20) * np.abs(ref) + 2.0 ** -126
    bad = np.argwhere(np.abs(got - ref) > tol)
    assert bad.size == 0, f"{label}: {len(bad)} outside the bound, first {bad[:3].tolist()}"


@pytest.mark.parametrize("f,k", [(37, 256), (1536, 1024), (500, 3072)])
@pytest.mark.parametrize("m", [1, 2, 5, 8, 40])
def test_swiglu_epilogue_gemv_and_gemm(f, k, m):
    layer, host = gate_up_layer(f, k, synth.seed_for(19, f, k % 1000), with_bias=(m % 2 == 0))
    x = torch.from_numpy(synth.activations(m, k, seed=synth.seed_for(19, m, 3))).to(torch.bfloat16).to(DEV)
    xq, xs = B.rotate_quant_act(x)
    say("swiglu", m, f, k)
    y_gemm = B.w4a8_gemm(xq, xs, layer, B.SWIGLU)
    assert tuple(y_gemm.shape) == (m, f) and y_gemm.dtype == torch.bfloat16
    check(y_gemm, reference(xq, xs, host), f"gemm {m}x{2 * f}x{k}")
    if m <= 8:
        y_gemv = B.w4a8_gemv(xq, xs, layer, B.SWIGLU)
        assert torch.equal(y_gemv.view(torch.int16), y_gemm.view(torch.int16)), "gemv != gemm"
        y_lin = B.linear(x, layer, B.SWIGLU)          # one-launch GEMV for one row
        assert torch.equal(y_lin.view(torch.int16), y_gemm.view(torch.int16)), "linear != gemm"
        if k <= B.gemv_act_max_k(m):
            y_act = B.w4a8_gemv_act(x, layer, B.SWIGLU)
            assert torch.equal(y_act.view(torch.int16), y_gemm.view(torch.int16)), "gemv_act != gemm"


@pytest.mark.parametrize("f", [128, 132])
def test_swiglu_whole_tiles(f):
    # 256 rows: whole GEMM tiles; 2f = 256 output rows per pair-row give 16-byte aligned
    # output rows (staged through LDS), 2f = 264 do not (direct stores)
    layer, host = gate_up_layer(f, 256, synth.seed_for(19, 300, f), with_bias=True)
    x = torch.from_numpy(synth.activations(256, 256, seed=synth.seed_for(19, 300, f + 1))).to(torch.bfloat16).to(DEV)
    xq, xs = B.rotate_quant_act(x)
    say("swiglu whole tiles", f)
    check(B.w4a8_gemm(xq, xs, layer, B.SWIGLU), reference(xq, xs, host), f"gemm 256x{2 * f}x256")


def test_swiglu_grouped_gemv_matches_single():
    items, singles = [], []
    for i, (f, k) in enumerate([(37, 256), (1536, 1024), (64, 512)] * 3):
        layer, _ = gate_up_layer(f, k, synth.seed_for(19, 100 + i, 0), with_bias=i % 2 == 0)
        x = torch.from_numpy(synth.activations(3, k, seed=synth.seed_for(19, 100 + i, 1))).to(torch.bfloat16).to(DEV)
        xq, xs = B.rotate_quant_act(x)
        items.append((xq, xs, layer, None))
        singles.append(B.w4a8_gemv(xq, xs, layer, B.SWIGLU))
    say("swiglu grouped")
    outs = B.w4a8_gemv_grouped(items, B.SWIGLU)
    for i, (a, b) in enumerate(zip(outs, singles)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"layer {i}"


def test_swiglu_mlp_up_projection_full_size_sampled_rows():
    # the MLP up projection of the prefill pair (N = 12288 = 2 x 6144, K = 3072) at
    # M = 4096 Student-t activations, 64 rows checked
    f, k, m = 6144, 3072, 4096
    wg = synth.gaussian_weight_device(f, k, seed=synth.seed_for(19, 7, 7), device=DEV)
    wu = synth.gaussian_weight_device(f, k, seed=synth.seed_for(19, 7, 17), device=DEV)
    layer = B.quantize_w4(torch.stack([wg, wu], dim=1).reshape(2 * f, k).contiguous())   # rows interleaved
    del wg, wu
    host = (layer.qpacked.cpu().numpy(), layer.srel.cpu().numpy(), layer.s_channel.cpu().numpy(),
            O.FIXED_CODEBOOK, None)
    x = torch.from_numpy(synth.activations(m, k, seed=synth.seed_for(19, 7, 8), kind="student_t")).to(
        torch.bfloat16).to(DEV)
    xq, xs = B.rotate_quant_act(x)
    say("swiglu 4096 x 12288 x 3072")
    y = B.w4a8_gemm(xq, xs, layer, B.SWIGLU)
    rows = np.sort(synth.rng(synth.seed_for(19, 7, 9)).choice(m, 64, replace=False))
    check(y[torch.from_numpy(rows).to(DEV)], reference(xq, xs, host, rows), "C3 up sampled")


def test_swiglu_prepared_calls():
    layer, _ = gate_up_layer(64, 512, synth.seed_for(19, 200, 0), with_bias=True)
    x = torch.from_numpy(synth.activations(1, 512, seed=synth.seed_for(19, 200, 1))).to(torch.bfloat16).to(DEV)
    xq, xs = B.rotate_quant_act(x)
    ref = B.w4a8_gemv(xq, xs, layer, B.SWIGLU)
    out_a = torch.empty(1, 64, dtype=torch.bfloat16, device=DEV)
    run_a = B.prepared_gemv_act(x, layer, out_a, out_dtype=B.SWIGLU)
    out_l = torch.empty(1, 64, dtype=torch.bfloat16, device=DEV)
    run_l = B.prepared_linear("w4a8_gemv", xq, xs, layer, out_l, B.SWIGLU)
    out_a.zero_()
    out_l.zero_()
    run_a()
    run_l()
    assert torch.equal(out_a.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out_l.view(torch.int16), ref.view(torch.int16))


def test_swiglu_rejects_odd_rows():
    packed, srel, sch = synth.random_layer_bytes(63, 256, seed=3)
    layer = B.W4A8Layer.from_host(packed, srel, O.FIXED_CODEBOOK, sch, None, device=DEV)
    xq, xs = B.rotate_quant_act(torch.zeros(2, 256, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        B.w4a8_gemv(xq, xs, layer, B.SWIGLU)
