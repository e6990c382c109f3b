"""GPU parity on random shapes (fixed seeds), bit for bit against the CPU oracle, for the
kernels whose LDS exchanges stay inside a wave: rotate_quant_act (one or many rows per
block, register-kept and recomputed long rows), the one-launch GEMV, the weight quantiser,
requantisation (nearest and stochastic), fake quantisation and dequantisation."""

import numpy as np
import pytest
import torch

import oracle as O
from bit_codebook_quantized_amd import synth
from bit_codebook_quantized_amd import w4a8 as B
from test_gpu_gemv_act import bits, layer_from_bytes, two_call
from test_gpu_regrid import dev, layer_of, say, trained_pair

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shape(tag, case, lo, hi):
    g = np.random.default_rng(synth.seed_for(31, tag, case))
    return [int(g.integers(a, b)) for a, b in zip(lo, hi)]


@pytest.mark.parametrize("case", range(8))
def test_rotate_quant_act_random_shapes(case):
    m, kb = _shape(0, case, (1, 1), (200, 161))    # K up to 40960 (recomputed long rows)
    k = 256 * kb
    x = synth.activations(m, k, seed=synth.seed_for(31, 0, 100 + case),
                          kind=("normal", "outliers", "student_t")[case % 3],
                          outlier_seed=synth.seed_for(31, 0, 200 + case))
    say("rotate_quant_act", m, k)
    xq, xs = B.rotate_quant_act(torch.from_numpy(x).to(torch.bfloat16).to(DEV))
    rq, rs = O.rotate_quant_act(x)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("case", range(6))
def test_gemv_act_random_shapes(case):
    m, n, kb = _shape(1, case, (1, 1, 1), (9, 600, 65))
    k = 256 * min(kb, B.gemv_act_max_k(m) // 256)
    layer = layer_from_bytes(n, k, synth.seed_for(31, 1, case), with_bias=case % 2 == 0)
    x = torch.from_numpy(synth.activations(m, k, seed=synth.seed_for(31, 1, 100 + case))).to(torch.bfloat16).to(DEV)
    say("gemv_act", m, n, k)
    ref, _, _ = two_call(x, layer, torch.bfloat16)
    assert np.array_equal(bits(B.w4a8_gemv_act(x, layer, torch.bfloat16)), bits(ref))


@pytest.mark.parametrize("case", range(4))
def test_weight_kernels_random_shapes(case):
    n, kb = _shape(2, case, (1, 1), (40, 56))
    k = 256 * kb
    w, w2, packed, srel, sch, cb = trained_pair(n, k, synth.seed_for(31, 2, case))
    say("quantize, requantize, fake quant, dequantize", n, k)
    lay = B.quantize_w4(dev(w))
    assert np.array_equal(lay.qpacked.cpu().numpy(), packed) and np.array_equal(lay.srel.cpu().numpy(), srel)
    assert np.array_equal(lay.s_channel.cpu().numpy().view(np.uint32), sch.view(np.uint32))
    layer = layer_of(packed, srel, sch, cb)
    assert np.array_equal(B.requantize_codes(dev(w2), layer).cpu().numpy(), O.requantize_codes(w2, srel, sch, cb))
    u = synth.rng(synth.seed_for(31, 2, 100 + case)).random((n, k), dtype=np.float32)
    assert np.array_equal(B.requantize_codes(dev(w2), layer, u=dev(u)).cpu().numpy(),
                          O.requantize_codes(w2, srel, sch, cb, u=u))
    w_rot = O.rotate_to_f32(w2)
    assert np.array_equal(B.fake_quant(dev(w_rot), layer).cpu().numpy().view(np.uint32),
                          O.fake_quant_rotated(w_rot, srel, sch, cb).view(np.uint32))
    assert np.array_equal(B.dequantize(layer).cpu().numpy().view(np.uint32),
                          O.dequantize_f32(packed, srel, sch, cb).view(np.uint32))
