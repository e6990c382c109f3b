"""GPU parity of the LoRA merge (lora_merge_w4, and the binding's merge_lora that feeds
it to quantize_w4) against the oracle's lora_merge_weight / quantize_w4.

Bar: the merged fp32 weight is bit-identical (the delta is formed in fp64 in a fixed
order on both sides and rounded once), and the requantised layer is bit-exact.  Covers
ranks 0, 1, 16 and 64, ragged chunks, and a full-size layer on sampled rows."""

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def adapter(n, k, r, seed):
    g = synth.rng(seed)
    return g.normal(0, 0.02, (r, k)).astype(np.float32), g.normal(0, 0.02, (n, r)).astype(np.float32)


@pytest.mark.parametrize("n,k,r", [(8, 256, 0), (37, 768, 1), (64, 4096, 16), (5, 13056, 64)])
def test_lora_merged_weight_and_requantised_layer(n, k, r):
    w = synth.gaussian_weight(n, k, seed=synth.seed_for(20, n, k % 1000))
    packed, srel, sch, cb = O.quantize_w4(w)
    layer = B.W4A8Layer.from_host(packed, srel, cb, sch, None, device=DEV)
    a, b = adapter(n, k, r, synth.seed_for(20, r, 1))
    scale = 0.75
    say("lora merge", n, k, r)
    got = B.lora_merged_weight(layer, dev(a), dev(b), scale).cpu().numpy()
    ref = O.lora_merge_weight(packed, srel, sch, cb, a, b, scale)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    merged = B.merge_lora(layer, dev(a), dev(b), scale)
    rp, rs, rc, _ = O.quantize_w4(ref)
    assert np.array_equal(merged.qpacked.cpu().numpy(), rp)
    assert np.array_equal(merged.srel.cpu().numpy(), rs)
    assert np.array_equal(merged.s_channel.cpu().numpy().view(np.uint32), rc.view(np.uint32))


def test_lora_merge_full_size_sampled_rows():
    n = k = 4096
    r = 64
    w = synth.gaussian_weight_device(n, k, seed=synth.seed_for(21, 0, synth.ROLE_WEIGHT), device=DEV)
    layer = B.quantize_w4(w)
    del w
    a, b = adapter(n, k, r, synth.seed_for(21, 0, 2))
    say("lora merge 4096 x 4096, rank 64")
    got = B.lora_merged_weight(layer, dev(a), dev(b), 0.5).cpu().numpy()
    rows = np.sort(synth.rng(synth.seed_for(21, 0, 3)).choice(n, 64, replace=False))
    packed, srel, sch = layer.qpacked.cpu().numpy(), layer.srel.cpu().numpy(), layer.s_channel.cpu().numpy()
    ref = O.lora_merge_weight(packed[rows], srel[rows], sch[rows], O.FIXED_CODEBOOK, a, b[rows], 0.5)
    assert np.array_equal(got[rows].view(np.uint32), ref.view(np.uint32))
