"""The prefill layer step (rotate_quant_act + w4a8_gemm) captured once as a HIP graph and
replayed: every replay must give the bytes the eager launches give, also when the inputs
change between replays and with other eager work and synchronisations in between.  The
step's launches hold no memory-set nodes; the eager results are themselves checked against
the oracle elsewhere, and here the first replay is checked against the oracle on sampled
rows as well."""

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


@pytest.mark.parametrize("M,N,K", [(300, 384, 1024), (2048, 4096, 4096)])
def test_step_graph_replays_match_eager(M, N, K):
    say("graph step", M, N, K)
    w = torch.from_numpy(synth.gaussian_weight(N, K, seed=synth.seed_for(7, 0, synth.ROLE_WEIGHT))).to(DEV)
    layer = B.quantize_w4(w)
    xs_np = [synth.activations(M, K, seed=synth.seed_for(7, i, synth.ROLE_ACT), kind="outliers",
                               outlier_seed=synth.seed_for(7, i, synth.ROLE_OUTLIER)) for i in range(3)]
    x = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    xq = torch.empty(M, K, dtype=torch.int8, device=DEV)
    xs = torch.empty(M, dtype=torch.float32, device=DEV)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    rq = B.prepared_rotate_quant(x, xq, xs)
    gm = B.prepared_linear("w4a8_gemm", xq, xs, layer, out)

    def step():
        rq()
        gm()

    graph = torch.cuda.CUDAGraph()
    x.copy_(torch.from_numpy(xs_np[0]).to(torch.bfloat16))
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(6):
        xi = torch.from_numpy(xs_np[rep % 3]).to(torch.bfloat16).to(DEV)
        # eager reference on separate buffers
        rq_e, s_e = B.rotate_quant_act(xi)
        y_e = B.w4a8_gemm(rq_e, s_e, layer)
        torch.cuda.synchronize()
        x.copy_(xi)
        out.fill_(0)
        graph.replay()
        if rep % 2:
            torch.cuda.synchronize()
            _ = (xi.float() * 2).sum()    # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(xq, rq_e), rep
        assert torch.equal(xs.view(torch.int32), s_e.view(torch.int32)), rep
        assert torch.equal(out.view(torch.int16), y_e.view(torch.int16)), rep
        if rep == 0:
            rows = np.unique(np.linspace(0, M - 1, 5).astype(np.int64))
            packed, srel, sch = (layer.qpacked.cpu().numpy(), layer.srel.cpu().numpy(),
                                 layer.s_channel.cpu().numpy())
            ref = O.linear(xi.float().cpu().numpy()[rows], packed, srel, sch, layer.codebook.cpu().numpy(),
                           out="bf16")[0]
            got = out.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
            assert np.array_equal(got, ref), "graph replay differs from the oracle"
