"""The decode layer captured in a HIP graph and replayed, as the benchmark
times it: every replay must equal, bit for bit, the same calls made eagerly.

Three layers (each its own hidden state and workspace, shared weights) are
captured once per token count (1-8 tokens: the decode kernels; 40: the chunk
kernels), with and without the shared expert, and replayed three times with
eager work of the program and synchronisations between the replays; every
replay's outputs are compared with the eager outputs.  The kernels sum in fixed orders, so the comparison is
exact.  Weights: the Ling shape with 64 experts (the kernels are the Ling ones;
fewer experts keep the upload small).
"""
import numpy as np
import pytest
import torch

from _moe_helpers import DevWeights, dev, host
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu

H, I, E, K, L = 2560, 768, 64, 8, 3


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


@pytest.fixture(scope="module")
def weights():
    w = synth.expert_weights(400, H, I, E)
    sh = synth.shared_expert(401, H, I)
    return DevWeights(w), tuple(dev(a) for a in sh), w


def _layer(moe, shp, M, x, dw, dsh, out, ws):
    if dsh is None:
        moe.moe_decode_forward(shp, M, x, dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    else:
        moe.moe_decode_forward_shared(shp, M, x, dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, dsh, out, ws)


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("M", [1, 2, 4, 8, 40])
def test_graph_replays_equal_eager_calls(moe, weights, M, shared):
    dw, dsh_all, w = weights
    dsh = dsh_all if shared else None
    shp = moe.shape(H, I, E, K)
    xs = [dev(synth.decode_tokens(410 + 10 * M + l, w, M, K=K).x) for l in range(L)]
    ws = [moe.workspace(shp, max(M, 8)) for _ in range(L)]
    eager = [torch.empty((M, H), dtype=torch.float32, device="cuda") for _ in range(L)]
    for l in range(L):
        _layer(moe, shp, M, xs[l], dw, dsh, eager[l], ws[l])
    torch.cuda.synchronize()
    ref = [host(o).copy() for o in eager]

    outs = [torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda") for _ in range(L)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for l in range(L):
            _layer(moe, shp, M, xs[l], dw, dsh, outs[l], ws[l])
    torch.cuda.synchronize()

    a = torch.randn(256, 256, device="cuda")
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            got = host(outs[l])
            assert np.array_equal(got.view(np.uint32), ref[l].view(np.uint32)), (M, shared, rep, l)
        # eager work of the program between replays
        _ = (a @ a).sum().item()
        torch.cuda.synchronize()
