"""End-to-end parity over many seeds: the whole layer (routing, activation
quantisation, gate/up, requantisation, down, combine) against the oracle at
every token count of the decode path (1-8 tokens) and at chunk sizes around the
tile edges (9, 16, 17, 64, 65 tokens), top-2 and top-8, ten hidden states each.
Where the oracle flags a near tie in the top-K (gap < 1e-4), both sides take
the oracle's selection.  Bar: relative L2 <= 1e-2 over the layer output.
Weights: hidden 256, intermediate 64, 16 experts."""
import pytest
import torch

import oracle
from _moe_helpers import DevWeights, dev, host, rel_l2
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu

H, I, E = 256, 64, 16


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


@pytest.fixture(scope="module")
def weights():
    w = synth.expert_weights(7, H, I, E)
    return w, DevWeights(w)


def _forward(moe, shp, li, dw, ws, sel):
    M = li.M
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    if sel is None:
        moe.moe_decode_forward(shp, M, dev(li.x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    else:                                            # the oracle's selection, through the staged entry points
        q = torch.empty((M, H), dtype=torch.uint8, device="cuda")
        s = torch.empty(M, dtype=torch.float32, device="cuda")
        moe.moe_quant_act(shp, M, dev(li.x), q, s)
        ids, w = sel
        moe.moe_experts_forward(shp, M, q, s, dev(ids.astype("int32")), dev(w.astype("float32")),
                                dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("K", [2, 8])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 17, 64, 65])
def test_layer_over_seeds(moe, weights, M, K):
    w, dw = weights
    shp = moe.shape(H, I, E, K)
    ws = moe.workspace(shp, M)
    for seed in range(2000 + 100 * M + 10 * K, 2000 + 100 * M + 10 * K + 10):
        li = synth.decode_tokens(seed, w, M, K=K)
        t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, K)
        sel = (t.route.ids, t.route.w) if t.flags.any() else None
        err = rel_l2(_forward(moe, shp, li, dw, ws, sel), t.out)
        assert err <= 1e-2, (M, K, seed, err)
