"""The entry point that allocates nothing (moe_decode_forward_noalloc: the
library's static device scratch instead of a workspace) against the same
layer through moe_decode_forward with a workspace, through the C ABI: two
calls in a row, the second with fewer tokens, each bit-identical to the
workspace call (the same kernels on the same inputs), plus the oracle's
whole-layer bound (relative L2 <= 1e-2), and the size limit's error."""
import numpy as np
import pytest
import torch

import oracle
from _moe_helpers import DevWeights, dev, host, rel_l2
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


@pytest.mark.parametrize("H,I,E,K,tokens", [(2560, 768, 256, 8, (4, 1)), (256, 64, 16, 2, (8, 3))])
def test_noalloc_equals_workspace_call(moe, H, I, E, K, tokens):
    w = synth.expert_weights(1300 + H, H, I, E)
    dw = DevWeights(w)
    shp = moe.shape(H, I, E, K)
    ws = moe.workspace(shp, max(tokens))
    for call, M in enumerate(tokens):
        li = synth.decode_tokens(1310 + 7 * call + M, w, M, K=K)
        x = dev(li.x)
        ref = torch.empty((M, H), dtype=torch.float32, device="cuda")
        got = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_decode_forward(shp, M, x, dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, ref, ws)
        moe.moe_decode_forward_noalloc(shp, M, x, dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, got)
        torch.cuda.synchronize()
        print(f"noalloc H={H} call {call} M={M}", flush=True)
        assert np.array_equal(host(got).view(np.uint32), host(ref).view(np.uint32))
        t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, K)
        if not t.flags.any():
            assert rel_l2(host(got), t.out) <= 1e-2


def test_noalloc_rejects_what_does_not_fit(moe):
    shp = moe.shape(2560, 768, 256, 8)
    need = moe.moe_workspace_bytes(shp, 512)
    assert need > 4 << 20
    x = torch.zeros((512, 2560), dtype=torch.int16, device="cuda")
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = torch.empty((512, 2560), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_decode_forward_noalloc(shp, 512, x, dummy, dummy, dummy, dummy, dummy, out)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED_SHAPE
    assert "static scratch" in str(ei.value)
