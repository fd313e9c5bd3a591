"""Top-K under exact ties, at 2-8 tokens (the decode path) and 16 tokens (the
chunk path), for 256 and 512 experts.

The routers repeat rows, so many logits are bit-identical (the same row and
the same token give the same fp32 dot product, in the kernels as in the
oracle's fp64).  The selection's threshold pass then either finds more than
64 candidates and hands the token to the K wave-wide rounds, or ranks tied
candidates by index; either way the ids must equal the oracle's (logit
descending, the lower expert index first among equal logits) and the weights
its softmax over the selected logits.  Tokens whose top-(K+1) logits hold two
distinct values closer than 1e-4 (a near-tie that fp32 may order either way)
are not compared; exact ties always are.
"""
import numpy as np
import pytest
import torch

import oracle
from _moe_helpers import DevWeights, dev, host, rel_l2
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu

H, I, K = 256, 64, 8


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


def _tied_router(seed: int, E: int, kind: str) -> np.ndarray:
    rng = np.random.default_rng(seed)
    base = synth.normal_bf16(rng, (E, H), 0.02)
    if kind == "all":          # one row everywhere: every logit of a token equal
        wr = np.repeat(base[:1], E, axis=0)
    elif kind == "blocks":     # 8 distinct rows, row e = base[e % 8]: E/8 copies of each logit
        wr = base[np.arange(E) % 8]
    else:                      # "half": the even rows copies of row 0, the odd rows random
        wr = base.copy()
        wr[::2] = base[0]
    return np.ascontiguousarray(wr)


def _comparable(logits: np.ndarray) -> np.ndarray:
    """Per token: no two distinct values among the top K + 1 logits lie within 1e-4."""
    ok = np.ones(logits.shape[0], bool)
    for t, row in enumerate(logits):
        top = np.sort(row)[::-1][:K + 1]
        d = np.abs(np.diff(top))
        ok[t] = not np.any((d > 0) & (d < 1e-4))
    return ok


@pytest.mark.parametrize("kind", ["all", "blocks", "half"])
@pytest.mark.parametrize("M", [2, 4, 8, 16])
@pytest.mark.parametrize("E", [256, 512])
def test_route_ties_match_oracle(moe, E, M, kind):
    w = synth.with_router(synth.expert_weights(11, H, I, E), _tied_router(E + M, E, kind))
    li = synth.decode_tokens(100 + M, w, M, K)
    shp = moe.shape(H, I, E, K)
    ids = torch.empty((M, K), dtype=torch.int32, device="cuda")
    ww = torch.empty((M, K), dtype=torch.float32, device="cuda")
    print(f"route ties: E={E} M={M} kind={kind}", flush=True)
    moe.moe_route(shp, M, dev(li.x), dev(w.wr), ids, ww, moe.workspace(shp, M))
    torch.cuda.synchronize()
    r = oracle.route(li.x, w.wr, K)
    ok = _comparable(r.logits)
    assert ok.sum() >= M // 2, "too few comparable tokens for the test to mean anything"
    got_ids, got_w = host(ids), host(ww)
    assert (got_ids[ok] == r.ids[ok]).all(), (got_ids[ok], r.ids[ok])
    assert np.allclose(got_w[ok], r.w[ok], rtol=0, atol=1e-5)
    if kind == "all":          # K equal logits: the K lowest experts, equal weights
        assert (got_ids == np.arange(K)).all()
        assert np.allclose(got_w, 1.0 / K, rtol=0, atol=1e-6)


@pytest.mark.parametrize("kind", ["all", "half"])
@pytest.mark.parametrize("M", [2, 4])
def test_layer_with_tied_router(moe, M, kind):
    """The gate/up kernel's own routing prologue (top-K per token, then the
    compaction) on the tied routers: the layer output against the oracle's."""
    E = 256
    w = synth.with_router(synth.expert_weights(12, H, I, E), _tied_router(E + 7 * M, E, kind))
    li = synth.decode_tokens(200 + M, w, M, K)
    ref = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, K)
    if not _comparable(ref.route.logits).all():
        pytest.skip("a near-tie (distinct logits within 1e-4) at the top-K boundary")
    shp = moe.shape(H, I, E, K)
    dw = DevWeights(w)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    print(f"layer ties: M={M} kind={kind}", flush=True)
    moe.moe_decode_forward(shp, M, dev(li.x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, out, moe.workspace(shp, M))
    torch.cuda.synchronize()
    assert rel_l2(host(out), ref.out) <= 1e-2
