"""Caller-given ids that name one expert more than once within a token.

For M > 8 the interface allows it: each (token, j) pair is computed and
weighted on its own, and an expert's pairs stay in (token, j) order, as in the
oracle's compaction.  The chunk path's pair sort then falls back from token
bitmasks to a full sort; it is checked against the oracle's stages run on the
same ids: P3 for h, the requantisation codes of the kernel's own h, P5 for the
layer output, and bit-identical h rows for the repeated pairs of a token.
For M <= 8 such ids are outside the contract (results unspecified); the calls
must still complete without error and leave the workspace usable.
"""
import numpy as np
import pytest
import torch

import oracle
from _moe_helpers import DevWeights, dev, host, rel_l2, requant_codes_match
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


def _ids_with_repeats(seed, M, K, E):
    """Seeded ids in [0, E) where every token repeats at least one expert."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(M, K)).astype(np.int32)
    for t in range(M):
        j = int(rng.integers(1, K))
        ids[t, j] = ids[t, int(rng.integers(0, j))]
    return ids


def _check(moe, w, x, ids):
    M, K = ids.shape
    H, I, E = w.H, w.I, w.E
    shp = moe.shape(H, I, E, K)
    dw, ws = DevWeights(w), moe.workspace(shp, M)
    rng = np.random.default_rng(int(ids.sum()) + M)
    wts = rng.uniform(0.05, 0.5, size=(M, K)).astype(np.float32)
    q, s = oracle.quant_act(x)
    h_ref = oracle.gate_up(q, s, ids, w.w13, w.s13, I)
    q2_ref, s2_ref = oracle.requant(h_ref)
    out_ref = oracle.down_combine(q2_ref, s2_ref, ids, wts, w.w2, w.s2, H)

    P = M * K
    taps = {"h": torch.empty((P, I), dtype=torch.float32, device="cuda"),
            "inter_fp8": torch.empty((P, I), dtype=torch.uint8, device="cuda"),
            "inter_scale": torch.empty(P, dtype=torch.float32, device="cuda")}
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    moe.moe_experts_forward(shp, M, dev(q), dev(s), dev(ids), dev(wts), dw.w13, dw.s13, dw.w2, dw.s2, out, ws,
                            taps=taps)
    torch.cuda.synchronize()
    h, q2, s2 = host(taps["h"]), host(taps["inter_fp8"]), host(taps["inter_scale"])
    assert rel_l2(h, h_ref) <= 1e-3
    requant_codes_match(q2, s2, h)
    assert rel_l2(host(out), out_ref) <= 1e-2
    # repeated pairs of a token are the same computation
    for t in range(M):
        for j in range(K):
            for jj in range(j):
                if ids[t, j] == ids[t, jj]:
                    assert np.array_equal(h[t * K + j].view(np.uint32), h[t * K + jj].view(np.uint32)), (t, j, jj)


@pytest.mark.parametrize("M", [9, 40])
def test_repeated_ids_chunk_tiny(moe, M):
    w = synth.expert_weights(56, 256, 64, 16)
    x = synth.decode_tokens(57 + M, w, M, K=2).x
    _check(moe, w, x, _ids_with_repeats(58 + M, M, 2, 16))


def test_repeated_ids_chunk_all_one_expert(moe):
    """Twelve tokens whose K = 2 ids all name expert 7: 24 pairs in one slot."""
    w = synth.expert_weights(61, 256, 64, 16)
    x = synth.decode_tokens(62, w, 12, K=2).x
    _check(moe, w, x, np.full((12, 2), 7, np.int32))


@pytest.mark.parametrize("M", [1, 3, 8])
def test_repeated_ids_decode_path_completes(moe, M):
    """Repeated ids on the decode path: the call succeeds, and a following
    call with routed ids on the same workspace matches the oracle."""
    w = synth.expert_weights(51, 256, 64, 16)
    li = synth.decode_tokens(52 + M, w, M, K=2)
    shp = moe.shape(256, 64, 16, 2)
    dw, ws = DevWeights(w), moe.workspace(shp, 8)
    q, s = oracle.quant_act(li.x)
    out = torch.empty((M, 256), dtype=torch.float32, device="cuda")
    moe.moe_experts_forward(shp, M, dev(q), dev(s), dev(_ids_with_repeats(53 + M, M, 2, 16)),
                            dev(np.full((M, 2), 0.5, np.float32)), dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    torch.cuda.synchronize()
    t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, 2)
    moe.moe_experts_forward(shp, M, dev(q), dev(s), dev(t.route.ids.astype(np.int32)),
                            dev(t.route.w.astype(np.float32)),
                            dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    torch.cuda.synchronize()
    assert rel_l2(host(out), t.out) <= 1e-2
