"""GPU parity of the shared expert against the CPU oracle, through the C ABI.

A Ling MoE layer sends every token to one shared expert besides its routed
ones ([EN] "What is Ling 3.0, and why does it suit DGX Spark?"); the library
runs it as one more slot of the same gate/up and down kernels (1..8 tokens) or
as one more expert of the grouped contractions (more tokens), with weight 1,
added after the routed terms.  The criteria are the routed layer's: the
intermediate h of every row (routed and shared) to rel L2 1e-3 (P3), the FP8
intermediate codes as in the routed tests, the layer output to 1e-2 (P5).
"""
import numpy as np
import pytest
import torch

import oracle
from _moe_helpers import DevWeights, dev, fp8_code_mismatches_ok, host, rel_l2, requant_codes_match
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


@pytest.fixture(scope="module")
def ling():
    w = synth.expert_weights(7, 2560, 768, 256)
    sh = synth.shared_expert(8, 2560, 768)
    return w, DevWeights(w), sh, tuple(dev(a) for a in sh)


def _tiny(seed):
    w = synth.expert_weights(seed, 256, 64, 16)
    sh = synth.shared_expert(seed + 500, 256, 64)
    return w, DevWeights(w), sh, tuple(dev(a) for a in sh)


def _forward(moe, shp, x, dw, dsh, ws):
    M = x.shape[0]
    out = torch.empty((M, shp.hidden), dtype=torch.float32, device="cuda")
    moe.moe_decode_forward_shared(shp, M, dev(x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, dsh, out, ws)
    torch.cuda.synchronize()
    return host(out)


def _experts(moe, shp, x, dw, dsh, ws, ids, w):
    """The experts entry point on given routing, with the M*K + M row taps."""
    M, I = x.shape[0], shp.inter
    R = M * shp.topk + (M if dsh is not None else 0)
    q = torch.empty((M, shp.hidden), dtype=torch.uint8, device="cuda")
    s = torch.empty(M, dtype=torch.float32, device="cuda")
    moe.moe_quant_act(shp, M, dev(x), q, s)
    taps = {"h": torch.empty((R, I), dtype=torch.float32, device="cuda"),
            "inter_fp8": torch.empty((R, I), dtype=torch.uint8, device="cuda"),
            "inter_scale": torch.empty(R, dtype=torch.float32, device="cuda")}
    out = torch.empty((M, shp.hidden), dtype=torch.float32, device="cuda")
    moe.moe_experts_forward_shared(shp, M, q, s, dev(ids.astype(np.int32)), dev(w.astype(np.float32)),
                                   dw.w13, dw.s13, dw.w2, dw.s2, dsh, out, ws, taps=taps)
    torch.cuda.synchronize()
    return host(out), {k: host(v) for k, v in taps.items()}


def _check_layer(moe, shp, x, w, dw, sh, dsh, ws, chunk):
    K = shp.topk
    t = oracle.moe_layer(x, w.wr, w.w13, w.s13, w.w2, w.s2, K, shared=oracle.SharedExpert(*sh))
    M = x.shape[0]
    assert t.h.shape[0] == M * K + M
    # P5 through the whole-layer entry point where the routing is decidable
    if not t.flags.any():
        err = rel_l2(_forward(moe, shp, x, dw, dsh, ws), t.out)
        assert err <= 1e-2, err
    # P3 and the FP8 intermediate on the oracle's routing, every row
    out, taps = _experts(moe, shp, x, dw, dsh, ws, t.route.ids, t.route.w)
    err = rel_l2(out, t.out)
    assert err <= 1e-2, err
    for rows in (slice(0, M * K), slice(M * K, M * K + M)):      # routed rows, then the shared rows
        e = rel_l2(taps["h"][rows], t.h[rows])
        assert e <= 1e-3, (rows, e)
    if chunk:
        # matrix-core sums: the FP8 intermediate is exactly the requantisation
        # of the kernel's own h; against the oracle's codes at most 1% differ
        requant_codes_match(taps["inter_fp8"], taps["inter_scale"], taps["h"])
        assert np.allclose(taps["inter_scale"], t.s2, rtol=1e-3, atol=0)
        assert (taps["inter_fp8"] != t.q2).sum() <= 0.01 * t.q2.size
    else:
        assert np.allclose(taps["inter_scale"], t.s2, rtol=1e-5, atol=0)
        y_ref = (t.h.astype(np.float32) / t.s2[:, None]).astype(np.float32)
        n_mis, bad = fp8_code_mismatches_ok(taps["inter_fp8"], t.q2, y_ref)
        assert not bad, (n_mis, bad[:5])
    return t


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_shared_tiny_decode(moe, M):
    w, dw, sh, dsh = _tiny(40 + M)
    shp = moe.shape(256, 64, 16, 2)
    x = synth.decode_tokens(60 + M, w, M, K=2).x
    _check_layer(moe, shp, x, w, dw, sh, dsh, moe.workspace(shp, 8), chunk=False)


@pytest.mark.parametrize("M", [9, 61, 200, 600, 2048])
def test_shared_tiny_chunk(moe, M):
    """Up to 2048 tokens: the shared expert's M rows are then cut into several
    chunk records of at most 256 rows (3 at 600 tokens, 8 at 2048)."""
    w, dw, sh, dsh = _tiny(80 + M)
    shp = moe.shape(256, 64, 16, 2)
    x = synth.decode_tokens(90 + M, w, M, K=2).x
    _check_layer(moe, shp, x, w, dw, sh, dsh, moe.workspace(shp, M), chunk=True)


def test_shared_ling_m1(moe, ling):
    w, dw, sh, dsh = ling
    shp = moe.shape(2560, 768, 256, 8)
    for seed in (500, 501):
        x = synth.decode_tokens(seed, w, 1).x
        _check_layer(moe, shp, x, w, dw, sh, dsh, moe.workspace(shp, 8), chunk=False)


@pytest.mark.parametrize("seed,distinct", [(510, 32), (511, 20)])
def test_shared_ling_verify_m4(moe, ling, seed, distinct):
    w, dw, sh, dsh = ling
    li = synth.verify_router(seed, w, distinct)
    shp = moe.shape(2560, 768, 256, 8)
    _check_layer(moe, shp, li.x, li.wts, dw.with_router(li.wts.wr), sh, dsh, moe.workspace(shp, 8), chunk=False)


def test_shared_ling_chunk_sampled(moe, ling):
    """40 tokens take the chunk path; the layer output of sampled tokens is
    compared (a token's output depends only on that token)."""
    w, dw, sh, dsh = ling
    shp = moe.shape(2560, 768, 256, 8)
    M = 40
    x = synth.decode_tokens(520, w, M).x
    got = _forward(moe, shp, x, dw, dsh, moe.workspace(shp, M))
    toks = [0, 17, 39]
    t = oracle.moe_layer(x[toks], w.wr, w.w13, w.s13, w.w2, w.s2, 8, shared=oracle.SharedExpert(*sh))
    ok = ~t.flags
    assert ok.any()
    err = rel_l2(got[toks][ok], t.out[ok])
    assert err <= 1e-2, err


def test_shared_none_is_the_routed_layer(moe):
    """shared = NULL gives the routed-only layer, bit for bit, and a workspace
    that served a shared call serves a routed-only call unchanged."""
    w, dw, sh, dsh = _tiny(120)
    shp = moe.shape(256, 64, 16, 2)
    for M in (4, 24):
        x = synth.decode_tokens(121, w, M, K=2).x
        ws_a, ws_b = moe.workspace(shp, M), moe.workspace(shp, M)
        plain = torch.empty((M, 256), dtype=torch.float32, device="cuda")
        moe.moe_decode_forward(shp, M, dev(x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, plain, ws_a)
        _forward(moe, shp, x, dw, dsh, ws_b)                       # leaves the shared slot in ws_b
        none = _forward(moe, shp, x, dw, None, ws_b)
        assert np.array_equal(none, host(plain))


def test_shared_expert_adds_its_own_term(moe):
    """(layer with shared) - (layer without) is the shared expert's own output
    for every token: compared with the oracle's K=1 layer routed to an expert
    that holds the shared weights (same steps, weight 1)."""
    w, dw, sh, dsh = _tiny(130)
    shp = moe.shape(256, 64, 16, 2)
    M = 5
    x = synth.decode_tokens(131, w, M, K=2).x
    ws = moe.workspace(shp, M)
    with_sh = _forward(moe, shp, x, dw, dsh, ws)
    without = _forward(moe, shp, x, dw, None, ws)
    one = synth.Weights(256, 64, 1, w.wr[:1].copy(), sh[0][None], sh[1][None], sh[2][None], sh[3][None])
    ref = oracle.moe_layer(x, one.wr, one.w13, one.s13, one.w2, one.s2, 1).out
    err = rel_l2(with_sh - without, ref)
    assert err <= 1e-2, err
