"""The one-kernel decode layer (layer_kernel, M <= 8) through the C ABI,
selected for this module with moe_set_decode_path (the default is the
three-kernel path).

Its workgroups hand results to each other through epoch-tagged words in the
workspace, and every wait is bounded.  Checked here: the path is the one
kernel at every decode token count; no wait runs out over many calls, graph
replays and token counts on one workspace (the sticky status stays 0); with
the wait bound forced to zero from the host the kernel still completes (the
status reports the waits that ran out), and after moe_workspace_init the
layer is exact again; caller ids that repeat an expert within a token are
computed pair by pair (against the oracle's stages on the same ids); and the
layer output against the oracle at the Ling shape for 1-8 tokens and both
verify constructions.
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
    binding.moe_set_decode_path(binding.PATH_ONE_KERNEL)
    yield binding
    binding.moe_set_decode_path(binding.PATH_THREE_KERNELS)


@pytest.fixture(scope="module")
def ling():
    w = synth.expert_weights(1500, 2560, 768, 256)
    return w, DevWeights(w)


def _fwd(moe, shp, li, dw, ws, out):
    moe.moe_decode_forward(shp, li.M, dev(li.x), dev(li.wts.wr), dw.w13, dw.s13, dw.w2, dw.s2, out, ws)


def test_decode_token_counts_run_one_kernel(moe):
    for shp in (moe.shape(2560, 768, 256, 8), moe.shape(2560, 768, 512, 8), moe.shape(256, 64, 16, 2)):
        for M in range(1, 9):
            st, info = moe.moe_path_info(shp, M)
            assert st == 0 and info.startswith("one-kernel") and "layer_kernel" in info, info


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_layer_ling_against_oracle(moe, ling, M):
    w, dw = ling
    shp = moe.shape(2560, 768, 256, 8)
    ws = moe.workspace(shp, 8)
    li = synth.decode_tokens(1510 + M, w, M)
    t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, 8)
    out = torch.empty((M, 2560), dtype=torch.float32, device="cuda")
    _fwd(moe, shp, li, dw, ws, out)
    torch.cuda.synchronize()
    if not t.flags.any():
        err = rel_l2(host(out), t.out)
        print(f"layer M={M}: rel_l2 {err:.2e}", flush=True)
        assert err <= 1e-2
    assert moe.sync_errors(ws) == 0


@pytest.mark.parametrize("distinct", [32, 20])
def test_layer_verify_window_against_oracle(moe, ling, distinct):
    w, dw = ling
    shp = moe.shape(2560, 768, 256, 8)
    ws = moe.workspace(shp, 4)
    for seed in (1520, 1521):
        li = synth.verify_router(seed, w, distinct)
        t = oracle.moe_layer(li.x, li.wts.wr, w.w13, w.s13, w.w2, w.s2, 8)
        assert len(set(t.route.ids.flatten().tolist())) == distinct
        out = torch.empty((4, 2560), dtype=torch.float32, device="cuda")
        _fwd(moe, shp, li, dw, ws, out)
        torch.cuda.synchronize()
        assert rel_l2(host(out), t.out) <= 1e-2
    assert moe.sync_errors(ws) == 0


def test_sync_status_clean_over_calls_and_replays(moe):
    w = synth.expert_weights(1530, 256, 64, 16)
    dw = DevWeights(w)
    shp = moe.shape(256, 64, 16, 2)
    ws = moe.workspace(shp, 8)
    outs = {M: torch.empty((M, 256), dtype=torch.float32, device="cuda") for M in (1, 4, 8)}
    xs = {M: dev(synth.decode_tokens(1531 + M, w, M, K=2).x) for M in (1, 4, 8)}
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(300):
            M = (1, 4, 8)[i % 3]
            moe.moe_decode_forward(shp, M, xs[M], dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, outs[M], ws)
        torch.cuda.synchronize()
        ref = {M: outs[M].clone() for M in outs}
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for M in (1, 4, 8, 4, 1):
                moe.moe_decode_forward(shp, M, xs[M], dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, outs[M], ws)
        for _ in range(50):
            g.replay()
        torch.cuda.synchronize()
    for M in outs:
        assert torch.equal(outs[M], ref[M])
    assert moe.sync_errors(ws) == 0


def test_forced_wait_timeout_completes_and_recovers(moe):
    """Every wait bounded by 1 us: the kernel must still finish (the status
    then names the waits that ran out); after moe_workspace_init and the
    default bound the layer matches the oracle again."""
    w = synth.expert_weights(1540, 256, 64, 16)
    dw = DevWeights(w)
    shp = moe.shape(256, 64, 16, 2)
    ws = moe.workspace(shp, 4)
    li = synth.decode_tokens(1541, w, 4, K=2)
    t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, 2)
    out = torch.empty((4, 256), dtype=torch.float32, device="cuda")
    moe.moe_set_wait_limit_us(1)
    try:
        print("forced wait bound 1 us: launching", flush=True)
        for _ in range(3):
            _fwd(moe, shp, li, dw, ws, out)
        torch.cuda.synchronize()
        errs = moe.sync_errors(ws)
        print(f"forced wait bound 1 us: completed, status {errs:#x}", flush=True)
        assert (errs & ~0xF) == 0
        if errs == 0:                       # every wait happened to find its data at once
            assert rel_l2(host(out), t.out) <= 1e-2
    finally:
        moe.moe_set_wait_limit_us(0)        # back to the default bound
    moe.moe_workspace_init(ws)
    _fwd(moe, shp, li, dw, ws, out)
    torch.cuda.synchronize()
    assert moe.sync_errors(ws) == 0
    if not t.flags.any():
        assert rel_l2(host(out), t.out) <= 1e-2


def _ids_with_repeats(seed, M, K, E):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(M, K)).astype(np.int32)
    for t in range(M):
        j = int(rng.integers(1, K))
        ids[t, j] = ids[t, int(rng.integers(0, j))]
    return ids


@pytest.mark.parametrize("H,I,E,K,M", [(256, 64, 16, 2, 1), (256, 64, 16, 2, 8), (2560, 768, 256, 8, 3)])
def test_repeated_ids_pair_by_pair(moe, H, I, E, K, M):
    """Caller ids naming one expert more than once within a token, one kernel:
    h (P3), the intermediate codes of the kernel's own h, the layer (P5), and
    bit-identical h rows for a token's repeated pairs."""
    w = synth.expert_weights(1550 + M, H, I, E)
    dw = DevWeights(w)
    shp = moe.shape(H, I, E, K)
    ws = moe.workspace(shp, M)
    x = synth.decode_tokens(1551 + M, w, M, K=K).x
    ids = _ids_with_repeats(1552 + M, M, K, E)
    if M * K >= 8:
        ids[:, :] = ids[0, 0]                # every pair of every token on one expert
    wts = np.random.default_rng(1553).uniform(0.05, 0.5, size=(M, K)).astype(np.float32)
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
    for t in range(M):
        for j in range(K):
            for jj in range(j):
                if ids[t, j] == ids[t, jj]:
                    assert np.array_equal(h[t * K + j].view(np.uint32), h[t * K + jj].view(np.uint32))
    assert moe.sync_errors(ws) == 0
