"""GPU parity of every stage of the layer against the CPU oracle, through the
C ABI, on seeded synthetic inputs.

Criteria (fixed before any kernel existed):
  P1 activation quantisation: codes and scales bit-exact;
  P2 routing: the K selected experts per token as a set, for tokens whose
     rank-K / rank-(K+1) logit gap in the oracle is >= 1e-4, plus bit-exact
     compaction; weights within 1e-5;
  P3 gate/up alone (oracle's q, s, ids): h relative L2 <= 1e-3; FP8
     intermediate codes may differ only by one code at a rounding midpoint;
  P4 down + combine alone (oracle's q2, s2, ids, w): relative L2 <= 1e-3;
  P5 whole layer: relative L2 <= 1e-2 (flagged tokens take the oracle's ids
     and weights through moe_experts_forward).
"""
import numpy as np
import pytest
import torch

import oracle
from _moe_helpers import DevWeights, dev, fp8_code_mismatches_ok, host, rel_l2
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


@pytest.fixture(scope="module")
def ling_weights():
    """One full Ling-shaped expert set (E=256, 802 MB) shared by the L tests."""
    w = synth.expert_weights(1, 2560, 768, 256)
    return w, DevWeights(w)


def _shape(moe, w: synth.Weights, K: int):
    return moe.shape(w.H, w.I, w.E, K)


def _ws(moe, shp, M=8):
    return moe.workspace(shp, M)


def _gpu_forward(moe, shp, li: synth.LayerInputs, dw: DevWeights, ws):
    M = li.M
    out = torch.empty((M, shp.hidden), dtype=torch.float32, device="cuda")
    moe.moe_decode_forward(shp, M, dev(li.x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    torch.cuda.synchronize()
    return host(out)


def _gpu_experts_forward(moe, shp, li, dw, ws, ids, w):
    M = li.M
    q = torch.empty((M, shp.hidden), dtype=torch.uint8, device="cuda")
    s = torch.empty(M, dtype=torch.float32, device="cuda")
    moe.moe_quant_act(shp, M, dev(li.x), q, s)
    out = torch.empty((M, shp.hidden), dtype=torch.float32, device="cuda")
    moe.moe_experts_forward(shp, M, q, s, dev(ids.astype(np.int32)), dev(w.astype(np.float32)),
                            dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    torch.cuda.synchronize()
    return host(out)


# ---------------------------------------------------------------------------
# E4M3 encoder: exhaustive over all 2^32 binary32 patterns
# ---------------------------------------------------------------------------
def test_fp8_encoder_exhaustive_against_torch(moe):
    """torch's float8_e4m3fn conversion is an independent round-to-nearest-even
    onto the finite E4M3 grid for |y| <= 464; above that torch gives NaN while
    the library saturates to +-448, and NaN encodes as 0x7F."""
    chunk = 1 << 26
    q = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for start in range(0, 1 << 32, chunk):
        moe.moe_fp8_encode_range(start, chunk, q)
        bits = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda")
        y = bits.to(torch.int32).view(torch.float32)
        ay = y.abs()
        inr = ay <= 464.0
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8)
        bad = (q != ref) & inr
        assert not bool(bad.any()), (start, int(bad.nonzero()[0]))
        sat = (~inr) & torch.isfinite(y) | torch.isinf(y)
        want_sat = torch.where(y < 0, 0xFE, 0x7E).to(torch.uint8)
        assert bool(((q == want_sat) | ~sat).all()), start
        nan = torch.isnan(y)
        assert bool(((q == 0x7F) | ~nan).all()), start
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# P1: activation quantisation
# ---------------------------------------------------------------------------
def _special_rows(H):
    rows = np.zeros((4, H), np.float32)
    rows[1, ::3] = -0.0                           # all-zero row with -0 entries
    rows[2, 0] = 448.0                            # scale exactly 1: ties 17, 19, 232, 2^-10
    rows[2, 1:9] = [17.0, 19.0, 232.0, 2.0 ** -10, -(2.0 ** -9), 1.5 * 2.0 ** -10, 240.0, -18.0]
    rows[3, :] = np.linspace(-3.0e38, 3.0e38, H, dtype=np.float32)    # near the bf16 maximum
    return synth.bf16_from_f32(rows)


@pytest.mark.parametrize("H", [256, 2560])
def test_quant_act_bit_exact(moe, H):
    I = 64 if H == 256 else 768
    shp = moe.shape(H, I, 16, 2)
    rng = np.random.default_rng(H)
    for M in (1, 3, 8):
        x = synth.normal_bf16(rng, (M, H), 1.0)
        if M == 8:
            x[4:] = _special_rows(H)
        q = torch.empty((M, H), dtype=torch.uint8, device="cuda")
        s = torch.empty(M, dtype=torch.float32, device="cuda")
        moe.moe_quant_act(shp, M, dev(x), q, s)
        rq, rs = oracle.quant_act(x)
        assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32)), (M, host(s), rs)
        assert np.array_equal(host(q), rq), np.nonzero(host(q) != rq)


# ---------------------------------------------------------------------------
# P2: routing and compaction
# ---------------------------------------------------------------------------
def _check_route(moe, shp, li, dw, ws):
    M, K = li.M, li.K
    ids = torch.empty((M, K), dtype=torch.int32, device="cuda")
    w = torch.empty((M, K), dtype=torch.float32, device="cuda")
    S = min(shp.num_experts, M * K)
    taps = {"logits": torch.empty((M, shp.num_experts), dtype=torch.float32, device="cuda"),
            "n_active": torch.empty(1, dtype=torch.int32, device="cuda"),
            "act_experts": torch.empty(S, dtype=torch.int32, device="cuda"),
            "offsets": torch.empty(S + 1, dtype=torch.int32, device="cuda"),
            "pair_token": torch.empty(M * K, dtype=torch.int32, device="cuda"),
            "pair_src": torch.empty(M * K, dtype=torch.int32, device="cuda"),
            "act_fp8": torch.empty((M, shp.hidden), dtype=torch.uint8, device="cuda"),
            "act_scale": torch.empty(M, dtype=torch.float32, device="cuda")}
    moe.moe_route(shp, M, dev(li.x), dw.wr, ids, w, ws, taps=taps)
    torch.cuda.synchronize()
    r = oracle.route(li.x, li.wts.wr, K)
    # P1 on the router kernel's own quantisation path
    rq, rs = oracle.quant_act(li.x)
    assert np.array_equal(host(taps["act_scale"]).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(taps["act_fp8"]), rq)
    gids, gw = host(ids), host(w)
    flags = r.gap < 1e-4
    for t in range(M):
        if flags[t]:
            continue
        assert set(gids[t].tolist()) == set(r.ids[t].tolist()), (t, gids[t], r.ids[t])
        assert np.array_equal(gids[t], r.ids[t]), "canonical order"
        assert np.abs(gw[t] - r.w[t]).max() <= 1e-5
    # fp32 logits against the exact values, within the usual dot-product bound
    # (a few ulps of the sum of |products|)
    scale = np.abs(synth.bf16_to_f32(li.x).astype(np.float64)) @ np.abs(
        synth.bf16_to_f32(li.wts.wr).astype(np.float64)).T
    assert (np.abs(host(taps["logits"]) - r.logits) <= 1e-6 * scale + 1e-30).all()
    # compaction of the GPU's own ids, bit-exact
    c = oracle.compact(gids, shp.num_experts)
    n = int(host(taps["n_active"])[0])
    assert n == c.n_act
    assert np.array_equal(host(taps["act_experts"])[:n], c.act_experts)
    assert np.array_equal(host(taps["offsets"])[:n + 1], c.offsets)
    assert np.array_equal(host(taps["pair_token"]), c.pair_token)
    assert np.array_equal(host(taps["pair_src"]), c.pair_src)
    return r, n


def test_route_quantises_special_rows(moe):
    """The router kernel's activation quantisation on zero, tie and huge rows."""
    w = synth.expert_weights(6, 256, 64, 16)
    x = synth.normal_bf16(np.random.default_rng(6), (8, 256), 1.0)
    x[4:] = _special_rows(256)
    li = synth.LayerInputs(x, w, 2)
    shp = _shape(moe, w, 2)
    _check_route(moe, shp, li, DevWeights(w), _ws(moe, shp))


def test_route_tiny(moe):
    for seed in range(10):
        li = synth.tiny(seed)
        shp = _shape(moe, li.wts, li.K)
        _check_route(moe, shp, li, DevWeights(li.wts), _ws(moe, shp))


def test_route_ling_m1(moe, ling_weights):
    w, dw = ling_weights
    shp = _shape(moe, w, 8)
    ws = _ws(moe, shp)
    for seed in range(100, 110):
        rng = np.random.default_rng(seed)
        wr = synth.normal_bf16(rng, (w.E, w.H), 0.02)
        li = synth.decode_tokens(seed, synth.with_router(w, wr), 1)
        _check_route(moe, shp, li, dw.with_router(wr), ws)


@pytest.mark.parametrize("seed,distinct", [(200, 32), (201, 20), (202, 32), (203, 20)])
def test_route_verify_m4_distinct(moe, ling_weights, seed, distinct):
    w, dw = ling_weights
    li = synth.verify_router(seed, w, distinct)
    shp = _shape(moe, w, 8)
    r, n = _check_route(moe, shp, li, dw.with_router(li.wts.wr), _ws(moe, shp))
    assert n == distinct


def test_route_exact_ties_go_to_lower_index(moe):
    """Duplicate router rows give bit-identical logits; the lower index must win,
    also across the K boundary."""
    w = synth.expert_weights(5, 256, 64, 16)
    wr = w.wr.copy()
    li0 = synth.tiny(5)
    r0 = oracle.route(li0.x, wr, 2)
    top = int(r0.ids[0, 0])
    # copy the best row onto a lower and a higher index: the tie sits at rank 1/2/3
    lo, hi = (top + 5) % 16, (top + 9) % 16
    wr[lo] = wr[top]
    wr[hi] = wr[top]
    li = synth.LayerInputs(li0.x, synth.with_router(w, wr), 2)
    shp = _shape(moe, li.wts, 2)
    ids = torch.empty((1, 2), dtype=torch.int32, device="cuda")
    ww = torch.empty((1, 2), dtype=torch.float32, device="cuda")
    moe.moe_route(shp, 1, dev(li.x), dev(wr), ids, ww, _ws(moe, shp))
    torch.cuda.synchronize()
    want = sorted([top, lo, hi])[:2]
    assert host(ids)[0].tolist() == want
    assert np.allclose(host(ww)[0], [0.5, 0.5])


# ---------------------------------------------------------------------------
# P3: gate/up in isolation
# ---------------------------------------------------------------------------
def _check_gate_up(moe, shp, li, dw, ws, r=None):
    M, K, I = li.M, li.K, shp.inter
    r = r or oracle.route(li.x, li.wts.wr, K)
    q, s = oracle.quant_act(li.x)
    h_ref = oracle.gate_up(q, s, r.ids, li.wts.w13, li.wts.s13, I)
    q2_ref, s2_ref = oracle.requant(h_ref)
    h = torch.empty((M * K, I), dtype=torch.float32, device="cuda")
    q2 = torch.empty((M * K, I), dtype=torch.uint8, device="cuda")
    s2 = torch.empty(M * K, dtype=torch.float32, device="cuda")
    moe.moe_gate_up(shp, M, dev(q), dev(s), dev(r.ids), dw.w13, dw.s13, h, q2, s2, ws)
    torch.cuda.synchronize()
    err = rel_l2(host(h), h_ref)
    assert err <= 1e-3, err
    assert np.allclose(host(s2), s2_ref, rtol=1e-5, atol=0)
    y_ref = (h_ref.astype(np.float32) / s2_ref[:, None]).astype(np.float32)
    n_mis, bad = fp8_code_mismatches_ok(host(q2), q2_ref, y_ref)
    assert not bad, (n_mis, bad[:5])
    return err, n_mis


def test_gate_up_tiny(moe):
    for seed in range(10):
        li = synth.tiny(seed)
        shp = _shape(moe, li.wts, li.K)
        _check_gate_up(moe, shp, li, DevWeights(li.wts), _ws(moe, shp))


def test_gate_up_ling_m1(moe, ling_weights):
    w, dw = ling_weights
    shp = _shape(moe, w, 8)
    for seed in (100, 101):
        li = synth.decode_tokens(seed, w, 1)
        _check_gate_up(moe, shp, li, dw, _ws(moe, shp))


@pytest.mark.parametrize("seed,distinct", [(200, 32), (201, 20)])
def test_gate_up_verify_m4(moe, ling_weights, seed, distinct):
    w, dw = ling_weights
    li = synth.verify_router(seed, w, distinct)
    shp = _shape(moe, w, 8)
    _check_gate_up(moe, shp, li, dw.with_router(li.wts.wr), _ws(moe, shp))


# ---------------------------------------------------------------------------
# P4: down + combine in isolation
# ---------------------------------------------------------------------------
def _check_down(moe, shp, li, dw, ws):
    M, K, H, I = li.M, li.K, shp.hidden, shp.inter
    t = oracle.moe_layer(li.x, li.wts.wr, li.wts.w13, li.wts.s13, li.wts.w2, li.wts.s2, K)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    moe.moe_down_combine(shp, M, dev(t.q2), dev(t.s2), dev(t.route.ids), dev(t.route.w.astype(np.float32)),
                         dw.w2, dw.s2, out, ws)
    torch.cuda.synchronize()
    err = rel_l2(host(out), t.out)
    assert err <= 1e-3, err
    return err


def test_down_tiny(moe):
    for seed in range(10):
        li = synth.tiny(seed)
        shp = _shape(moe, li.wts, li.K)
        _check_down(moe, shp, li, DevWeights(li.wts), _ws(moe, shp))


def test_down_ling(moe, ling_weights):
    w, dw = ling_weights
    shp = _shape(moe, w, 8)
    _check_down(moe, shp, synth.decode_tokens(102, w, 1), dw, _ws(moe, shp))
    li = synth.verify_router(201, w, 20)
    _check_down(moe, shp, li, dw.with_router(li.wts.wr), _ws(moe, shp))


# ---------------------------------------------------------------------------
# P5: whole layer
# ---------------------------------------------------------------------------
def _check_layer(moe, shp, li, dw, ws):
    t = oracle.moe_layer(li.x, li.wts.wr, li.wts.w13, li.wts.s13, li.wts.w2, li.wts.s2, li.K)
    if t.flags.any():
        got = _gpu_experts_forward(moe, shp, li, dw, ws, t.route.ids, t.route.w)
    else:
        got = _gpu_forward(moe, shp, li, dw, ws)
    err = rel_l2(got, t.out)
    assert err <= 1e-2, err
    return err


def test_layer_tiny(moe):
    for seed in range(10):
        li = synth.tiny(seed)
        shp = _shape(moe, li.wts, li.K)
        _check_layer(moe, shp, li, DevWeights(li.wts), _ws(moe, shp))


def test_layer_ling_m1(moe, ling_weights):
    w, dw = ling_weights
    shp = _shape(moe, w, 8)
    ws = _ws(moe, shp)
    for seed in (103, 104, 105):
        _check_layer(moe, shp, synth.decode_tokens(seed, w, 1), dw, ws)


@pytest.mark.parametrize("seed,distinct", [(202, 32), (203, 20)])
def test_layer_verify_m4(moe, ling_weights, seed, distinct):
    w, dw = ling_weights
    li = synth.verify_router(seed, w, distinct)
    shp = _shape(moe, w, 8)
    _check_layer(moe, shp, li, dw.with_router(li.wts.wr), _ws(moe, shp))


@pytest.mark.parametrize("M", [2, 3, 5, 7, 8])
def test_layer_ragged_token_counts(moe, M):
    w = synth.expert_weights(11, 256, 64, 16)
    li = synth.decode_tokens(50 + M, w, M, K=2)
    shp = _shape(moe, w, 2)
    _check_layer(moe, shp, li, DevWeights(w), _ws(moe, shp))


def test_layer_all_experts_selected(moe):
    """K = E: every expert is active for every token (gap is infinite)."""
    w = synth.expert_weights(12, 256, 64, 8)
    li = synth.decode_tokens(60, w, 3, K=8)
    shp = _shape(moe, w, 8)
    _check_layer(moe, shp, li, DevWeights(w), _ws(moe, shp))


@pytest.mark.parametrize("E,K", [(40, 4), (100, 8), (200, 8), (300, 8)])
def test_route_and_layer_partial_logit_loads(moe, E, K):
    """Expert counts that fill a lane's last logits load only in part (E % 64
    != 0, one to eight logits per lane): the top-K masks the lanes past E.
    Routing (P1, P2, compaction) and the whole layer (P5) at 1 token (gate/up
    ranks in rank order) and 3 tokens (the compaction path)."""
    w = synth.expert_weights(80 + E, 256, 64, E)
    shp = _shape(moe, w, K)
    dw = DevWeights(w)
    for M in (1, 3):
        li = synth.decode_tokens(81 + E + M, w, M, K=K)
        _check_route(moe, shp, li, dw, _ws(moe, shp))
        _check_layer(moe, shp, li, dw, _ws(moe, shp))


def test_layer_zero_hidden(moe):
    w = synth.expert_weights(13, 256, 64, 16)
    x = synth.bf16_from_f32(np.zeros((2, 256), np.float32))
    li = synth.LayerInputs(x, w, 2)
    shp = _shape(moe, w, 2)
    got = _gpu_forward(moe, shp, li, DevWeights(w), _ws(moe, shp))
    assert np.all(got == 0.0)


def test_workspace_reuse_across_token_counts(moe):
    """One workspace sized for 8 tokens serves interleaved calls of 1..8 tokens."""
    w = synth.expert_weights(14, 256, 64, 16)
    dw = DevWeights(w)
    shp = _shape(moe, w, 2)
    ws = _ws(moe, shp, 8)
    for M in (8, 1, 4, 1, 6, 2):
        li = synth.decode_tokens(70 + M, w, M, K=2)
        _check_layer(moe, shp, li, dw, ws)


def test_requant_inside_down_matches_requant_kernel(moe, ling_weights):
    """The forward path requantises inside the down kernel; its codes and
    scales (the experts taps) must equal the standalone requant kernel's."""
    w, dw = ling_weights
    li = synth.verify_router(205, w, 20)
    shp = _shape(moe, w, 8)
    ws = _ws(moe, shp)
    t = oracle.route(li.x, li.wts.wr, 8)
    M, K, I = 4, 8, shp.inter
    q = torch.empty((M, shp.hidden), dtype=torch.uint8, device="cuda")
    s = torch.empty(M, dtype=torch.float32, device="cuda")
    moe.moe_quant_act(shp, M, dev(li.x), q, s)
    ids, wts = dev(t.ids.astype(np.int32)), dev(t.w.astype(np.float32))
    taps = {"h": torch.empty((M * K, I), dtype=torch.float32, device="cuda"),
            "inter_fp8": torch.empty((M * K, I), dtype=torch.uint8, device="cuda"),
            "inter_scale": torch.empty(M * K, dtype=torch.float32, device="cuda")}
    out = torch.empty((M, shp.hidden), dtype=torch.float32, device="cuda")
    moe.moe_experts_forward(shp, M, q, s, ids, wts, dw.w13, dw.s13, dw.w2, dw.s2, out, ws, taps=taps)
    h2 = torch.empty_like(taps["h"])
    q2 = torch.empty_like(taps["inter_fp8"])
    s2 = torch.empty_like(taps["inter_scale"])
    moe.moe_gate_up(shp, M, q, s, ids, dw.w13, dw.s13, h2, q2, s2, ws)
    torch.cuda.synchronize()
    assert torch.equal(taps["h"], h2)
    assert torch.equal(taps["inter_fp8"], q2)
    assert torch.equal(taps["inter_scale"], s2)


def test_deterministic_repeat(moe, ling_weights):
    w, dw = ling_weights
    li = synth.verify_router(204, w, 32)
    shp = _shape(moe, w, 8)
    ws = _ws(moe, shp)
    dwr = dw.with_router(li.wts.wr)
    a = _gpu_forward(moe, shp, li, dwr, ws)
    b = _gpu_forward(moe, shp, li, dwr, ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _fused_and_staged(moe, shp, li, dw, ws, shared=None):
    """The fused forward, and the staged path on the same inputs: moe_route
    (its quantisation taps, ids and weights), then moe_experts_forward."""
    M, H, K = li.M, shp.hidden, shp.topk
    x = dev(li.x)
    out_f = torch.empty((M, H), dtype=torch.float32, device="cuda")
    if shared is None:
        moe.moe_decode_forward(shp, M, x, dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, out_f, ws)
    else:
        moe.moe_decode_forward_shared(shp, M, x, dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, shared, out_f, ws)
    ids = torch.empty((M, K), dtype=torch.int32, device="cuda")
    w = torch.empty((M, K), dtype=torch.float32, device="cuda")
    q = torch.empty((M, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(M, dtype=torch.float32, device="cuda")
    moe.moe_route(shp, M, x, dw.wr, ids, w, ws, taps={"act_fp8": q, "act_scale": s})
    out_s = torch.empty((M, H), dtype=torch.float32, device="cuda")
    if shared is None:
        moe.moe_experts_forward(shp, M, q, s, ids, w, dw.w13, dw.s13, dw.w2, dw.s2, out_s, ws)
    else:
        moe.moe_experts_forward_shared(shp, M, q, s, ids, w, dw.w13, dw.s13, dw.w2, dw.s2, shared, out_s, ws)
    torch.cuda.synchronize()
    return host(out_f), host(out_s), host(q), host(s)


@pytest.mark.parametrize("M,seed", [(1, 0), (1, 1), (1, 2), (2, 3), (2, 4)])
def test_small_forward_equals_staged_path(moe, ling_weights, M, seed):
    """At one or two tokens the gate/up kernel quantises the activations
    itself (the router then computes logits only).  The layer output must
    equal, bit for bit, the staged path whose codes come from the router's
    quantisation, and those codes are bit-exact with the oracle (P1)."""
    w, dw = ling_weights
    li = synth.decode_tokens(300 + seed, w, M, K=8)
    shp = _shape(moe, w, 8)
    ws = _ws(moe, shp)
    fused, staged, q, s = _fused_and_staged(moe, shp, li, dw, ws)
    assert np.array_equal(fused.view(np.uint32), staged.view(np.uint32))
    rq, rs = oracle.quant_act(li.x)
    assert np.array_equal(q, rq) and np.array_equal(s.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("M", [1, 2])
def test_small_forward_equals_staged_path_tiny_shared(moe, M):
    """The same at the tiny shape (one wave quantises a whole token), without
    and with a shared expert."""
    w = synth.expert_weights(71, 256, 64, 16)
    li = synth.decode_tokens(72 + M, w, M, K=2)
    shp = _shape(moe, w, 2)
    dw, ws = DevWeights(w), _ws(moe, shp)
    fused, staged, _, _ = _fused_and_staged(moe, shp, li, dw, ws)
    assert np.array_equal(fused.view(np.uint32), staged.view(np.uint32))
    sh = [dev(t) for t in synth.shared_expert(73, 256, 64)]
    fused, staged, _, _ = _fused_and_staged(moe, shp, li, dw, ws, shared=sh)
    assert np.array_equal(fused.view(np.uint32), staged.view(np.uint32))
