"""GPU parity of kernels compiled at run time (moe_jit_load) against the CPU
oracle, through the C ABI: a layer shape outside the ahead-of-time set
(hidden 1024, intermediate 384, 64 experts, top-4) on the decode path, the
chunk path, with a shared expert and for the LM-head GEMV at hidden 1024;
and the Ling shape's own kernels compiled at run time and preferred over the
compiled-in ones.  The criteria are those of the compiled-in kernels
(P1-P5, LM-head logits within 1e-6 of their magnitude sums).
"""
import numpy as np
import pytest
import torch

import oracle
from _moe_helpers import DevWeights, dev, fp8_code_mismatches_ok, host, rel_l2
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu

H, I, E, K = 1024, 384, 64, 4


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


@pytest.fixture(scope="module")
def cache_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("jit_cache"))


@pytest.fixture(scope="module")
def loaded(moe, cache_dir):
    shp = moe.shape(H, I, E, K)
    st, info = moe.moe_path_info(shp, 1)
    assert st == moe.MOE_ERR_UNSUPPORTED_SHAPE, info         # nothing compiled implicitly
    first = moe.moe_jit_load(shp, cache_dir)
    second = moe.moe_jit_load(shp, cache_dir)               # reloads the module from the cache file
    print(f"jit: compile+load {first['seconds']:.2f} s, cached load {second['seconds']:.3f} s", flush=True)
    assert not first["from_cache"] and second["from_cache"]
    assert first["has_chunk_path"] and first["has_lm_head"]
    yield shp
    assert moe.moe_jit_unload(shp) == 1


@pytest.fixture(scope="module")
def weights():
    w = synth.expert_weights(900, H, I, E)
    return w, DevWeights(w)


def test_path_reports_run_time_kernels(moe, loaded):
    for M in (1, 4, 40):
        st, info = moe.moe_path_info(loaded, M)
        assert st == 0 and "compiled at run time" in info, info


@pytest.mark.parametrize("M", [1, 3, 4, 8])
def test_jit_decode_layer(moe, loaded, weights, M):
    w, dw = weights
    li = synth.decode_tokens(910 + M, w, M, K=K)
    ws = moe.workspace(loaded, 8)
    # P2 + bit-exact compaction
    ids = torch.empty((M, K), dtype=torch.int32, device="cuda")
    wts = torch.empty((M, K), dtype=torch.float32, device="cuda")
    taps = {"act_fp8": torch.empty((M, H), dtype=torch.uint8, device="cuda"),
            "act_scale": torch.empty(M, dtype=torch.float32, device="cuda")}
    moe.moe_route(loaded, M, dev(li.x), dw.wr, ids, wts, ws, taps=taps)
    torch.cuda.synchronize()
    r = oracle.route(li.x, w.wr, K)
    q_ref, s_ref = oracle.quant_act(li.x)
    assert np.array_equal(host(taps["act_fp8"]), q_ref)                      # P1
    assert np.array_equal(host(taps["act_scale"]).view(np.uint32), s_ref.view(np.uint32))
    ok = r.gap >= 1e-4
    assert np.array_equal(host(ids)[ok], r.ids[ok])                          # P2
    # P3: gate/up in isolation on the oracle's routing
    h = torch.empty((M * K, I), dtype=torch.float32, device="cuda")
    q2 = torch.empty((M * K, I), dtype=torch.uint8, device="cuda")
    s2 = torch.empty(M * K, dtype=torch.float32, device="cuda")
    moe.moe_gate_up(loaded, M, dev(q_ref), dev(s_ref), dev(r.ids), dw.w13, dw.s13, h, q2, s2, ws)
    torch.cuda.synchronize()
    h_ref = oracle.gate_up(q_ref, s_ref, r.ids, w.w13, w.s13, I)
    assert rel_l2(host(h), h_ref) <= 1e-3
    q2_ref, s2_ref = oracle.requant(h_ref)
    y_ref = (h_ref.astype(np.float32) / s2_ref[:, None]).astype(np.float32)
    n_mis, bad = fp8_code_mismatches_ok(host(q2), q2_ref, y_ref)
    assert not bad, (n_mis, bad[:5])
    # P4: down on the oracle's intermediate
    t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, K)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    moe.moe_down_combine(loaded, M, dev(t.q2), dev(t.s2), dev(t.route.ids), dev(t.route.w.astype(np.float32)),
                         dw.w2, dw.s2, out, ws)
    torch.cuda.synchronize()
    assert rel_l2(host(out), t.out) <= 1e-3
    # P5: the whole layer
    if not t.flags.any():
        moe.moe_decode_forward(loaded, M, dev(li.x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
        torch.cuda.synchronize()
        assert rel_l2(host(out), t.out) <= 1e-2


@pytest.mark.parametrize("M", [9, 40, 130])
def test_jit_chunk_layer(moe, loaded, weights, M):
    w, dw = weights
    li = synth.decode_tokens(930 + M, w, M, K=K)
    ws = moe.workspace(loaded, M)
    t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, K)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    if t.flags.any():
        q = torch.empty((M, H), dtype=torch.uint8, device="cuda")
        s = torch.empty(M, dtype=torch.float32, device="cuda")
        moe.moe_quant_act(loaded, M, dev(li.x), q, s)
        moe.moe_experts_forward(loaded, M, q, s, dev(t.route.ids), dev(t.route.w.astype(np.float32)),
                                dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    else:
        moe.moe_decode_forward(loaded, M, dev(li.x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
    torch.cuda.synchronize()
    assert rel_l2(host(out), t.out) <= 1e-2


@pytest.mark.parametrize("M", [2, 24])
def test_jit_shared_expert(moe, loaded, weights, M):
    w, dw = weights
    sh = synth.shared_expert(950, H, I)
    li = synth.decode_tokens(951 + M, w, M, K=K)
    ws = moe.workspace(loaded, M)
    t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, K, shared=oracle.SharedExpert(*sh))
    q = torch.empty((M, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(M, dtype=torch.float32, device="cuda")
    moe.moe_quant_act(loaded, M, dev(li.x), q, s)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    moe.moe_experts_forward_shared(loaded, M, q, s, dev(t.route.ids), dev(t.route.w.astype(np.float32)),
                                   dw.w13, dw.s13, dw.w2, dw.s2, tuple(dev(a) for a in sh), out, ws)
    torch.cuda.synchronize()
    assert rel_l2(host(out), t.out) <= 1e-2


@pytest.mark.parametrize("M", [1, 3, 8])
def test_jit_lm_head(moe, loaded, M):
    rng = np.random.default_rng(960 + M)
    V = 3001
    w = synth.bf16_from_f32((rng.standard_normal((V, H)) * 0.02).astype(np.float32))
    x = synth.normal_bf16(rng, (M, H), 1.0)
    q = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(V, dtype=torch.float32, device="cuda")
    moe.moe_lm_head_quantize(dev(w), q, s)
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    moe.moe_lm_head_forward(dev(x), q, s, logits)
    torch.cuda.synchronize()
    rq, rs = oracle.lm_head_quant(w)
    assert np.array_equal(host(q), rq) and np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    ref = oracle.lm_head_gemv(x, rq, rs)
    e4 = torch.from_numpy(rq).view(torch.float8_e4m3fn).double().numpy()
    mag = np.abs(synth.bf16_to_f32(x).astype(np.float64)) @ np.abs(e4).T * rs.astype(np.float64)[None, :]
    assert np.all(np.abs(host(logits) - ref) <= 1e-6 * mag + 1e-30)


def test_jit_ling_kernels_preferred(moe, cache_dir):
    """The Ling shape compiled at run time and preferred over the compiled-in
    kernels: oracle parity and agreement with the compiled-in result (8 tokens
    put 98 KiB of intermediate rows in the down kernel's LDS); after
    unloading, the compiled-in kernels run again."""
    w = synth.expert_weights(970, 2560, 768, 256)
    dw = DevWeights(w)
    shp = moe.shape(2560, 768, 256, 8)
    ws = moe.workspace(shp, 8)
    cases = [synth.decode_tokens(971, w, 1), synth.verify_router(972, w, 32), synth.decode_tokens(973, w, 8)]
    aot = []
    for li in cases:
        out = torch.empty((li.M, 2560), dtype=torch.float32, device="cuda")
        moe.moe_decode_forward(shp, li.M, dev(li.x), dev(li.wts.wr), dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
        torch.cuda.synchronize()
        aot.append(host(out))
    rep = moe.moe_jit_load(shp, cache_dir, prefer=True)
    try:
        st, info = moe.moe_path_info(shp, 1)
        assert st == 0 and "compiled at run time" in info, info
        for li, a in zip(cases, aot):
            t = oracle.moe_layer(li.x, li.wts.wr, w.w13, w.s13, w.w2, w.s2, 8)
            out = torch.empty((li.M, 2560), dtype=torch.float32, device="cuda")
            moe.moe_decode_forward(shp, li.M, dev(li.x), dev(li.wts.wr), dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
            torch.cuda.synchronize()
            got = host(out)
            if not t.flags.any():
                assert rel_l2(got, t.out) <= 1e-2
            assert rel_l2(got, a) <= 1e-5, rel_l2(got, a)
        print(f"jit ling: {rep}", flush=True)
    finally:
        assert moe.moe_jit_unload(shp) == 1
    st, info = moe.moe_path_info(shp, 1)
    assert st == 0 and "compiled at run time" not in info


@pytest.mark.parametrize("shared", [False, True])
def test_jit_one_token_items_beyond_the_grid(moe, cache_dir, shared):
    """One token routed from its logits where the gate/up items outnumber the
    512-workgroup grid (hidden 2560, intermediate 1088: 68 items per expert,
    8 x 68 = 544 items, 612 with the shared expert), so that workgroups also
    take an item of a higher-ranked slot than their first: the whole layer
    against the oracle (P5) and its routing (P2)."""
    Hj, Ij, Ej, Kj = 2560, 1088, 16, 8
    shp = moe.shape(Hj, Ij, Ej, Kj)
    moe.moe_jit_load(shp, cache_dir)
    try:
        w = synth.expert_weights(980, Hj, Ij, Ej)
        dw = DevWeights(w)
        ws = moe.workspace(shp, 1)
        sh = synth.shared_expert(981, Hj, Ij) if shared else None
        for seed in (982, 983, 984):
            li = synth.decode_tokens(seed, w, 1, K=Kj)
            t = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, Kj,
                                 shared=oracle.SharedExpert(*sh) if shared else None)
            if t.flags.any():
                continue
            out = torch.empty((1, Hj), dtype=torch.float32, device="cuda")
            if shared:
                moe.moe_decode_forward_shared(shp, 1, dev(li.x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2,
                                              tuple(dev(a) for a in sh), out, ws)
            else:
                moe.moe_decode_forward(shp, 1, dev(li.x), dw.wr, dw.w13, dw.s13, dw.w2, dw.s2, out, ws)
            torch.cuda.synchronize()
            err = rel_l2(host(out), t.out)
            print(f"one token, {Ij}-wide experts, shared={shared}, seed {seed}: rel_l2 {err:.2e}", flush=True)
            assert err <= 1e-2, err
    finally:
        assert moe.moe_jit_unload(shp) == 1
