"""Pins for the CPU oracle: each one checks it against something other than
itself -- a format definition evaluated a different way, a library routine
(torch's OCP float8 conversion), a closed form, an invariant, or brute force.

Each test is chosen so that a plausible mistake in the oracle fails it: a wrong
nibble order or scale-block index, a transposed operand, a dropped sign, a
wrong tie-break, a reciprocal instead of a division, a missing requantisation.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore")


# ---------------------------------------------------------------------------
# Formats
# ---------------------------------------------------------------------------
def test_e2m1_all_16_codes_from_bit_fields():
    """MX v1.0 E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa, decoded from
    the bit fields here (the oracle uses a magnitude table)."""
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (0.5 * m) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
        v = -v if s else v
        got = oracle.e2m1_value(c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), c
    assert [oracle.e2m1_value(c) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_matches_f16_bit_placement():
    """A second, independent decode path: placing S at bit 15 and EEM at bits
    11..9 of an IEEE half gives the E2M1 value times 2^-14, for all 16 codes."""
    codes = np.arange(16, dtype=np.uint16)
    bits = ((codes & 8) << 12) | ((codes & 7) << 9)
    via_half = bits.view(np.float16).astype(np.float64) * 2.0 ** 14
    for c in range(16):
        assert oracle.e2m1_value(c) == via_half[c]


def test_e8m0_power_of_two_invariant():
    assert oracle.e8m0_value(127) == 1.0
    for c in range(0, 254):
        assert oracle.e8m0_value(c + 1) == 2.0 * oracle.e8m0_value(c)
        assert oracle.e8m0_value(c) == math.ldexp(1.0, c - 127)
    assert math.isnan(oracle.e8m0_value(255))


def test_e4m3_decode_all_256_against_torch():
    """torch's OCP float8_e4m3fn type is an independent library decode."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        got = oracle.e4m3_value(c)
        if c in (0x7F, 0xFF):
            assert math.isnan(got) and math.isnan(ref[c])
        else:
            assert got == ref[c], hex(c)
            assert math.copysign(1, got) == math.copysign(1, ref[c])
    assert oracle.e4m3_value(0x7E) == 448.0


def test_e4m3_encode_roundtrip_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c, hex(c)


# Hand-derived from the OFP8 E4M3 definition (grid spacing 2^(e-3) in binade
# [2^e, 2^(e+1)), subnormal spacing 2^-9, largest finite 448); see also
# tests/golden/e4m3_cases.txt.
E4M3_CASES = [
    (448.0, 0x7E), (-448.0, 0xFE), (1.0, 0x38), (0.0, 0x00), (-0.0, 0x80),
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01),
    (240.0, 0x77), (232.0, 0x76), (17.0, 0x58), (18.0, 0x59), (19.0, 0x5A),
    (500.0, 0x7E), (-1e-30, 0x80), (1e30, 0x7E), (464.0, 0x7E), (-3.0e38, 0xFE),
]


def test_e4m3_encode_printed_cases():
    for y, c in E4M3_CASES:
        assert oracle.e4m3_encode(y) == c, (y, hex(c))


def test_golden_e4m3_file_matches():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3_cases.txt")
    rows = [ln.split("#")[0].split() for ln in open(path)]
    rows = [r for r in rows if r]
    assert len(rows) >= 10
    for val, code in rows:
        assert oracle.e4m3_encode(float.fromhex(val)) == int(code, 16), (val, code)


def _e4m3_sweep_values():
    """Every E4M3 midpoint and its float32 neighbours, plus a dense stratified
    sample of every binade from 2^-12 to 2^9, both signs."""
    vals = [oracle.e4m3_value(c) for c in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    pts = []
    for m in mids + vals:
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    rng = np.random.default_rng(5)
    for e in range(-12, 9):
        mant = np.concatenate([np.arange(0, 1 << 23, 4099), rng.integers(0, 1 << 23, 4000)])
        pts.append((np.float32(2.0 ** e) * (1 + mant.astype(np.float64) / 2 ** 23)).astype(np.float32))
    pts = np.concatenate([np.atleast_1d(np.asarray(p, np.float32)) for p in pts])
    pts = np.concatenate([pts, -pts])
    return pts[np.abs(pts) <= 464.0]


def test_e4m3_encode_matches_torch_rne_sweep():
    """Within [-464, 464] torch's float8_e4m3fn conversion is round-to-nearest-
    even onto the finite grid (464 is the tie between 448 and the NaN slot).
    Above that torch gives NaN while the library saturates, tested separately."""
    y = _e4m3_sweep_values()
    ours = oracle.e4m3_encode_array(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(y[i]), hex(ours[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_saturates():
    y = np.array([448.0001, 470, 480, 512, 1e6, 3.4e38, np.inf], np.float32)
    assert (oracle.e4m3_encode_array(y) == 0x7E).all()
    assert (oracle.e4m3_encode_array(-y) == 0xFE).all()


# ---------------------------------------------------------------------------
# Activation quantisation
# ---------------------------------------------------------------------------
def test_quant_act_scale_and_nearest_code():
    rng = np.random.default_rng(3)
    x = synth.normal_bf16(rng, (3, 256), 1.0)
    x[2] = synth.bf16_from_f32(np.zeros(256, np.float32))
    q, s = oracle.quant_act(x)
    xf = synth.bf16_to_f32(x)
    for t in range(2):
        amax = np.float32(np.abs(xf[t]).max())
        assert s[t] == np.float32(amax / np.float32(448.0))   # numpy float32 division is IEEE
        y = (xf[t] / s[t]).astype(np.float32)
        dec = np.array([oracle.e4m3_value(c) for c in q[t]])
        # nearest: no finite code is strictly closer
        grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
        for yi, di, ci in zip(y, dec, q[t]):
            best = np.min(np.abs(grid - abs(float(yi))))
            assert abs(abs(di) - abs(float(yi))) == best
            assert bool(ci >= 0x80) == bool(np.signbit(yi))
        i = int(np.argmax(np.abs(xf[t])))
        assert q[t][i] in (0x7E, 0xFE)                         # the max maps to +-448
    assert s[2] == 1.0 and (q[2] == 0).all()


def test_quant_act_division_not_reciprocal():
    """With amax = 448 the scale is exactly 1 and codes equal direct encodes;
    with amax = 1 the scale is fl32(1/448) and y = x / s (a division) puts 1.0
    on 448 exactly, while the reciprocal form would give 447.99997."""
    x = np.zeros((1, 64), np.float32)
    x[0, 0] = 1.0
    x[0, 1] = -0.5
    q, s = oracle.quant_act(synth.bf16_from_f32(x))
    assert s[0] == np.float32(1.0) / np.float32(448.0)
    assert q[0, 0] == 0x7E and q[0, 1] == oracle.e4m3_encode(np.float32(-0.5) / s[0])


# ---------------------------------------------------------------------------
# Router and top-K
# ---------------------------------------------------------------------------
def _one_hot_router(logits, H=64):
    E = len(logits)
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    wr = np.zeros((E, H), np.float32)
    wr[:, 0] = logits
    return synth.bf16_from_f32(x), synth.bf16_from_f32(wr)


@pytest.mark.parametrize("logits,K,ids,w", [
    ([1, 3, 3, 2], 2, [1, 2], [0.5, 0.5]),
    ([1, 3, 2, 3, 0], 1, [1], [1.0]),
    ([0.5, 0.5, 0.5, 0.5], 3, [0, 1, 2], [1 / 3] * 3),
])
def test_route_hand_cases(logits, K, ids, w):
    x, wr = _one_hot_router(logits)
    r = oracle.route(x, wr, K)
    assert list(r.logits[0]) == [float(v) for v in logits]
    assert list(r.ids[0]) == ids
    np.testing.assert_allclose(r.w[0], w, rtol=0, atol=1e-15)


def test_route_gap_and_weights_closed_form():
    x, wr = _one_hot_router([0.0, 2.0, 1.0, -1.0, 0.5])
    r = oracle.route(x, wr, 2)
    assert list(r.ids[0]) == [1, 2] and r.gap[0] == 0.5
    e = math.exp(-1.0)
    np.testing.assert_allclose(r.w[0], [1 / (1 + e), e / (1 + e)], rtol=1e-15)
    r = oracle.route(x, wr, 5)
    assert r.gap[0] == math.inf


def test_route_logits_match_library_dot():
    rng = np.random.default_rng(11)
    x = synth.normal_bf16(rng, (3, 256), 1.0)
    wr = synth.normal_bf16(rng, (16, 256), 0.02)
    r = oracle.route(x, wr, 4)
    ref = synth.bf16_to_f32(x).astype(np.float64) @ synth.bf16_to_f32(wr).astype(np.float64).T
    np.testing.assert_allclose(r.logits, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r.w.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_topk_brute_force_over_subsets():
    """For E <= 12 and K <= 4, exactly one K-subset puts every member ahead of
    every non-member under (logit descending, index ascending); it must be the
    oracle's selection.  Logits are drawn from a small set so ties are common."""
    rng = np.random.default_rng(2)
    for trial in range(120):
        E = int(rng.integers(2, 13))
        K = int(rng.integers(1, min(4, E) + 1))
        logits = rng.choice([-1.0, 0.0, 0.5, 1.0, 2.0], size=E)
        x, wr = _one_hot_router(logits)
        r = oracle.route(x, wr, K)
        ahead = lambda a, b: logits[a] > logits[b] or (logits[a] == logits[b] and a < b)
        winners = [S for S in itertools.combinations(range(E), K)
                   if all(ahead(a, b) for a in S for b in range(E) if b not in S)]
        assert len(winners) == 1
        assert sorted(r.ids[0].tolist()) == list(winners[0])
        # canonical order within the selection
        sel = r.ids[0].tolist()
        assert all(ahead(sel[i], sel[i + 1]) for i in range(K - 1))


# ---------------------------------------------------------------------------
# Compaction
# ---------------------------------------------------------------------------
def test_compaction_invariants():
    rng = np.random.default_rng(4)
    for trial in range(50):
        M = int(rng.integers(1, 9))
        E = int(rng.integers(8, 40))
        K = int(rng.integers(1, min(8, E) + 1))
        ids = np.stack([rng.choice(E, size=K, replace=False) for _ in range(M)]).astype(np.int32)
        c = oracle.compact(ids, E)
        assert c.act_experts.tolist() == sorted(set(ids.ravel().tolist()))
        assert c.offsets[0] == 0 and c.offsets[-1] == M * K
        assert (np.diff(c.offsets) >= 1).all()
        for a, e in enumerate(c.act_experts):
            lo, hi = c.offsets[a], c.offsets[a + 1]
            toks = c.pair_token[lo:hi]
            assert (np.diff(toks) > 0).all()
            for i in range(lo, hi):
                assert ids.ravel()[c.pair_src[i]] == e
                assert c.pair_src[i] // K == c.pair_token[i]
        assert sorted(c.pair_src.tolist()) == list(range(M * K))
        assert (c.pair_of[c.pair_src] == np.arange(M * K)).all()


# ---------------------------------------------------------------------------
# Gate/up projection
# ---------------------------------------------------------------------------
H_T, I_T, E_T = 256, 64, 3


def _pack(codes):
    """Pack E2M1 codes [.., K] into bytes: element 2i low nibble, 2i+1 high."""
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _act_with_scale_one(seed, M=1, H=H_T):
    """bf16 activations whose amax is exactly 448, so the scale is exactly 1."""
    rng = np.random.default_rng(seed)
    xf = (rng.standard_normal((M, H)) * 8).astype(np.float32)
    xf[:, 5] = 448.0
    x = synth.bf16_from_f32(xf)
    q, s = oracle.quant_act(x)
    assert (s == 1.0).all()
    return x, q, s


def _e4m3_decode_lib(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double().numpy()


def test_gate_up_all_ones_closed_form():
    """Every weight 1.0 (code 0x2, scale 2^0): g = u = sum_k E4M3(q_k) exactly."""
    x, q, s = _act_with_scale_one(1)
    ids = np.array([[1]], np.int32)
    w13 = np.full((E_T, 2 * I_T, H_T // 2), 0x22, np.uint8)
    s13 = np.full((E_T, 2 * I_T, H_T // 32), 127, np.uint8)
    h = oracle.gate_up(q, s, ids, w13, s13, I_T)
    S = _e4m3_decode_lib(q[0]).sum()
    assert abs(S) < 700
    assert np.all(h[0] == S / (1 + math.exp(-S)) * S)


def _one_hot_w13(seed):
    """Row r of expert e has a single 1.0 at k = (7r + 3e + 1) mod H; block
    scales vary as 2^((r + b + e) mod 4 - 1)."""
    codes = np.zeros((E_T, 2 * I_T, H_T), np.uint8)
    kk = np.zeros((E_T, 2 * I_T), np.int64)
    for e in range(E_T):
        for r in range(2 * I_T):
            k = (7 * r + 3 * e + 1) % H_T
            codes[e, r, k] = 0x2
            kk[e, r] = k
    sc = np.zeros((E_T, 2 * I_T, H_T // 32), np.uint8)
    for e in range(E_T):
        for r in range(2 * I_T):
            for b in range(H_T // 32):
                sc[e, r, b] = 126 + (r + b + e) % 4
    return _pack(codes), sc, kk


def test_gate_up_one_hot_pins_layout_nibbles_and_scales():
    x, q, s = _act_with_scale_one(2, M=2)
    w13, s13, kk = _one_hot_w13(0)
    ids = np.array([[2, 0], [1, 2]], np.int32)
    h = oracle.gate_up(q, s, ids, w13, s13, I_T)
    A = _e4m3_decode_lib(q) * s[:, None]
    for t in range(2):
        for j in range(2):
            e = ids[t, j]
            for i in range(I_T):
                kg, ku = kk[e, i], kk[e, I_T + i]
                g = A[t, kg] * 2.0 ** (int(s13[e, i, kg // 32]) - 127)
                u = A[t, ku] * 2.0 ** (int(s13[e, I_T + i, ku // 32]) - 127)
                assert h[t * 2 + j, i] == g / (1 + math.exp(-g)) * u


def test_gate_up_sign_flip_and_scale_doubling_on_up_rows():
    rng = np.random.default_rng(9)
    x = synth.normal_bf16(rng, (1, H_T), 1.0)
    q, s = oracle.quant_act(x)
    w = synth.expert_weights(9, H_T, I_T, E_T)
    ids = np.array([[2, 1]], np.int32)
    h = oracle.gate_up(q, s, ids, w.w13, w.s13, I_T)
    flipped = w.w13.copy()
    flipped[:, I_T:, :] ^= 0x88                  # negate every up weight
    assert np.array_equal(oracle.gate_up(q, s, ids, flipped, w.s13, I_T), -h)
    scaled = w.s13.copy()
    scaled[:, I_T:, :] += 1                       # double every up weight
    assert np.array_equal(oracle.gate_up(q, s, ids, w.w13, scaled, I_T), 2 * h)


def test_gate_up_silu_zero_and_reflection():
    """SiLU(0) = 0 and SiLU(-z) = SiLU(z) - z, on the one-hot construction."""
    x, q, s = _act_with_scale_one(4)
    w13, s13, kk = _one_hot_w13(0)
    ids = np.array([[0]], np.int32)
    h = oracle.gate_up(q, s, ids, w13, s13, I_T)
    neg = w13.copy()
    neg[:, :I_T, :] ^= 0x88                       # negate the gate rows
    hn = oracle.gate_up(q, s, ids, neg, s13, I_T)
    A = _e4m3_decode_lib(q[0])
    for i in range(I_T):
        g = A[kk[0, i]] * 2.0 ** (int(s13[0, i, kk[0, i] // 32]) - 127)
        u = A[kk[0, I_T + i]] * 2.0 ** (int(s13[0, I_T + i, kk[0, I_T + i] // 32]) - 127)
        assert math.isclose(hn[0, i], h[0, i] - g * u, rel_tol=1e-14, abs_tol=1e-12)
    zero = w13.copy()
    zero[:, :I_T, :] = 0
    assert np.all(oracle.gate_up(q, s, ids, zero, s13, I_T) == 0)


# ---------------------------------------------------------------------------
# Requantisation
# ---------------------------------------------------------------------------
def test_requant_scale_max_and_zero_row():
    rng = np.random.default_rng(6)
    h = rng.standard_normal((3, 64)) * 5
    h[2] = 0.0
    q2, s2 = oracle.requant(h)
    for p in range(2):
        b = np.float32(np.abs(h[p].astype(np.float32)).max())
        assert s2[p] == b / np.float32(448.0)
        i = int(np.argmax(np.abs(h[p])))
        assert q2[p, i] in (0x7E, 0xFE)
        y = (h[p].astype(np.float32) / s2[p]).astype(np.float32)
        ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q2[p], ref)
    assert s2[2] == 1.0 and (q2[2] == 0).all()


# ---------------------------------------------------------------------------
# Down projection and combine
# ---------------------------------------------------------------------------
def test_down_permutation_closed_form():
    """W2[e, n, k] = 1.0 iff k == n mod I (scale 2^0): d_n = s2 * E4M3(q2[n mod I])
    and out = sum_j w_j * d_n exactly."""
    H, I, E, K, M = 256, 64, 4, 2, 2
    codes = np.zeros((E, H, I), np.uint8)
    for n in range(H):
        codes[:, n, n % I] = 0x2
    w2 = _pack(codes)
    sc2 = np.full((E, H, I // 32), 127, np.uint8)
    rng = np.random.default_rng(8)
    q2 = rng.integers(0, 0x7F, (M * K, I)).astype(np.uint8)
    s2 = np.array([0.5, 0.25, 2.0, 1.5], np.float32)
    ids = np.array([[3, 0], [1, 3]], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5]])
    out = oracle.down_combine(q2, s2, ids, w, w2, sc2, H)
    dec = _e4m3_decode_lib(q2)
    for t in range(M):
        for n in range(H):
            ref = sum(w[t, j] * (float(s2[t * K + j]) * dec[t * K + j, n % I]) for j in range(K))
            assert out[t, n] == ref


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def test_layer_doubles_with_every_down_scale_code():
    li = synth.tiny(3)
    w = li.wts
    a = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, li.K)
    b = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2 + 1, li.K)
    assert np.array_equal(b.out, 2 * a.out)


def test_layer_invariant_under_expert_relabelling():
    li = synth.tiny(4)
    w = li.wts
    a = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, li.K)
    assert not a.flags.any()
    perm = np.random.default_rng(1).permutation(w.E)
    b = oracle.moe_layer(li.x, w.wr[perm], w.w13[perm], w.s13[perm], w.w2[perm], w.s2[perm], li.K)
    assert np.array_equal(b.out, a.out)
    assert np.array_equal(perm[b.route.ids], a.route.ids)


def test_verify_router_construction_hits_distinct_counts():
    w = synth.expert_weights(200, 256, 64, 64)
    for seed, distinct in [(200, 32), (201, 20)]:
        li = synth.verify_router(seed, w, distinct)
        r = oracle.route(li.x, li.wts.wr, 8)
        assert len(set(r.ids.ravel().tolist())) == distinct
        assert r.gap.min() > 1e-2


# ---------------------------------------------------------------------------
# FP8 LM head: load-time row quantisation and the FP8-weight GEMV
# ---------------------------------------------------------------------------
def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    """Decode with torch's float8_e4m3fn (a decoder independent of the oracle)."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def test_lm_head_quant_hand_row():
    # amax 448 gives scale 1: 448 -> 0x7E, -224 = -1.75*2^7 -> 0xF6, 1 -> 0x38, 0 -> 0
    row = np.zeros((2, 16), np.float32)
    row[0, :4] = [448.0, -224.0, 1.0, 0.0]
    row[1, :4] = [448.0 * 2 ** -10, -224.0 * 2 ** -10, 2 ** -10, 0.0]   # same codes, scale 2^-10
    q, s = oracle.lm_head_quant(synth.bf16_from_f32(row))
    assert s[0] == np.float32(1.0) and s[1] == np.float32(2.0 ** -10)
    assert q[0, :4].tolist() == [0x7E, 0xF6, 0x38, 0x00] and q[1, :4].tolist() == q[0, :4].tolist()
    assert np.all(q[:, 4:] == 0)
    qz, sz = oracle.lm_head_quant(np.zeros((1, 8), np.uint16))
    assert sz[0] == 1.0 and np.all(qz == 0)


def test_lm_head_quant_error_bound():
    """Each dequantised weight is within half an E4M3 step of the bf16 weight
    (relative 2^-4 for normal codes, 2^-10 * s absolute for subnormals)."""
    rng = np.random.default_rng(5)
    w = synth.normal_bf16(rng, (64, 256), 0.02)
    q, s = oracle.lm_head_quant(w)
    wf = synth.bf16_to_f32(w).astype(np.float64)
    deq = _torch_e4m3(q) * s[:, None].astype(np.float64)
    bound = np.maximum(np.abs(wf) * 2.0 ** -4, s[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(np.abs(deq - wf) <= bound * (1 + 1e-12))
    assert np.allclose(s, np.abs(wf).max(axis=1).astype(np.float32) / np.float32(448.0), rtol=0, atol=0)


def test_lm_head_gemv_one_hot_and_ones():
    rng = np.random.default_rng(6)
    V, H = 40, 64
    q = rng.integers(0, 256, (V, H), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x30
    s = (2.0 ** rng.uniform(-12, -4, V)).astype(np.float32)
    for k in (0, 17, 63):
        x = np.zeros((1, H), np.float32)
        x[0, k] = 1.0
        got = oracle.lm_head_gemv(synth.bf16_from_f32(x), q, s)
        assert np.array_equal(got[0], s.astype(np.float64) * _torch_e4m3(q[:, k]))
    ones = synth.bf16_from_f32(np.ones((1, H), np.float32))
    got = oracle.lm_head_gemv(ones, q, s)
    assert np.allclose(got[0], s.astype(np.float64) * _torch_e4m3(q).sum(axis=1), rtol=1e-15, atol=0)
    x = synth.normal_bf16(rng, (3, H), 1.0)
    x2 = synth.bf16_from_f32(2.0 * synth.bf16_to_f32(x))
    assert np.array_equal(oracle.lm_head_gemv(x2, q, s), 2.0 * oracle.lm_head_gemv(x, q, s))


# ---------------------------------------------------------------------------
# Shared expert
# ---------------------------------------------------------------------------
def _shared_from(w: synth.Weights, e: int) -> oracle.SharedExpert:
    return oracle.SharedExpert(w.w13[e].copy(), w.s13[e].copy(), w.w2[e].copy(), w.s2[e].copy())


def test_shared_expert_equals_top1_routing_to_that_expert():
    """A shared expert with expert j's weights adds exactly what a K=1 layer
    that routes every token to j (weight 1) produces."""
    w = synth.expert_weights(41, 256, 64, 16)
    rng = np.random.default_rng(42)
    xf = synth.bf16_to_f32(synth.normal_bf16(rng, (5, 256), 1.0))
    xf[:, 0] = 1.0
    x = synth.bf16_from_f32(xf)
    j = 9
    wr1 = synth.bf16_to_f32(w.wr).copy()
    wr1[:, 0] = -40.0
    wr1[j, 0] = 40.0
    top1 = oracle.moe_layer(x, synth.bf16_from_f32(wr1), w.w13, w.s13, w.w2, w.s2, 1)
    assert np.all(top1.route.ids[:, 0] == j) and np.all(top1.route.w == 1.0)
    base = oracle.moe_layer(x, w.wr, w.w13, w.s13, w.w2, w.s2, 2)
    with_shared = oracle.moe_layer(x, w.wr, w.w13, w.s13, w.w2, w.s2, 2, shared=_shared_from(w, j))
    np.testing.assert_allclose(with_shared.out - base.out, top1.out, rtol=1e-12, atol=1e-12 * np.abs(top1.out).max())
    assert with_shared.h.shape[0] == 5 * 2 + 5
    np.testing.assert_array_equal(with_shared.q2[10:], top1.q2)


def test_shared_expert_zero_down_and_scale_doubling():
    w = synth.expert_weights(43, 256, 64, 16)
    li = synth.decode_tokens(44, w, 3, K=2)
    base = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, 2)
    sh = _shared_from(w, 3)
    sh0 = oracle.SharedExpert(sh.w13, sh.s13, np.zeros_like(sh.w2), sh.s2)
    np.testing.assert_array_equal(oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, 2, shared=sh0).out, base.out)
    one = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, 2, shared=sh).out - base.out
    sh2 = oracle.SharedExpert(sh.w13, sh.s13, sh.w2, (sh.s2.astype(np.int32) + 1).astype(np.uint8))
    two = oracle.moe_layer(li.x, w.wr, w.w13, w.s13, w.w2, w.s2, 2, shared=sh2).out - base.out
    np.testing.assert_allclose(two, 2.0 * one, rtol=1e-12, atol=1e-12 * np.abs(one).max())
