"""GPU parity of the FP8 LM head (load-time per-row E4M3 quantisation and the
FP8-weight decode GEMV) against the CPU oracle, through the C ABI.

Quantisation codes and scales must be bit-exact.  The logits are fp32 sums of
exact products (E4M3 and bf16 are both exact in the bf16 x bf16 -> fp32 dot
instruction), so each must lie within 1e-6 of the sum of the magnitudes of its
terms, times the row scale, of the oracle's double value.  At the pages'
vocabulary (157,184 x 2,560) rows are sampled for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from _moe_helpers import dev, host
from mxfp4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


def _quant(moe, w):
    V, H = w.shape
    q = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(V, dtype=torch.float32, device="cuda")
    moe.moe_lm_head_quantize(dev(w), q, s)
    torch.cuda.synchronize()
    return q, s


def _e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _check_logits(got, x, q, s):
    ref = oracle.lm_head_gemv(x, q, s)
    mag = np.abs(synth.bf16_to_f32(x).astype(np.float64)) @ np.abs(_e4m3(q)).T * s.astype(np.float64)[None, :]
    assert np.all(np.abs(got - ref) <= 1e-6 * mag + 1e-30), np.max(np.abs(got - ref) / (mag + 1e-30))


def test_lm_head_quant_bit_exact_small(moe):
    rng = np.random.default_rng(1)
    wf = (rng.standard_normal((301, 512)) * 0.02).astype(np.float32)
    wf[0] = 0.0                                   # all-zero row: scale 1
    wf[1] = 0.0
    wf[1, 7] = -3.0e38                            # huge
    wf[2] = 1.0                                   # all equal
    wf[3, ::2] = -wf[3, ::2]
    w = synth.bf16_from_f32(wf)
    q, s = _quant(moe, w)
    rq, rs = oracle.lm_head_quant(w)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


@pytest.mark.parametrize("M", [1, 3, 8])
def test_lm_head_gemv_small(moe, M):
    rng = np.random.default_rng(10 + M)
    w = synth.normal_bf16(rng, (1000, 512), 0.02)
    x = synth.normal_bf16(rng, (M, 512), 1.0)
    q, s = _quant(moe, w)
    logits = torch.empty((M, 1000), dtype=torch.float32, device="cuda")
    moe.moe_lm_head_forward(dev(x), q, s, logits)
    torch.cuda.synchronize()
    _check_logits(host(logits), x, host(q), host(s))


@pytest.mark.slow
def test_lm_head_ling_vocab_sampled(moe):
    V, H = 157184, 2560
    rng = np.random.default_rng(20)
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    w_dev = (torch.randn((V, H), generator=g, device="cuda") * 0.02).to(torch.bfloat16).view(torch.int16)
    q = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(V, dtype=torch.float32, device="cuda")
    moe.moe_lm_head_quantize(w_dev, q, s)
    rows = np.unique(np.concatenate([[0, 1, V - 1], rng.integers(0, V, 400)]))
    w_rows = host(w_dev[torch.from_numpy(rows).cuda()]).view(np.uint16)
    rq, rs = oracle.lm_head_quant(w_rows)
    qh = host(q[torch.from_numpy(rows).cuda()])
    sh = host(s)[rows]
    assert np.array_equal(sh.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(qh, rq)
    for M in (1, 4):
        x = synth.normal_bf16(rng, (M, H), 1.0)
        logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
        moe.moe_lm_head_forward(dev(x), q, s, logits)
        torch.cuda.synchronize()
        _check_logits(host(logits)[:, rows], x, qh, sh)
