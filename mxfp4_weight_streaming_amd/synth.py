"""Seeded synthetic inputs for the MoE decode layer.

This module holds no arithmetic of the layer itself: it only draws random
numbers and rounds them to the storage formats (bf16 by round-to-nearest-even,
uniform MXFP4 codes, uniform E8M0 scale codes).  The same arrays feed both the
GPU path and the CPU oracle.

Shapes and distributions follow the workloads the library is measured on:

* tiny      -- hidden 256, expert intermediate 64, 16 experts, top-2, 1 token;
* ling      -- hidden 2560, expert intermediate 768 (the Ling-3.0-flash expert
               shape), 256 experts, top-8, 1 token (plain decode);
* verify    -- the same shapes with 4 tokens (the MTP verify window) and a
               router biased so that the 4 tokens pick 32 distinct experts, or
               share 4 experts and pick 20 distinct;
* chunk     -- the same shapes with 512 tokens and a router biased so that
               expert popularity falls off as rank^-1.1 (Zipf);
* stack     -- 40 independent ling layers (about 30 GiB of MXFP4 weights), drawn
               directly on the GPU with torch's generator so that they never
               exist on the host.

Hidden values are N(0,1), router weights N(0, 0.02), every MXFP4 code is
uniform over all 16 values (two uniform nibbles per byte, -0 included) and
every E8M0 scale code is uniform over 119..123 (block scales 2^-8 .. 2^-4).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SCALE_LO, SCALE_HI = 119, 123          # E8M0 codes for 2^-8 .. 2^-4


def bf16_from_f32(a) -> np.ndarray:
    """Round binary32 values to bf16 bit patterns (round to nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to binary32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return bf16_from_f32((rng.standard_normal(shape) * std).astype(np.float32))


def mxfp4_codes(rng: np.random.Generator, E: int, N: int, K: int) -> np.ndarray:
    """Uniform random packed E2M1 codes, [E, N, K/2] bytes."""
    n = E * N * (K // 2)
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(E, N, K // 2).copy()


def e8m0_scales(rng: np.random.Generator, E: int, N: int, K: int) -> np.ndarray:
    """Uniform E8M0 codes in [119, 123], [E, N, K/32] bytes."""
    return rng.integers(SCALE_LO, SCALE_HI + 1, size=(E, N, K // 32), dtype=np.uint8)


@dataclass
class Weights:
    """One layer's router and expert weights, in the library's storage layout."""
    H: int
    I: int
    E: int
    wr: np.ndarray        # bf16 bits [E, H]
    w13: np.ndarray       # u8 [E, 2I, H/2]
    s13: np.ndarray       # u8 [E, 2I, H/32]
    w2: np.ndarray        # u8 [E, H, I/2]
    s2: np.ndarray        # u8 [E, H, I/32]


@dataclass
class LayerInputs:
    x: np.ndarray         # bf16 bits [M, H]
    wts: Weights
    K: int
    note: dict = field(default_factory=dict)

    @property
    def M(self) -> int:
        return self.x.shape[0]


def expert_weights(seed: int, H: int, I: int, E: int) -> Weights:
    """Expert tensors (w13, w2 and their scales) plus an unbiased router."""
    rng = np.random.default_rng(seed)
    wr = normal_bf16(rng, (E, H), 0.02)
    w13 = mxfp4_codes(rng, E, 2 * I, H)
    s13 = e8m0_scales(rng, E, 2 * I, H)
    w2 = mxfp4_codes(rng, E, H, I)
    s2 = e8m0_scales(rng, E, H, I)
    return Weights(H, I, E, wr, w13, s13, w2, s2)


def shared_expert(seed: int, H: int, I: int):
    """One shared expert drawn like a routed one: (w13 [2I,H/2], s13 [2I,H/32],
    w2 [H,I/2], s2 [H,I/32])."""
    rng = np.random.default_rng(seed)
    return (mxfp4_codes(rng, 1, 2 * I, H)[0], e8m0_scales(rng, 1, 2 * I, H)[0],
            mxfp4_codes(rng, 1, H, I)[0], e8m0_scales(rng, 1, H, I)[0])


def with_router(w: Weights, wr: np.ndarray) -> Weights:
    return Weights(w.H, w.I, w.E, np.ascontiguousarray(wr, np.uint16), w.w13, w.s13, w.w2, w.s2)


def tiny(seed: int) -> LayerInputs:
    """Hidden 256, intermediate 64, 16 experts, top-2, 1 token."""
    w = expert_weights(seed, 256, 64, 16)
    rng = np.random.default_rng(seed + 7_000_000)
    return LayerInputs(normal_bf16(rng, (1, 256), 1.0), w, 2)


def decode_tokens(seed: int, wts: Weights, M: int, K: int = 8) -> LayerInputs:
    """M tokens of N(0,1) hidden state with the weights' own (unbiased) router."""
    rng = np.random.default_rng(seed)
    return LayerInputs(normal_bf16(rng, (M, wts.H), 1.0), wts, K)


def verify_router(seed: int, wts: Weights, distinct: int, M: int = 4, K: int = 8,
                  bias: float = 0.2) -> LayerInputs:
    """MTP verify window: M=4 tokens whose router is biased toward chosen experts.

    distinct == 32: every token gets K experts of its own (Wr[e] += bias * u_t).
    distinct == 20: 4 experts are shared by all tokens (Wr[e] += bias * sum_t u_t)
    and every token gets K-4 of its own.  u_t is the unit vector of token t.
    """
    assert distinct in (M * K, 4 + M * (K - 4))
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (M, wts.H), 1.0)
    wr = rng.standard_normal((wts.E, wts.H)) * 0.02
    xf = bf16_to_f32(x).astype(np.float64)
    u = xf / np.linalg.norm(xf, axis=1, keepdims=True)
    perm = rng.permutation(wts.E)
    if distinct == M * K:
        for t in range(M):
            wr[perm[K * t:K * (t + 1)]] += bias * u[t]
    else:
        wr[perm[:4]] += bias * u.sum(axis=0)
        own = K - 4
        for t in range(M):
            wr[perm[4 + own * t:4 + own * (t + 1)]] += bias * u[t]
    return LayerInputs(x, with_router(wts, bf16_from_f32(wr.astype(np.float32))), K,
                       {"distinct": distinct})


def zipf_router(seed: int, wts: Weights, M: int = 512, K: int = 8, tau: float = 0.5,
                exponent: float = 1.1) -> LayerInputs:
    """Chunk of M tokens whose expert popularity falls off with rank.

    Channel 0 of every token is a constant 1.0 (a bias channel) and the router's
    channel-0 weight of the expert with popularity rank r is tau * (-exponent * ln r).
    """
    rng = np.random.default_rng(seed)
    xf = (rng.standard_normal((M, wts.H))).astype(np.float32)
    xf[:, 0] = 1.0
    wr = (rng.standard_normal((wts.E, wts.H)) * 0.02).astype(np.float32)
    ranks = rng.permutation(wts.E) + 1
    wr[:, 0] = tau * (-exponent * np.log(ranks.astype(np.float64)))
    return LayerInputs(bf16_from_f32(xf), with_router(wts, bf16_from_f32(wr)), K,
                       {"tau": tau, "exponent": exponent, "ranks": ranks})


# --------------------------------------------------------------------------
# device-side stacks (torch is used only as a random-number source and for
# device memory; nothing here is layer arithmetic)
# --------------------------------------------------------------------------
def device_stack(n_layers: int, H: int, I: int, E: int, seed: int, device="cuda"):
    """A list of n_layers dicts of device tensors: wr, w13, s13, w2, s2."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    layers = []
    for _ in range(n_layers):
        wr = (torch.randn((E, H), generator=g, device=device) * 0.02).to(torch.bfloat16).view(torch.uint16)
        w13 = torch.randint(0, 256, (E, 2 * I, H // 2), generator=g, device=device, dtype=torch.uint8)
        s13 = torch.randint(SCALE_LO, SCALE_HI + 1, (E, 2 * I, H // 32), generator=g, device=device,
                            dtype=torch.uint8)
        w2 = torch.randint(0, 256, (E, H, I // 2), generator=g, device=device, dtype=torch.uint8)
        s2 = torch.randint(SCALE_LO, SCALE_HI + 1, (E, H, I // 32), generator=g, device=device,
                           dtype=torch.uint8)
        layers.append({"wr": wr, "w13": w13, "s13": s13, "w2": w2, "s2": s2})
    return layers


def device_shared(n_layers: int, H: int, I: int, seed: int, device="cuda"):
    """n_layers shared experts on the device: tuples (w13, s13, w2, s2) drawn
    like one routed expert each."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(n_layers):
        w13 = torch.randint(0, 256, (2 * I, H // 2), generator=g, device=device, dtype=torch.uint8)
        s13 = torch.randint(SCALE_LO, SCALE_HI + 1, (2 * I, H // 32), generator=g, device=device, dtype=torch.uint8)
        w2 = torch.randint(0, 256, (H, I // 2), generator=g, device=device, dtype=torch.uint8)
        s2 = torch.randint(SCALE_LO, SCALE_HI + 1, (H, I // 32), generator=g, device=device, dtype=torch.uint8)
        out.append((w13, s13, w2, s2))
    return out


def device_hidden(n: int, M: int, H: int, seed: int, device="cuda"):
    """n independent [M, H] bf16 hidden batches (as uint16 bit views)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return [torch.randn((M, H), generator=g, device=device).to(torch.bfloat16).view(torch.uint16)
            for _ in range(n)]


def device_verify_router(wr_bits, x_bits, distinct: int, gen, K: int = 8, bias: float = 0.2):
    """The verify-window router construction of verify_router, on the device:
    a copy of the bf16 router wr_bits [E,H] with Wr[e] += bias * u_t for the
    experts each token t of x_bits [M,H] is meant to pick (u_t = x_t/|x_t|,
    in float64), the experts taken from a seeded permutation (generator gen).
    distinct == M*K: every token gets K experts of its own; otherwise 4
    experts are shared by all tokens (bias * sum_t u_t) and every token gets
    K - 4 of its own.  Rounded back to bf16 through binary32 as verify_router."""
    import torch
    M = x_bits.shape[0]
    E = wr_bits.shape[0]
    assert distinct in (M * K, 4 + M * (K - 4))
    wr = wr_bits.view(torch.bfloat16).double()
    x = x_bits.view(torch.bfloat16).double()
    u = x / x.norm(dim=1, keepdim=True)
    perm = torch.randperm(E, generator=gen, device=wr.device)
    if distinct == M * K:
        for t in range(M):
            wr[perm[K * t:K * (t + 1)]] += bias * u[t]
    else:
        wr[perm[:4]] += bias * u.sum(dim=0)
        own = K - 4
        for t in range(M):
            wr[perm[4 + own * t:4 + own * (t + 1)]] += bias * u[t]
    return wr.float().to(torch.bfloat16).view(torch.uint16).contiguous()
