"""TEST INFRASTRUCTURE ONLY: Python access to the plain CPU oracle.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
must not: it is the independent reference the GPU path is checked against.

The arithmetic lives in ``moe_oracle.c`` (single-threaded, fp64 accumulation,
binary32 quantisation steps); this module only compiles it with ``gcc`` when
needed and marshals numpy arrays through ``ctypes``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

# Strict IEEE: no contraction into FMA, no fast-math; float division stays a
# single correctly rounded binary32 division.
GCC_CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-shared", "-fPIC", _SRC, "-o", _LIB, "-lm"]


def build(force: bool = False) -> str:
    """Compile the oracle library (gcc) and return its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int


def _declare(L: ctypes.CDLL) -> None:
    L.orc_e2m1_value.restype = ctypes.c_double
    L.orc_e2m1_value.argtypes = [ctypes.c_uint]
    L.orc_e8m0_value.restype = ctypes.c_double
    L.orc_e8m0_value.argtypes = [ctypes.c_uint]
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_e4m3_value.argtypes = [ctypes.c_uint]
    L.orc_bf16_value.restype = ctypes.c_double
    L.orc_bf16_value.argtypes = [ctypes.c_uint16]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3_encode_n.restype = None
    L.orc_e4m3_encode_n.argtypes = [ctypes.c_int64, _P, _P]
    L.orc_route.restype = None
    L.orc_route.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    L.orc_compact.restype = _I
    L.orc_compact.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P]
    L.orc_quant_act.restype = None
    L.orc_quant_act.argtypes = [_I, _I, _P, _P, _P]
    L.orc_gate_up.restype = None
    L.orc_gate_up.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    L.orc_requant.restype = None
    L.orc_requant.argtypes = [_I, _I, _P, _P, _P]
    L.orc_down_combine.restype = None
    L.orc_down_combine.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
    L.orc_time_layer.restype = None
    L.orc_time_layer.argtypes = [_I, _I, _I, _I, _I, _I] + [_P] * 17
    L.orc_lm_head_quant.restype = None
    L.orc_lm_head_quant.argtypes = [_I, _I, _P, _P, _P]
    L.orc_lm_head_gemv.restype = None
    L.orc_lm_head_gemv.argtypes = [_I, _I, _I, _P, _P, _P, _P]


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# scalar formats
# --------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(code)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(bits)


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(ctypes.c_float(y))


def e4m3_encode_array(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32).ravel()
    q = np.zeros(y.size, np.uint8)
    lib().orc_e4m3_encode_n(y.size, _ptr(y), _ptr(q))
    return q


# --------------------------------------------------------------------------
# layer stages
# --------------------------------------------------------------------------
@dataclass
class Route:
    logits: np.ndarray   # f64 [M,E]
    ids: np.ndarray      # i32 [M,K]
    w: np.ndarray        # f64 [M,K]
    gap: np.ndarray      # f64 [M]


def route(x: np.ndarray, wr: np.ndarray, K: int) -> Route:
    x = _c(x, np.uint16)
    wr = _c(wr, np.uint16)
    M, H = x.shape
    E = wr.shape[0]
    assert wr.shape == (E, H) and 1 <= K <= E
    r = Route(np.zeros((M, E)), np.zeros((M, K), np.int32), np.zeros((M, K)), np.zeros(M))
    lib().orc_route(M, H, E, K, _ptr(x), _ptr(wr), _ptr(r.logits), _ptr(r.ids), _ptr(r.w), _ptr(r.gap))
    return r


@dataclass
class Compaction:
    n_act: int
    act_experts: np.ndarray  # i32 [n_act]
    offsets: np.ndarray      # i32 [n_act+1]
    pair_token: np.ndarray   # i32 [M*K]
    pair_src: np.ndarray     # i32 [M*K]
    pair_of: np.ndarray      # i32 [M*K]


def compact(ids: np.ndarray, E: int) -> Compaction:
    ids = _c(ids, np.int32)
    M, K = ids.shape
    P = M * K
    act = np.zeros(min(E, P), np.int32)
    off = np.zeros(min(E, P) + 1, np.int32)
    pt = np.zeros(P, np.int32)
    ps = np.zeros(P, np.int32)
    po = np.zeros(P, np.int32)
    n = lib().orc_compact(M, K, E, _ptr(ids), _ptr(act), _ptr(off), _ptr(pt), _ptr(ps), _ptr(po))
    return Compaction(n, act[:n].copy(), off[:n + 1].copy(), pt, ps, po)


def quant_act(x: np.ndarray):
    x = _c(x, np.uint16)
    M, H = x.shape
    q = np.zeros((M, H), np.uint8)
    s = np.zeros(M, np.float32)
    lib().orc_quant_act(M, H, _ptr(x), _ptr(q), _ptr(s))
    return q, s


def gate_up(q, s, ids, w13, s13, I: int) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    ids = _c(ids, np.int32)
    w13 = _c(w13, np.uint8)
    s13 = _c(s13, np.uint8)
    M, H = q.shape
    K = ids.shape[1]
    assert w13.shape[1:] == (2 * I, H // 2) and s13.shape[1:] == (2 * I, H // 32)
    h = np.zeros((M * K, I))
    lib().orc_gate_up(M, H, I, K, _ptr(q), _ptr(s), _ptr(ids), _ptr(w13), _ptr(s13), _ptr(h))
    return h


def requant(h: np.ndarray):
    h = _c(h, np.float64)
    P, I = h.shape
    q2 = np.zeros((P, I), np.uint8)
    s2 = np.zeros(P, np.float32)
    lib().orc_requant(P, I, _ptr(h), _ptr(q2), _ptr(s2))
    return q2, s2


def down_combine(q2, s2, ids, w, w2, sc2, H: int) -> np.ndarray:
    q2 = _c(q2, np.uint8)
    s2 = _c(s2, np.float32)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    w2 = _c(w2, np.uint8)
    sc2 = _c(sc2, np.uint8)
    M, K = ids.shape
    I = q2.shape[1]
    assert w2.shape[1:] == (H, I // 2) and sc2.shape[1:] == (H, I // 32)
    out = np.zeros((M, H))
    lib().orc_down_combine(M, H, I, K, _ptr(q2), _ptr(s2), _ptr(ids), _ptr(w), _ptr(w2), _ptr(sc2), _ptr(out))
    return out


@dataclass
class LayerTaps:
    route: Route
    q: np.ndarray
    s: np.ndarray
    h: np.ndarray
    q2: np.ndarray
    s2: np.ndarray
    out: np.ndarray

    @property
    def flags(self) -> np.ndarray:
        """Tokens whose rank-K / rank-(K+1) logit gap is below 1e-4."""
        return self.route.gap < 1e-4


@dataclass
class SharedExpert:
    """One dense MXFP4 expert applied to every token: w13 [2I,H/2], s13 [2I,H/32],
    w2 [H,I/2], s2 [H,I/32] (one expert of the routed layout)."""
    w13: np.ndarray
    s13: np.ndarray
    w2: np.ndarray
    s2: np.ndarray


def moe_layer(x, wr, w13, s13, w2, sc2, K: int, shared: SharedExpert | None = None) -> LayerTaps:
    """The whole layer, stage by stage, returning every tap.

    With a shared expert ([EN] "What is Ling 3.0, and why does it suit DGX
    Spark?": one shared expert per MoE layer beside the 8 routed ones) every
    token also goes through that expert with weight 1, by the same W4A8 steps
    (the token's FP8 activations, gate/up + SiLU, its own per-row FP8
    requantisation, down), and the result is added to the routed sum.  Its rows
    of h, q2 and s2 follow the M*K routed pairs (row M*K + t for token t)."""
    x = _c(x, np.uint16)
    M, H = x.shape
    I = w2.shape[2] * 2
    r = route(x, wr, K)
    q, s = quant_act(x)
    h = gate_up(q, s, r.ids, w13, s13, I)
    q2, s2 = requant(h)
    out = down_combine(q2, s2, r.ids, r.w, w2, sc2, H)
    if shared is not None:
        zero = np.zeros((M, 1), np.int32)
        hs = gate_up(q, s, zero, shared.w13[None], shared.s13[None], I)
        q2s, s2s = requant(hs)
        out = out + down_combine(q2s, s2s, zero, np.ones((M, 1)), shared.w2[None], shared.s2[None], H)
        h, q2, s2 = np.vstack([h, hs]), np.vstack([q2, q2s]), np.concatenate([s2, s2s])
    return LayerTaps(r, q, s, h, q2, s2, out)


def time_layer(x, wr, w13, s13, w2, sc2, K: int, runs: int = 3) -> np.ndarray:
    """Wall time (seconds) of each of `runs` calls of the oracle's whole layer on
    the same inputs, clocked inside the oracle library around the call only
    (the CPU baseline; every buffer is made before the first run)."""
    x = _c(x, np.uint16)
    wr = _c(wr, np.uint16)
    w13, s13, w2, sc2 = (_c(a, np.uint8) for a in (w13, s13, w2, sc2))
    M, H = x.shape
    E = wr.shape[0]
    I = w2.shape[2] * 2
    bufs = [np.zeros((M, E)), np.zeros((M, K), np.int32), np.zeros((M, K)), np.zeros(M),
            np.zeros((M, H), np.uint8), np.zeros(M, np.float32), np.zeros((M * K, I)),
            np.zeros((M * K, I), np.uint8), np.zeros(M * K, np.float32), np.zeros((M, H))]
    sec = np.zeros(runs)
    lib().orc_time_layer(runs, M, H, I, E, K, _ptr(x), _ptr(wr), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(sc2),
                         *[_ptr(b) for b in bufs], _ptr(sec))
    return sec


def lm_head_quant(w: np.ndarray):
    """Load-time FP8 quantisation of a bf16 LM head [V,H]: codes [V,H] and one
    binary32 scale per row (the activation scheme applied to weight rows)."""
    w = _c(w, np.uint16)
    V, H = w.shape
    q = np.zeros((V, H), np.uint8)
    s = np.zeros(V, np.float32)
    lib().orc_lm_head_quant(V, H, _ptr(w), _ptr(q), _ptr(s))
    return q, s


def lm_head_gemv(x: np.ndarray, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """logits [M,V] = s_v * sum_k E4M3(q[v,k]) * x[t,k], in double."""
    x = _c(x, np.uint16)
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    M, H = x.shape
    V = q.shape[0]
    out = np.zeros((M, V), np.float64)
    lib().orc_lm_head_gemv(M, V, H, _ptr(x), _ptr(q), _ptr(s), _ptr(out))
    return out

