"""Helpers shared by the GPU tests: device upload of the synthetic inputs and
the comparison metrics.  No layer arithmetic lives here."""
from __future__ import annotations

import numpy as np
import torch

from mxfp4_weight_streaming_amd import synth

DEV = "cuda"


def dev(a: np.ndarray) -> torch.Tensor:
    """Copy a numpy array to the GPU, keeping its bytes (uint16 goes as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


class DevWeights:
    def __init__(self, w: synth.Weights):
        self.H, self.I, self.E = w.H, w.I, w.E
        self.wr = dev(w.wr)
        self.w13 = dev(w.w13)
        self.s13 = dev(w.s13)
        self.w2 = dev(w.w2)
        self.s2 = dev(w.s2)

    def with_router(self, wr: np.ndarray) -> "DevWeights":
        c = object.__new__(DevWeights)
        c.__dict__.update(self.__dict__)
        c.wr = dev(wr)
        return c


def rel_l2(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.linalg.norm(gpu) == 0.0 else np.inf
    return float(np.linalg.norm(gpu - ref) / nr)


def e4m3_values() -> np.ndarray:
    """Decoded values of all 256 E4M3 codes (torch's float8_e4m3fn decode)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def fp8_code_mismatches_ok(gpu_q: np.ndarray, ref_q: np.ndarray, ref_y: np.ndarray, rel: float = 1e-5):
    """Every differing code must be an adjacent code (+-1 in magnitude, same
    sign) and the reference's pre-quantisation value must sit within `rel`
    (relative) of the midpoint between the two codes' values.  Returns
    (n_mismatch, list of offending indices)."""
    vals = e4m3_values()
    bad = []
    idx = np.nonzero(gpu_q != ref_q)
    for i in zip(*idx):
        g, r = int(gpu_q[i]), int(ref_q[i])
        if vals[g] == vals[r]:          # +0 and -0
            continue
        same_sign = (g & 0x80) == (r & 0x80)
        adjacent = abs((g & 0x7F) - (r & 0x7F)) == 1
        mid = 0.5 * (vals[g] + vals[r])
        y = float(ref_y[i])
        near = abs(y - mid) <= rel * max(abs(mid), 2.0 ** -9)
        if not (same_sign and adjacent and near):
            bad.append(i)
    return len(idx[0]), bad


def requant_codes_match(q2, s2, h, rel: float = 1e-6):
    """The kernel's FP8 intermediate (q2, s2) against the oracle's
    requantisation of the kernel's own h: scales bit-exact; codes equal except
    where h / s2 lies within `rel` of a rounding midpoint (the kernels
    multiply by the correctly rounded reciprocal of s2 where the oracle
    divides).  Returns the number of differing codes."""
    import oracle
    q2_own, s2_own = oracle.requant(h)
    assert np.array_equal(np.asarray(s2, np.float32).view(np.uint32), s2_own.view(np.uint32))
    y = (np.asarray(h, np.float32) / s2_own[:, None]).astype(np.float32)
    n_mis, bad = fp8_code_mismatches_ok(q2, q2_own, y, rel=rel)
    assert not bad, (n_mis, bad[:5])
    return n_mis

