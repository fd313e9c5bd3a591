"""ctypes binding of libmoe_decode.so (the C ABI in include/moe_decode.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  Tensors are passed as device pointers (``tensor.data_ptr()``),
streams as ``hipStream_t`` handles (default: torch's current stream).  Importing
this module fails loudly if the library has not been built; there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_decode.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe_decode.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; build it with `python -m mxfp4_weight_streaming_amd.build` "
        "(hipcc, gfx950). The MoE layer has no non-HIP implementation.")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED_SHAPE = -2
MOE_ERR_ALIGNMENT = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_JIT = -6


class MoeShape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("topk", ctypes.c_int32)]

    def __repr__(self):
        return f"MoeShape(H={self.hidden}, I={self.inter}, E={self.num_experts}, K={self.topk})"


class MoeRouteTaps(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("n_active", ctypes.c_void_p), ("act_experts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("pair_token", ctypes.c_void_p), ("pair_src", ctypes.c_void_p),
                ("act_fp8", ctypes.c_void_p), ("act_scale", ctypes.c_void_p)]


class MoeExpertTaps(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("inter_fp8", ctypes.c_void_p), ("inter_scale", ctypes.c_void_p)]


class MoeSharedExpert(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p)]


class MoeJitReport(ctypes.Structure):
    _fields_ = [("from_cache", ctypes.c_int32), ("has_chunk_path", ctypes.c_int32), ("has_lm_head", ctypes.c_int32),
                ("num_kernels", ctypes.c_int32), ("seconds", ctypes.c_double), ("cache_file", ctypes.c_char * 1024)]

    def as_dict(self) -> dict:
        return {"from_cache": bool(self.from_cache), "has_chunk_path": bool(self.has_chunk_path),
                "has_lm_head": bool(self.has_lm_head), "num_kernels": self.num_kernels, "seconds": self.seconds,
                "cache_file": self.cache_file.decode()}


_V = ctypes.c_void_p
_S = ctypes.POINTER(MoeShape)
_SH = ctypes.POINTER(MoeSharedExpert)
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

_SIGNATURES = {
    "moe_workspace_bytes": (_sz, [_S, _i32]),
    "moe_workspace_init": (ctypes.c_int, [_V, _sz, _V]),
    "moe_decode_forward": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, _V, _V, _V, _V, _sz, _V]),
    "moe_decode_forward_events": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, _V, _V, _V, _V, _sz, _V,
                                                  ctypes.POINTER(ctypes.c_void_p)]),
    "moe_decode_forward_shared": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, _V, _V, _SH, _V, _V, _sz, _V,
                                                  ctypes.POINTER(ctypes.c_void_p)]),
    "moe_decode_forward_noalloc": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, _V, _V, _V, _V]),
    "moe_route": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, ctypes.POINTER(MoeRouteTaps), _V, _sz, _V]),
    "moe_quant_act": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V]),
    "moe_experts_forward": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, _V, _V, _V, _V, _V,
                                           ctypes.POINTER(MoeExpertTaps), _V, _sz, _V]),
    "moe_experts_forward_shared": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, _V, _V, _V, _V, _SH, _V,
                                                  ctypes.POINTER(MoeExpertTaps), _V, _sz, _V]),
    "moe_gate_up": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, _V, _V, _V, _V, _V, _sz, _V]),
    "moe_down_combine": (ctypes.c_int, [_S, _i32, _V, _V, _V, _V, _V, _V, _V, _V, _sz, _V]),
    "moe_fp8_encode_range": (ctypes.c_int, [ctypes.c_uint32, ctypes.c_int64, _V, _V]),
    "moe_lm_head_quantize": (ctypes.c_int, [_V, _i32, _i32, _V, _V, _V]),
    "moe_lm_head_forward": (ctypes.c_int, [_V, _i32, _V, _V, _i32, _i32, _V, _V]),
    "moe_path_info": (ctypes.c_int, [_S, _i32, ctypes.c_char_p, _sz]),
    "moe_jit_build": (ctypes.c_int, [_S, ctypes.c_char_p, ctypes.c_char_p, ctypes.POINTER(MoeJitReport)]),
    "moe_jit_load": (ctypes.c_int, [_S, ctypes.c_char_p, _i32, ctypes.POINTER(MoeJitReport)]),
    "moe_jit_unload": (_i32, [_S]),
    "moe_workspace_sync_status": (ctypes.c_int, [_V, _sz, _V, _V]),
    "moe_set_wait_limit_us": (None, [ctypes.c_uint32]),
    "moe_set_decode_path": (ctypes.c_int, [_i32]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def header_functions() -> list[str]:
    """Names of the functions declared in include/moe_decode.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(moe_\w+)\s*\(", text, re.M)))


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.moe_last_error().decode()
        super().__init__(f"{where}: {_lib.moe_status_string(status).decode()} ({status}): {msg}")


def _check(status: int, where: str) -> int:
    if status != MOE_OK:
        raise MoeError(status, where)
    return status


def _p(t):
    """Device pointer of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def shape(hidden: int, inter: int, num_experts: int, topk: int) -> MoeShape:
    return MoeShape(hidden, inter, num_experts, topk)


def moe_workspace_bytes(shp: MoeShape, max_tokens: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(shp), max_tokens)


def moe_workspace_init(ws, stream=None) -> None:
    _check(_lib.moe_workspace_init(_p(ws), _nbytes(ws), _stream(stream)), "moe_workspace_init")


def workspace(shp: MoeShape, max_tokens: int, device="cuda"):
    """Allocate (through torch) and initialise a workspace for up to max_tokens."""
    import torch
    n = moe_workspace_bytes(shp, max_tokens)
    if n == 0:
        raise MoeError(MOE_ERR_UNSUPPORTED_SHAPE, "moe_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    moe_workspace_init(ws)
    torch.cuda.current_stream().synchronize()   # usable from any stream afterwards
    return ws


def moe_decode_forward(shp, M, hidden, router_w, w13, w13_scale, w2, w2_scale, out, ws, stream=None):
    _check(_lib.moe_decode_forward(ctypes.byref(shp), M, _p(hidden), _p(router_w), _p(w13), _p(w13_scale),
                                   _p(w2), _p(w2_scale), _p(out), _p(ws), _nbytes(ws), _stream(stream)),
           "moe_decode_forward")


def moe_decode_forward_noalloc(shp, M, hidden, router_w, w13, w13_scale, w2, w2_scale, out, stream=None):
    """moe_decode_forward on the library's static scratch (no workspace)."""
    _check(_lib.moe_decode_forward_noalloc(ctypes.byref(shp), M, _p(hidden), _p(router_w), _p(w13), _p(w13_scale),
                                           _p(w2), _p(w2_scale), _p(out), _stream(stream)),
           "moe_decode_forward_noalloc")


def moe_decode_forward_events(shp, M, hidden, router_w, w13, w13_scale, w2, w2_scale, out, ws, events,
                              stream=None):
    """events: 6 torch.cuda.Event (timing enabled, each recorded once so that it
    exists), start/stop pairs stamped by the router, gate/up and down launches."""
    if len(events) != 6:
        raise ValueError("moe_decode_forward_events takes 6 events (start/stop of 3 kernels)")
    arr = (ctypes.c_void_p * 6)(*[None if e is None else e.cuda_event for e in events])
    _check(_lib.moe_decode_forward_events(ctypes.byref(shp), M, _p(hidden), _p(router_w), _p(w13), _p(w13_scale),
                                          _p(w2), _p(w2_scale), _p(out), _p(ws), _nbytes(ws), _stream(stream),
                                          arr),
           "moe_decode_forward_events")


def _shared(shared):
    """A MoeSharedExpert from (w13, w13_scale, w2, w2_scale) tensors, or None."""
    if shared is None:
        return None
    if len(shared) != 4:
        raise ValueError("a shared expert is (w13, w13_scale, w2, w2_scale)")
    return MoeSharedExpert(*[_p(t) for t in shared])


def _events(events):
    if events is None:
        return None
    if len(events) != 6:
        raise ValueError("events: 6 torch.cuda.Event (start/stop of 3 kernels)")
    return (ctypes.c_void_p * 6)(*[None if e is None else e.cuda_event for e in events])


def moe_decode_forward_shared(shp, M, hidden, router_w, w13, w13_scale, w2, w2_scale, shared, out, ws,
                              events=None, stream=None):
    """moe_decode_forward plus the shared expert; shared = (w13, w13_scale, w2,
    w2_scale) of one expert, or None.  events as in moe_decode_forward_events."""
    sh = _shared(shared)
    _check(_lib.moe_decode_forward_shared(ctypes.byref(shp), M, _p(hidden), _p(router_w), _p(w13), _p(w13_scale),
                                          _p(w2), _p(w2_scale), ctypes.byref(sh) if sh is not None else None,
                                          _p(out), _p(ws), _nbytes(ws), _stream(stream), _events(events)),
           "moe_decode_forward_shared")


def moe_route(shp, M, hidden, router_w, topk_ids, topk_w, ws, taps: dict | None = None, stream=None):
    t = None
    if taps is not None:
        t = MoeRouteTaps(*[_p(taps.get(k)) for k, _ in MoeRouteTaps._fields_])
    _check(_lib.moe_route(ctypes.byref(shp), M, _p(hidden), _p(router_w), _p(topk_ids), _p(topk_w),
                          ctypes.byref(t) if t is not None else None, _p(ws), _nbytes(ws), _stream(stream)),
           "moe_route")


def moe_quant_act(shp, M, hidden, act_fp8, act_scale, stream=None):
    _check(_lib.moe_quant_act(ctypes.byref(shp), M, _p(hidden), _p(act_fp8), _p(act_scale), _stream(stream)),
           "moe_quant_act")


def moe_experts_forward(shp, M, act_fp8, act_scale, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, out, ws,
                        taps: dict | None = None, stream=None):
    t = None
    if taps is not None:
        t = MoeExpertTaps(*[_p(taps.get(k)) for k, _ in MoeExpertTaps._fields_])
    _check(_lib.moe_experts_forward(ctypes.byref(shp), M, _p(act_fp8), _p(act_scale), _p(topk_ids), _p(topk_w),
                                    _p(w13), _p(w13_scale), _p(w2), _p(w2_scale), _p(out),
                                    ctypes.byref(t) if t is not None else None, _p(ws), _nbytes(ws),
                                    _stream(stream)),
           "moe_experts_forward")


def moe_experts_forward_shared(shp, M, act_fp8, act_scale, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, shared,
                               out, ws, taps: dict | None = None, stream=None):
    """moe_experts_forward plus the shared expert; taps then hold M*K + M rows."""
    t = None
    if taps is not None:
        t = MoeExpertTaps(*[_p(taps.get(k)) for k, _ in MoeExpertTaps._fields_])
    sh = _shared(shared)
    _check(_lib.moe_experts_forward_shared(ctypes.byref(shp), M, _p(act_fp8), _p(act_scale), _p(topk_ids),
                                           _p(topk_w), _p(w13), _p(w13_scale), _p(w2), _p(w2_scale),
                                           ctypes.byref(sh) if sh is not None else None, _p(out),
                                           ctypes.byref(t) if t is not None else None, _p(ws), _nbytes(ws),
                                           _stream(stream)),
           "moe_experts_forward_shared")


def moe_gate_up(shp, M, act_fp8, act_scale, topk_ids, w13, w13_scale, h, inter_fp8, inter_scale, ws, stream=None):
    _check(_lib.moe_gate_up(ctypes.byref(shp), M, _p(act_fp8), _p(act_scale), _p(topk_ids), _p(w13),
                            _p(w13_scale), _p(h), _p(inter_fp8), _p(inter_scale), _p(ws), _nbytes(ws),
                            _stream(stream)),
           "moe_gate_up")


def moe_down_combine(shp, M, inter_fp8, inter_scale, topk_ids, topk_w, w2, w2_scale, out, ws, stream=None):
    _check(_lib.moe_down_combine(ctypes.byref(shp), M, _p(inter_fp8), _p(inter_scale), _p(topk_ids), _p(topk_w),
                                 _p(w2), _p(w2_scale), _p(out), _p(ws), _nbytes(ws), _stream(stream)),
           "moe_down_combine")


def moe_fp8_encode_range(first_bits: int, n: int, q, stream=None):
    _check(_lib.moe_fp8_encode_range(first_bits & 0xFFFFFFFF, n, _p(q), _stream(stream)), "moe_fp8_encode_range")


def moe_lm_head_quantize(w_bf16, q, scale, stream=None):
    """w_bf16 [V,H] -> q [V,H] E4M3 codes and scale [V] (one fp32 scale per row)."""
    V, H = w_bf16.shape
    _check(_lib.moe_lm_head_quantize(_p(w_bf16), V, H, _p(q), _p(scale), _stream(stream)), "moe_lm_head_quantize")


def moe_lm_head_forward(x_bf16, q, scale, logits, stream=None):
    """logits [M,V] = scale[v] * sum_k E4M3(q[v,k]) * x[t,k]."""
    M, H = x_bf16.shape
    V = q.shape[0]
    _check(_lib.moe_lm_head_forward(_p(x_bf16), M, _p(q), _p(scale), V, H, _p(logits), _stream(stream)),
           "moe_lm_head_forward")


def _path_arg(p):
    return None if p is None else os.fsencode(p)


def moe_jit_build(shp: MoeShape, arch: str = "gfx950", cache_dir=None) -> dict:
    """Compile the kernels of (H, I) for `arch` into the cache (no GPU needed)."""
    r = MoeJitReport()
    _check(_lib.moe_jit_build(ctypes.byref(shp), arch.encode(), _path_arg(cache_dir), ctypes.byref(r)),
           "moe_jit_build")
    return r.as_dict()


def moe_jit_load(shp: MoeShape, cache_dir=None, prefer: bool = False) -> dict:
    """Compile or find (H, I) in the cache and load it on the current device."""
    r = MoeJitReport()
    _check(_lib.moe_jit_load(ctypes.byref(shp), _path_arg(cache_dir), 1 if prefer else 0, ctypes.byref(r)),
           "moe_jit_load")
    return r.as_dict()


def moe_jit_unload(shp: MoeShape) -> int:
    return _lib.moe_jit_unload(ctypes.byref(shp))


def moe_path_info(shp: MoeShape, M: int) -> tuple[int, str]:
    buf = ctypes.create_string_buffer(1024)
    st = _lib.moe_path_info(ctypes.byref(shp), M, buf, len(buf))
    return st, buf.value.decode()


def moe_workspace_sync_status(ws, status, stream=None) -> None:
    """Copy the workspace's sticky wait-error bits into `status` (a device
    int32/uint32 tensor of one element)."""
    _check(_lib.moe_workspace_sync_status(_p(ws), _nbytes(ws), _p(status), _stream(stream)),
           "moe_workspace_sync_status")


def sync_errors(ws) -> int:
    """The workspace's wait-error bits, read back (synchronises the current stream)."""
    import torch
    st = torch.zeros(1, dtype=torch.int32, device=ws.device)
    moe_workspace_sync_status(ws, st)
    return int(st.item())


def moe_set_wait_limit_us(us: int) -> None:
    _lib.moe_set_wait_limit_us(us)


PATH_THREE_KERNELS = 0
PATH_ONE_KERNEL = 1


def moe_set_decode_path(path: int) -> None:
    """Select how M <= 8 runs for later calls: PATH_THREE_KERNELS (default) or
    PATH_ONE_KERNEL (layer_kernel)."""
    _check(_lib.moe_set_decode_path(path), "moe_set_decode_path")


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def raw():
    """The underlying ctypes library (for argument-validation tests)."""
    return _lib
