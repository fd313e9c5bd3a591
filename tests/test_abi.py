"""CPU-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
enqueuing anything (no GPU is touched by these calls)."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mxfp4_weight_streaming_amd", "libmoe_decode.so")


@pytest.fixture(scope="module")
def moe():
    if not os.path.exists(LIB):
        from mxfp4_weight_streaming_amd import build
        build.build()
    from mxfp4_weight_streaming_amd import binding
    return binding


def test_every_declared_function_is_exported(moe):
    names = moe.header_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(moe.raw(), n), n


def test_binding_covers_the_header(moe):
    assert set(moe.header_functions()) == set(moe._SIGNATURES)


def _shape(moe, H=2560, I=768, E=256, K=8):
    return moe.shape(H, I, E, K)


def test_workspace_bytes(moe):
    s = _shape(moe)
    sizes = [moe.moe_workspace_bytes(s, m) for m in list(range(1, 10)) + [512, 2048]]
    assert all(b > 0 for b in sizes)
    assert sizes == sorted(sizes)      # a workspace sized for M serves every smaller M
    # h [M*K, I] fp32 alone is 8*768*4 bytes at M=1
    assert sizes[0] >= 8 * 768 * 4
    # the chunk path also keeps the weighted expert outputs y [M*K, H] fp32
    assert sizes[-1] >= 2048 * 8 * 2560 * 4
    assert moe.moe_workspace_bytes(s, 0) == 0
    assert moe.moe_workspace_bytes(s, 2049) == 0
    assert moe.moe_workspace_bytes(_shape(moe, H=512, I=128), 1) == 0
    assert moe.moe_workspace_bytes(_shape(moe, 256, 64, 16, 2), 1) > 0


@pytest.mark.parametrize("shape,M,status", [
    ((2560, 768, 256, 8), 0, -1),          # M must be positive
    ((2560, 768, 256, 8), 2049, -2),       # chunk path compiled up to 2048 tokens
    ((2560, 768, 200, 8), 9, -2),          # chunk path needs E % 16 == 0
    ((2560, 768, 4, 8), 1, -1),            # K > E
    ((2560, 768, 256, 9), 1, -2),          # K above 8
    ((2560, 768, 1024, 8), 1, -2),         # E above 512
    ((2560, 760, 256, 8), 1, -1),          # I not a multiple of 32
    ((2048, 768, 256, 8), 1, -2),          # shape not compiled
    ((0, 768, 256, 8), 1, -1),
])
def test_shape_validation(moe, shape, M, status):
    s = moe.shape(*shape)
    st, info = moe.moe_path_info(s, M)
    assert st == status, info
    fake = 1 << 20   # aligned, never dereferenced: validation fails first
    r = moe.raw().moe_decode_forward(ctypes.byref(s), M, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 30, None)
    assert r == status
    assert moe.moe_last_error() != ""


def test_null_and_alignment_and_workspace(moe):
    s = _shape(moe)
    L = moe.raw()
    a = 1 << 20
    ws_need = moe.moe_workspace_bytes(s, 4)
    assert L.moe_decode_forward(ctypes.byref(s), 4, None, a, a, a, a, a, a, a, ws_need, None) == -1
    assert "hidden" in moe.moe_last_error()
    assert L.moe_decode_forward(ctypes.byref(s), 4, a + 2, a, a, a, a, a, a, a, ws_need, None) == -3
    assert L.moe_decode_forward(ctypes.byref(s), 4, a, a, a, a, a, a, a, None, ws_need, None) == -4
    assert L.moe_decode_forward(ctypes.byref(s), 4, a, a, a, a, a, a, a, a + 16, ws_need, None) == -4
    assert L.moe_decode_forward(ctypes.byref(s), 4, a, a, a, a, a, a, a, a, ws_need - 1, None) == -4
    assert L.moe_route(ctypes.byref(s), 1, a, a, None, a, None, a, ws_need, None) == -1
    assert L.moe_gate_up(ctypes.byref(s), 1, a, a, a, a, a, None, a, a, a, ws_need, None) == -1
    assert L.moe_down_combine(ctypes.byref(s), 1, a, a, a, a, a, a, a + 4, a, ws_need, None) == -3
    assert L.moe_experts_forward(ctypes.byref(s), 1, a, a, a, a, a, a, a, a, a, None, a, 16, None) == -4
    assert L.moe_quant_act(None, 1, a, a, a, None) == -1
    assert L.moe_fp8_encode_range(0, 16, None, None) == -1
    assert L.moe_fp8_encode_range(0, -1, a, None) == -1
    assert L.moe_workspace_init(None, 1024, None) == -4
    assert L.moe_workspace_init(a + 8, 1024, None) == -4
    assert L.moe_workspace_sync_status(None, 1024, a, None) == -4
    assert L.moe_workspace_sync_status(a + 8, 1024, a, None) == -4
    assert L.moe_workspace_sync_status(a, 1024, None, None) == -1
    assert L.moe_decode_forward_noalloc(None, 1, a, a, a, a, a, a, a, None) == -1
    assert L.moe_decode_forward_noalloc(ctypes.byref(s), 1, None, a, a, a, a, a, a, None) == -1
    assert L.moe_decode_forward_noalloc(ctypes.byref(s), 1, a + 4, a, a, a, a, a, a, None) == -3


def test_status_strings_and_path_info(moe):
    for st in (0, -1, -2, -3, -4, -5):
        assert moe.moe_status_string(st)
    st, info = moe.moe_path_info(_shape(moe), 1)
    assert st == 0 and info.startswith("gemv path") and "gate_up_kernel" in info
    moe.moe_set_decode_path(moe.PATH_ONE_KERNEL)
    try:
        st, info = moe.moe_path_info(_shape(moe), 1)
        assert st == 0 and info.startswith("one-kernel gemv path") and "layer_kernel<H=2560,I=768>" in info
        st, info = moe.moe_path_info(_shape(moe), 512)       # the chunk path is not affected
        assert st == 0 and info.startswith("chunk path")
    finally:
        moe.moe_set_decode_path(moe.PATH_THREE_KERNELS)
    assert moe.raw().moe_set_decode_path(2) == -1
    assert moe.raw().moe_set_decode_path(-1) == -1
    st, info = moe.moe_path_info(_shape(moe), 1)
    assert info.startswith("gemv path")
    st, info = moe.moe_path_info(_shape(moe, 256, 64, 16, 2), 4)
    assert st == 0 and "H=256" in info
    st, info = moe.moe_path_info(_shape(moe), 512)
    assert st == 0 and info.startswith("chunk path") and "chunk_gate_up_kernel<2560,768>" in info


def test_lm_head_validation(moe):
    L = moe.raw()
    a = 1 << 20
    assert L.moe_lm_head_quantize(None, 16, 512, a, a, None) == -1
    assert L.moe_lm_head_quantize(a, 16, 500, a, a, None) == -1          # hidden % 8
    assert L.moe_lm_head_quantize(a + 2, 16, 512, a, a, None) == -3      # alignment
    assert L.moe_lm_head_forward(a, 1, a, a, 16, 1024, a, None) == -2     # hidden not compiled
    assert L.moe_lm_head_forward(a, 9, a, a, 16, 2560, a, None) == -2     # above 8 tokens
    assert L.moe_lm_head_forward(a, 0, a, a, 16, 2560, a, None) == -1
    assert L.moe_lm_head_forward(a, 1, a, None, 16, 2560, a, None) == -1


def test_shared_expert_validation(moe):
    s = _shape(moe)
    L = moe.raw()
    a = 1 << 20
    ws_need = moe.moe_workspace_bytes(s, 4)
    # the workspace of moe_workspace_bytes already covers the shared expert's rows
    assert ws_need >= (4 * 8 + 4) * 768 * 4
    bad = moe.MoeSharedExpert(a, None, a, a)
    assert L.moe_decode_forward_shared(ctypes.byref(s), 4, a, a, a, a, a, a, ctypes.byref(bad), a, a, ws_need,
                                       None, None) == -1
    assert "shared" in moe.moe_last_error()
    mis = moe.MoeSharedExpert(a + 4, a, a, a)
    assert L.moe_decode_forward_shared(ctypes.byref(s), 4, a, a, a, a, a, a, ctypes.byref(mis), a, a, ws_need,
                                       None, None) == -3
    mis2 = moe.MoeSharedExpert(a, a, a + 8, a)
    assert L.moe_experts_forward_shared(ctypes.byref(s), 1, a, a, a, a, a, a, a, a, ctypes.byref(mis2), a, None, a,
                                        ws_need, None) == -3
    ok = moe.MoeSharedExpert(a, a, a, a)
    assert L.moe_experts_forward_shared(ctypes.byref(s), 1, a, a, a, a, a, a, a, a, ctypes.byref(ok), a, None, a,
                                        16, None) == -4
    assert L.moe_decode_forward_shared(ctypes.byref(s), 0, a, a, a, a, a, a, ctypes.byref(ok), a, a, ws_need,
                                       None, None) == -1
