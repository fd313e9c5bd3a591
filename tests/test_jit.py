"""CPU checks of run-time compilation (moe_jit_build): hipRTC compiles the
library's own device headers for a layer shape outside the ahead-of-time set,
without a GPU, into an on-disk cache that later calls reuse; damaged cache
files are rebuilt, and shapes or targets the kernels cannot serve are
rejected with the documented status."""
import ctypes
import os
import struct
import subprocess

import pytest
import torch  # noqa: F401  (loaded first, as in use: the library then runs on torch's HIP runtime and hipRTC)

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.fixture(scope="module")
def moe():
    from mxfp4_weight_streaming_amd import binding
    return binding


@pytest.fixture(scope="module")
def built(moe, tmp_path_factory):
    """One compile of (H=1024, I=384) into a fresh cache directory."""
    d = tmp_path_factory.mktemp("jit_cache")
    rep = moe.moe_jit_build(moe.shape(1024, 384, 64, 4), "gfx950", str(d))
    return d, rep


def test_compile_fills_the_cache(built):
    d, rep = built
    assert not rep["from_cache"]
    # decode path: quant, requant, and router/gate_up/down(x2)/layer at 4 token
    # bounds; chunk path: router, gate_up, down(x2), combine; LM head at 4 token bounds
    assert rep["has_chunk_path"] and rep["has_lm_head"] and rep["num_kernels"] == 2 + 20 + 5 + 4
    path = rep["cache_file"]
    assert os.path.dirname(path) == str(d) and os.path.basename(path).startswith("moe_H1024_I384_gfx950_")
    assert os.path.getsize(path) > 10_000
    assert [f for f in os.listdir(d) if ".tmp." in f] == []      # no temporary left behind


def test_second_build_is_a_cache_hit(moe, built):
    d, rep = built
    again = moe.moe_jit_build(moe.shape(1024, 384, 128, 8), "gfx950", str(d))   # E, K do not enter the kernels
    assert again["from_cache"] and again["cache_file"] == rep["cache_file"]
    assert again["seconds"] < 1.0


def test_damaged_entries_are_rebuilt(moe, built):
    d, rep = built
    path = rep["cache_file"]
    good = open(path, "rb").read()
    try:
        bad = bytearray(good)
        bad[-100] ^= 0x40                                          # inside the code object
        open(path, "wb").write(bytes(bad))
        r = moe.moe_jit_build(moe.shape(1024, 384, 64, 4), "gfx950", str(d))
        assert not r["from_cache"]
        assert moe.moe_jit_build(moe.shape(1024, 384, 64, 4), "gfx950", str(d))["from_cache"]   # whole again
        open(path, "wb").write(good[: len(good) // 2])             # truncated
        assert not moe.moe_jit_build(moe.shape(1024, 384, 64, 4), "gfx950", str(d))["from_cache"]
        assert moe.moe_jit_build(moe.shape(1024, 384, 64, 4), "gfx950", str(d))["from_cache"]
    finally:
        open(path, "wb").write(good)


def test_shapes_and_targets_without_kernels_are_rejected(moe, tmp_path):
    L = moe.raw()
    for H, I in ((1000, 384), (1024, 96), (128, 64), (16384, 768)):
        s = moe.shape(H, I, 64, 4)
        assert L.moe_jit_build(ctypes.byref(s), b"gfx950", str(tmp_path).encode(), None) == moe.MOE_ERR_UNSUPPORTED_SHAPE
        assert "kernel geometry" in moe.moe_last_error()
    s = moe.shape(1024, 384, 64, 4)
    assert L.moe_jit_build(ctypes.byref(s), b"gfx942", str(tmp_path).encode(), None) == moe.MOE_ERR_UNSUPPORTED_SHAPE
    assert "gfx950" in moe.moe_last_error()
    assert L.moe_jit_build(None, b"gfx950", None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_jit_build(ctypes.byref(s), None, None, None) == moe.MOE_ERR_INVALID_ARG
    blocker = tmp_path / "file"
    blocker.write_bytes(b"x")                                       # a file where the directory should be
    assert L.moe_jit_build(ctypes.byref(s), b"gfx950", str(blocker / "sub").encode(), None) == moe.MOE_ERR_JIT
    assert listed(tmp_path) == ["file"]


def listed(p):
    return sorted(os.listdir(p))


def _code_object(path):
    """The code object of a cache entry (format: magic, key, kernel list, size, checksum, code)."""
    b = open(path, "rb").read()
    at = 16
    (n,) = struct.unpack_from("<I", b, at)
    at += 4
    for _ in range(n):
        ln = struct.unpack_from("<iiiiI", b, at)[4]
        at += 20 + ln
    size = struct.unpack_from("<Q", b, at)[0]
    return b[at + 16: at + 16 + size]


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="no llvm-objdump")
def test_compiled_code_has_valid_operands(built, tmp_path):
    """Every instruction of the compiled module disassembles with valid
    operands; in particular the scaled MFMAs of the chunk kernels take their
    scale codes from VGPRs (a compiler release once encoded a constant scale
    as an SGPR, which the instruction misreads)."""
    _, rep = built
    co = tmp_path / "module.co"
    co.write_bytes(_code_object(rep["cache_file"]))
    dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(co)], capture_output=True, text=True, check=True).stdout
    assert dis.count("v_mfma_scale_f32_16x16x128_f8f6f4") > 0
    assert "Invalid register" not in dis


def test_without_a_device_load_fails_cleanly(moe, built):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d, _ = built
    s = moe.shape(1024, 384, 64, 4)
    assert moe.raw().moe_jit_load(ctypes.byref(s), str(d).encode(), 0, None) == moe.MOE_ERR_HIP
    assert moe.raw().moe_jit_unload(ctypes.byref(s)) == 0
    # an unloaded shape stays unsupported: nothing is compiled implicitly
    st, info = moe.moe_path_info(s, 1)
    assert st == moe.MOE_ERR_UNSUPPORTED_SHAPE and "moe_jit_load" in info


def test_ahead_of_time_shapes_need_no_module(moe):
    for shp in (moe.shape(2560, 768, 256, 8), moe.shape(256, 64, 16, 2)):
        st, info = moe.moe_path_info(shp, 1)
        assert st == 0 and "compiled at run time" not in info
    # the down kernel's LDS bound on the decode path
    st, info = moe.moe_path_info(moe.shape(2560, 768, 256, 8), 8)
    assert st == 0
