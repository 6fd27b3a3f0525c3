"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, sizes workspaces, and rejects bad arguments on the
host before any HIP call (nothing enqueued, outputs untouched)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (the binding binds to torch's HIP runtime)
    from group_limited_routing_router_amd import moe
    return moe


def _declared():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = _declared()
    assert set(names) == set(lib.EXPORTS)
    cdll = lib.load_library()
    for n in names:
        assert hasattr(cdll, n), n


def test_single_hip_runtime(lib):
    lib.load_library()
    assert len(lib._hip_runtimes_mapped()) <= 1


def _beam(T=128):
    from group_limited_routing_router_amd.moe import MoEProblem
    return MoEProblem(T, 5120, 2560, 256, 8, 4, 8, 2.5)


def test_workspace_bytes(lib):
    for T in (1, 128, 8192, 65536):
        p = _beam(T)
        n = lib.moe_workspace_bytes(p)
        assert n >= T * 8 * 2560 * 2          # bf16 SwiGLU product
        assert n < T * 8 * 2560 * 2 + T * 8 * 64 + (1 << 22)
    assert lib.moe_workspace_bytes(_beam(0)) >= 0


@pytest.mark.parametrize("field,value,status", [
    ("T", -1, 1), ("H", 100, 1), ("H", 0, 1), ("I", 96, 1), ("E", 0, 1), ("G", 7, 1),
    ("TG", 0, 1), ("TG", 9, 1), ("k", 0, 1), ("k", 129, 1), ("E", 512, 1), ("k", 17, 2),
    ("H", 192, 2), ("H", 65536 + 128, 2), ("I", 65536 + 64, 2),
])
def test_problem_validation(lib, field, value, status):
    p = _beam()
    setattr(p, field, value)
    if field == "E" and value == 512:
        p.G = 8  # divisible, valid shape but beyond the kernels' limit
        status = 2
    cdll = lib.load_library()
    buf = np.zeros(64, np.int32)
    out = np.full(64, 7, np.float32)
    ptr = buf.ctypes.data
    rc = cdll.moe_route(ctypes.byref(p), ptr, ptr, None, ptr, out.ctypes.data, None)
    assert rc == status, cdll.moe_last_error()
    assert cdll.moe_last_error()
    assert np.all(out == 7)
    assert lib.moe_workspace_bytes(p) == 0


def _aligned(n=4096, offset=0):
    raw = np.zeros(n + 64, np.uint8)
    base = (-raw.ctypes.data) % 64
    return raw, raw.ctypes.data + base + offset


def test_pointer_and_workspace_errors(lib):
    cdll = lib.load_library()
    p = _beam()
    keep, good = _aligned()
    keep2, odd = _aligned(offset=4)
    guard = np.full(16, 3, np.int32)
    # NULL inputs
    assert cdll.moe_route(ctypes.byref(p), None, good, None, good, good, None) == 1
    assert b"x" in cdll.moe_last_error()
    # misaligned output
    assert cdll.moe_route(ctypes.byref(p), good, good, None, odd, good, None) == 1
    assert b"aligned" in cdll.moe_last_error()
    # workspace too small / NULL
    need = lib.moe_workspace_bytes(p)
    assert cdll.moe_permute(ctypes.byref(p), good, good, good, good, good, need - 1, None) == 3
    assert cdll.moe_permute(ctypes.byref(p), good, good, good, good, None, need, None) == 3
    assert cdll.moe_expert_ffn(ctypes.byref(p), good, good, good, good, good, good, good, good,
                               16, None) == 3
    # bad output dtype
    assert cdll.moe_combine(ctypes.byref(p), good, good, good, good, 5, None) == 1
    assert cdll.moe_forward(ctypes.byref(p), good, good, None, good, good, good,
                            guard.ctypes.data, 9, None, None, good, good, need, None) == 1
    # forward: y missing
    assert cdll.moe_forward(ctypes.byref(p), good, good, None, good, good, good,
                            guard.ctypes.data, 0, None, None, None, good, need, None) == 1
    assert np.all(guard == 3)
    assert cdll.moe_status_string(3) == b"MOE_ERR_WORKSPACE"
    # fused epilogue: eps, step, missing pointers, hidden size beyond the limit
    f, i32 = ctypes.c_float, ctypes.c_int32
    assert cdll.moe_combine_residual(ctypes.byref(p), good, good, good, good, f(0.0), i32(2),
                                     good, None) == 1
    assert b"eps" in cdll.moe_last_error()
    assert cdll.moe_combine_residual(ctypes.byref(p), good, good, good, good, f(float("nan")),
                                     i32(2), good, None) == 1
    assert cdll.moe_combine_residual(ctypes.byref(p), good, good, good, good, f(1e-6), i32(0),
                                     good, None) == 1
    assert b"step" in cdll.moe_last_error()
    assert cdll.moe_combine_residual(ctypes.byref(p), good, good, good, None, f(1e-6), i32(2),
                                     good, None) == 1
    assert b"norm_weight" in cdll.moe_last_error()
    assert cdll.moe_combine_residual(ctypes.byref(p), good, good, good, good, f(1e-6), i32(2),
                                     odd, None) == 1
    # dense MLP: needs one expert, one group, k = 1, and a workspace
    assert cdll.moe_dense_mlp(ctypes.byref(p), good, good, good, good, good, good, need,
                              None) == 1
    assert b"E=G=TG=k=1" in cdll.moe_last_error()
    dense = _beam()
    dense.E = dense.G = dense.TG = dense.k = 1
    assert cdll.moe_dense_mlp(ctypes.byref(dense), good, good, good, good, good, None, 0,
                              None) == 3
    assert cdll.moe_dense_mlp(ctypes.byref(dense), good, good, None, good, good, good, 1 << 40,
                              None) == 1
    wide = _beam()
    wide.H = 16384 + 128
    assert cdll.moe_combine_residual(ctypes.byref(wide), good, good, good, good, f(1e-6), i32(2),
                                     good, None) == 2


def test_zero_tokens_is_a_noop(lib):
    cdll = lib.load_library()
    p = _beam(0)
    assert cdll.moe_route(ctypes.byref(p), None, None, None, None, None, None) == 0
    assert cdll.moe_permute(ctypes.byref(p), None, None, None, None, None, 0, None) == 0
    assert cdll.moe_expert_ffn(ctypes.byref(p), None, None, None, None, None, None, None, None,
                               0, None) == 0
    assert cdll.moe_combine(ctypes.byref(p), None, None, None, None, 0, None) == 0
    assert cdll.moe_combine_residual(ctypes.byref(p), None, None, None, None, ctypes.c_float(1e-6),
                                     ctypes.c_int32(3), None, None) == 0
    dense = _beam(0)
    dense.E = dense.G = dense.TG = dense.k = 1
    assert cdll.moe_dense_mlp(ctypes.byref(dense), None, None, None, None, None, None, 0,
                              None) == 0
    assert cdll.moe_forward(ctypes.byref(p), None, None, None, None, None, None, None, 0, None,
                            None, None, None, 0, None) == 0


def test_binding_raises_with_message(lib):
    p = _beam()
    p.G = 3
    with pytest.raises(lib.MoEError) as ei:
        lib.moe_route(p, 0, 0, None, 0, 0, stream=0)
    assert "G=3" in str(ei.value)


def test_header_serves_a_plain_c_program(tmp_path, lib):
    """include/moe.h compiles as C11 with every gcc warning an error, and a C
    program links against libmoe.so and the HIP runtime's C API.  Run with no
    arguments it prints its usage before any HIP call."""
    import subprocess
    import sys

    sys.path.insert(0, ROOT)
    import __graft_entry__

    lib.load_library()  # libmoe.so is built
    exe = __graft_entry__.build_c_client(out=str(tmp_path / "moe_client"), werror=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr



def test_measurement_kernels_reject_bad_arguments(lib):
    cdll = lib.load_library()
    keep, good = _aligned()
    keep2, odd = _aligned(offset=4)
    i64 = ctypes.c_int64
    assert cdll.moe_peak_stream_read(None, 4096, 0, good, 16, None) == 1
    assert cdll.moe_peak_stream_read(good, 4096, 0, None, 16, None) == 1
    assert cdll.moe_peak_stream_read(good, 4008, 0, good, 16, None) == 1   # not a multiple of 16
    assert cdll.moe_peak_stream_read(odd, 4096, 0, good, 16, None) == 1    # misaligned
    assert cdll.moe_peak_stream_read(good, 4096, 0, good, 0, None) == 1    # no workgroups
    assert cdll.moe_peak_mfma_bf16(i64(0), 1, good, 16, None) == 1
    assert cdll.moe_peak_mfma_bf16(i64(10), 0, None, 16, None) == 1
    assert cdll.moe_peak_mfma_bf16(i64(10), 1, good, 0, None) == 1      # no workgroups
    # the MFMA loop with an HBM stream: steps a multiple of 8, loads 0/1/2/4,
    # and a buffer holding every chunk the launch reads
    sz = ctypes.c_size_t
    need = (64 + 8) * 2 * 16 * 256 * 16
    assert cdll.moe_peak_mfma_stream(good, sz(need), 2, i64(60), good, 16, None) == 1  # not x8
    assert cdll.moe_peak_mfma_stream(good, sz(need), 3, i64(64), good, 16, None) == 1  # loads
    assert cdll.moe_peak_mfma_stream(good, sz(need - 16), 2, i64(64), good, 16, None) == 1
    assert cdll.moe_peak_mfma_stream(odd, sz(need), 2, i64(64), good, 16, None) == 1
    assert cdll.moe_peak_mfma_stream(None, sz(need), 2, i64(64), good, 16, None) == 1
    assert cdll.moe_peak_mfma_stream(good, sz(need), 2, i64(64), None, 16, None) == 1
    assert cdll.moe_peak_mfma_stream(good, sz(need), 2, i64(64), good, 0, None) == 1
    assert lib.load_library().moe_peak_mfma_stream_flops(i64(64), 3) == 3 * 4 * 64 * 16 * 32768
    assert lib.load_library().moe_peak_mfma_stream_bytes(i64(64), 2, 3) == 3 * 256 * 64 * 2 * 16
    # FLOPs of one call: waves x steps x 8 chains x 2*32*32*16
    assert lib.load_library().moe_peak_mfma_bf16_flops(i64(100), 3) == 3 * 4 * 100 * 8 * 32768


def test_noalloc_forward_host_checks(lib):
    """moe_forward_noalloc: T = 0 is a no-op; a problem whose workspace would
    not fit the static scratch is refused before anything is enqueued."""
    cdll = lib.load_library()
    keep, good = _aligned()
    guard = np.full(16, 3, np.int32)
    assert cdll.moe_forward_noalloc(ctypes.byref(_beam(0)), None, None, None, None, None, None,
                                    None, 0, None, None, None, None) == 0
    big = _beam(4096)
    assert lib.moe_workspace_bytes(big) > lib.NOALLOC_SCRATCH_BYTES
    assert cdll.moe_forward_noalloc(ctypes.byref(big), good, good, None, good, good, good,
                                    guard.ctypes.data, 0, None, None, good, None) == 2
    assert b"static scratch" in cdll.moe_last_error()
    assert cdll.moe_forward_noalloc(ctypes.byref(_beam()), good, good, None, good, good, good,
                                    guard.ctypes.data, 0, None, None, None, None) == 1
    assert np.all(guard == 3)
    # the header's limit and the binding's copy of it agree
    text = open(HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    assert lib.NOALLOC_SCRATCH_BYTES == 64 << 20
