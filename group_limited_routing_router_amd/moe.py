"""ctypes binding of libmoe.so (C ABI in include/moe.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the current HIP stream to
the library, and raises MoEError when the library returns an error status.
No step of the computation runs here; if libmoe.so is missing or cannot be
loaded, ``load_library`` raises and nothing falls back to another path.

torch is imported before the library is loaded so that libmoe.so binds to the
HIP runtime torch already holds (both carry the soname libamdhip64.so.7); the
loader then checks that only one HIP runtime is mapped in the process.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoe.so"
_lock = threading.Lock()
_lib = None

MOE_OK = 0
DTYPE_F32 = 0
DTYPE_BF16 = 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES of moe.h

_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
           3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class MoEProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("G", ctypes.c_int32), ("TG", ctypes.c_int32),
                ("k", ctypes.c_int32), ("scale", ctypes.c_float)]

    @classmethod
    def from_config(cls, cfg, T=None):
        return cls(cfg.T if T is None else T, cfg.H, cfg.I, cfg.E, cfg.G, cfg.TG, cfg.k,
                   cfg.scale)


EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_permute", "moe_expert_ffn",
           "moe_expert_gate_up", "moe_expert_down", "moe_combine", "moe_combine_residual",
           "moe_dense_mlp", "moe_expert_ffn_fp8", "moe_forward", "moe_forward_fp8",
           "moe_forward_noalloc", "moe_status_string", "moe_last_error",
           # measurement kernels (include/moe_peak.h)
           "moe_peak_stream_read", "moe_peak_mfma_bf16", "moe_peak_mfma_bf16_flops",
           "moe_peak_mfma_stream", "moe_peak_mfma_stream_flops", "moe_peak_mfma_stream_bytes")


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load_library():
    """Load libmoe.so once and declare its signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m group_limited_routing_router_amd.build`")
        lib = ctypes.CDLL(path)
        rts = _hip_runtimes_mapped()
        if len(rts) > 1:
            raise ImportError(f"two HIP runtimes are mapped: {sorted(rts)}")
        P = ctypes.c_void_p
        prob = ctypes.POINTER(MoEProblem)
        st = ctypes.c_int
        lib.moe_workspace_bytes.argtypes = [prob]
        lib.moe_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_route.argtypes = [prob, P, P, P, P, P, P]
        lib.moe_route.restype = st
        lib.moe_permute.argtypes = [prob, P, P, P, P, P, ctypes.c_size_t, P]
        lib.moe_permute.restype = st
        lib.moe_expert_ffn.argtypes = [prob, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.moe_expert_ffn.restype = st
        lib.moe_expert_gate_up.argtypes = [prob, P, P, P, P, P, P, P]
        lib.moe_expert_gate_up.restype = st
        lib.moe_expert_down.argtypes = [prob, P, P, P, P, P]
        lib.moe_expert_down.restype = st
        lib.moe_combine.argtypes = [prob, P, P, P, P, ctypes.c_int, P]
        lib.moe_combine.restype = st
        lib.moe_combine_residual.argtypes = [prob, P, P, P, P, ctypes.c_float, ctypes.c_int32, P,
                                             P]
        lib.moe_combine_residual.restype = st
        lib.moe_expert_ffn_fp8.argtypes = [prob, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t,
                                           P]
        lib.moe_expert_ffn_fp8.restype = st
        lib.moe_forward_fp8.argtypes = [prob, P, P, P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P,
                                        P, ctypes.c_size_t, P]
        lib.moe_forward_fp8.restype = st
        lib.moe_dense_mlp.argtypes = [prob, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.moe_dense_mlp.restype = st
        lib.moe_forward.argtypes = [prob, P, P, P, P, P, P, P, ctypes.c_int, P, P, P, P,
                                    ctypes.c_size_t, P]
        lib.moe_forward.restype = st
        lib.moe_forward_noalloc.argtypes = [prob, P, P, P, P, P, P, P, ctypes.c_int, P, P, P, P]
        lib.moe_forward_noalloc.restype = st
        lib.moe_peak_stream_read.argtypes = [P, ctypes.c_size_t, ctypes.c_int, P, ctypes.c_int, P]
        lib.moe_peak_stream_read.restype = st
        lib.moe_peak_mfma_bf16.argtypes = [ctypes.c_int64, ctypes.c_int, P, ctypes.c_int, P]
        lib.moe_peak_mfma_bf16.restype = st
        lib.moe_peak_mfma_bf16_flops.argtypes = [ctypes.c_int64, ctypes.c_int]
        lib.moe_peak_mfma_bf16_flops.restype = ctypes.c_double
        lib.moe_peak_mfma_stream.argtypes = [P, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64, P,
                                             ctypes.c_int, P]
        lib.moe_peak_mfma_stream.restype = st
        lib.moe_peak_mfma_stream_flops.argtypes = [ctypes.c_int64, ctypes.c_int]
        lib.moe_peak_mfma_stream_flops.restype = ctypes.c_double
        lib.moe_peak_mfma_stream_bytes.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        lib.moe_peak_mfma_stream_bytes.restype = ctypes.c_double
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_last_error.argtypes = []
        lib.moe_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != MOE_OK:
        raise MoEError(status, load_library().moe_last_error().decode())


def _dtype_code(out):
    if isinstance(out, int):
        raise TypeError("out must be a tensor")
    if out.dtype == torch.float32:
        return DTYPE_F32
    if out.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"out dtype {out.dtype} is not float32/bfloat16")


def moe_workspace_bytes(p: MoEProblem) -> int:
    return int(load_library().moe_workspace_bytes(ctypes.byref(p)))


def moe_route(p, x, w_router, bias, topk_ids, topk_weights, stream=None):
    _check(load_library().moe_route(ctypes.byref(p), _p(x), _p(w_router), _p(bias), _p(topk_ids),
                                     _p(topk_weights), _stream(stream)))


def moe_permute(p, topk_ids, expert_offsets, sorted_pairs, pair_rows, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().moe_permute(ctypes.byref(p), _p(topk_ids), _p(expert_offsets),
                                       _p(sorted_pairs), _p(pair_rows), _p(ws), nbytes,
                                       _stream(stream)))


def moe_expert_ffn(p, x, sorted_pairs, expert_offsets, w_gate, w_up, w_down, y, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().moe_expert_ffn(ctypes.byref(p), _p(x), _p(sorted_pairs),
                                          _p(expert_offsets), _p(w_gate), _p(w_up), _p(w_down),
                                          _p(y), _p(ws), nbytes, _stream(stream)))


def moe_expert_gate_up(p, x, sorted_pairs, expert_offsets, w_gate, w_up, h, stream=None):
    _check(load_library().moe_expert_gate_up(ctypes.byref(p), _p(x), _p(sorted_pairs),
                                              _p(expert_offsets), _p(w_gate), _p(w_up), _p(h),
                                              _stream(stream)))


def moe_expert_down(p, h, expert_offsets, w_down, y, stream=None):
    _check(load_library().moe_expert_down(ctypes.byref(p), _p(h), _p(expert_offsets),
                                           _p(w_down), _p(y), _stream(stream)))


def moe_combine(p, y, pair_rows, topk_weights, out, stream=None):
    _check(load_library().moe_combine(ctypes.byref(p), _p(y), _p(pair_rows), _p(topk_weights),
                                       _p(out), _dtype_code(out), _stream(stream)))


def moe_combine_residual(p, y, pair_rows, topk_weights, norm_weight, eps, step, residual,
                         stream=None):
    _check(load_library().moe_combine_residual(ctypes.byref(p), _p(y), _p(pair_rows),
                                                _p(topk_weights), _p(norm_weight), float(eps),
                                                int(step), _p(residual), _stream(stream)))


def moe_expert_ffn_fp8(p, x, sorted_pairs, expert_offsets, q_gate, s_gate, q_up, s_up, q_down,
                       s_down, y, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().moe_expert_ffn_fp8(ctypes.byref(p), _p(x), _p(sorted_pairs),
                                              _p(expert_offsets), _p(q_gate), _p(s_gate), _p(q_up),
                                              _p(s_up), _p(q_down), _p(s_down), _p(y), _p(ws),
                                              nbytes, _stream(stream)))


def moe_forward_fp8(p, x, w_router, bias, q_gate, s_gate, q_up, s_up, q_down, s_down, out,
                    topk_ids, topk_weights, y, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().moe_forward_fp8(ctypes.byref(p), _p(x), _p(w_router), _p(bias),
                                           _p(q_gate), _p(s_gate), _p(q_up), _p(s_up), _p(q_down),
                                           _p(s_down), _p(out), _dtype_code(out), _p(topk_ids),
                                           _p(topk_weights), _p(y), _p(ws), nbytes,
                                           _stream(stream)))


def moe_dense_mlp(p, x, w_gate, w_up, w_down, out, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().moe_dense_mlp(ctypes.byref(p), _p(x), _p(w_gate), _p(w_up), _p(w_down),
                                         _p(out), _p(ws), nbytes, _stream(stream)))


def moe_forward(p, x, w_router, bias, w_gate, w_up, w_down, out, topk_ids, topk_weights, y, ws,
                stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().moe_forward(ctypes.byref(p), _p(x), _p(w_router), _p(bias), _p(w_gate),
                                       _p(w_up), _p(w_down), _p(out), _dtype_code(out),
                                       _p(topk_ids), _p(topk_weights), _p(y), _p(ws), nbytes,
                                       _stream(stream)))


def moe_forward_noalloc(p, x, w_router, bias, w_gate, w_up, w_down, out, topk_ids, topk_weights,
                        y, stream=None):
    _check(load_library().moe_forward_noalloc(ctypes.byref(p), _p(x), _p(w_router), _p(bias),
                                               _p(w_gate), _p(w_up), _p(w_down), _p(out),
                                               _dtype_code(out), _p(topk_ids), _p(topk_weights),
                                               _p(y), _stream(stream)))


def moe_peak_stream_read(buf, sink, workgroups, nontemporal=False, stream=None):
    """One streaming read of the whole of `buf` (a GPU tensor) by the
    measurement kernel; `sink` is a GPU tensor of at least 4 bytes."""
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().moe_peak_stream_read(_p(buf), nbytes, int(bool(nontemporal)), _p(sink),
                                                int(workgroups), _stream(stream)))


def moe_peak_mfma_bf16(iters, sink, workgroups, random_operands=True, stream=None):
    """The back-to-back bf16 MFMA loop on pseudo-random (default) or fixed
    register operands; `sink` holds 4 * workgroups floats.  Returns the FLOPs
    of the call."""
    lib = load_library()
    _check(lib.moe_peak_mfma_bf16(int(iters), int(bool(random_operands)), _p(sink),
                                  int(workgroups), _stream(stream)))
    return float(lib.moe_peak_mfma_bf16_flops(int(iters), int(workgroups)))


def moe_peak_mfma_stream(buf, loads_per_step, steps, sink, workgroups, stream=None):
    """LDS-fed bf16 MFMAs with `loads_per_step` 16-byte HBM loads a lane per
    step from `buf` (a GPU tensor, or None with 0 loads); `sink` holds
    4 * workgroups floats.  Returns (FLOPs, bytes) of the call."""
    lib = load_library()
    nbytes = 0 if buf is None else buf.numel() * buf.element_size()
    _check(lib.moe_peak_mfma_stream(_p(buf) if buf is not None else None, nbytes,
                                    int(loads_per_step), int(steps), _p(sink), int(workgroups),
                                    _stream(stream)))
    return (float(lib.moe_peak_mfma_stream_flops(int(steps), int(workgroups))),
            float(lib.moe_peak_mfma_stream_bytes(int(steps), int(loads_per_step), int(workgroups))))


def alloc_buffers(p: MoEProblem, device="cuda", out_dtype=torch.float32):
    """Caller-side buffers for one forward pass (torch allocations)."""
    T, k, H, E = p.T, p.k, p.H, p.E
    ws_bytes = moe_workspace_bytes(p)
    if ws_bytes == 0 and T > 0:
        raise MoEError(1, load_library().moe_last_error().decode())
    return dict(
        out=torch.empty((T, H), dtype=out_dtype, device=device),
        topk_ids=torch.empty((T, k), dtype=torch.int32, device=device),
        topk_weights=torch.empty((T, k), dtype=torch.float32, device=device),
        expert_offsets=torch.empty((E + 1,), dtype=torch.int32, device=device),
        sorted_pairs=torch.empty((T * k,), dtype=torch.int32, device=device),
        pair_rows=torch.empty((T * k,), dtype=torch.int32, device=device),
        y=torch.empty((T * k, H), dtype=torch.float32, device=device),
        h=torch.empty((T * k, p.I), dtype=torch.bfloat16, device=device),
        ws=torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=device),
    )
