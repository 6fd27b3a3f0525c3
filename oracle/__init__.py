"""CPU oracle for the Beam-style MoE block forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

The arithmetic lives in ``moe_oracle.c`` (plain C loops, fp32 where the pages
fix fp32, bf16 inputs widened exactly); this module only builds that file with
gcc, loads it with ctypes and marshals numpy arrays.  The compositions
``forward`` and ``forward_with_routing`` chain the C steps in the order the
page "Welcome Beam: a 501B open model you can own, customize, and scale",
section "Mixture of Experts", describes them: score, group-limited selection,
normalised weights, SwiGLU experts, weighted sum times the scale.

Arrays of bf16 values are passed as ``numpy.uint16`` bit patterns.

Parity pins (see ``tests/test_oracle_*.py``): routing is pinned by two-stage
brute-force enumeration on tiny inputs, invariants and special cases that
reduce to ``numpy.argsort`` / ``argmax``; the scores by a float64 library
matmul; the permutation by ``numpy.bincount`` and a stable ``argsort``; the
SwiGLU expert by ``torch.nn.functional`` on the CPU; the combine by the k=1
and identical-experts closed forms; the whole block by the dense all-experts
sum when k=E and G=1; the sublayer epilogue (``residual_norm``) by
``torch.nn.functional.rms_norm`` at step 1 and by the closed forms of the
stream update (scale of the stream, zero stream, orthogonal inputs); the FP8
expert (``ffn_pairs_fp8``) by torch's float8_e4m3fn decoding of every code
and by bit equality with the bf16 expert when every channel scale is a power
of two (the scaled weights are then exact in bf16).  No function here is
parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into oracle/liboracle.so."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        lib.oracle_route.argtypes = [i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, P]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_select.argtypes = [i64, i32, i32, i32, i32, P, P, P]
        lib.oracle_select.restype = ctypes.c_int
        lib.oracle_permute.argtypes = [i64, i32, i32, P, P, P, P]
        lib.oracle_permute.restype = ctypes.c_int
        lib.oracle_ffn_pairs.argtypes = [i64, i32, i32, P, P, P, P, P, P, P, P]
        lib.oracle_ffn_pairs.restype = ctypes.c_int
        lib.oracle_ffn_pairs_fp8.argtypes = [i64, i32, i32, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_ffn_pairs_fp8.restype = ctypes.c_int
        lib.oracle_e4m3_decode.argtypes = [i64, P, P]
        lib.oracle_e4m3_decode.restype = None
        lib.oracle_combine.argtypes = [i64, i32, i32, P, P, f32, P]
        lib.oracle_combine.restype = ctypes.c_int
        lib.oracle_residual_norm.argtypes = [i64, i32, P, P, f32, i32, P]
        lib.oracle_residual_norm.restype = ctypes.c_int
        lib.oracle_f32_to_bf16_rne.argtypes = [i64, P, P]
        lib.oracle_f32_to_bf16_rne.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc == -2:
        raise FloatingPointError(f"oracle {what}: non-finite router score")
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def route(x, w_router, bias, G, TG, k, want_scores=False):
    """Score, select and weight.  x [T,H] and w_router [E,H] as uint16 bf16 bits,
    bias [E] float32 or None.  Returns (ids [T,k] int32, weights [T,k] float32,
    scores [T,E] float32 or None, group_scores [T,G] float32 or None)."""
    lib = _load()
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.uint16)
    T, H = x.shape
    E = w_router.shape[0]
    assert w_router.shape[1] == H
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    s = np.empty((T, E), np.float32) if want_scores else None
    gs = np.empty((T, G), np.float32) if want_scores else None
    rc = lib.oracle_route(T, H, E, G, TG, k, _ptr(x), _ptr(w_router), _ptr(b), _ptr(ids),
                          _ptr(w), _ptr(s), _ptr(gs))
    _check(rc, "route")
    return ids, w, s, gs


def select(scores, G, TG, k):
    """Selection and weights from given fp32 scores [T,E]."""
    lib = _load()
    s = _c(scores, np.float32)
    T, E = s.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(lib.oracle_select(T, E, G, TG, k, _ptr(s), _ptr(ids), _ptr(w)), "select")
    return ids, w


def permute(ids, E):
    """Stable counting sort of pairs p=t*k+j by expert.  Returns
    (offsets [E+1], sorted_pairs [T*k], pair_rows [T*k]), all int32."""
    lib = _load()
    ids = _c(ids, np.int32)
    T, k = ids.shape
    off = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    pr = np.empty(T * k, np.int32)
    _check(lib.oracle_permute(T, k, E, _ptr(ids), _ptr(off), _ptr(sp), _ptr(pr)), "permute")
    return off, sp, pr


def ffn_pairs(tok, exp, x, w_gate, w_up, w_down, want_h=False):
    """SwiGLU expert outputs for (token, expert) pairs.  x [*,H], w_gate/w_up
    [*,I,H], w_down [*,H,I] as uint16 bf16 bits.  Returns (y [n,H] float32,
    h [n,I] uint16 or None)."""
    lib = _load()
    tok = _c(tok, np.int32).ravel()
    exp = _c(exp, np.int32).ravel()
    x = _c(x, np.uint16)
    w_gate = _c(w_gate, np.uint16)
    w_up = _c(w_up, np.uint16)
    w_down = _c(w_down, np.uint16)
    n = tok.shape[0]
    H = x.shape[1]
    I = w_gate.shape[1]
    assert w_gate.shape[2] == H and w_up.shape == w_gate.shape
    assert w_down.shape[1] == H and w_down.shape[2] == I
    assert n == 0 or (tok.max() < x.shape[0] and exp.max() < w_gate.shape[0])
    y = np.empty((n, H), np.float32)
    h = np.empty((n, I), np.uint16) if want_h else None
    _check(lib.oracle_ffn_pairs(n, H, I, _ptr(tok), _ptr(exp), _ptr(x), _ptr(w_gate),
                                _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(y)), "ffn")
    return y, h


def ffn_pairs_fp8(tok, exp, x, q_gate, s_gate, q_up, s_up, q_down, s_down, want_h=False):
    """ffn_pairs with FP8 (E4M3 codes, uint8) weights and fp32 per-channel
    scales: q_gate/q_up [*,I,H], s_gate/s_up [*,I], q_down [*,H,I], s_down [*,H]."""
    lib = _load()
    tok = _c(tok, np.int32).ravel()
    exp = _c(exp, np.int32).ravel()
    x = _c(x, np.uint16)
    qg, qu, qd = _c(q_gate, np.uint8), _c(q_up, np.uint8), _c(q_down, np.uint8)
    sg, su, sd = _c(s_gate, np.float32), _c(s_up, np.float32), _c(s_down, np.float32)
    n = tok.shape[0]
    H = x.shape[1]
    I = qg.shape[1]
    assert qg.shape[2] == H and qd.shape[1:] == (H, I) and sg.shape == qg.shape[:2]
    assert sd.shape == qd.shape[:2]
    y = np.empty((n, H), np.float32)
    h = np.empty((n, I), np.uint16) if want_h else None
    _check(lib.oracle_ffn_pairs_fp8(n, H, I, _ptr(tok), _ptr(exp), _ptr(x), _ptr(qg), _ptr(sg),
                                    _ptr(qu), _ptr(su), _ptr(qd), _ptr(sd), _ptr(h), _ptr(y)),
           "ffn_pairs_fp8")
    return y, h


def forward_with_routing_fp8(x, ids, weights, q_gate, s_gate, q_up, s_up, q_down, s_down,
                             scale, want_h=False):
    """FP8-weight expert FFN and combine for given routing (ids, weights) [T,k]."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    tok = np.repeat(np.arange(T, dtype=np.int32), k)
    y, h = ffn_pairs_fp8(tok, ids.ravel(), x, q_gate, s_gate, q_up, s_up, q_down, s_down,
                         want_h=want_h)
    out = combine(y, weights, scale)
    return out, y, h


def e4m3_decode(codes):
    """The oracle's decoding of E4M3 codes (uint8) to float32."""
    lib = _load()
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float32)
    lib.oracle_e4m3_decode(c.size, _ptr(c), _ptr(out))
    return out


def combine(y, weights, scale):
    """out[t] = scale * sum_j weights[t,j] * y[t*k+j] (y rows in pair order)."""
    lib = _load()
    w = _c(weights, np.float32)
    T, k = w.shape
    y = _c(y, np.float32)
    H = y.shape[1]
    assert y.shape[0] == T * k
    out = np.empty((T, H), np.float32)
    _check(lib.oracle_combine(T, k, H, _ptr(y), _ptr(w), float(scale), _ptr(out)), "combine")
    return out


def residual_norm(o, gain, eps, step, residual):
    """Post-norm of the sublayer output o [T,H] (RMSNorm with gain [H]) and the
    residual-stream update at step `step`; returns the new stream [T,H]."""
    lib = _load()
    o = _c(o, np.float32)
    T, H = o.shape
    g = _c(gain, np.float32)
    assert g.shape == (H,)
    res = np.array(residual, dtype=np.float32, order="C", copy=True)
    assert res.shape == (T, H)
    _check(lib.oracle_residual_norm(T, H, _ptr(o), _ptr(g), float(eps), int(step), _ptr(res)),
           "residual_norm")
    return res


def forward_with_routing(x, ids, weights, w_gate, w_up, w_down, scale, want_h=False):
    """Expert FFN and combine for given routing (ids, weights) [T,k]."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    tok = np.repeat(np.arange(T, dtype=np.int32), k)
    y, h = ffn_pairs(tok, ids.ravel(), x, w_gate, w_up, w_down, want_h=want_h)
    out = combine(y, weights, scale)
    return out, y, h


def forward(x, w_router, bias, w_gate, w_up, w_down, G, TG, k, scale, want_h=False):
    """The whole block: returns a dict with ids, weights, scores, group_scores,
    y (pair order), h (pair order, if asked) and out [T,H] float32."""
    ids, w, s, gs = route(x, w_router, bias, G, TG, k, want_scores=True)
    out, y, h = forward_with_routing(x, ids, w, w_gate, w_up, w_down, scale, want_h=want_h)
    return dict(ids=ids, weights=w, scores=s, group_scores=gs, y=y, h=h, out=out)


def f32_to_bf16(a):
    """Round-to-nearest-even float32 -> bf16 bits (the oracle's own rounding)."""
    lib = _load()
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib.oracle_f32_to_bf16_rne(a.size, _ptr(a), _ptr(out))
    return out


def num_threads():
    """Threads the oracle's OpenMP loops run on."""
    return int(_load().oracle_num_threads())


def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns to float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)
