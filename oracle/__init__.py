"""CPU oracle for the W2A8 ternary linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never links,
imports or calls it, and it shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, built here with gcc); this
module only builds it and marshals numpy arrays.  Each function names the
step it follows on the page "BitMTP: When Multi-Token Prediction Meets
Low-Bit Large Language Models" (ai.info AI summary); the formulas are the
readings stated at the top of ``oracle.c``.

Parity status: every function below is pinned by a ``-m "not gpu"`` test
(brute force, closed forms, invariants or hand-derived fixtures); none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc into ``oracle/liboracle.so``."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.orc_ternarize_absmean.argtypes = [p, i64, i64, p, p]
    lib.orc_ternarize_absmean.restype = ctypes.c_int
    lib.orc_quantize_act.argtypes = [p, i64, i64, p, p]
    lib.orc_quantize_act.restype = ctypes.c_int
    lib.orc_unpack.argtypes = [p, i64, i64, p]
    lib.orc_unpack.restype = ctypes.c_int
    lib.orc_linear.argtypes = [p, p, i64, i64, i64, p, ctypes.c_int]
    lib.orc_linear.restype = None
    lib.orc_dequant.argtypes = [p, p, p, i64, i64, p]
    lib.orc_dequant.restype = None
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def ternarize_absmean(W: np.ndarray):
    """Absmean ternarization of one tensor (BitNet b1.58, named in "What This
    Paper Is About"; the rule itself is a reading).  W: fp32 [N, K].
    Returns (t int8 [N, K], gamma float)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    t = np.empty((N, K), dtype=np.int8)
    g = np.zeros(1, dtype=np.float32)
    rc = _load().orc_ternarize_absmean(_ptr(W), N, K, _ptr(t), _ptr(g))
    if rc != 0:
        raise ValueError("non-finite weight")
    return t, float(g[0])


def ternarize_segments(W: np.ndarray, seg_rows):
    """Fused projections: each row segment is ternarized on its own with its
    own gamma.  Returns (t [N, K], gamma per segment list, gamma per row)."""
    N, K = W.shape
    if sum(seg_rows) != N:
        raise ValueError("segments do not cover N")
    ts, gammas, grow = [], [], np.empty(N, dtype=np.float32)
    r0 = 0
    for rows in seg_rows:
        t, g = ternarize_absmean(W[r0:r0 + rows])
        ts.append(t)
        gammas.append(g)
        grow[r0:r0 + rows] = g
        r0 += rows
    return np.concatenate(ts, axis=0), gammas, grow


def quantize_act(x_bf16: np.ndarray):
    """Per-token absmax int8 quantization ("Main Findings": 8-bit
    activations).  x_bf16: uint16 bf16 bit patterns [M, K].
    Returns (q int8 [M, K], scale fp32 [M])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    rc = _load().orc_quantize_act(_ptr(x), M, K, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("non-finite activation")
    return q, s


def unpack(packed: np.ndarray, N: int, K: int):
    """Decode the 2-bit packed format (layout stated in oracle.c) into
    ternary int8 [N, K].  Raises on the invalid code 3."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    if p.size != N * K // 4:
        raise ValueError("packed size mismatch")
    t = np.empty((N, K), dtype=np.int8)
    rc = _load().orc_unpack(_ptr(p), N, K, _ptr(t))
    if rc == -1:
        raise ValueError("invalid code 3 in packed weights")
    if rc != 0:
        raise ValueError("K must be a multiple of 16")
    return t


def linear(q: np.ndarray, t: np.ndarray, threads: int = 1):
    """int32 accumulators acc[m, n] = sum_k q[m, k] t[n, k]: the contraction
    the packed W2A8 operators compute ("Methodology in Plain English")."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    t = np.ascontiguousarray(t, dtype=np.int8)
    M, K = q.shape
    N, K2 = t.shape
    if K != K2:
        raise ValueError("K mismatch")
    acc = np.empty((M, N), dtype=np.int32)
    _load().orc_linear(_ptr(q), _ptr(t), M, N, K, _ptr(acc), int(threads))
    return acc


def dequant(acc: np.ndarray, scale: np.ndarray, gamma_row: np.ndarray):
    """y = acc * s_m * gamma(n) in double."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    M, N = acc.shape
    s = np.ascontiguousarray(scale, dtype=np.float32)
    g = np.ascontiguousarray(gamma_row, dtype=np.float32)
    if s.size != M or g.size != N:
        raise ValueError("scale sizes")
    y = np.empty((M, N), dtype=np.float64)
    _load().orc_dequant(_ptr(acc), _ptr(s), _ptr(g), M, N, _ptr(y))
    return y


def max_threads() -> int:
    return int(_load().orc_max_threads())


def forward(W: np.ndarray, seg_rows, x_bf16: np.ndarray, threads: int = 1):
    """Whole path on the CPU: ternarize (per segment), quantize, contract,
    dequantize.  Returns a dict of every intermediate."""
    t, gammas, grow = ternarize_segments(W, seg_rows)
    q, s = quantize_act(x_bf16)
    acc = linear(q, t, threads)
    y = dequant(acc, s, grow)
    return dict(t=t, gammas=gammas, gamma_row=grow, q=q, scale=s, acc=acc, y=y)
