"""CPU oracle for the W2A8 ternary linear layer and the role-dependent
(FP8 fast / bf16 critical) projections -- TEST INFRASTRUCTURE ONLY.

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


NATIVE_FLAGS = ["-O3", "-march=native"]


def build_native(path=None) -> str:
    """Compile ``oracle.c`` with ``-O3 -march=native`` (plain loops, still no
    fast-math or contraction) into a separate library for timing the oracle
    on the machine it runs on; the tests keep the portable ``-O2`` build."""
    import tempfile
    path = path or os.path.join(tempfile.gettempdir(), f"liboracle_native_{os.getpid()}.so")
    cmd = ["gcc", "-std=c11", *NATIVE_FLAGS, "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-o", path, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return path


def select(path) -> None:
    """Use the oracle library at ``path`` (e.g. from build_native) for the
    calls that follow in this process."""
    global _lib, _LIB_PATH
    _LIB_PATH = path
    _lib = None
    _load()


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
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float, p]
    lib.orc_e4m3_encode.restype = ctypes.c_int
    lib.orc_quantize_fp8_rows.argtypes = [p, i64, i64, p, p]
    lib.orc_quantize_fp8_rows.restype = ctypes.c_int
    lib.orc_quantize_act_fp8.argtypes = [p, i64, i64, p, p]
    lib.orc_quantize_act_fp8.restype = ctypes.c_int
    lib.orc_fp8_linear.argtypes = [p, p, i64, i64, i64, p, p]
    lib.orc_fp8_linear.restype = ctypes.c_int
    lib.orc_bf16_linear.argtypes = [p, p, i64, i64, i64, p, p]
    lib.orc_bf16_linear.restype = None
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


# ---------------------------------------------------------------------------
# Role-dependent projections ("Methodology in Plain English", the paragraph
# on M1: "fast" projections for drafting, "critical" ones for autoregressive
# steps and verification, FP8 draft projections on H20).  Readings stated at
# the top of oracle.c.
# ---------------------------------------------------------------------------

def e4m3_decode(code: int) -> float:
    """Value of an OCP E4M3 code (NaN for 0x7F / 0xFF)."""
    return float(_load().orc_e4m3_decode(int(code) & 0xFF))


def e4m3_encode(v: float) -> int:
    """fp32 value -> E4M3 code, round to nearest, ties to even.  Raises if v
    is not finite or rounds beyond 448."""
    out = ctypes.c_uint8(0)
    rc = _load().orc_e4m3_encode(ctypes.c_float(v), ctypes.byref(out))
    if rc != 0:
        raise ValueError(f"{v!r} has no finite E4M3 code")
    return int(out.value)


def quantize_fp8_rows(W: np.ndarray):
    """Per-output-row absmax FP8 quantization of weights (fp32 [N, K]).
    Returns (codes uint8 [N, K], scale fp32 [N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes = np.empty((N, K), dtype=np.uint8)
    s = np.empty(N, dtype=np.float32)
    if _load().orc_quantize_fp8_rows(_ptr(W), N, K, _ptr(codes), _ptr(s)) != 0:
        raise ValueError("non-finite weight")
    return codes, s


def quantize_act_fp8(x_bf16: np.ndarray):
    """Per-token absmax FP8 quantization of bf16 activations [M, K].
    Returns (codes uint8 [M, K], scale fp32 [M])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    codes = np.empty((M, K), dtype=np.uint8)
    s = np.empty(M, dtype=np.float32)
    rc = _load().orc_quantize_act_fp8(_ptr(x), M, K, _ptr(codes), _ptr(s))
    if rc != 0:
        raise ValueError("non-finite activation or K > 8192")
    return codes, s


def fp8_linear(xq: np.ndarray, wq: np.ndarray):
    """Exact sum_k dec(xq[m, k]) dec(wq[n, k]) and the same sum of absolute
    products, as float64 [M, N] each."""
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("K mismatch")
    dot = np.empty((M, N), dtype=np.float64)
    absdot = np.empty((M, N), dtype=np.float64)
    if _load().orc_fp8_linear(_ptr(xq), _ptr(wq), M, N, K, _ptr(dot), _ptr(absdot)) != 0:
        raise ValueError("NaN code")
    return dot, absdot


def bf16_linear(x_bf16: np.ndarray, w_bf16: np.ndarray):
    """sum_k x[m, k] w[n, k] over bf16 bit patterns, in double, and the sum of
    absolute products, as float64 [M, N] each."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("K mismatch")
    dot = np.empty((M, N), dtype=np.float64)
    absdot = np.empty((M, N), dtype=np.float64)
    _load().orc_bf16_linear(_ptr(x), _ptr(w), M, N, K, _ptr(dot), _ptr(absdot))
    return dot, absdot


def fast_projection(W: np.ndarray, x_bf16: np.ndarray):
    """The fast (FP8) projection on the CPU: quantize the weights per row and
    the activations per token, contract exactly, dequantize in double.
    Returns a dict of every intermediate."""
    wq, ws = quantize_fp8_rows(W)
    xq, xs = quantize_act_fp8(x_bf16)
    dot, absdot = fp8_linear(xq, wq)
    scale = xs.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]
    return dict(wq=wq, wscale=ws, xq=xq, xscale=xs, dot=dot, absdot=absdot,
                y=dot * scale, yabs=absdot * scale)
