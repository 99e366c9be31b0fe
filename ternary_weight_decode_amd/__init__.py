"""Python binding of libtwd, the gfx950 W2A8 ternary linear library.

Argument marshalling only: every step runs in the C/HIP library
(``libtwd.so``, built in-tree by ``build.py``).  PyTorch supplies device
memory and the current HIP stream.  Importing this package without the built
library raises ``ImportError`` -- there is no fallback implementation.

Names follow the C ABI in ``include/twd.h``: ``quantize_act``,
``ternary_linear``, ``ternary_linear_fused``, ``ternary_linear_bf16``,
``pack_ternary``,
``unpack_ternary``, ``ternarize_absmean``, ``select_kernel``,
``stream_read``, ``stream_copy``; ``Sweep`` wraps ``twd_sweep_table_bytes``,
``twd_sweep_encode`` and ``twd_ternary_sweep``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtwd.so")

TWD_OK = 0
KERNEL_AUTO, KERNEL_DOT, KERNEL_MFMA, KERNEL_MFMA_STAGED, KERNEL_MFMA_TILE = 0, 1, 2, 3, 4
KERNEL_NAMES = {KERNEL_DOT: "dot", KERNEL_MFMA: "mfma", KERNEL_MFMA_STAGED: "mfma_staged",
                KERNEL_MFMA_TILE: "mfma_tile"}
MAX_M, MAX_K, MAX_SEGMENTS = 16, 8192, 4
_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "BAD_CODE", 4: "HIP"}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python ternary_weight_decode_amd/build.py` "
        "or `python -c 'import __graft_entry__ as g; g.build()'` (hipcc --offload-arch=gfx950)")

# PyTorch ships its own HIP runtime with the same soname as ROCm's; loading
# torch first makes libtwd bind to that one, so a process never holds two
# HIP runtimes (device tensors come from torch).
try:
    import torch  # noqa: F401
except ImportError:  # host-side functions still work without torch
    pass

_lib = ctypes.CDLL(LIB_PATH)
_p, _i64, _int, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_lib_version = _sig("twd_version", [], ctypes.c_char_p)
_lib_last_error = _sig("twd_last_error", [], ctypes.c_char_p)
_lib_ternarize = _sig("twd_ternarize_absmean", [_p, _i64, _i64, _p, _p])
_lib_pack = _sig("twd_pack_ternary", [_p, _i64, _i64, _p])
_lib_unpack = _sig("twd_unpack_ternary", [_p, _i64, _i64, _p])
_lib_quantize = _sig("twd_quantize_act", [_p, _i64, _i64, _p, _p, _p])
_lib_linear = _sig("twd_ternary_linear", [_p, _f32, _p, _p, _i64, _i64, _i64, _p, _p, _p])
_lib_fused = _sig("twd_ternary_linear_fused",
                  [_p, _int, _p, _p, _p, _p, _i64, _i64, _p, _p, _p])
_lib_fused_kernel = _sig("twd_ternary_linear_fused_kernel",
                         [_p, _int, _p, _p, _p, _p, _i64, _i64, _p, _p, _int, _p])
_lib_bf16 = _sig("twd_ternary_linear_bf16",
                 [_p, _int, _p, _p, _p, _i64, _i64, _p, _p, _int, _p])
_lib_bf16_ws = _sig("twd_ternary_linear_bf16_ws",
                    [_p, _int, _p, _p, _p, _i64, _i64, _p, _p, _int, _p, _i64, _p])
_lib_bf16_noalloc = _sig("twd_ternary_linear_bf16_noalloc",
                         [_p, _int, _p, _p, _p, _i64, _i64, _p, _p, _int, _p])
_lib_select = _sig("twd_select_kernel", [_i64, _i64, _i64, _int])
_lib_quantize_fp8_rows = _sig("twd_quantize_fp8_rows", [_p, _i64, _i64, _p, _p])
_lib_proj_fp8 = _sig("twd_projection_fp8", [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p])
_lib_proj_bf16 = _sig("twd_projection_bf16", [_p, _p, _i64, _i64, _i64, _p, _p])
_lib_kv_commit = _sig("twd_kv_commit",
                      [_p, _int, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p])
_lib_stream_read = _sig("twd_stream_read", [_p, _i64, _p, _p])


class SweepProjDesc(ctypes.Structure):
    """twd_sweep_proj (include/twd.h)."""
    _fields_ = [("wpacked", _p), ("x_bf16", _p), ("acc", _p), ("y", _p),
                ("K", _i64), ("nseg", _i64), ("seg_rows", _i64 * MAX_SEGMENTS),
                ("seg_gamma", _f32 * MAX_SEGMENTS)]


class SweepPlan(ctypes.Structure):
    """twd_sweep_plan (include/twd.h)."""
    _fields_ = [("table", _p), ("table_bytes", _i64), ("weight_bytes", _i64),
                ("nproj", ctypes.c_int32), ("M", ctypes.c_int32), ("nwg", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("check", ctypes.c_uint32),
                ("reserved", ctypes.c_int32 * 3)]


_lib_tiled_bytes = _sig("twd_sweep_tiled_bytes", [_i64, _i64], _i64)
_lib_ws_bytes = _sig("twd_linear_bf16_workspace_bytes", [_i64, _i64], _i64)
_lib_tile = _sig("twd_sweep_tile_weights", [_p, _i64, _i64, _p])
_lib_sweep_bytes = _sig("twd_sweep_table_bytes", [_p, _int, _i64, _p])
_lib_sweep_encode = _sig("twd_sweep_encode", [_p, _int, _i64, _p, _p, _i64, _p])
_lib_sweep = _sig("twd_ternary_sweep", [_p, _p])
_lib_stream_copy = _sig("twd_stream_copy", [_p, _p, _i64, _p])

EXPORTS = ("twd_version", "twd_last_error", "twd_ternarize_absmean",
           "twd_pack_ternary", "twd_unpack_ternary", "twd_quantize_act",
           "twd_ternary_linear", "twd_ternary_linear_fused",
           "twd_ternary_linear_fused_kernel", "twd_ternary_linear_bf16",
           "twd_linear_bf16_workspace_bytes", "twd_ternary_linear_bf16_ws",
           "twd_ternary_linear_bf16_noalloc",
           "twd_select_kernel", "twd_quantize_fp8_rows", "twd_projection_fp8",
           "twd_projection_bf16", "twd_kv_commit", "twd_stream_read", "twd_stream_copy",
           "twd_sweep_tiled_bytes", "twd_sweep_tile_weights",
           "twd_sweep_table_bytes", "twd_sweep_encode", "twd_ternary_sweep")


class TwdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"twd {_STATUS.get(status, status)}: {message}")
        self.status = status


def _check(status: int):
    if status != TWD_OK:
        raise TwdError(status, _lib_last_error().decode(errors="replace"))


def version() -> str:
    return _lib_version().decode()


# ----------------------------------------------------------------- host side

def _np_ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def ternarize_absmean(W: np.ndarray):
    """Absmean ternarization of one fp32 tensor [N, K] -> (int8 codes, gamma)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes = np.empty((N, K), np.int8)
    g = np.zeros(1, np.float32)
    _check(_lib_ternarize(_np_ptr(W), N, K, _np_ptr(codes), _np_ptr(g)))
    return codes, float(g[0])


def pack_ternary(codes: np.ndarray) -> np.ndarray:
    """int8 codes [N, K] in {-1, 0, 1} -> packed uint8 [N, K/4]."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = codes.shape
    out = np.empty((N, K // 4), np.uint8)
    _check(_lib_pack(_np_ptr(codes), N, K, _np_ptr(out)))
    return out


def unpack_ternary(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if packed.size != N * K // 4:
        raise ValueError("packed size does not match N*K/4")
    codes = np.empty((N, K), np.int8)
    _check(_lib_unpack(_np_ptr(packed), N, K, _np_ptr(codes)))
    return codes


def prepare_weights(W: np.ndarray, seg_rows=None):
    """Offline weight preparation of a (fused) projection: each row segment
    is ternarized with its own gamma, then the whole matrix is packed.
    Returns (packed uint8 [N, K/4], [gamma per segment])."""
    N, K = W.shape
    seg_rows = tuple(seg_rows) if seg_rows is not None else (N,)
    if sum(seg_rows) != N:
        raise ValueError("segments do not cover N")
    codes = np.empty((N, K), np.int8)
    gammas = []
    r0 = 0
    for rows in seg_rows:
        c, g = ternarize_absmean(W[r0:r0 + rows])
        codes[r0:r0 + rows] = c
        gammas.append(g)
        r0 += rows
    return pack_ternary(codes), gammas


# --------------------------------------------------------------- device side

def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtypes=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return t.numel() * t.element_size()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def quantize_act(x, xq=None, xscale=None, stream=None):
    """Per-token absmax int8 quantization of a bf16 [M, K] device tensor.
    Returns (xq int8 [M, K], xscale fp32 [M])."""
    torch = _torch()
    _need(x.dim() == 2, "x must be [M, K]")
    M, K = x.shape
    _need(xq is None or tuple(xq.shape) == (M, K), "xq must be [M, K]")
    _need(xscale is None or xscale.numel() >= M, "xscale must hold M values")
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if xscale is None:
        xscale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(_lib_quantize(_dev_ptr(x, "x", (torch.bfloat16, torch.int16)), M, K,
                         _dev_ptr(xq, "xq", (torch.int8,)),
                         _dev_ptr(xscale, "xscale", (torch.float32,)),
                         _stream(stream)))
    return xq, xscale


def _outputs(M, N, device, acc, y, want_acc, want_y):
    torch = _torch()
    _need(acc is None or tuple(acc.shape) == (M, N), "acc must be [M, N]")
    _need(y is None or tuple(y.shape) == (M, N), "y must be [M, N]")
    if acc is None and want_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=device)
    if y is None and want_y:
        y = torch.empty((M, N), dtype=torch.float32, device=device)
    return acc, y


def ternary_linear(wpacked, gamma, xq, xscale, N, acc=None, y=None,
                   want_acc=True, want_y=True, stream=None):
    """acc = xq . t^T (int32), y = acc * xscale[m] * gamma (fp32).
    wpacked: uint8 device tensor of N*K/4 bytes.  Returns (acc, y)."""
    torch = _torch()
    _need(xq.dim() == 2, "xq must be [M, K]")
    M, K = xq.shape
    _need(_nbytes(wpacked) >= N * K // 4, "wpacked holds fewer than N*K/4 bytes")
    _need(xscale.numel() >= M, "xscale must hold M values")
    acc, y = _outputs(M, N, xq.device, acc, y, want_acc, want_y)
    _check(_lib_linear(_dev_ptr(wpacked, "wpacked", (torch.uint8,)), float(gamma),
                       _dev_ptr(xq, "xq", (torch.int8,)),
                       _dev_ptr(xscale, "xscale", (torch.float32,)), M, K, N,
                       _dev_ptr(acc, "acc", (torch.int32,)),
                       _dev_ptr(y, "y", (torch.float32,)), _stream(stream)))
    return acc, y


def ternary_linear_fused(wpacked, seg_rows, seg_gamma, xq, xscale, acc=None,
                         y=None, want_acc=True, want_y=True, kernel=KERNEL_AUTO,
                         stream=None):
    """One launch over concatenated row segments (fused Q/K/V or gate/up),
    each dequantized with its own gamma.  Returns (acc, y)."""
    torch = _torch()
    _need(xq.dim() == 2, "xq must be [M, K]")
    M, K = xq.shape
    seg_rows = [int(r) for r in seg_rows]
    nseg = len(seg_rows)
    _need(len(seg_gamma) == nseg, "one gamma per segment")
    N = int(sum(seg_rows))
    _need(_nbytes(wpacked) >= N * K // 4, "wpacked holds fewer than N*K/4 bytes")
    _need(xscale.numel() >= M, "xscale must hold M values")
    rows = (ctypes.c_int64 * max(nseg, 1))(*seg_rows)
    gam = (ctypes.c_float * max(nseg, 1))(*[float(g) for g in seg_gamma])
    acc, y = _outputs(M, N, xq.device, acc, y, want_acc, want_y)
    args = (_dev_ptr(wpacked, "wpacked", (torch.uint8,)), nseg, rows, gam,
            _dev_ptr(xq, "xq", (torch.int8,)),
            _dev_ptr(xscale, "xscale", (torch.float32,)), M, K,
            _dev_ptr(acc, "acc", (torch.int32,)), _dev_ptr(y, "y", (torch.float32,)))
    if kernel == KERNEL_AUTO:
        _check(_lib_fused(*args, _stream(stream)))
    else:
        _check(_lib_fused_kernel(*args, int(kernel), _stream(stream)))
    return acc, y


def ternary_linear_bf16(wpacked, seg_rows, seg_gamma, x, acc=None, y=None,
                        want_acc=True, want_y=True, kernel=KERNEL_AUTO, stream=None):
    """Whole projection in one launch: bf16 activations x [M, K] are
    quantized per token inside the kernel, then contracted with the packed
    ternary weights over the row segments.  Returns (acc, y)."""
    torch = _torch()
    _need(x.dim() == 2, "x must be [M, K]")
    M, K = x.shape
    seg_rows = [int(r) for r in seg_rows]
    nseg = len(seg_rows)
    _need(len(seg_gamma) == nseg, "one gamma per segment")
    N = int(sum(seg_rows))
    _need(_nbytes(wpacked) >= N * K // 4, "wpacked holds fewer than N*K/4 bytes")
    rows = (ctypes.c_int64 * max(nseg, 1))(*seg_rows)
    gam = (ctypes.c_float * max(nseg, 1))(*[float(g) for g in seg_gamma])
    acc, y = _outputs(M, N, x.device, acc, y, want_acc, want_y)
    _check(_lib_bf16(_dev_ptr(wpacked, "wpacked", (torch.uint8,)), nseg, rows, gam,
                     _dev_ptr(x, "x", (torch.bfloat16, torch.int16)), M, K,
                     _dev_ptr(acc, "acc", (torch.int32,)), _dev_ptr(y, "y", (torch.float32,)),
                     int(kernel), _stream(stream)))
    return acc, y


def linear_bf16_workspace_bytes(M: int, K: int) -> int:
    """Workspace bytes ternary_linear_bf16_ws needs for (M, K); -1 if invalid."""
    return int(_lib_ws_bytes(int(M), int(K)))


def ternary_linear_bf16_ws(wpacked, seg_rows, seg_gamma, x, workspace=None, acc=None, y=None,
                           want_acc=True, want_y=True, kernel=KERNEL_AUTO, stream=None):
    """ternary_linear_bf16 with the form picked by width and shape: two
    launches (quantizer into `workspace`, a device uint8 tensor of at least
    linear_bf16_workspace_bytes(M, K) bytes, then the int8 linear) where they
    are faster, else one.  workspace=None: always one launch."""
    torch = _torch()
    _need(x.dim() == 2, "x must be [M, K]")
    M, K = x.shape
    seg_rows = [int(r) for r in seg_rows]
    nseg = len(seg_rows)
    _need(len(seg_gamma) == nseg, "one gamma per segment")
    N = int(sum(seg_rows))
    _need(_nbytes(wpacked) >= N * K // 4, "wpacked holds fewer than N*K/4 bytes")
    rows = (ctypes.c_int64 * max(nseg, 1))(*seg_rows)
    gam = (ctypes.c_float * max(nseg, 1))(*[float(g) for g in seg_gamma])
    acc, y = _outputs(M, N, x.device, acc, y, want_acc, want_y)
    ws = _dev_ptr(workspace, "workspace", (torch.uint8,)) if workspace is not None else None
    _check(_lib_bf16_ws(_dev_ptr(wpacked, "wpacked", (torch.uint8,)), nseg, rows, gam,
                        _dev_ptr(x, "x", (torch.bfloat16, torch.int16)), M, K,
                        _dev_ptr(acc, "acc", (torch.int32,)), _dev_ptr(y, "y", (torch.float32,)),
                        int(kernel), ws, _nbytes(workspace) if workspace is not None else 0,
                        _stream(stream)))
    return acc, y


def ternary_linear_bf16_noalloc(wpacked, seg_rows, seg_gamma, x, acc, y, kernel=KERNEL_AUTO,
                                stream=None):
    """ternary_linear_bf16_ws with the library's own per-device workspace: the
    call itself allocates nothing, so acc [M, N] int32 and y [M, N] fp32 are
    required (either may be None to skip it).  Calls that overlap on one
    device race on that workspace."""
    torch = _torch()
    _need(x.dim() == 2, "x must be [M, K]")
    M, K = x.shape
    seg_rows = [int(r) for r in seg_rows]
    nseg = len(seg_rows)
    _need(len(seg_gamma) == nseg, "one gamma per segment")
    N = int(sum(seg_rows))
    _need(_nbytes(wpacked) >= N * K // 4, "wpacked holds fewer than N*K/4 bytes")
    for t, name in ((acc, "acc"), (y, "y")):
        _need(t is None or tuple(t.shape) == (M, N), f"{name} must be [M, N]")
    rows = (ctypes.c_int64 * max(nseg, 1))(*seg_rows)
    gam = (ctypes.c_float * max(nseg, 1))(*[float(g) for g in seg_gamma])
    _check(_lib_bf16_noalloc(_dev_ptr(wpacked, "wpacked", (torch.uint8,)), nseg, rows, gam,
                             _dev_ptr(x, "x", (torch.bfloat16, torch.int16)), M, K,
                             _dev_ptr(acc, "acc", (torch.int32,)),
                             _dev_ptr(y, "y", (torch.float32,)), int(kernel), _stream(stream)))
    return acc, y


def select_kernel(M: int, K: int, N: int, bf16_input: bool = True) -> int:
    """Kernel family the width dispatch picks (a KERNEL_* value other than
    KERNEL_AUTO) for ternary_linear_bf16 (bf16_input) or for the int8 entry
    points, or -1 for an unsupported shape."""
    return int(_lib_select(M, K, N, 1 if bf16_input else 0))


def quantize_fp8_rows(W: np.ndarray):
    """Per-output-row FP8 (OCP E4M3) quantization of fp32 weights [N, K] for
    the fast projection -> (codes uint8 [N, K], scale fp32 [N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes = np.empty((N, K), np.uint8)
    scale = np.empty(N, np.float32)
    _check(_lib_quantize_fp8_rows(_np_ptr(W), N, K, _np_ptr(codes), _np_ptr(scale)))
    return codes, scale


def projection_fp8(wq, wscale, x, y=None, want_codes=False, stream=None):
    """Fast (FP8) projection of bf16 activations x [M, K] with E4M3 weight
    codes wq [N, K] and per-row scales wscale [N].  Returns y fp32 [M, N],
    or (y, xq uint8 [M, K], xscale fp32 [M]) with want_codes."""
    torch = _torch()
    _need(x.dim() == 2 and wq.dim() == 2, "x must be [M, K], wq [N, K]")
    M, K = x.shape
    N = wq.shape[0]
    _need(wq.shape[1] == K, "wq must be [N, K]")
    _need(wscale.numel() >= N, "wscale must hold N values")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(tuple(y.shape) == (M, N), "y must be [M, N]")
    xq = xs = None
    if want_codes:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(_lib_proj_fp8(_dev_ptr(wq, "wq", (torch.uint8,)),
                         _dev_ptr(wscale, "wscale", (torch.float32,)),
                         _dev_ptr(x, "x", (torch.bfloat16, torch.int16)), M, K, N,
                         _dev_ptr(y, "y", (torch.float32,)),
                         _dev_ptr(xq, "xq", (torch.uint8,)),
                         _dev_ptr(xs, "xscale", (torch.float32,)), _stream(stream)))
    return (y, xq, xs) if want_codes else y


def projection_bf16(w, x, y=None, stream=None):
    """Critical (bf16) projection: y fp32 [M, N] = x [M, K] . w [N, K]^T."""
    torch = _torch()
    _need(x.dim() == 2 and w.dim() == 2, "x must be [M, K], w [N, K]")
    M, K = x.shape
    N = w.shape[0]
    _need(w.shape[1] == K, "w must be [N, K]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(tuple(y.shape) == (M, N), "y must be [M, N]")
    _check(_lib_proj_bf16(_dev_ptr(w, "w", (torch.bfloat16, torch.int16)),
                          _dev_ptr(x, "x", (torch.bfloat16, torch.int16)), M, K, N,
                          _dev_ptr(y, "y", (torch.float32,)), _stream(stream)))
    return y


def kv_segment_positions(c0: int, nseg: int):
    """Positions held by each KV segment: c0, 2 c0, 4 c0, ..."""
    return [c0 << s for s in range(nseg)]


def kv_commit(segments, c0: int, layers: int, row_bytes: int, block, W: int, n_mat, n_new,
              state_in, state_out, stream=None):
    """Accepted-prefix KV commit: store the first n_mat rows of block
    ([layers][2][W][row_bytes] bytes on the device) into the segment buffers
    at positions L.., and write the new (P, L, S, error) state to state_out.
    segments: device tensors, segment s holding [layers][2][c0 2^s][row_bytes]
    bytes; n_mat, n_new: device int32 (one element used); state_in /
    state_out: device int32[4], distinct."""
    torch = _torch()
    nseg = len(segments)
    seg_ptrs = []
    for s, t in enumerate(segments):
        seg_ptrs.append(_dev_ptr(t, f"segment {s}").value)
        _need(_nbytes(t) >= layers * 2 * (c0 << s) * row_bytes,
              f"segment {s} smaller than layers * 2 * c0 * 2^s * row_bytes")
    _need(_nbytes(block) >= layers * 2 * W * row_bytes, "block smaller than its rows")
    for name, t, n in (("n_mat", n_mat, 1), ("n_new", n_new, 1), ("state_in", state_in, 4),
                       ("state_out", state_out, 4)):
        _dev_ptr(t, name, (torch.int32,))
        _need(t.numel() >= n, f"{name} must hold at least {n} int32 value(s)")
    ptrs = (ctypes.c_void_p * max(nseg, 1))(*seg_ptrs)
    _check(_lib_kv_commit(ptrs, nseg, int(c0), int(layers), int(row_bytes),
                          _dev_ptr(block, "block"), int(W), _dev_ptr(n_mat, "n_mat"),
                          _dev_ptr(n_new, "n_new"), _dev_ptr(state_in, "state_in"),
                          _dev_ptr(state_out, "state_out"), _stream(stream)))


def stream_read(buf, nbytes: int, sink, stream=None):
    """Launch the plain streaming-read reference kernel over nbytes of buf."""
    _need(_nbytes(buf) >= nbytes, "buf smaller than nbytes")
    _need(_nbytes(sink) >= 1024, "sink needs 1024 bytes")
    _check(_lib_stream_read(_dev_ptr(buf, "buf"), int(nbytes), _dev_ptr(sink, "sink"),
                            _stream(stream)))


def stream_copy(src, dst, nbytes: int, stream=None):
    """Launch the plain copy kernel: nbytes from src to dst."""
    _need(_nbytes(src) >= nbytes and _nbytes(dst) >= nbytes, "buffers smaller than nbytes")
    _check(_lib_stream_copy(_dev_ptr(src, "src"), _dev_ptr(dst, "dst"), int(nbytes),
                            _stream(stream)))


# ------------------------------------------------------ multi-projection sweep

def sweep_tiled_bytes(N: int, K: int) -> int:
    """Bytes of [N, K] weights in the sweep's tiled layout."""
    n = int(_lib_tiled_bytes(int(N), int(K)))
    if n < 0:
        raise ValueError("N must be >= 0 and K a multiple of 64")
    return n


def tile_for_sweep(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Packed weights [N, K/4] (host) -> the sweep's tiled layout (host
    uint8, sweep_tiled_bytes(N, K) bytes)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    _need(packed.size == N * K // 4, "packed size does not match N*K/4")
    out = np.empty(sweep_tiled_bytes(N, K), np.uint8)
    _check(_lib_tile(_np_ptr(packed), int(N), int(K), _np_ptr(out)))
    return out


def sweep_descs(projs, M: int):
    """ctypes array of twd_sweep_proj from (wpacked_ptr, x_ptr, acc_ptr, y_ptr,
    K, seg_rows, seg_gamma) tuples of plain integers (host-side planning)."""
    arr = (SweepProjDesc * len(projs))()
    for i, (w, x, acc, y, K, seg_rows, seg_gamma) in enumerate(projs):
        seg_rows = [int(r) for r in seg_rows]
        if not 1 <= len(seg_rows) <= MAX_SEGMENTS or len(seg_gamma) != len(seg_rows):
            raise ValueError("1..4 segments, one gamma each")
        d = arr[i]
        d.wpacked, d.x_bf16, d.acc, d.y = w, x, acc, y
        d.K, d.nseg = int(K), len(seg_rows)
        for s, (r, g) in enumerate(zip(seg_rows, seg_gamma)):
            d.seg_rows[s] = r
            d.seg_gamma[s] = float(g)
    return arr


def sweep_encode(descs, M: int, table_dev_ptr: int):
    """Plan a sweep on the host: returns (table image as uint8 numpy, plan)."""
    n = ctypes.c_int64(0)
    _check(_lib_sweep_bytes(descs, len(descs), int(M), ctypes.byref(n)))
    img = np.zeros(n.value, np.uint8)
    plan = SweepPlan()
    _check(_lib_sweep_encode(descs, len(descs), int(M), ctypes.c_void_p(table_dev_ptr),
                             _np_ptr(img), n.value, ctypes.byref(plan)))
    return img, plan


class Sweep:
    """One launch over a list of independent projections at width M.

    projs: sequence of (wtiled, seg_rows, seg_gamma, x, acc, y) with device
    tensors wtiled (uint8, the weights in the sweep's tiled layout:
    tile_for_sweep), x (bf16 [M, K]), acc (int32 [M, N]
    or None), y (fp32 [M, N] or None).  The table is planned on the host,
    copied once to a device buffer held by this object, and every run() is a
    single asynchronous launch on the stream (capturable into a graph).  The
    tensors must stay alive and in place while the object is used."""

    def __init__(self, projs):
        torch = _torch()
        if not projs:
            raise ValueError("empty projection list")
        M = None
        rows = []
        keep = []
        for (w, seg_rows, seg_gamma, x, acc, y) in projs:
            _need(x.dim() == 2, "x must be [M, K]")
            m, K = x.shape
            M = m if M is None else M
            _need(m == M, "every projection takes the same M")
            N = int(sum(int(r) for r in seg_rows))
            need = int(_lib_tiled_bytes(N, int(K)))  # -1: a K the library rejects below
            _need(_nbytes(w) >= need,
                  "the tiled weights hold fewer than sweep_tiled_bytes(N, K) bytes")
            _need(acc is None or tuple(acc.shape) == (M, N), "acc must be [M, N]")
            _need(y is None or tuple(y.shape) == (M, N), "y must be [M, N]")
            ptr = lambda t, name, dt: (_dev_ptr(t, name, dt).value if t is not None else None)
            rows.append((ptr(w, "wpacked", (torch.uint8,)),
                         ptr(x, "x", (torch.bfloat16, torch.int16)),
                         ptr(acc, "acc", (torch.int32,)), ptr(y, "y", (torch.float32,)),
                         K, seg_rows, seg_gamma))
            keep.append((w, x, acc, y))
        descs = sweep_descs(rows, M)
        n = ctypes.c_int64(0)
        _check(_lib_sweep_bytes(descs, len(descs), int(M), ctypes.byref(n)))
        self.table = torch.empty(n.value, dtype=torch.uint8, device=projs[0][3].device)
        img, self.plan = sweep_encode(descs, M, self.table.data_ptr())
        self.table.copy_(torch.from_numpy(img))
        torch.cuda.synchronize()
        self._keep = keep
        self.M = M

    @property
    def weight_bytes(self) -> int:
        return int(self.plan.weight_bytes)

    def run(self, stream=None):
        _check(_lib_sweep(ctypes.byref(self.plan), _stream(stream)))
