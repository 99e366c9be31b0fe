"""CPU tests of the C ABI: every symbol the header declares is exported, the
host-side weight preparation matches the oracle bit for bit, and argument
checks reject bad calls before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT, read_golden
import workloads as wl


@pytest.fixture(scope="module")
def twd():
    from ternary_weight_decode_amd import build as libbuild
    if not os.path.exists(libbuild.LIB):
        libbuild.build()
    import ternary_weight_decode_amd as twd
    return twd


def header_functions():
    src = open(os.path.join(ROOT, "include", "twd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(twd_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(twd):
    names = header_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(twd.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(names) == set(twd.EXPORTS)


def test_version(twd):
    assert "gfx950" in twd.version()


# ------------------------------------------------------------- pack / unpack

@pytest.mark.parametrize("N,K", [(1, 16), (3, 64), (17, 256), (5, 2560), (2, 8192)])
def test_pack_roundtrip_against_oracle_unpack(twd, orc, N, K):
    rng = np.random.default_rng([N, K])
    codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    packed = twd.pack_ternary(codes)
    assert packed.shape == (N, K // 4)
    np.testing.assert_array_equal(orc.unpack(packed, N, K), codes)
    np.testing.assert_array_equal(twd.unpack_ternary(packed, N, K), codes)


def test_pack_golden(twd):
    g = read_golden("packed_word.txt")
    codes = np.array([[int(v) for v in g["T"]]], np.int8)
    assert twd.pack_ternary(codes)[0].tolist() == [int(v, 16) for v in g["BYTES"]]
    h = read_golden("hand_case_k16.txt")
    codes = np.array([[int(v) for v in h["T0"]], [int(v) for v in h["T1"]]], np.int8)
    packed = twd.pack_ternary(codes)
    assert packed[0].tolist() == [int(v, 16) for v in h["PACKED0"]]
    assert packed[1].tolist() == [int(v, 16) for v in h["PACKED1"]]


def test_pack_rejects_bad_codes(twd):
    codes = np.zeros((2, 32), np.int8)
    codes[1, 5] = 2
    with pytest.raises(twd.TwdError) as e:
        twd.pack_ternary(codes)
    assert e.value.status == 3
    with pytest.raises(twd.TwdError) as e:
        twd.pack_ternary(np.zeros((2, 24), np.int8))
    assert e.value.status == 1


def test_unpack_rejects_code3_everywhere(twd):
    base = twd.pack_ternary(np.zeros((1, 16), np.int8))
    for byte in range(4):
        for field in range(4):
            p = base.copy()
            p[0, byte] |= np.uint8(3 << (2 * field))
            with pytest.raises(twd.TwdError) as e:
                twd.unpack_ternary(p, 1, 16)
            assert e.value.status == 3


# ------------------------------------------------------------------ ternarize

@pytest.mark.parametrize("shape,sigma", [((512, 256), 1.0), ((640, 2560), 0.02),
                                         ((7, 48), 3.0), ((1, 16), 1.0)])
def test_ternarize_bit_exact_vs_oracle(twd, orc, shape, sigma):
    rng = np.random.default_rng(list(shape))
    W = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    c1, g1 = twd.ternarize_absmean(W)
    c2, g2 = orc.ternarize_absmean(W)
    assert np.float32(g1).view(np.uint32) == np.float32(g2).view(np.uint32)
    np.testing.assert_array_equal(c1, c2)


def test_ternarize_ties_zero_and_nonfinite(twd):
    c, g = twd.ternarize_absmean(np.array([[1, 7, 0, 0]], np.float32))
    assert g == 2.0 and c.tolist() == [[0, 1, 0, 0]]
    c, g = twd.ternarize_absmean(np.zeros((4, 16), np.float32))
    assert g == 0.0 and not c.any()
    W = np.ones((2, 16), np.float32)
    W[0, 0] = np.nan
    with pytest.raises(twd.TwdError):
        twd.ternarize_absmean(W)


def test_prepare_weights_segments_vs_oracle(twd, orc):
    W = wl.layer_weights(wl.SET_2B, 0, 0)[:, :256]  # qkv segments, narrowed K
    segs = wl.SET_2B.projs[0].segs
    packed, gammas = twd.prepare_weights(W, segs)
    t, og, _ = orc.ternarize_segments(W, segs)
    assert gammas == og
    np.testing.assert_array_equal(orc.unpack(packed, W.shape[0], W.shape[1]), t)


# ---------------------------------------------------- argument checks (no GPU)

def _fused(twd, wp=0x1000, nseg=1, rows=(64,), gam=(1.0,), xq=0x2000, xs=0x3000,
           M=1, K=256, acc=0x4000, y=0x5000, kernel=0):
    r = (ctypes.c_int64 * 4)(*rows)
    g = (ctypes.c_float * 4)(*gam)
    return twd._lib_fused_kernel(wp, nseg, r, g, xq, xs, M, K, acc, y, kernel, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=17), 2), (dict(M=-1), 2), (dict(K=100), 2), (dict(K=0), 2),
    (dict(K=8256), 2), (dict(nseg=0), 1), (dict(nseg=5), 1),
    (dict(rows=(-1,)), 1), (dict(wp=None), 1), (dict(xq=None), 1),
    (dict(xs=None), 1), (dict(acc=None, y=None), 1), (dict(wp=0x1008), 1),
    (dict(xq=0x2004), 1), (dict(y=0x5002), 1), (dict(kernel=7), 1),
    (dict(kernel=1, M=5), 2),
])
def test_linear_rejects_before_launch(twd, kw, status):
    assert _fused(twd, **kw) == status
    assert twd._lib_last_error()


def test_bf16_linear_rejects_before_launch(twd):
    f = twd._lib_bf16
    r = (ctypes.c_int64 * 1)(64)
    g = (ctypes.c_float * 1)(1.0)
    assert f(0x1000, 1, r, g, 0x2000, 17, 256, 0x4000, 0x5000, 0, None) == 2
    assert f(0x1000, 1, r, g, 0x2000, 1, 96, 0x4000, 0x5000, 0, None) == 2
    assert f(0x1000, 1, r, g, None, 1, 256, 0x4000, 0x5000, 0, None) == 1
    assert f(0x1000, 1, r, g, 0x2008, 1, 256, 0x4000, 0x5000, 0, None) == 1
    assert f(0x1000, 1, r, g, 0x2000, 5, 256, 0x4000, 0x5000, 1, None) == 2
    assert f(0x1000, 1, r, g, 0x2000, 0, 256, 0x4000, 0x5000, 0, None) == 0


def test_linear_empty_is_noop(twd):
    # M == 0 or N == 0: nothing to compute, nothing launched, even with
    # placeholder pointers
    assert _fused(twd, M=0) == 0
    assert _fused(twd, rows=(0,)) == 0


def test_quantize_rejects_before_launch(twd):
    q = twd._lib_quantize
    assert q(0x1000, 1, 12, 0x2000, 0x3000, None) == 2       # K % 8
    assert q(0x1000, 1, 0, 0x2000, 0x3000, None) == 2        # K == 0
    assert q(0x1000, -1, 64, 0x2000, 0x3000, None) == 1      # M < 0
    assert q(None, 1, 64, 0x2000, 0x3000, None) == 1         # null
    assert q(0x1008, 1, 64, 0x2000, 0x3000, None) == 1       # alignment
    assert q(0x1000, 0, 64, None, None, None) == 0           # empty


def test_select_kernel(twd):
    for bf16 in (True, False):
        assert twd.select_kernel(1, 2560, 2560, bf16) == twd.KERNEL_DOT
        assert twd.select_kernel(16, 1024, 2560, bf16) == twd.KERNEL_MFMA
        assert twd.select_kernel(16, 2560, 2560, bf16) == twd.KERNEL_MFMA
        # wide outputs take the tile-owner kernel (K <= 3072): from M = 2
        # with the bf16 quantization inside, from M = 3 for int8 activations
        for M in (3, 5, 6, 16):
            assert twd.select_kernel(M, 2560, 13824, bf16) == twd.KERNEL_MFMA_TILE
        assert twd.select_kernel(4, 8192, 2560, bf16) == twd.KERNEL_MFMA
        # M = 2: the tile kernel for a wide output and the straight-line one
        # otherwise with the quantization inside, the dot kernel for int8
        # activations
        assert twd.select_kernel(2, 2560, 13824, bf16) == (
            twd.KERNEL_MFMA_TILE if bf16 else twd.KERNEL_DOT)
        assert twd.select_kernel(2, 2560, 2560, bf16) == (
            twd.KERNEL_MFMA if bf16 else twd.KERNEL_DOT)
        # a long K past four waves' register budget: int8 activations split
        # K over more waves of the straight-line kernel; with the bf16
        # quantization inside, the staged kernel is faster
        for M, K, N in ((16, 6912, 2560), (16, 8192, 3072), (7, 6912, 2560)):
            assert twd.select_kernel(M, K, N, bf16) == (
                twd.KERNEL_MFMA_STAGED if bf16 else twd.KERNEL_MFMA)
        assert twd.select_kernel(6, 6912, 2560, bf16) == twd.KERNEL_MFMA
        for M in range(1, 17):
            assert twd.select_kernel(M, 2560, 13824, bf16) in (
                twd.KERNEL_DOT, twd.KERNEL_MFMA, twd.KERNEL_MFMA_STAGED, twd.KERNEL_MFMA_TILE)
        assert twd.select_kernel(17, 2560, 2560, bf16) == -1
        assert twd.select_kernel(1, 100, 2560, bf16) == -1
        assert twd.select_kernel(1, 2560, 0, bf16) == -1
    assert twd.select_kernel(16, 6912, 2560) == twd.KERNEL_MFMA_STAGED  # default: bf16


def test_measurement_helpers_reject_before_launch(twd):
    r, c = twd._lib_stream_read, twd._lib_stream_copy
    assert r(0x1000, 24, 0x2000, None) == 1          # bytes % 16
    assert r(0x1000, -16, 0x2000, None) == 1         # negative
    assert r(None, 16, 0x2000, None) == 1            # null
    assert r(0x1008, 16, 0x2000, None) == 1          # alignment
    assert r(0x1000, 0, None, None) == 0             # empty: no launch
    assert c(0x1000, 0x2000, 24, None) == 1
    assert c(0x1000, None, 16, None) == 1
    assert c(0x1000, 0x2008, 16, None) == 1
    assert c(0x1000, 0x2000, 0, None) == 0


# ------------------------------------------------ role-dependent projections

@pytest.mark.parametrize("shape,sigma", [((7, 48), 0.02), ((33, 320), 1.0), ((4, 4096), 3.0)])
def test_quantize_fp8_rows_bit_exact_vs_oracle(twd, orc, shape, sigma):
    rng = np.random.default_rng(sum(shape))
    W = rng.standard_normal(shape).astype(np.float32) * np.float32(sigma)
    W[0] = 0.0                      # zero row
    W[1, 3] = 57.0                  # an outlier sets the row scale
    W[2, :] = np.float32(2.0 ** -20)  # one large value; the rest scale below
    W[2, 1] = np.float32(1.0)         # the smallest E4M3 subnormal -> zero codes
    W[3, :5] = np.float32(2.0 ** -9) * np.arange(1, 6, dtype=np.float32)  # subnormals
    codes, scale = twd.quantize_fp8_rows(W)
    rc, rs = orc.quantize_fp8_rows(W)
    np.testing.assert_array_equal(codes, rc)
    np.testing.assert_array_equal(scale.view(np.uint32), rs.view(np.uint32))


def test_quantize_fp8_rows_hand_and_errors(twd):
    g = read_golden("fp8_e4m3_hand.txt")
    W = np.array([[float(v) for v in g["W"]]], dtype=np.float32)
    codes, scale = twd.quantize_fp8_rows(W)
    assert [int(c) for c in codes[0]] == [int(c, 16) for c in g["WQ"]] and scale[0] == 1.0
    with pytest.raises(twd.TwdError):
        twd.quantize_fp8_rows(np.array([[1.0, np.inf]], np.float32))


def test_projection_rejects_before_launch(twd):
    f8, f16 = twd._lib_proj_fp8, twd._lib_proj_bf16
    ok = (0x1000, 0x2000, 0x3000)
    assert f8(*ok, 17, 256, 64, 0x4000, None, None, None) == 2     # M > 16
    assert f8(*ok, 1, 8, 64, 0x4000, None, None, None) == 2        # K % 16
    assert f8(*ok, 1, 4112, 64, 0x4000, None, None, None) == 2     # K > 4096
    assert f8(*ok, 1, 256, (1 << 24) + 1, 0x4000, None, None, None) == 2
    assert f8(*ok, 1, 256, -1, 0x4000, None, None, None) == 1
    assert f8(0x1000, None, 0x3000, 1, 256, 64, 0x4000, None, None, None) == 1
    assert f8(0x1008, 0x2000, 0x3000, 1, 256, 64, 0x4000, None, None, None) == 1
    assert f8(*ok, 1, 256, 64, 0x4002, None, None, None) == 1      # y alignment
    assert f8(*ok, 1, 256, 64, 0x4000, 0x5004, None, None) == 1    # xq alignment
    assert f8(*ok, 0, 256, 64, None, None, None, None) == 0        # empty
    assert f8(*ok, 3, 256, 0, None, None, None, None) == 0
    assert f16(0x1000, 0x3000, 1, 12, 64, 0x4000, None) == 2       # K % 8
    assert f16(0x1000, 0x3000, 1, 4104, 64, 0x4000, None) == 2
    assert f16(None, 0x3000, 1, 256, 64, 0x4000, None) == 1
    assert f16(0x1000, 0x3008, 1, 256, 64, 0x4000, None) == 1
    assert f16(0x1000, 0x3000, 0, 256, 64, None, None) == 0
    assert twd._lib_last_error()


def test_linear_bf16_workspace_bytes(twd):
    """The two-launch form's workspace: int8 rows [M][K], then the fp32
    scales [M] at the next 16-byte boundary."""
    assert twd.linear_bf16_workspace_bytes(16, 6912) == 16 * 6912 + 64
    assert twd.linear_bf16_workspace_bytes(1, 64) == 64 + 4
    assert twd.linear_bf16_workspace_bytes(3, 64) == 192 + 12
    assert twd.linear_bf16_workspace_bytes(0, 64) == 0
    for M, K in ((17, 64), (-1, 64), (1, 100), (1, 0), (1, 16384)):
        assert twd.linear_bf16_workspace_bytes(M, K) == -1


def test_linear_bf16_ws_rejects_before_launch(twd):
    """A misaligned or short workspace is refused before anything launches;
    the linear's own checks apply as for twd_ternary_linear_bf16."""
    f = twd._lib_bf16_ws
    rows = (ctypes.c_int64 * 1)(16)
    gam = (ctypes.c_float * 1)(1.0)
    w, x, y, ws = 0x10000, 0x20000, 0x30000, 0x40000
    need = twd.linear_bf16_workspace_bytes(16, 6912)

    def call(M=16, K=6912, ws_ptr=ws, ws_bytes=need, kernel=0):
        return f(w, 1, rows, gam, x, M, K, None, y, kernel, ws_ptr, ws_bytes, None)

    assert call(ws_ptr=ws + 8) == 1
    assert call(ws_bytes=need - 1) == 1 and b"needed" in twd._lib_last_error()
    assert call(K=100) == 2 and call(M=17) == 2
    assert call(M=0) == 0  # nothing to do, nothing launched


def test_linear_bf16_noalloc_rejects_before_launch(twd):
    """The allocation-free form applies the linear's checks before it looks up
    its static workspace or launches anything."""
    f = twd._lib_bf16_noalloc
    rows = (ctypes.c_int64 * 1)(16)
    gam = (ctypes.c_float * 1)(1.0)
    w, x, y = 0x10000, 0x20000, 0x30000

    def call(M=16, K=6912, kernel=0):
        return f(w, 1, rows, gam, x, M, K, None, y, kernel, None)

    assert call(K=100) == 2 and call(M=17) == 2 and call(K=8256) == 2
    assert call(kernel=99) == 1
    assert call(M=0) == 0  # nothing to do, nothing looked up or launched


def test_kv_commit_rejects_before_launch(twd):
    f = twd._lib_kv_commit
    segs = (ctypes.c_void_p * 4)(0x10000, 0x20000, 0x30000, 0x40000)
    ok = dict(seg=segs, nseg=4, c0=8, layers=30, row=1280, block=0x50000, W=9,
              nm=0x60000, nn=0x60010, si=0x70000, so=0x70010)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["seg"], a["nseg"], a["c0"], a["layers"], a["row"], a["block"], a["W"],
                 a["nm"], a["nn"], a["si"], a["so"], None)

    assert call(nseg=0) == 2 and call(nseg=25) == 2
    assert call(W=0) == 1 and call(W=65) == 1
    assert call(row=24) == 1 and call(row=0) == 1 and call(c0=0) == 1
    assert call(c0=1 << 30, nseg=2) == 2                 # capacity >= 2^31
    assert call(layers=40000) == 2
    assert call(block=None) == 1 and call(si=None) == 1
    assert call(block=0x50008) == 1                       # alignment
    assert call(so=0x70008) == 1                          # overlapping state words
    bad = (ctypes.c_void_p * 4)(0x10000, 0x20008, 0x30000, 0x40000)
    assert call(seg=bad) == 1
    nul = (ctypes.c_void_p * 4)(0x10000, None, 0x30000, 0x40000)
    assert call(seg=nul) == 1
    assert twd._lib_last_error()


class _FakeDev:
    """Stands in for a device tensor in binding checks that must fail before
    any library call (no GPU here)."""

    def __init__(self, n, dtype="int32", contiguous=True, cuda=True, esize=4):
        import torch
        self.n, self.dtype = n, getattr(torch, dtype)
        self._contig, self.is_cuda, self.esize = contiguous, cuda, esize

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        return 0x100000

    def numel(self):
        return self.n

    def element_size(self):
        return self.esize


def test_kv_commit_binding_checks_tensors(twd):
    """The binding refuses host, non-contiguous or short tensors for the
    segments, counts and state words before calling the library."""
    pytest.importorskip("torch")
    c0, layers, row = 2, 2, 16
    segs = [_FakeDev(layers * 2 * (c0 << s) * row, "uint8", esize=1) for s in range(2)]
    block = _FakeDev(layers * 2 * 4 * row, "uint8", esize=1)
    good = dict(n_mat=_FakeDev(1), n_new=_FakeDev(1), state_in=_FakeDev(4),
                state_out=_FakeDev(4))

    def call(segments=segs, **kw):
        a = dict(good, **kw)
        twd.kv_commit(segments, c0, layers, row, block, 4, a["n_mat"], a["n_new"],
                      a["state_in"], a["state_out"])

    for bad in (dict(segments=[segs[0], _FakeDev(10 ** 6, "uint8", cuda=False, esize=1)]),
                dict(segments=[segs[0], _FakeDev(10 ** 6, "uint8", contiguous=False, esize=1)]),
                dict(n_mat=_FakeDev(0)), dict(n_new=_FakeDev(1, cuda=False)),
                dict(state_in=_FakeDev(3)), dict(state_out=_FakeDev(4, contiguous=False)),
                dict(state_in=_FakeDev(4, "float32"))):
        with pytest.raises(ValueError):
            call(**bad)


def test_profile_summary_refuses_runs_of_other_sources(tmp_path):
    """A counter record is stamped with the kernel-source hash of the run it
    summarizes: a run that printed another hash is refused, so stale counters
    can never carry the current sources' hash."""
    import json
    import subprocess
    import sys
    run = tmp_path / "run.json"
    run.write_text(json.dumps({"kernel_source_hash": "0" * 16,
                               "projection_source_hash": "0" * 16,
                               "sweep_source_hash": "0" * 16}) + "\n")
    d = str(tmp_path)
    for flag in ("--summarize-profile", "--summarize-projection", "--summarize-sweep"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), flag, d, d, d,
                            "--profile-run-json", str(run), "--profile-out", d],
                           capture_output=True, text=True, cwd=ROOT)
        assert r.returncode != 0 and "profile" in r.stderr
        assert not any(p.suffix == ".json" and p.name != "run.json" for p in tmp_path.iterdir())


def test_linear_bf16_noalloc_binding_checks_tensors(twd):
    """The allocation-free binding refuses host tensors and outputs of the
    wrong shape before calling the library."""
    torch = pytest.importorskip("torch")
    M, K, N = 4, 128, 16
    wp = torch.zeros(N * K // 4, dtype=torch.uint8)
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    acc = torch.zeros((M, N), dtype=torch.int32)
    y = torch.zeros((M, N), dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensor"):
        twd.ternary_linear_bf16_noalloc(wp, (N,), (1.0,), x, acc, y)
    with pytest.raises(ValueError, match=r"acc must be \[M, N\]"):
        twd.ternary_linear_bf16_noalloc(wp, (N,), (1.0,), x, acc[:, :8], y)
    with pytest.raises(ValueError, match="one gamma per segment"):
        twd.ternary_linear_bf16_noalloc(wp, (8, 8), (1.0,), x, acc, y)
