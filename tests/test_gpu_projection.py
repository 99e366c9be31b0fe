"""GPU parity of the role-dependent projections (fast FP8 / critical bf16)
through the C ABI, against the CPU oracle.

Bar.  Activation codes and scales (fast role) bit-exact.  y: the kernels
multiply exact values (E4M3 and bf16 products are exact in fp32) and add
them in fp32, then scale twice, so per element
    |y - y_ref| <= gamma_K * sum_k |x_k w_k| * s + 3 u |y_ref|,
gamma_K = K u / (1 - K u), u = 2^-24 (the standard bound for a K-term fp32
sum; s = s_m s_n for the fast role, 1 for the critical one), with y_ref
the oracle's exact (fast) or double (critical) value.  Zero rows and columns
give exact zeros.
"""
import sys

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    import ternary_weight_decode_amd as twd
    oracle.build(force=False)
    return torch, twd, oracle


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def check_bound(y, yref, yabs, K, what):
    y = np.asarray(y, dtype=np.float64)
    g = K * U / (1 - K * U)
    bound = g * yabs + 3 * U * np.abs(yref)
    err = np.abs(y - yref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} values outside the fp32 summation bound, "
                           f"worst err {err[bad].max()} vs bound {bound[bad].min()}")
    zero = yabs == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero y where every product is zero"
    ratio = float((err / np.maximum(yabs, 1e-300)).max())
    log(f"  {what}: max |err| / sum|products| = {ratio:.3g} (bound {g:.3g})")


def fast_case(env, W, x_bits, tag):
    torch, twd, orc = env
    M, K = x_bits.shape
    N = W.shape[0]
    log(f"fast case {tag} M={M} K={K} N={N}")
    wq, ws = orc.quantize_fp8_rows(W)
    r = orc.fast_projection(W, x_bits)
    y, xq, xs = twd.projection_fp8(torch.from_numpy(wq).cuda(), torch.from_numpy(ws).cuda(),
                                   dev_bf16(torch, x_bits), want_codes=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq.cpu().numpy(), r["xq"])
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32), r["xscale"].view(np.uint32))
    check_bound(y.cpu().numpy(), r["y"], r["yabs"], K, f"fast {tag}")
    return y


def critical_case(env, W, x_bits, tag):
    torch, twd, orc = env
    M, K = x_bits.shape
    N = W.shape[0]
    log(f"critical case {tag} M={M} K={K} N={N}")
    wb = wl.f32_to_bf16_bits(W)
    dot, absdot = orc.bf16_linear(x_bits, wb)
    y = twd.projection_bf16(dev_bf16(torch, wb), dev_bf16(torch, x_bits))
    torch.cuda.synchronize()
    check_bound(y.cpu().numpy(), dot, absdot, K, f"critical {tag}")
    return y


SHAPES = [(16, 17), (256, 40), (1040, 129), (2560, 300), (3072, 64), (4096, 70)]


@pytest.mark.parametrize("K,N", SHAPES)
@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_fast_projection_parity(env, M, K, N):
    W, _, x = wl.random_case(40 + M, M, K, (N,), w_sigma=0.02)
    fast_case(env, W, x, f"K{K}N{N}")


@pytest.mark.parametrize("K,N", [(8, 9), (24, 33)] + SHAPES)
@pytest.mark.parametrize("M", [1, 3, 16])
def test_critical_projection_parity(env, M, K, N):
    W, _, x = wl.random_case(60 + M, M, K, (N,), w_sigma=0.02)
    critical_case(env, W, x, f"K{K}N{N}")


def test_zero_rows_columns_and_outliers(env):
    M, K, N = 6, 2560, 100
    W, _, x = wl.random_case(7, M, K, (N,), w_sigma=0.02)
    W[5] = 0.0
    W[17, 9] = 3.0
    xf = wl.bf16_bits_to_f32(x)
    xf[2] = 0.0
    xf[4, ::97] *= 40.0
    x = wl.f32_to_bf16_bits(xf)
    y = fast_case(env, W, x, "zeros").cpu().numpy()
    assert not y[2].any() and not y[:, 5].any()
    y = critical_case(env, W, x, "zeros").cpu().numpy()
    assert not y[2].any() and not y[:, 5].any()


def test_span_split_and_determinism(env):
    """More rows than one launch covers (every wave keeps at most 4 tiles'
    weight scales): the call runs as several launches over row spans."""
    torch, twd, orc = env
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    span = 4 * 16 * cus * 16
    M, K, N = 2, 16, span + 37
    W, _, x = wl.random_case(9, M, K, (N,), w_sigma=0.02)
    y1 = fast_case(env, W, x, "span")
    wq, ws = orc.quantize_fp8_rows(W)
    y2 = twd.projection_fp8(torch.from_numpy(wq).cuda(), torch.from_numpy(ws).cuda(),
                            dev_bf16(torch, x))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    critical_case(env, W, x, "span")


_head = {}


def head_prepared(twd):
    if not _head:
        W = wl.head_weights()
        wq, ws = twd.quantize_fp8_rows(W)
        _head.update(W=W, wq=wq, ws=ws, wb=wl.f32_to_bf16_bits(W))
    return _head


@pytest.mark.parametrize("M", [1, 16])
def test_full_output_projection_sampled(env, M):
    """The 2B-class output projection, 2560 -> 128256, at full size in the
    launch configuration the benchmark times; 320 sampled rows against the
    oracle (the weight codes of those rows also against the oracle's)."""
    torch, twd, orc = env
    K, N = wl.HEAD_K, wl.HEAD_N
    log(f"full output projection M={M}: preparing weights")
    h = head_prepared(twd)
    W, wq, ws, wb = h["W"], h["wq"], h["ws"], h["wb"]
    x = wl.head_activations(M)
    rows = np.sort(np.random.default_rng(M).choice(N, 320, replace=False))
    rows[-1] = N - 1
    oq, os_ = orc.quantize_fp8_rows(W[rows])
    np.testing.assert_array_equal(wq[rows], oq)
    np.testing.assert_array_equal(ws[rows].view(np.uint32), os_.view(np.uint32))
    log(f"full output projection M={M}: running")
    y, xq, xs = twd.projection_fp8(torch.from_numpy(wq).cuda(), torch.from_numpy(ws).cuda(),
                                   dev_bf16(torch, x), want_codes=True)
    yc = twd.projection_bf16(dev_bf16(torch, wb), dev_bf16(torch, x))
    torch.cuda.synchronize()
    rq, rs = orc.quantize_act_fp8(x)
    np.testing.assert_array_equal(xq.cpu().numpy(), rq)
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    dot, absdot = orc.fp8_linear(rq, oq)
    s = rs.astype(np.float64)[:, None] * os_.astype(np.float64)[None, :]
    check_bound(y.cpu().numpy()[:, rows], dot * s, absdot * s, K, f"fast full M={M}")
    dot, absdot = orc.bf16_linear(x, wb[rows])
    check_bound(yc.cpu().numpy()[:, rows], dot, absdot, K, f"critical full M={M}")


def test_graph_replays_match_oracle(env):
    """Both roles captured into one graph: three replays, with eager work and
    synchronization between them, each within the fp32 summation bound of the
    oracle and bit-identical to the eager results."""
    torch, twd, orc = env
    M, K, N = 5, 2560, 1000
    W, _, x = wl.random_case(11, M, K, (N,), w_sigma=0.02)
    r8 = orc.fast_projection(W, x)
    d16, a16 = orc.bf16_linear(x, wl.f32_to_bf16_bits(W))
    wq, ws = orc.quantize_fp8_rows(W)
    wq_d, ws_d = torch.from_numpy(wq).cuda(), torch.from_numpy(ws).cuda()
    wb = dev_bf16(torch, wl.f32_to_bf16_bits(W))
    xd = dev_bf16(torch, x)
    y8 = torch.empty((M, N), device="cuda")
    y16 = torch.empty((M, N), device="cuda")

    def both():
        twd.projection_fp8(wq_d, ws_d, xd, y=y8)
        twd.projection_bf16(wb, xd, y=y16)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        both()
    torch.cuda.synchronize()
    ref8, ref16 = y8.clone(), y16.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            both()
    for rep in range(3):
        y8.fill_(float("nan"))
        y16.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y8.view(torch.int32), ref8.view(torch.int32)), f"fast replay {rep}"
        assert torch.equal(y16.view(torch.int32), ref16.view(torch.int32)), f"critical replay {rep}"
        check_bound(y8.cpu().numpy(), r8["y"], r8["yabs"], K, f"fast replay {rep}")
        check_bound(y16.cpu().numpy(), d16, a16, K, f"critical replay {rep}")
        _ = (y8.sum() + y16.sum()).item()  # eager work between replays
