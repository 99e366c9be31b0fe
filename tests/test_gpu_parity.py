"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: quantized activations, scales and int32 accumulators bit-exact; fp32
outputs within 1e-6 relative of the oracle's double-precision value, per
element.  Cases span several 16-row tiles, partial 256-wide K slices and
ragged N tails, every width M = 1..16 for the matrix-core kernel and 1..4 for
the VALU kernel, fused segments, the single-linear workload and full-size
2B / 4B projections.
"""
import sys

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6


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


def to_dev_bf16(torch, x_bits):
    return torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)


def check_y(y, yref):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - yref)
    bad = err > REL_TOL * np.abs(yref)
    assert not bad.any(), f"{bad.sum()} y values outside 1e-6 relative, worst {err[bad].max()}"


_prep_cache = {}


def prepared(twd, torch, W, segs, key):
    if key not in _prep_cache:
        packed, gammas = twd.prepare_weights(W, segs)
        _prep_cache.clear()
        _prep_cache[key] = (torch.from_numpy(packed).cuda(), gammas)
    return _prep_cache[key]


def run_case(env, W, segs, x, kernel, key, ref=None, fused=False):
    """Run one case through the C ABI and compare with the oracle.  fused:
    the one-launch bf16 entry point instead of quantize_act + linear."""
    torch, twd, orc = env
    wp, gammas = prepared(twd, torch, W, segs, key)
    M, K = x.shape
    log(f"case {key} M={M} K={K} N={W.shape[0]} segs={segs} kernel={kernel} fused={fused}")
    if ref is None:
        ref = orc.forward(W, segs, x)
    assert gammas == ref["gammas"]
    xd = to_dev_bf16(torch, x)
    if fused:
        acc, y = twd.ternary_linear_bf16(wp, segs, gammas, xd, kernel=kernel)
        torch.cuda.synchronize()
    else:
        xq, xs = twd.quantize_act(xd)
        acc, y = twd.ternary_linear_fused(wp, segs, gammas, xq, xs, kernel=kernel)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(xq.cpu().numpy(), ref["q"])
        np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32),
                                      ref["scale"].view(np.uint32))
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(y.cpu().numpy(), ref["y"])
    return acc, y


# ------------------------------------------------------------ quantize_act

@pytest.mark.parametrize("M,K", [(1, 256), (3, 2560), (16, 6912), (16, 8192), (2, 8),
                                 (5, 65536), (300, 64)])
def test_quantize_act_bit_exact(env, M, K):
    torch, twd, orc = env
    rng = np.random.default_rng([M, K])
    xf = rng.standard_normal((M, K), dtype=np.float32)
    if M > 2:
        xf[1] = 0.0                       # all-zero row
        xf[2, :: max(K // 50, 1)] *= 20  # outlier channels
    x = wl.f32_to_bf16_bits(xf)
    log(f"quantize M={M} K={K}")
    xq, xs = twd.quantize_act(to_dev_bf16(torch, x))
    torch.cuda.synchronize()
    q, s = orc.quantize_act(x)
    np.testing.assert_array_equal(xq.cpu().numpy(), q)
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32), s.view(np.uint32))


def test_quantize_act_ties(env):
    torch, twd, orc = env
    row = np.zeros((1, 64), np.float32)
    row[0, :6] = [127, 62.5, -62.5, 0.5, 1.5, 2.5]
    x = wl.f32_to_bf16_bits(row)
    xq, xs = twd.quantize_act(to_dev_bf16(torch, x))
    torch.cuda.synchronize()
    assert xq.cpu().numpy()[0, :6].tolist() == [127, 62, -62, 0, 2, 2]
    assert float(xs.cpu()[0]) == 1.0


# ------------------------------------------------------------------- linear

SMALL_SHAPES = [
    (64, (1,)),            # one partial slice, one row; three waves idle
    (320, (17,)),          # partial last slice, ragged tile
    (2560, (130,)),        # ten full slices, ragged tail
    (1536, (64, 33, 33)),  # three segments, ragged
    (768, (50, 50)),       # two segments
    (6912, (33,)),         # 27 slices: seven per wave, one wave a slice short
    (8192, (20,)),         # the largest K
    (512, (4104, 4104)),   # N >= 6400: the dot kernel's 8 rows x 4 waves shape at M=1
    (256, (6400, 6417)),   # N >= 12800: 8 rows x 8 waves at M=1, ragged
]

# (kernel family, widest M it takes); KERNEL_MFMA runs the straight-line
# matrix-core kernel where its registers allow and KERNEL_MFMA_TILE the
# tile-owner one for K <= 3072; both run the staged kernel otherwise
FAMILIES = [("dot", 4), ("mfma", 16), ("mfma_staged", 16), ("mfma_tile", 16)]
# every (family, width) pair a family takes
FAMILY_WIDTHS = [(fam, M) for fam, max_m in FAMILIES for M in range(1, max_m + 1)]


def family(twd, name):
    return {"dot": twd.KERNEL_DOT, "mfma": twd.KERNEL_MFMA,
            "mfma_staged": twd.KERNEL_MFMA_STAGED, "mfma_tile": twd.KERNEL_MFMA_TILE}[name]


@pytest.mark.parametrize("fused", [False, True], ids=["int8", "bf16"])
@pytest.mark.parametrize("K,segs", SMALL_SHAPES)
@pytest.mark.parametrize("fam,M", FAMILY_WIDTHS)
def test_kernel_parity(env, fam, M, K, segs, fused):
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=1, M=M, K=K, seg_rows=segs)
    run_case(env, W, segs, x, family(twd, fam), ("rand", 1, K, segs), fused=fused)


@pytest.mark.parametrize("M", [1, 2, 3, 8, 16])
def test_fused_bf16_zero_rows_and_outliers(env, M):
    """All-zero token rows (scale 0, output 0) and x20 outlier channels."""
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=7, M=M, K=2560, seg_rows=(48,))
    xf = wl.bf16_bits_to_f32(x).copy()
    xf[0] = 0.0
    if M > 1:
        xf[1, ::97] *= 20.0
    x = wl.f32_to_bf16_bits(xf)
    for kernel in ((twd.KERNEL_MFMA, twd.KERNEL_MFMA_STAGED, twd.KERNEL_MFMA_TILE,
                    twd.KERNEL_DOT) if M <= 4
                   else (twd.KERNEL_MFMA, twd.KERNEL_MFMA_STAGED, twd.KERNEL_MFMA_TILE)):
        acc, y = run_case(env, W, segs, x, kernel, ("rand", 7), fused=True)
        assert not acc[0].any() and not y[0].any()


@pytest.mark.parametrize("M", [1, 2, 4, 5, 8, 16])
def test_auto_dispatch_parity_and_determinism(env, M):
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=2, M=M, K=1024, seg_rows=(200,))
    a1, y1 = run_case(env, W, segs, x, twd.KERNEL_AUTO, ("rand", 2, 1024, segs))
    a2, y2 = run_case(env, W, segs, x, twd.KERNEL_AUTO, ("rand", 2, 1024, segs))
    assert torch.equal(a1, a2) and torch.equal(y1, y2)


def test_single_linear_workload(env):
    """The single-linear case: M=1, K=256, N=512, seed 0."""
    torch, twd, orc = env
    W, segs, x = wl.single_case(seed=0)
    for kernel in (twd.KERNEL_AUTO, twd.KERNEL_DOT, twd.KERNEL_MFMA, twd.KERNEL_MFMA_STAGED,
                   twd.KERNEL_MFMA_TILE):
        for fused in (False, True):
            run_case(env, W, segs, x, kernel, ("single", 0), fused=fused)


def test_width_invariance(env):
    """Row m of an M-wide call equals the 1-wide call on that row."""
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=3, M=16, K=2560, seg_rows=(96,))
    wp, gammas = prepared(twd, torch, W, segs, ("rand", 3))
    xq, xs = twd.quantize_act(to_dev_bf16(torch, x))
    full = {}
    for kernel in (twd.KERNEL_MFMA_STAGED, twd.KERNEL_MFMA, twd.KERNEL_MFMA_TILE,
                   twd.KERNEL_DOT):
        for M in (4, 2, 1) if kernel == twd.KERNEL_DOT else (16, 13, 10, 8, 5, 4, 1):
            acc, _ = twd.ternary_linear_fused(wp, segs, gammas, xq[:M].contiguous(),
                                              xs[:M].contiguous(), kernel=kernel)
            full[(kernel, M)] = acc
    torch.cuda.synchronize()
    ref = full[(twd.KERNEL_MFMA_STAGED, 16)]
    for (kernel, M), acc in full.items():
        assert torch.equal(acc, ref[:M]), (kernel, M)


def test_fused_equals_separate_calls(env):
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=4, M=4, K=512, seg_rows=(48, 16, 16))
    wp, gammas = prepared(twd, torch, W, segs, ("rand", 4))
    xq, xs = twd.quantize_act(to_dev_bf16(torch, x))
    acc, y = twd.ternary_linear_fused(wp, segs, gammas, xq, xs)
    r0 = 0
    for rows, g in zip(segs, gammas):
        part = wp.view(-1)[r0 * 512 // 4:(r0 + rows) * 512 // 4]
        a2, y2 = twd.ternary_linear(part, g, xq, xs, rows)
        torch.cuda.synchronize()
        assert torch.equal(acc[:, r0:r0 + rows], a2)
        assert torch.equal(y[:, r0:r0 + rows], y2)
        r0 += rows


def test_timing_mode_outputs_optional(env):
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=5, M=2, K=256, seg_rows=(40,))
    wp, gammas = prepared(twd, torch, W, segs, ("rand", 5))
    xq, xs = twd.quantize_act(to_dev_bf16(torch, x))
    acc, y = twd.ternary_linear_fused(wp, segs, gammas, xq, xs)
    a_only, none_y = twd.ternary_linear_fused(wp, segs, gammas, xq, xs, want_y=False)
    none_a, y_only = twd.ternary_linear_fused(wp, segs, gammas, xq, xs, want_acc=False)
    torch.cuda.synchronize()
    assert none_y is None and none_a is None
    assert torch.equal(acc, a_only) and torch.equal(y, y_only)


def test_invariants_on_gpu(env):
    """Zero weights give zero; an all-+1 row gives the activation row sum."""
    torch, twd, orc = env
    M, K, N = 3, 512, 20
    x = wl.f32_to_bf16_bits(np.random.default_rng(6).standard_normal((M, K),
                                                                     dtype=np.float32))
    codes = np.zeros((N, K), np.int8)
    codes[1] = 1
    codes[2] = -1
    wp = torch.from_numpy(twd.pack_ternary(codes)).cuda()
    xq, xs = twd.quantize_act(to_dev_bf16(torch, x))
    for kernel in (twd.KERNEL_DOT, twd.KERNEL_MFMA, twd.KERNEL_MFMA_STAGED,
                   twd.KERNEL_MFMA_TILE):
        acc, y = twd.ternary_linear_fused(wp, (N,), (1.0,), xq, xs, kernel=kernel)
        torch.cuda.synchronize()
        a = acc.cpu().numpy()
        rowsum = xq.cpu().numpy().astype(np.int64).sum(axis=1)
        assert not a[:, 0].any() and not a[:, 3:].any()
        np.testing.assert_array_equal(a[:, 1], rowsum)
        np.testing.assert_array_equal(a[:, 2], -rowsum)
        assert not y.cpu().numpy()[:, 0].any()


def test_extreme_values(env):
    """|acc| at its maximum: q = +-127 everywhere, every weight +-1, K = 8192."""
    torch, twd, orc = env
    M, K, N = 16, 8192, 32
    xf = np.full((M, K), 1.0, np.float32)
    xf[1::2] = -1.0
    x = wl.f32_to_bf16_bits(xf)
    W = np.ones((N, K), np.float32)
    W[::3] = -1.0
    for kernel in (twd.KERNEL_MFMA_STAGED, twd.KERNEL_MFMA, twd.KERNEL_MFMA_TILE,
                   twd.KERNEL_DOT):
        xs_ = x[:4] if kernel == twd.KERNEL_DOT else x
        acc, _ = run_case(env, W, (N,), xs_, kernel, ("extreme",))
        assert abs(int(acc.abs().max())) == 127 * K


# ---------------------------------------------------------- full-size layers

@pytest.mark.parametrize("set_name,workload,layer,M", [
    ("2b", "2b_decode", 0, 1),
    ("2b", "2b_decode", 29, 1),
    ("2b", "2b_verify", 11, 2),
    ("2b", "2b_verify", 19, 3),
    ("2b", "2b_verify", 7, 4),
    ("2b", "2b_verify", 7, 8),
    ("2b", "2b_verify", 23, 16),
    ("4b", "4b_stack", 35, 1),
    ("4b", "4b_stack", 17, 4),
    ("4b", "4b_stack", 0, 16),
] + [("2b", "2b_sweep_outlier", (5 * M + 3) % 30, M) for M in range(1, 17)])
def test_full_size_layer(env, set_name, workload, layer, M):
    """Every projection of one full-size layer, in the dispatch the benchmark
    times (one launch per projection, AUTO), in both forms, compared element
    by element; the outlier workload at every width 1..16."""
    torch, twd, orc = env
    ls = wl.LAYER_SETS[set_name]
    threads = orc.max_threads()
    for pi, proj in enumerate(ls.projs):
        W = wl.layer_weights(ls, layer, pi)
        x = wl.layer_activations(workload, proj.K, M, layer, pi,
                                 outliers=workload == "2b_sweep_outlier")
        ref = orc.forward(W, proj.segs, x, threads=threads)
        run_case(env, W, proj.segs, x, twd.KERNEL_AUTO, (set_name, layer, pi), ref=ref)
        run_case(env, W, proj.segs, x, twd.KERNEL_AUTO, (set_name, layer, pi), ref=ref,
                 fused=True)


# ------------------------------------------------------------ graph replay

def test_linear_graph_replays_match_oracle(env):
    """Every linear kernel family, in the one-launch bf16 form and in the
    two-launch form (quantize_act, then the int8 linear), captured into one
    graph: three replays, with eager work and synchronization between them,
    each checked against the oracle (quantized activations and scales
    bit-exact, acc bit-exact, y within 1e-6) and bit-identical to the eager
    results."""
    torch, twd, orc = env
    cases = [("dot", 1, 2560, (96,)), ("dot", 3, 768, (40, 24)),
             ("mfma", 2, 2560, (64, 32, 32)), ("mfma", 9, 6912, (33,)),
             ("mfma_tile", 5, 1536, (130,)), ("mfma_staged", 16, 8192, (20,))]
    runs = []
    for i, (fam, M, K, segs) in enumerate(cases):
        W, segs, x = wl.random_case(seed=40 + i, M=M, K=K, seg_rows=segs)
        packed, gammas = twd.prepare_weights(W, segs)
        N = int(sum(segs))
        runs.append(dict(
            ref=orc.forward(W, segs, x),
            fam=family(twd, fam), segs=segs, gammas=gammas,
            wp=torch.from_numpy(packed).cuda(), x=to_dev_bf16(torch, x),
            acc_f=torch.empty((M, N), dtype=torch.int32, device="cuda"),
            y_f=torch.empty((M, N), device="cuda"),
            xq=torch.empty((M, K), dtype=torch.int8, device="cuda"),
            xs=torch.empty(M, device="cuda"),
            acc_i=torch.empty((M, N), dtype=torch.int32, device="cuda"),
            y_i=torch.empty((M, N), device="cuda")))
    outs = ("acc_f", "y_f", "xq", "xs", "acc_i", "y_i")

    def all_cases():
        for r in runs:
            twd.ternary_linear_bf16(r["wp"], r["segs"], r["gammas"], r["x"], acc=r["acc_f"],
                                    y=r["y_f"], kernel=r["fam"])
            twd.quantize_act(r["x"], xq=r["xq"], xscale=r["xs"])
            twd.ternary_linear_fused(r["wp"], r["segs"], r["gammas"], r["xq"], r["xs"],
                                     acc=r["acc_i"], y=r["y_i"], kernel=r["fam"])

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        all_cases()
    torch.cuda.synchronize()
    refs = [{k: r[k].clone() for k in outs} for r in runs]
    for r, ref in zip(runs, refs):  # the two forms agree with each other
        assert torch.equal(ref["acc_f"], ref["acc_i"])
        assert torch.equal(ref["y_f"].view(torch.int32), ref["y_i"].view(torch.int32))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            all_cases()
    for rep in range(3):
        for r in runs:
            for k in outs:
                r[k].fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for i, (r, ref) in enumerate(zip(runs, refs)):
            for k in outs:
                a, b = r[k], ref[k]
                if a.dtype == torch.float32:
                    a, b = a.view(torch.int32), b.view(torch.int32)
                assert torch.equal(a, b), f"replay {rep}, case {cases[i]}, {k}"
            o = r["ref"]
            np.testing.assert_array_equal(r["xq"].cpu().numpy(), o["q"])
            np.testing.assert_array_equal(r["xs"].cpu().numpy().view(np.uint32),
                                          o["scale"].view(np.uint32))
            for acc_k, y_k in (("acc_f", "y_f"), ("acc_i", "y_i")):
                np.testing.assert_array_equal(r[acc_k].cpu().numpy(), o["acc"])
                check_y(r[y_k].cpu().numpy(), o["y"])
        _ = sum(float(r["y_f"].sum()) for r in runs)  # eager work between replays


# ------------------------------------------------------------- error paths

def test_fused_errors_on_gpu(env):
    torch, twd, orc = env
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    wp = torch.zeros(64 * 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(twd.TwdError) as e:
        twd.ternary_linear_bf16(wp, (64,), (1.0,),
                                torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == 2
    with pytest.raises(twd.TwdError) as e:
        twd.ternary_linear_bf16(wp, (64,), (1.0,), torch.zeros((5, 256), dtype=torch.bfloat16,
                                                               device="cuda"), kernel=twd.KERNEL_DOT)
    assert e.value.status == 2
    acc, y = twd.ternary_linear_bf16(wp, (64,), (1.0,), x[:0])
    assert acc.shape == (0, 64)


def test_errors_on_gpu(env):
    torch, twd, orc = env
    xq = torch.zeros((17, 256), dtype=torch.int8, device="cuda")
    xs = torch.ones(17, device="cuda")
    wp = torch.zeros(64 * 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(twd.TwdError) as e:
        twd.ternary_linear(wp, 1.0, xq, xs, 64)
    assert e.value.status == 2
    with pytest.raises(twd.TwdError) as e:
        twd.ternary_linear(wp, 1.0, xq[:4, :100].contiguous(), xs[:4], 64)
    assert e.value.status == 2
    with pytest.raises(twd.TwdError) as e:
        twd.ternary_linear(wp[1:], 1.0, xq[:4], xs[:4], 32)  # misaligned weights
    assert e.value.status == 1
    # empty width: no launch, outputs untouched
    acc, y = twd.ternary_linear(wp, 1.0, xq[:0], xs[:0], 64)
    assert acc.shape == (0, 64)


def test_measurement_helpers(env):
    """The copy kernel copies exactly its bytes (its counter readings
    calibrate the HBM byte counts); the read kernel runs without error."""
    torch, twd, orc = env
    n = (1 << 20) + 48
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n + 64, dtype=torch.uint8, device="cuda")
    twd.stream_copy(src, dst, n)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    twd.stream_read(src, n, sink)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert not dst[n:].any()


def _random_shapes(seed=2024):
    """One seeded random draw per width M = 1..16: K a multiple of 64 up to
    4096, 1..4 segments of 1..400 rows."""
    rng = np.random.default_rng(seed)
    shapes = []
    for M in range(1, 17):
        K = 64 * int(rng.integers(1, 65))
        nseg = int(rng.integers(1, 5))
        segs = tuple(int(v) for v in rng.integers(1, 401, size=nseg))
        shapes.append((M, K, segs))
    return shapes


@pytest.mark.parametrize("fam,M,K,segs",
                         [(fam, M, K, segs) for fam, max_m in FAMILIES
                          for M, K, segs in _random_shapes() if M <= max_m])
def test_random_shapes(env, fam, M, K, segs):
    """Random shapes through every family, both forms, against the oracle."""
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=11, M=M, K=K, seg_rows=segs)
    ref = orc.forward(W, segs, x)
    for fused in (False, True):
        run_case(env, W, segs, x, family(twd, fam), ("rand", 11, K, segs), ref=ref, fused=fused)
