"""GPU parity of the multi-projection sweep (twd_ternary_sweep) against the
CPU oracle, through the C ABI.

Bar, as for the one-launch linear: int32 accumulators bit-exact, fp32 outputs
within 1e-6 relative of the oracle's double-precision value.  Cases: random
projection lists at every width M = 1..16 (ragged K and N, 1..4 segments,
empty projections, K = 64 and K = 8192), one full-size 2B-class layer at
every width on the outlier workload, whole layer sets in the benchmark's
launch (the 2B set at M = 1, 2, 4, 8, 11 and on the outlier workload at
M = 16, the 4B stack at M = 1, 4, 16; sampled rows against the oracle, every
row against the per-projection launches), outputs deferred as 24-bit
accumulators on ragged and misaligned outputs, graph replays checked against
the oracle, and a table that does not match its plan (nothing written).
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


def dev_bf16(torch, x_bits):
    return torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)


def check_y(y, yref, what=""):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - yref)
    bad = err > REL_TOL * np.abs(yref)
    assert not bad.any(), f"{what}: {bad.sum()} y values outside 1e-6 relative"


class Case:
    """One projection of a sweep: host inputs, device tensors, oracle."""

    def __init__(self, env, W, segs, x, want_acc=True, want_y=True):
        torch, twd, orc = env
        self.W, self.segs, self.x = W, tuple(segs), x
        M, K = x.shape
        N = int(sum(segs))
        packed, self.gammas = twd.prepare_weights(W, segs)
        self.wp = torch.from_numpy(packed).cuda()
        self.wt = torch.from_numpy(twd.tile_for_sweep(packed, N, K)).cuda()
        self.xd = dev_bf16(torch, x)
        self.acc = (torch.full((M, N), -7, dtype=torch.int32, device="cuda")
                    if want_acc else None)
        self.y = torch.full((M, N), -7.0, device="cuda") if want_y else None

    def entry(self):
        return (self.wt, self.segs, self.gammas, self.xd, self.acc, self.y)

    def check(self, orc, ref=None):
        ref = ref if ref is not None else orc.forward(self.W, self.segs, self.x)
        assert self.gammas == ref["gammas"]
        if self.acc is not None:
            np.testing.assert_array_equal(self.acc.cpu().numpy(), ref["acc"])
        if self.y is not None:
            check_y(self.y.cpu().numpy(), ref["y"])
        return ref


def random_list(env, M, seed, n=6):
    rng = np.random.default_rng([91, seed, M])
    cases = []
    for i in range(n):
        K = 64 * int(rng.integers(1, 129))
        nseg = int(rng.integers(1, 5))
        segs = tuple(int(v) for v in rng.integers(0 if i == 2 else 1, 300, size=nseg))
        W, segs, x = wl.random_case(seed=1000 * seed + i, M=M, K=K, seg_rows=segs)
        cases.append(Case(env, W, segs, x, want_acc=i != 4, want_y=i != 5))
    # the extremes of K
    W, segs, x = wl.random_case(seed=1000 * seed + 77, M=M, K=64, seg_rows=(17,))
    cases.append(Case(env, W, segs, x))
    W, segs, x = wl.random_case(seed=1000 * seed + 78, M=M, K=8192, seg_rows=(40, 9))
    cases.append(Case(env, W, segs, x))
    return cases


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_sweep_random_lists(env, M):
    torch, twd, orc = env
    cases = random_list(env, M, seed=M)
    log(f"sweep random list M={M}: " + ", ".join(
        f"K={c.x.shape[1]} segs={c.segs}" for c in cases))
    sw = twd.Sweep([c.entry() for c in cases])
    sw.run()
    torch.cuda.synchronize()
    for c in cases:
        c.check(orc)


@pytest.mark.parametrize("M", [1, 2, 5, 9, 16])
def test_sweep_tiny_projections_cross_spans(env, M):
    """Many projections of one or two 16-row tiles (ragged N): each workgroup
    holds four spans and most of its waves own no tile in most of them, so
    the loads that run ahead skip from span to span."""
    torch, twd, orc = env
    rng = np.random.default_rng([17, M])
    cases = []
    for i in range(40):
        K = 64 * int(rng.integers(1, 41))
        N = int(rng.integers(1, 33))
        W, segs, x = wl.random_case(seed=4000 + 50 * M + i, M=M, K=K, seg_rows=(N,))
        cases.append(Case(env, W, segs, x, want_acc=i % 3 != 1, want_y=i % 3 != 2))
    sw = twd.Sweep([c.entry() for c in cases])
    log(f"sweep tiny projections M={M}: {len(cases)} projections, {sw.plan.nwg} workgroups")
    sw.run()
    torch.cuda.synchronize()
    for c in cases:
        c.check(orc)


@pytest.mark.parametrize("M", [1, 3, 16])
def test_sweep_zero_rows_and_empty_projections(env, M):
    """All-zero token rows (scale 0, outputs 0) and projections with N = 0."""
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=5, M=M, K=2560, seg_rows=(70, 3))
    xf = wl.bf16_bits_to_f32(x).copy()
    xf[0] = 0.0
    x = wl.f32_to_bf16_bits(xf)
    W0, segs0, x0 = wl.random_case(seed=6, M=M, K=512, seg_rows=(0,))
    cases = [Case(env, W0, segs0, x0), Case(env, W, segs, x), Case(env, W0, segs0, x0)]
    sw = twd.Sweep([c.entry() for c in cases])
    sw.run()
    torch.cuda.synchronize()
    cases[1].check(orc)
    assert not cases[1].acc[0].any() and not cases[1].y[0].any()
    # a list of empty projections only: one workgroup that stages nothing
    empty = twd.Sweep([cases[0].entry(), cases[2].entry()])
    assert empty.plan.nwg == 1 and empty.weight_bytes == 0
    empty.run()
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_sweep_full_size_layer_every_width(env, M):
    """One full-size 2B-class layer (all four projections) on the outlier
    workload, at every width, in one sweep."""
    torch, twd, orc = env
    ls = wl.SET_2B
    layer = (7 * M) % ls.layers
    cases = []
    for pi, proj in enumerate(ls.projs):
        W = wl.layer_weights(ls, layer, pi)
        x = wl.layer_activations("2b_sweep_outlier", proj.K, M, layer, pi, outliers=True)
        cases.append(Case(env, W, proj.segs, x))
    log(f"sweep full-size 2B layer {layer} M={M}")
    sw = twd.Sweep([c.entry() for c in cases])
    sw.run()
    torch.cuda.synchronize()
    threads = orc.max_threads()
    for c in cases:
        c.check(orc, orc.forward(c.W, c.segs, c.x, threads=threads))


SAMPLED_ROWS = 24


def _threads():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@pytest.fixture(scope="module")
def whole_sets(env):
    """Each layer set once: tiled and row-major packed weights on the device,
    and for a fixed sample of rows per projection the oracle's ternary codes
    and per-row gamma (ternarized over the whole segment)."""
    from concurrent.futures import ThreadPoolExecutor
    torch, twd, orc = env
    cache = {}

    def get(name):
        if name in cache:
            return cache[name]
        ls = wl.LAYER_SETS[name]
        keys = [(layer, pi) for layer in range(ls.layers) for pi in range(len(ls.projs))]

        def prep(key):
            layer, pi = key
            proj = ls.projs[pi]
            W = wl.layer_weights(ls, layer, pi)
            packed, gammas = twd.prepare_weights(W, proj.segs)
            t, gam, grow = orc.ternarize_segments(W, proj.segs)
            assert gam == list(gammas)
            rows = np.sort(np.random.default_rng([123, layer, pi]).choice(
                proj.N, SAMPLED_ROWS, replace=False))
            tiled = twd.tile_for_sweep(packed, proj.N, proj.K)
            return key, packed, tiled, gammas, t[rows].copy(), grow[rows].copy(), rows

        out = {}
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            for key, packed, tiled, gammas, trows, grows, rows in ex.map(prep, keys):
                out[key] = (torch.from_numpy(tiled).cuda(), torch.from_numpy(packed).cuda(),
                            gammas, trows, grows, rows)
        torch.cuda.synchronize()
        cache.clear()  # hold one set on the device at a time
        cache[name] = (ls, keys, out)
        log(f"whole-set fixture {name}: {len(keys)} projections prepared")
        return cache[name]

    return get


WHOLE_SET_CASES = [("2b", "2b_decode", 1), ("2b", "2b_verify", 2), ("2b", "2b_verify", 4),
                   ("2b", "2b_verify", 8), ("2b", "2b_verify", 11),
                   ("2b", "2b_sweep_outlier", 16),
                   ("4b", "4b_stack", 1), ("4b", "4b_stack", 4), ("4b", "4b_stack", 16)]


@pytest.mark.parametrize("set_name,workload,M", WHOLE_SET_CASES)
def test_sweep_whole_layer_set(env, whole_sets, set_name, workload, M):
    """The benchmark's launch at full size: every projection of a layer set
    (the 30-layer 2B set, the 36-layer 4B stack) in one sweep at width M.
    Every output equals the per-projection launch; sampled rows of every
    projection equal the oracle."""
    torch, twd, orc = env
    ls, keys, dev = whole_sets(set_name)
    log(f"sweep whole set {set_name} {workload} M={M}")
    outliers = workload == "2b_sweep_outlier"
    entries, checks = [], []
    for key in keys:
        layer, pi = key
        proj = ls.projs[pi]
        wt, wp, gammas, trows, grows, rows = dev[key]
        x = wl.layer_activations(workload, proj.K, M, layer, pi, outliers=outliers)
        q, s = orc.quantize_act(x)
        ra = orc.linear(q, trows)
        xd = dev_bf16(torch, x)
        entries.append((wt, proj.segs, gammas, xd,
                        torch.full((M, proj.N), -7, dtype=torch.int32, device="cuda"),
                        torch.full((M, proj.N), -7.0, device="cuda")))
        checks.append((key, wp, rows, ra, orc.dequant(ra, s, grows)))
    sw = twd.Sweep(entries)
    assert sw.weight_bytes == ls.packed_bytes
    sw.run()
    torch.cuda.synchronize()
    for (wt, segs, gammas, xd, acc, y), (key, wp, rows, ra, ry) in zip(entries, checks):
        a2, y2 = twd.ternary_linear_bf16(wp, segs, gammas, xd)
        torch.cuda.synchronize()
        assert torch.equal(acc, a2), key
        assert torch.equal(y, y2), key
        np.testing.assert_array_equal(acc.cpu().numpy()[:, rows], ra)
        check_y(y.cpu().numpy()[:, rows], ry, f"{key}")


@pytest.mark.parametrize("scale", [1, 2])
def test_sweep_packed_deferral_ragged(env, scale):
    """Workgroups whose outputs fit in LDS only as 24-bit accumulators (M =
    16, K = 64 and 128, about 2800 rows per workgroup; at scale 2 about 5600,
    so that only each span's first tiles fit and the rest store in the
    stream), on ragged N (N % 4 != 0) and on a y that is not 16-byte
    aligned, so the packed write-out takes both of its store forms: every
    output equals the per-projection launch, sampled rows equal the oracle."""
    torch, twd, orc = env
    M = 16
    specs = [(64, (145001 * scale,), True, True, False),
             (64, (70000 * scale, 74999 * scale), False, True, False),
             (128, (72999 * scale,), True, False, False), (64, (144997 * scale,), True, True, True),
             (64, (145003 * scale, 2), False, True, False)]
    entries, checks = [], []
    for i, (K, segs, want_acc, want_y, misaligned) in enumerate(specs):
        W, segs, x = wl.random_case(seed=5100 + i, M=M, K=K, seg_rows=segs)
        N = int(sum(segs))
        packed, gammas = twd.prepare_weights(W, segs)
        t, gam, grow = orc.ternarize_segments(W, segs)
        assert gam == list(gammas)
        rows = np.sort(np.random.default_rng([5200, i]).choice(N, SAMPLED_ROWS, replace=False))
        q, sc = orc.quantize_act(x)
        ra = orc.linear(q, t[rows].copy())
        ry = orc.dequant(ra, sc, grow[rows].copy())
        del W, t
        wt = torch.from_numpy(twd.tile_for_sweep(packed, N, K)).cuda()
        wp = torch.from_numpy(packed).cuda()
        xd = dev_bf16(torch, x)
        acc = torch.full((M, N), -7, dtype=torch.int32, device="cuda") if want_acc else None
        y = None
        if want_y:
            buf = torch.full((M * N + 1,), -7.0, device="cuda")
            y = (buf[1:] if misaligned else buf[:-1]).view(M, N)
            assert (y.data_ptr() % 16 != 0) == misaligned
        entries.append((wt, segs, gammas, xd, acc, y))
        checks.append((wp, segs, gammas, xd, rows, ra, ry))
    sw = twd.Sweep(entries)
    img = sw.table.cpu().numpy()
    nwg, work_off = (int(v) for v in img[:32].view(np.int32)[[3, 7]])
    work = img[work_off:work_off + 144 * nwg].view(np.int32).reshape(nwg, 36)
    defer = work[:, 1]
    spans = work[:, 4:].reshape(nwg, 4, 8)  # q, t0, t1, xoff, yoff, aoff, nd, pad
    partial = sum(int(spans[i, k, 6]) < int(spans[i, k, 2] - spans[i, k, 1])
                  for i in range(nwg) if defer[i] == 2 for k in range(int(work[i, 0])))
    log(f"sweep packed deferral x{scale}: {nwg} workgroups, {int((defer == 2).sum())} packed "
        f"({partial} spans in part), {int((defer == 1).sum())} with values, "
        f"{int((defer == 0).sum())} in the stream")
    assert (defer == 2).sum() > nwg // 2
    assert (partial > 0) == (scale == 2)
    sw.run()
    torch.cuda.synchronize()
    for (wt, segs, gammas, xd, acc, y), (wp, _, _, _, rows, ra, ry) in zip(entries, checks):
        a2, y2 = twd.ternary_linear_bf16(wp, segs, gammas, xd)
        torch.cuda.synchronize()
        if acc is not None:
            assert torch.equal(acc, a2)
            np.testing.assert_array_equal(acc.cpu().numpy()[:, rows], ra)
        if y is not None:
            assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
            check_y(y.cpu().numpy()[:, rows], ry, "packed deferral")


def test_sweep_graph_replays_match_oracle(env):
    """A sweep captured into a graph: three replays, with eager work and
    synchronization between them, each checked against the oracle."""
    torch, twd, orc = env
    cases = random_list(env, 5, seed=50, n=4)
    refs = [orc.forward(c.W, c.segs, c.x) for c in cases]
    sw = twd.Sweep([c.entry() for c in cases])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sw.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sw.run()
    for rep in range(3):
        for c in cases:
            if c.acc is not None:
                c.acc.fill_(-1)
            if c.y is not None:
                c.y.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        for c, ref in zip(cases, refs):
            c.check(orc, ref)
        _ = sum(float(c.y.sum()) for c in cases if c.y is not None)  # eager work


def test_sweep_table_mismatch_writes_nothing(env):
    """A plan whose check value is not the table's: the launch returns
    without writing any output."""
    torch, twd, orc = env
    cases = random_list(env, 2, seed=60, n=2)
    sw = twd.Sweep([c.entry() for c in cases])
    sw.plan.check ^= 0x5A5A5A5A
    sw.run()
    torch.cuda.synchronize()
    for c in cases:
        if c.acc is not None:
            assert bool((c.acc == -7).all())
        if c.y is not None:
            assert bool((c.y == -7.0).all())
    sw.plan.check ^= 0x5A5A5A5A
    sw.run()
    torch.cuda.synchronize()
    for c in cases:
        c.check(orc)


def test_sweep_errors(env):
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=8, M=2, K=256, seg_rows=(16,))
    c = Case(env, W, segs, x)
    with pytest.raises(ValueError):
        twd.Sweep([])
    bad = wl.random_case(seed=8, M=2, K=100, seg_rows=(16,))
    with pytest.raises(twd.TwdError) as e:
        xb = torch.zeros((2, 100), dtype=torch.bfloat16, device="cuda")
        twd.Sweep([(c.wt, segs, c.gammas, xb, None, c.y)])
    assert e.value.status == 2
    with pytest.raises(twd.TwdError) as e:
        twd.Sweep([(c.wt, segs, c.gammas, c.xd, None, None)])
    assert e.value.status == 1
    with pytest.raises(ValueError):
        x3 = torch.zeros((3, 256), dtype=torch.bfloat16, device="cuda")
        twd.Sweep([c.entry(), (c.wt, segs, c.gammas, x3, None, None)])
    del bad


def test_sweep_width_atlas_replays_match_oracle(env):
    """A width-keyed atlas: one captured graph per width, all held at once
    over the same weights (each width with its own activation and output
    buffers), replayed in an interleaved order, every replay checked against
    the oracle."""
    torch, twd, orc = env
    shapes = [(2560, (96, 40, 40)), (6912, (48,)), (1024, (130,))]
    base = []
    for i, (K, segs) in enumerate(shapes):
        W, segs, _ = wl.random_case(seed=300 + i, M=1, K=K, seg_rows=segs)
        packed, gammas = twd.prepare_weights(W, segs)
        N = int(sum(segs))
        base.append((W, segs, gammas, torch.from_numpy(twd.tile_for_sweep(packed, N, K)).cuda()))
    atlas = {}
    for M in (1, 2, 5, 9, 16):
        cases, entries = [], []
        for i, (W, segs, gammas, wt) in enumerate(base):
            _, _, x = wl.random_case(seed=400 + 17 * M + i, M=M, K=W.shape[1], seg_rows=segs)
            N = int(sum(segs))
            acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
            y = torch.empty((M, N), device="cuda")
            entries.append((wt, segs, gammas, dev_bf16(torch, x), acc, y))
            cases.append((W, segs, x, acc, y, orc.forward(W, segs, x)))
        sw = twd.Sweep(entries)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            sw.run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                sw.run()
        atlas[M] = (g, sw, cases)
    log(f"atlas of {len(atlas)} graphs held")
    for rep, M in enumerate((16, 1, 9, 2, 5, 1, 16, 9)):
        g, _, cases = atlas[M]
        for (_, _, _, acc, y, _) in cases:
            acc.fill_(-3)
            y.fill_(-3.0)
        g.replay()
        torch.cuda.synchronize()
        for (W, segs, x, acc, y, ref) in cases:
            np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
            check_y(y.cpu().numpy(), ref["y"], f"atlas M={M} replay {rep}")
        _ = float(cases[0][4].sum())  # eager work between replays
