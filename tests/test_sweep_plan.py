"""Host logic of the multi-projection sweep (no GPU): the planner's table
image, decoded field by field, must cover every 16-row tile of every
projection exactly once, in order, with at most four projections per
workgroup, consistent LDS offsets (staged activations, then the deferred
outputs where they fit) and a check value bound to the table's device
address; bad arguments must be rejected before anything is written.
"""
import ctypes

import numpy as np
import pytest

import ternary_weight_decode_amd as twd

HEADER = np.dtype([("magic", "<u4"), ("check", "<u4"), ("nproj", "<i4"), ("nwg", "<i4"),
                   ("M", "<i4"), ("lds", "<i4"), ("proj_off", "<i4"), ("work_off", "<i4"),
                   ("weight_bytes", "<i8"), ("pad", "<i4", 6)])
PROJ = np.dtype([("w", "<u8"), ("x", "<u8"), ("acc", "<u8"), ("y", "<u8"), ("K", "<i4"),
                 ("N", "<i4"), ("passes", "<i4"), ("slices", "<i4"), ("stride", "<i4"),
                 ("nseg", "<i4"), ("bound", "<i4", 4), ("gamma", "<f4", 4), ("pad", "<i4", 2)])
WORK = np.dtype([("nspan", "<i4"), ("defer", "<i4"), ("pad", "<i4", 2),
                 ("span", "<i4", (4, 8))])  # q, t0, t1, xoff, yoff, aoff, nd, pad
LDS_HEADER = 64 + 3 * 4 * 16 * 4 + 16
MAX_SPANS = 4


def fake_list(shapes, base=1 << 32, outputs=lambda i: (True, True)):
    """(K, seg_rows) list -> descriptors with distinct aligned fake pointers
    (the planner never dereferences them); outputs(i) -> (acc?, y?)."""
    rows = []
    for i, (K, segs) in enumerate(shapes):
        p = base + (i << 24)
        a, y = outputs(i)
        rows.append((p, p + (1 << 20), p + (2 << 20) if a else None, p + (3 << 20) if y else None,
                     K, segs, [0.5 + i] * len(segs)))
    return rows


def decode(img):
    h = np.frombuffer(img[:64].tobytes(), HEADER)[0]
    projs = np.frombuffer(img[h["proj_off"]:h["proj_off"] + 96 * h["nproj"]].tobytes(), PROJ)
    work = np.frombuffer(img[h["work_off"]:h["work_off"] + 144 * h["nwg"]].tobytes(), WORK)
    return h, projs, work


def plan(shapes, M, table_dev=0x7F0000000000, outputs=lambda i: (True, True)):
    descs = twd.sweep_descs(fake_list(shapes, outputs=outputs), M)
    img, p = twd.sweep_encode(descs, M, table_dev)
    return img, p


def stride(K):
    return -(-K // 256) * 256 + 16


SHAPE_LISTS = [
    [(2560, (2560, 640, 640)), (2560, (2560,)), (2560, (6912, 6912)), (6912, (2560,))] * 3,
    [(3072, (3072, 1024, 1024)), (3072, (3072,)), (3072, (8192, 8192)), (8192, (3072,))] * 3,
    [(64, (1,)), (8192, (33, 7)), (320, (0,)), (1536, (64, 33, 33, 5)), (256, (700,))],
    [(256, (16,))] * 40,           # many small projections: span limit
    [(8192, (5000,)), (64, (3,))],
]


OUTPUTS = {"both": lambda i: (True, True), "y": lambda i: (False, True),
           "mixed": lambda i: (i % 3 != 1, i % 3 != 2)}


@pytest.mark.parametrize("outs", sorted(OUTPUTS))
@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("li", range(len(SHAPE_LISTS)))
def test_plan_covers_every_tile_once(li, M, outs):
    check_plan(SHAPE_LISTS[li], M, OUTPUTS[outs])


def check_plan(shapes, M, outputs):
    """Decode the plan of (K, seg_rows) list `shapes` at width M and check
    every field against the planner's rules."""
    img, p = plan(shapes, M, outputs=outputs)
    h, projs, work = decode(img)
    assert h["magic"] == 0x53445754 and h["nproj"] == len(shapes) and h["M"] == M
    assert p.nwg == h["nwg"] == len(work) and p.lds_bytes == h["lds"]
    assert p.check == h["check"] != 0 and p.table_bytes == img.size
    total = sum(K * sum(s) // 4 for K, s in shapes)
    assert h["weight_bytes"] == total == p.weight_bytes
    for i, (K, segs) in enumerate(shapes):
        d = projs[i]
        assert (d["K"], d["N"]) == (K, sum(segs))
        assert d["slices"] == -(-K // 256) and d["passes"] == -(-d["slices"] // 4)
        assert d["stride"] == stride(K) and d["nseg"] == len(segs)
        assert list(d["bound"][:len(segs)]) == list(np.cumsum(segs))
    seen = []
    for w in work:
        n = int(w["nspan"])
        assert 1 <= n <= MAX_SPANS or (n == 0 and total == 0)
        lds = LDS_HEADER
        for s in range(n):
            q, t0, t1, xoff = (int(v) for v in w["span"][s][:4])
            assert xoff == lds - LDS_HEADER
            lds += M * stride(shapes[q][0])
            assert t0 < t1
            seen.extend((q, t) for t in range(t0, t1))
        assert lds <= h["lds"] <= 160 * 1024
        # deferred outputs, from the first 16-byte boundary past the staged
        # rows: when the rows of all its spans fit in 160 KiB, per span, y
        # then acc rows [M][16 (t1 - t0)] fp32 / int32 (defer = 1); else,
        # per span with any output, the first nd tiles as [M][16 nd] 24-bit
        # accumulators (3 bytes each) at yoff, nd as large as fits, span
        # after span (defer = 2, if any tile fits)
        off = (lds + 15) & ~15
        expect = []
        for s in range(n):
            q, t0, t1 = (int(v) for v in w["span"][s][:3])
            a, y = outputs(q)
            b = 4 * M * 16 * (t1 - t0)
            ey = off if y else -1
            off += b if y else 0
            ea = off if a else -1
            off += b if a else 0
            expect.append((ey, ea))
        packed_off = (lds + 15) & ~15
        packed = []
        for s in range(n):
            q, t0, t1 = (int(v) for v in w["span"][s][:3])
            a, y = outputs(q)
            nd = min(max(160 * 1024 - packed_off, 0) // (48 * M), t1 - t0) if a or y else 0
            packed.append((packed_off if nd else -1, -1, nd))
            packed_off += 48 * M * nd
        got = [(int(w["span"][s][4]), int(w["span"][s][5])) for s in range(n)]
        nds = [int(w["span"][s][6]) for s in range(n)]
        if n and off <= 160 * 1024:
            assert w["defer"] == 1 and got == expect and nds == [0] * n
            assert off <= h["lds"]
        elif n and any(p[2] for p in packed):
            assert w["defer"] == 2 and [p[:2] for p in packed] == got
            assert nds == [p[2] for p in packed]
            assert packed_off <= h["lds"] <= 160 * 1024
        else:
            assert w["defer"] == 0 and all(g == (-1, -1) for g in got)
    expect = [(q, t) for q, (K, s) in enumerate(shapes) for t in range(-(-sum(s) // 16))]
    assert seen == expect


@pytest.mark.parametrize("seed", range(40))
def test_plan_random_lists(seed):
    """Seeded random lists (1-24 projections, K from 64 to 8192, up to four
    segments of 0-3000 rows, acc or y or both) at random widths: every
    rule of the plan holds, whichever deferral form each workgroup takes."""
    rng = np.random.default_rng([91, seed])
    n = int(rng.integers(1, 25))
    shapes = []
    for _ in range(n):
        K = 64 * int(rng.integers(1, 129))
        segs = tuple(int(v) for v in rng.integers(0, 3001, int(rng.integers(1, 5))))
        shapes.append((K, segs))
    M = int(rng.integers(1, 17))
    mask = rng.integers(1, 4, n)  # acc, y or both (a projection needs an output)
    check_plan(shapes, M, lambda i: (bool(mask[i] & 1), bool(mask[i] & 2)))


def test_plan_balances_bytes():
    """The 2B-class layer set: workgroups carry about equal weight bytes."""
    ls = [(2560, (2560, 640, 640)), (2560, (2560,)), (2560, (6912, 6912)), (6912, (2560,))] * 30
    img, p = plan(ls, 1)
    h, projs, work = decode(img)
    sizes = []
    for w in work:
        b = 0
        for s in range(int(w["nspan"])):
            q, t0, t1, _ = (int(v) for v in w["span"][s][:4])
            b += (t1 - t0) * 16 * ls[q][0] // 4
        sizes.append(b)
    sizes = np.array(sizes)
    assert sizes.sum() == h["weight_bytes"]
    # one workgroup per compute unit, a few more where a range is closed at
    # the span limit
    assert 256 <= len(sizes) <= 300
    # the cuts fall on tile boundaries: no workgroup exceeds the mean share
    # by more than a tile
    assert sizes.max() <= h["weight_bytes"] / 256 + 16 * 6912 // 4


@pytest.mark.parametrize("M,acc,deferring", [(1, False, 256), (4, False, 256), (1, True, 256),
                                             (8, False, 256), (8, True, 256), (12, False, 256),
                                             (16, False, 256), (16, True, 256)])
def test_plan_defers_where_outputs_fit(M, acc, deferring):
    """The 2B-class layer set: at M = 1 and 4 every workgroup gathers its
    outputs in LDS as values; up to M = 8 every workgroup gathers all of
    them (as values where they fit, else as 24-bit accumulators, with or
    without acc); at M = 12 and 16 the staged activations leave room for
    only part of them in some workgroups, which defer the first tiles of
    their spans and store the rest in the stream."""
    ls = [(2560, (2560, 640, 640)), (2560, (2560,)), (2560, (6912, 6912)), (6912, (2560,))] * 30
    img, p = plan(ls, M, outputs=lambda i: (acc, True))
    h, projs, work = decode(img)
    n = int(sum(int(w["defer"]) > 0 for w in work))
    assert n == min(deferring, len(work))
    partial = sum(int(w["span"][s][6]) < int(w["span"][s][2]) - int(w["span"][s][1])
                  for w in work if int(w["defer"]) == 2 for s in range(int(w["nspan"])))
    if M <= 4:
        assert all(int(w["defer"]) == 1 for w in work)
    if M <= 8:
        assert partial == 0
    else:
        assert partial > 0
    assert h["lds"] <= 160 * 1024


@pytest.mark.parametrize("M", [1, 8, 12, 14, 15, 16])
def test_plan_stays_resident(M):
    """The 4B-class stack: where the staged rows of a K = 8192 projection
    leave no room for a neighbour (M >= 15), the ranges must end at those
    boundaries; the plan still fits one workgroup per compute unit (no second
    round) and no workgroup carries more than a range's share of its
    segment: at most 10% above the mean here."""
    ls = [(3072, (3072, 1024, 1024)), (3072, (3072,)), (3072, (8192, 8192)), (8192, (3072,))] * 36
    img, p = plan(ls, M, outputs=lambda i: (False, True))
    h, projs, work = decode(img)
    assert len(work) <= 256
    sizes = []
    for w in work:
        b = 0
        for s in range(int(w["nspan"])):
            q, t0, t1 = (int(v) for v in w["span"][s][:3])
            b += (t1 - t0) * 16 * ls[q][0] // 4
        sizes.append(b)
    sizes = np.array(sizes)
    assert sizes.sum() == h["weight_bytes"]
    assert sizes.max() <= 1.1 * sizes.mean()


def test_check_binds_device_address():
    shapes = SHAPE_LISTS[0]
    img1, p1 = plan(shapes, 2, table_dev=0x7F0000000000)
    img2, p2 = plan(shapes, 2, table_dev=0x7F0000001000)
    assert p1.check != p2.check
    assert p1.table == 0x7F0000000000


def test_plan_errors():
    good = fake_list([(256, (16,))])
    with pytest.raises(twd.TwdError) as e:
        plan([(100, (16,))], 1)
    assert e.value.status == 2
    with pytest.raises(twd.TwdError) as e:
        plan([(256, (16,))], 0)
    assert e.value.status == 2
    with pytest.raises(twd.TwdError) as e:
        plan([(256, (16,))], 17)
    assert e.value.status == 2
    with pytest.raises(twd.TwdError) as e:
        plan([(16384, (16,))], 1)
    assert e.value.status == 2
    # misaligned weights, missing outputs, negative segment
    for mutate in (lambda r: (r[0] + 8,) + r[1:], lambda r: r[:2] + (None, None) + r[4:],
                   lambda r: r[:5] + ((-1,),) + r[6:]):
        descs = twd.sweep_descs([mutate(good[0])], 1)
        with pytest.raises(twd.TwdError) as e:
            twd.sweep_encode(descs, 1, 0x7F0000000000)
        assert e.value.status == 1
    # a table too small, a misaligned device table
    descs = twd.sweep_descs(good, 1)
    n = ctypes.c_int64(0)
    assert twd._lib_sweep_bytes(descs, 1, 1, ctypes.byref(n)) == 0
    img = np.zeros(n.value, np.uint8)
    pl = twd.SweepPlan()
    assert twd._lib_sweep_encode(descs, 1, 1, ctypes.c_void_p(0x7F0000000000),
                                 twd._np_ptr(img), n.value - 1, ctypes.byref(pl)) == 1
    assert twd._lib_sweep_encode(descs, 1, 1, ctypes.c_void_p(0x7F0000000008),
                                 twd._np_ptr(img), n.value, ctypes.byref(pl)) == 1
    # a launch with a plan out of range is refused before anything runs
    pl.table = 0x7F0000000000
    pl.M = 0
    assert twd._lib_sweep(ctypes.byref(pl), None) == 1


def tile_reference(packed, N, K):
    """The tiled layout written out with numpy indexing: tile t, slice u,
    position l = 16 g + r holds bytes 64 u + 16 g .. + 15 of row 16 t + r."""
    RB = K // 4
    T, S = -(-N // 16), -(-K // 256)
    rows = np.zeros((T * 16, S * 64), np.uint8)
    rows[:N, :RB] = packed.reshape(N, RB)
    # [t, r, u, g, b] -> [t, u, g, r, b]
    v = rows.reshape(T, 16, S, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(v).reshape(-1)


@pytest.mark.parametrize("N,K", [(1, 64), (16, 256), (17, 320), (130, 2560), (33, 6912),
                                 (20, 8192), (0, 256), (5, 0)])
def test_tile_weights_layout(N, K):
    rng = np.random.default_rng([N, K])
    codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    packed = twd.pack_ternary(codes)
    tiled = twd.tile_for_sweep(packed, N, K)
    assert tiled.size == twd.sweep_tiled_bytes(N, K) == -(-N // 16) * -(-K // 256) * 1024
    np.testing.assert_array_equal(tiled, tile_reference(packed, N, K))
    if tiled.size:
        # padding (rows past N, bytes past K / 4) is zero
        T, S = -(-N // 16), -(-K // 256)
        v = tiled.reshape(T, S, 4, 16, 16)
        r = np.arange(16)[None, None, None, :] + 16 * np.arange(T)[:, None, None, None]
        col = 64 * np.arange(S)[None, :, None, None] + 16 * np.arange(4)[None, None, :, None]
        pad = (r >= N) | (col >= K // 4)
        assert not v[np.broadcast_to(pad, v.shape[:4])].any()


def test_tile_weights_errors():
    with pytest.raises(ValueError):
        twd.sweep_tiled_bytes(16, 100)
    assert twd._lib_tiled_bytes(-1, 64) == -1
    with pytest.raises(twd.TwdError):
        twd._check(twd._lib_tile(None, 16, 64, None))
