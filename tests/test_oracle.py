"""Pins of the CPU oracle against things other than itself: numpy's integer
matmul (brute force), closed forms of the absmean rule on Gaussian weights,
invariants of the contraction, and hand-derived fixtures under tests/golden/.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden, read_golden_rows
from workloads import bf16_bits_to_f32, f32_to_bf16_bits


# ---------------------------------------------------------------- contraction

@pytest.mark.parametrize("seed", range(8))
def test_linear_matches_int64_matmul(orc, seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 5))
    K = int(rng.integers(1, 65))
    N = int(rng.integers(1, 17))
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    ref = q.astype(np.int64) @ t.astype(np.int64).T
    acc = orc.linear(q, t)
    assert acc.dtype == np.int32
    np.testing.assert_array_equal(acc.astype(np.int64), ref)


def test_linear_extremes(orc):
    K = 8192
    q = np.full((2, K), 127, dtype=np.int8)
    q[1] = -127
    t = np.ones((3, K), dtype=np.int8)
    t[1] = -1
    t[2, ::2] = -1
    acc = orc.linear(q, t)
    ref = q.astype(np.int64) @ t.astype(np.int64).T
    np.testing.assert_array_equal(acc, ref)
    assert acc[0, 0] == 127 * 8192 and acc[1, 0] == -127 * 8192


def test_linear_invariants(orc):
    rng = np.random.default_rng(5)
    M, K, N = 3, 96, 7
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    # zero weights give zero
    assert not orc.linear(q, np.zeros((N, K), np.int8)).any()
    # all +1 row gives the activation row sum, all -1 its negation
    t = np.zeros((N, K), np.int8)
    t[0] = 1
    t[1] = -1
    k0 = 17
    t[2, k0] = 1  # one-hot
    acc = orc.linear(q, t)
    rowsum = q.astype(np.int64).sum(axis=1)
    np.testing.assert_array_equal(acc[:, 0], rowsum)
    np.testing.assert_array_equal(acc[:, 1], -rowsum)
    np.testing.assert_array_equal(acc[:, 2], q[:, k0])
    # negating the weights negates the result
    tr = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    np.testing.assert_array_equal(orc.linear(q, -tr), -orc.linear(q, tr))
    # width invariance: row m of an M-wide call equals the 1-wide call
    full = orc.linear(q, tr)
    for m in range(M):
        np.testing.assert_array_equal(full[m], orc.linear(q[m:m + 1], tr)[0])
    # bound
    assert np.all(np.abs(full) <= 127 * np.count_nonzero(tr, axis=1)[None, :])


# --------------------------------------------------------------- ternarize

def test_ternarize_gaussian_closed_form(orc):
    # For W ~ N(0, s^2) and gamma = E|W| = s*sqrt(2/pi), t = 0 iff
    # |W| <= gamma/2, so P(t = 0) = 2*Phi(sqrt(2/pi)/2) - 1 = 0.3101 for any s.
    p0 = math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    assert abs(p0 - 0.3101) < 1e-4
    for sigma in (1.0, 0.02):
        rng = np.random.default_rng(0)
        W = rng.standard_normal((512, 256), dtype=np.float32) * np.float32(sigma)
        t, g = orc.ternarize_absmean(W)
        frac0 = np.mean(t == 0)
        assert abs(frac0 - p0) < 0.01
        assert abs(np.mean(t == 1) - (1 - p0) / 2) < 0.01
        # gamma is the mean absolute value, rounded once to fp32
        mean = float(np.mean(np.abs(W.astype(np.float64))))
        assert abs(g - mean) <= 2 ** -23 * mean
        assert abs(g / sigma - math.sqrt(2 / math.pi)) < 0.01


def test_ternarize_threshold_characterisation(orc):
    # clamp(rint(v), -1, 1) with ties to even equals sign(v) for |v| > 1/2 and
    # 0 for |v| <= 1/2; check that form on random weights, using the fp32
    # quotient, and check signs.
    rng = np.random.default_rng(3)
    W = rng.standard_normal((64, 160), dtype=np.float32)
    t, g = orc.ternarize_absmean(W)
    v = W / np.float32(g)
    expect = np.where(np.abs(v) > 0.5, np.sign(v), 0).astype(np.int8)
    np.testing.assert_array_equal(t, expect)
    assert set(np.unique(t)) <= {-1, 0, 1}


def test_ternarize_ties_and_zero(orc):
    # gamma = (1 + 7) / 4 = 2: W/gamma = 0.5, 3.5 -> 0 (half-even) and 1.
    t, g = orc.ternarize_absmean(np.array([[1, 7, 0, 0]], np.float32))
    assert g == 2.0
    assert t.tolist() == [[0, 1, 0, 0]]
    t, g = orc.ternarize_absmean(np.array([[-1, 7, 0, 0]], np.float32))
    assert t.tolist() == [[0, 1, 0, 0]]
    t, g = orc.ternarize_absmean(np.zeros((3, 32), np.float32))
    assert g == 0.0 and not t.any()
    # negation symmetry
    W = np.random.default_rng(9).standard_normal((8, 48), dtype=np.float32)
    t1, g1 = orc.ternarize_absmean(W)
    t2, g2 = orc.ternarize_absmean(-W)
    assert g1 == g2
    np.testing.assert_array_equal(t2, -t1)


def test_ternarize_rejects_nonfinite(orc):
    W = np.ones((2, 16), np.float32)
    W[1, 3] = np.inf
    with pytest.raises(ValueError):
        orc.ternarize_absmean(W)


# ---------------------------------------------------------------- quantize

def test_quantize_crafted_ties(orc):
    x = f32_to_bf16_bits(np.array([[127, 62.5, -62.5, 0.5, 1.5, 2.5]], np.float32))
    q, s = orc.quantize_act(x)
    assert q.tolist() == [[127, 62, -62, 0, 2, 2]]
    assert s[0] == np.float32(1.0)
    # absmax 254 gives inv = 0.5 exactly: 125 * 0.5 = 62.5 -> 62, 3 * .5 -> 2
    x = f32_to_bf16_bits(np.array([[254, 125, 3, -5, 1]], np.float32))
    q, s = orc.quantize_act(x)
    assert q.tolist() == [[127, 62, 2, -2, 0]]
    assert s[0] == np.float32(2.0)


def test_quantize_properties(orc):
    rng = np.random.default_rng(11)
    xf = rng.standard_normal((16, 512), dtype=np.float32)
    xf[3, 10:40] *= 20.0
    xf[5] = 0.0
    xb = f32_to_bf16_bits(xf)
    q, s = orc.quantize_act(xb)
    xw = bf16_bits_to_f32(xb).astype(np.float64)
    a = np.abs(xw).max(axis=1)
    for m in range(16):
        if a[m] == 0:
            assert not q[m].any() and s[m] == 0
            continue
        assert np.abs(q[m]).max() == 127
        assert q[m][np.argmax(np.abs(xw[m]))] == np.sign(xw[m][np.argmax(np.abs(xw[m]))]) * 127
        # exact-real view: q is a nearest integer of x*127/a, up to the fp32
        # rounding of 127/a and of the product (relative 2^-23 together)
        v = xw[m] * 127.0 / a[m]
        assert np.all(np.abs(q[m] - v) <= 0.5 + 128 * 2.0 ** -22)
        assert np.all((np.sign(q[m]) == np.sign(v)) | (q[m] == 0))
        # the scale is a/127 to within half an fp32 ulp
        assert abs(float(s[m]) - a[m] / 127.0) <= 2.0 ** -24 * a[m] / 127.0


# ---------------------------------------------------------------- format

def test_unpack_golden_word(orc):
    g = read_golden("packed_word.txt")
    packed = np.array([int(v, 16) for v in g["BYTES"]], np.uint8)
    t = orc.unpack(packed, 1, 16)
    assert t[0].tolist() == [int(v) for v in g["T"]]


def test_unpack_exhaustive_bytes(orc):
    # every byte value at every byte position of a word: exactly the 81 bytes
    # whose four fields are all < 3 decode; the other 175 are rejected.
    for pos in range(4):
        valid = 0
        for byte in range(256):
            word = np.full(4, 0x55, np.uint8)  # 0x55 = four zero-valued codes
            word[pos] = byte
            try:
                t = orc.unpack(word, 1, 16)
            except ValueError:
                continue
            valid += 1
            # only the 4 elements held by this byte may be nonzero
            nz = set(np.nonzero(t[0])[0].tolist())
            assert nz <= {pos, pos + 4, pos + 8, pos + 12}
        assert valid == 81


def test_unpack_bad_shapes(orc):
    with pytest.raises(ValueError):
        orc.unpack(np.zeros(3, np.uint8), 1, 12)


# ---------------------------------------------------------------- dequant

def test_dequant_exact_product(orc):
    rng = np.random.default_rng(2)
    acc = rng.integers(-10 ** 6, 10 ** 6, size=(3, 5)).astype(np.int32)
    acc[0, 0] = 0
    s = rng.random(3).astype(np.float32)
    g = rng.random(5).astype(np.float32)
    y = orc.dequant(acc, s, g)
    assert y[0, 0] == 0.0
    for m in range(3):
        for n in range(5):
            exact = Fraction(int(acc[m, n])) * Fraction(float(s[m])) * Fraction(float(g[n]))
            if exact == 0:
                assert y[m, n] == 0
            else:
                assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 51)


# ---------------------------------------------------------------- end to end

def test_hand_worked_example(orc):
    g = read_golden("hand_case_k16.txt")
    W = np.array([[float(v) for v in g["W0"]], [float(v) for v in g["W1"]]], np.float32)
    x = f32_to_bf16_bits(np.array([[float(v) for v in g["X0"]]], np.float32))
    r = orc.forward(W, (2,), x)
    assert r["gammas"] == [float(g["gamma"][0])]
    assert r["t"][0].tolist() == [int(v) for v in g["T0"]]
    assert r["t"][1].tolist() == [int(v) for v in g["T1"]]
    assert r["q"][0].tolist() == [int(v) for v in g["Q0"]]
    assert float(r["scale"][0]) == float(g["scale"][0])
    assert r["acc"][0].tolist() == [int(v) for v in g["ACC0"]]
    assert r["y"][0].tolist() == [float(v) for v in g["Y0"]]
    packed = np.array([[int(v, 16) for v in g["PACKED0"]],
                       [int(v, 16) for v in g["PACKED1"]]], np.uint8)
    np.testing.assert_array_equal(orc.unpack(packed, 2, 16), r["t"])


def test_segments_concatenate(orc):
    rng = np.random.default_rng(4)
    W = rng.standard_normal((48, 64), dtype=np.float32)
    W[32:] *= 5.0
    t, gammas, grow = orc.ternarize_segments(W, (32, 16))
    t0, g0 = orc.ternarize_absmean(W[:32])
    t1, g1 = orc.ternarize_absmean(W[32:])
    assert gammas == [g0, g1] and g1 > 4 * g0
    np.testing.assert_array_equal(t, np.concatenate([t0, t1]))
    assert np.all(grow[:32] == g0) and np.all(grow[32:] == g1)


# ------------------------------------------- role-dependent projections (FP8)

def _torch_e4m3():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    return torch


def test_e4m3_decode_against_torch_and_hand(orc):
    torch = _torch_e4m3()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([orc.e4m3_decode(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    g = read_golden("fp8_e4m3_hand.txt")
    for key, vals in g.items():
        if key.startswith("DECODE_"):
            c = int(key[7:], 16)
            v = orc.e4m3_decode(c)
            assert v == float(vals[0]) and math.copysign(1, v) == math.copysign(1, float(vals[0]))


def test_e4m3_encode_hand_ties(orc):
    rows = read_golden_rows("fp8_e4m3_hand.txt", "ENCODE")
    assert len(rows) == 8
    for v, c in rows:
        assert orc.e4m3_encode(float(v)) == int(c, 16), v
    with pytest.raises(ValueError):
        orc.e4m3_encode(470.0)  # rounds to 480, beyond the largest finite value
    with pytest.raises(ValueError):
        orc.e4m3_encode(float("inf"))


def test_e4m3_encode_against_torch(orc):
    torch = _torch_e4m3()
    rng = np.random.default_rng(11)
    finite = np.array([orc.e4m3_decode(c) for c in range(0x7F)])  # 0 .. 448
    mids = (finite[:-1] + finite[1:]) / 2  # every tie between neighbours
    f32 = mids.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), mids)  # ties are exact in fp32
    up = np.nextafter(f32, np.float32(np.inf))
    dn = np.nextafter(f32, np.float32(0))
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 3000)).astype(np.float32)
    vals = np.concatenate([f32, up, dn, rand, finite.astype(np.float32)])
    vals = vals[np.abs(vals) < 464.0]
    vals = np.concatenate([vals, -vals])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_round_trip_every_code(orc):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c


def test_fp8_quantizer_properties(orc):
    rng = np.random.default_rng(12)
    M, K = 6, 320
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(3.0)
    x[2] = 0.0
    x[3, 7] = 500.0  # a single outlier dominates the scale
    xb = f32_to_bf16_bits(x)
    codes, s = orc.quantize_act_fp8(xb)
    xf = bf16_bits_to_f32(xb)
    dec = np.vectorize(orc.e4m3_decode)(codes)
    for m in range(M):
        a = np.float32(np.abs(xf[m]).max())
        if a == 0:
            assert not codes[m].any() and s[m] == 0
            continue
        assert s[m] == np.float32(a / np.float32(448.0))
        assert np.abs(dec[m]).max() == 448.0
        inv = np.float32(448.0) / a
        p = (xf[m] * inv).astype(np.float64)
        # |rounding error| <= half the spacing at |p| (2^-10 below 2^-6)
        spacing = np.where(np.abs(p) < 2.0 ** -6, 2.0 ** -9,
                           2.0 ** (np.floor(np.log2(np.maximum(np.abs(p), 2.0 ** -6))) - 3))
        assert np.all(np.abs(dec[m] - p) <= spacing / 2)
        assert np.all((dec[m] == 0) | (np.sign(dec[m]) == np.sign(p)))
    # the weight quantizer applies the same rule per output row
    wc, ws = orc.quantize_fp8_rows(xf)
    np.testing.assert_array_equal(wc, codes)
    np.testing.assert_array_equal(ws, s)


def test_fp8_linear_exact_against_fractions(orc):
    rng = np.random.default_rng(13)
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    M, N, K = 3, 4, 37
    xq = rng.choice(finite, size=(M, K)).astype(np.uint8)
    wq = rng.choice(finite, size=(N, K)).astype(np.uint8)
    dot, absdot = orc.fp8_linear(xq, wq)
    val = {c: Fraction(orc.e4m3_decode(c)) for c in finite}
    for m in range(M):
        for n in range(N):
            exact = sum(val[int(xq[m, k])] * val[int(wq[n, k])] for k in range(K))
            assert Fraction(dot[m, n]) == exact
            assert Fraction(absdot[m, n]) == sum(abs(val[int(xq[m, k])] * val[int(wq[n, k])])
                                                 for k in range(K))
    # extremes: 8192 products of 448 * 448 stay exact
    big = np.full((1, 8192), 0x7E, np.uint8)
    d, _ = orc.fp8_linear(big, big)
    assert d[0, 0] == 448.0 * 448.0 * 8192
    with pytest.raises(ValueError):
        orc.fp8_linear(np.array([[0x7F]], np.uint8), np.array([[0x38]], np.uint8))


def test_fast_projection_hand_example(orc):
    g = read_golden("fp8_e4m3_hand.txt")
    W = np.array([[float(v) for v in g["W"]]], dtype=np.float32)
    x = np.array([[float(v) for v in g["X0"]], [float(v) for v in g["X1"]]], dtype=np.float32)
    r = orc.fast_projection(W, f32_to_bf16_bits(x))
    np.testing.assert_array_equal(r["wq"][0], [int(c, 16) for c in g["WQ"]])
    np.testing.assert_array_equal(r["xq"][0], [int(c, 16) for c in g["XQ0"]])
    np.testing.assert_array_equal(r["xq"][1], [int(c, 16) for c in g["XQ1"]])
    np.testing.assert_array_equal(r["xscale"], [float(v) for v in g["XSCALE"]])
    assert r["wscale"][0] == 1.0
    np.testing.assert_array_equal(r["y"][:, 0], [float(v) for v in g["Y"]])


def test_bf16_linear_against_fractions(orc):
    rng = np.random.default_rng(14)
    M, N, K = 2, 3, 29
    x = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    dot, absdot = orc.bf16_linear(x, w)
    xf, wf = bf16_bits_to_f32(x), bf16_bits_to_f32(w)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xf[m, k])) * Fraction(float(wf[n, k])) for k in range(K))
            bound = K * 2.0 ** -53 * absdot[m, n]
            assert abs(Fraction(dot[m, n]) - exact) <= Fraction(bound)
    # one-hot weight rows pick single activations; a zero row gives zero
    w1 = np.zeros((2, K), np.uint16)
    w1[0, 5] = 0x3F80  # 1.0
    d, _ = orc.bf16_linear(x, w1)
    np.testing.assert_array_equal(d[:, 0], xf[:, 5].astype(np.float64))
    assert not d[:, 1].any()


# ------------------------------------------- accepted-prefix KV commit

def _kv():
    from oracle import kv_commit
    return kv_commit


def test_kv_segment_geometry_closed_form():
    kv = _kv()
    for c0 in (1, 2, 16, 128):
        nseg = 9
        for s in range(nseg):
            start = c0 * (2 ** s - 1)           # after c0 (1 + 2 + ... + 2^(s-1))
            end = c0 * (2 ** (s + 1) - 1)
            assert kv.locate(start, c0, nseg) == (s, 0)
            assert kv.locate(end - 1, c0, nseg) == (s, c0 * 2 ** s - 1)
        assert kv.locate(c0 * (2 ** nseg - 1), c0, nseg) is None
        # a history of H positions needs ceil(log2(H / c0 + 1)) segments
        for H in range(1, c0 * 200, max(1, c0 // 3)):
            last = kv.locate(H - 1, c0, 12)[0]
            assert last + 1 == math.ceil(math.log2(H / c0 + 1) - 1e-12)


def test_kv_commit_hand_sequence():
    kv = _kv()
    st = kv.KVStore(c0=2, nseg=3, layers=1, row=2)
    commits = read_golden_rows("kv_commit_hand.txt", "COMMIT")
    states = read_golden_rows("kv_commit_hand.txt", "STATE")
    assert len(commits) == len(states) == 6
    for (c, W, n_mat, n_new), state in zip(commits, states):
        c, W = int(c), int(W)
        block = np.zeros((1, 2, W, 2), np.uint16)
        for j in range(W):
            for k in range(2):
                block[0, k, j] = [100 * c + 10 * j + k, 100 * c + 10 * j + k + 500]
        st.commit(block, int(n_mat), int(n_new))
        assert st.state == [int(v) for v in state]
    want = [np.zeros((1, 2, cap, 2), np.uint16) for cap in (2, 4, 8)]
    for s, o, k0, k1, v0, v1 in read_golden_rows("kv_commit_hand.txt", "SEG"):
        want[int(s)][0, 0, int(o)] = [int(k0), int(k1)]
        want[int(s)][0, 1, int(o)] = [int(v0), int(v1)]
    for got, w in zip(st.segs, want):
        np.testing.assert_array_equal(got, w)


def test_kv_commit_invariants_and_errors():
    kv = _kv()
    rng = np.random.default_rng(21)
    st = kv.KVStore(c0=4, nseg=5, layers=2, row=3)
    dense = []  # the materialized rows, kept independently in order
    for it in range(40):
        P, L, S, _ = st.state
        W = int(rng.integers(1, 7))
        block = rng.integers(0, 65535, (2, 2, W, 3)).astype(np.uint16)
        mode = rng.integers(0, 3)
        if mode == 0 and S <= W:            # verify: S pending + drafts
            a = int(rng.integers(0, W - S + 1))
            n_mat, n_new = S + a, a + 1
        elif mode == 1:                     # confidence-only
            n_mat, n_new = 0, int(rng.integers(1, 3))
        else:                               # autoregressive-like
            n_mat, n_new = min(1, S, W), 1
        if L + n_mat > st.capacity:
            break
        st.commit(block, n_mat, n_new)
        assert st.state[3] == 0
        P2, L2, S2, _ = st.state
        assert P2 == L2 + S2 and L2 == L + n_mat and P2 == P + n_new and S2 >= 0
        dense.extend(block[:, :, j, :] for j in range(n_mat))
        hist = st.history()
        np.testing.assert_array_equal(hist, np.stack(dense, axis=2) if dense else hist)
    assert len(dense) > 20
    # error paths leave every segment untouched
    before = [s.copy() for s in st.segs]
    bad = kv.KVStore(c0=4, nseg=5, layers=2, row=3, state=(5, 2, 2, 0))
    bad.commit(np.ones((2, 2, 2, 3), np.uint16), 1, 1)
    assert bad.state == [5, 2, 2, kv.ERR_IDENTITY] and not any(s.any() for s in bad.segs)
    neg = kv.KVStore(c0=4, nseg=5, layers=2, row=3, state=(1, -2, 3, 0))
    neg.commit(np.ones((2, 2, 2, 3), np.uint16), 1, 1)
    assert neg.state[3] == kv.ERR_IDENTITY and not any(s.any() for s in neg.segs)
    full = kv.KVStore(c0=2, nseg=3, layers=1, row=2, state=(14, 13, 1, 0))
    full.commit(np.ones((1, 2, 2, 2), np.uint16), 2, 1)
    assert full.state == [14, 13, 1, kv.ERR_CAPACITY]
    st2 = kv.KVStore(c0=2, nseg=3, layers=1, row=2)
    st2.commit(np.ones((1, 2, 2, 2), np.uint16), 3, 1)    # n_mat > W
    assert st2.state[3] == kv.ERR_COUNTS
    for a, b in zip(before, st.segs):
        np.testing.assert_array_equal(a, b)
