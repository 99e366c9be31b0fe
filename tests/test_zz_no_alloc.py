"""GPU check of twd_ternary_linear_bf16_noalloc (the bf16 linear on the
library's own static per-device workspace, for callers that cannot allocate)
against twd_ternary_linear_bf16_ws with a caller's workspace, through the C
ABI.

Both run the same launches on the same inputs, so the bar is equality: int32
accumulators and fp32 y bit for bit (stricter than the 1e-6 relative bar
against the oracle, which is checked too).  Calls in a row share the static
array: the first (M = 16, K = 6912) fills it, the second (M = 7, K = 4096, a
smaller input that also runs two launches) must not see what the first left,
and a third (M = 4) runs the one-launch form.
"""
import sys

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6
SEQUENCE = [(16, 6912, (2560,)), (7, 4096, (37, 200)), (4, 2560, (96, 40, 40)),
            (16, 8192, (33,))]


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


def test_noalloc_matches_workspace_form_on_calls_in_a_row(env):
    torch, twd, orc = env
    for i, (M, K, segs) in enumerate(SEQUENCE):
        W, segs, x = wl.random_case(seed=980 + i, M=M, K=K, seg_rows=segs)
        N = int(sum(segs))
        log(f"noalloc call {i}: M={M} K={K} segs={segs}")
        packed, gammas = twd.prepare_weights(W, segs)
        wp = torch.from_numpy(packed).cuda()
        xd = dev_bf16(torch, x)
        ws = torch.full((twd.linear_bf16_workspace_bytes(M, K),), 0xA5, dtype=torch.uint8,
                        device="cuda")
        acc_ws, y_ws = twd.ternary_linear_bf16_ws(wp, segs, gammas, xd, workspace=ws)
        acc = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
        y = torch.full((M, N), float("nan"), device="cuda")
        twd.ternary_linear_bf16_noalloc(wp, segs, gammas, xd, acc, y)
        torch.cuda.synchronize()
        assert torch.equal(acc, acc_ws), f"call {i}: acc differs from the workspace form"
        assert torch.equal(y.view(torch.int32), y_ws.view(torch.int32)), \
            f"call {i}: y differs from the workspace form"
        ref = orc.forward(W, segs, x)
        assert gammas == ref["gammas"]
        np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref["y"])
        assert not (err > REL_TOL * np.abs(ref["y"])).any(), f"call {i}: y outside 1e-6 relative"


def test_noalloc_rejects_before_launch(env):
    torch, twd, _ = env
    W, segs, x = wl.random_case(seed=990, M=4, K=128, seg_rows=(16,))
    packed, gammas = twd.prepare_weights(W, segs)
    wp = torch.from_numpy(packed).cuda()
    xd = dev_bf16(torch, x)
    acc = torch.zeros((4, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        twd.ternary_linear_bf16_noalloc(wp, segs, gammas, xd, acc, None, kernel=99)
    torch.cuda.synchronize()
    assert bool((acc == 0).all())


def test_noalloc_graph_replays_match_oracle(env):
    """A caller that cannot allocate under capture: after one eager call has
    set the device up, the two-launch call is captured into a graph and
    replayed three times, with eager work between replays; every replay
    equals the oracle."""
    torch, twd, orc = env
    M, K, segs = 16, 6912, (300,)
    W, segs, x = wl.random_case(seed=995, M=M, K=K, seg_rows=segs)
    N = int(sum(segs))
    packed, gammas = twd.prepare_weights(W, segs)
    wp = torch.from_numpy(packed).cuda()
    xd = dev_bf16(torch, x)
    ref = orc.forward(W, segs, x)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = torch.empty((M, N), device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        twd.ternary_linear_bf16_noalloc(wp, segs, gammas, xd, acc, y)
    torch.cuda.synchronize()
    log("noalloc graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            twd.ternary_linear_bf16_noalloc(wp, segs, gammas, xd, acc, y)
    for rep in range(3):
        acc.fill_(-1)
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref["y"])
        assert not (err > REL_TOL * np.abs(ref["y"])).any(), f"replay {rep}: y outside 1e-6"
        _ = float(y.sum())  # eager work between replays
