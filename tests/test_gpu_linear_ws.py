"""GPU parity of twd_ternary_linear_bf16_ws (the bf16 linear that runs as
two launches through a workspace where that is faster) against the CPU
oracle, through the C ABI.

Bar, as for the one-launch form: int32 accumulators bit-exact, y within 1e-6
relative of the oracle; and, since both forms use the same quantization and
epilogue, the workspace form's outputs equal the one-launch form's bit for
bit.  Cases on both sides of the form switch (M >= 14, or M >= 7 with
K >= 4096), ragged N, 1-3 segments, no workspace, a forced kernel, and a
captured graph replayed with eager work between replays.
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


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def check_y(y, yref, what):
    err = np.abs(np.asarray(y, dtype=np.float64) - yref)
    bad = err > REL_TOL * np.abs(yref)
    assert not bad.any(), f"{what}: {bad.sum()} y values outside 1e-6 relative"


def two_launch(M, K):
    return M >= 14 or (K >= 4096 and M >= 7)


CASES = [(6912, (2560,), M) for M in (1, 6, 7, 8, 13, 16)] + \
        [(2560, (96, 40, 40), M) for M in (8, 13, 14, 16)] + \
        [(4096, (37,), M) for M in (6, 7, 15)] + \
        [(8192, (33, 7), 16), (64, (17,), 16)]


@pytest.mark.parametrize("K,segs,M", CASES)
def test_linear_bf16_ws_matches_oracle(env, K, segs, M):
    torch, twd, orc = env
    W, segs, x = wl.random_case(seed=900 + M, M=M, K=K, seg_rows=segs)
    log(f"ws case M={M} K={K} segs={segs} two-launch={two_launch(M, K)}")
    packed, gammas = twd.prepare_weights(W, segs)
    wp = torch.from_numpy(packed).cuda()
    xd = dev_bf16(torch, x)
    ref = orc.forward(W, segs, x)
    assert gammas == ref["gammas"]
    ws = torch.full((twd.linear_bf16_workspace_bytes(M, K),), 0xA5, dtype=torch.uint8,
                    device="cuda")
    acc, y = twd.ternary_linear_bf16_ws(wp, segs, gammas, xd, workspace=ws)
    acc1, y1 = twd.ternary_linear_bf16(wp, segs, gammas, xd)
    acc0, y0 = twd.ternary_linear_bf16_ws(wp, segs, gammas, xd, workspace=None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(y.cpu().numpy(), ref["y"], "workspace form")
    # the same outputs as the one-launch form, with and without a workspace
    assert torch.equal(acc, acc1) and torch.equal(acc0, acc1)
    assert torch.equal(y.view(torch.int32), y1.view(torch.int32))
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    if two_launch(M, K):
        # the workspace holds the quantized rows and scales of the oracle
        n = M * K
        np.testing.assert_array_equal(ws[:n].cpu().numpy().view(np.int8).reshape(M, K), ref["q"])
        off = -(-n // 16) * 16
        xs = ws[off:off + 4 * M].cpu().numpy().view(np.float32)
        np.testing.assert_array_equal(xs.view(np.uint32), ref["scale"].view(np.uint32))


def test_linear_bf16_ws_forced_kernel_ignores_workspace(env):
    """A forced kernel family runs the one-launch form: the workspace is left
    as it was."""
    torch, twd, orc = env
    M, K = 16, 6912
    W, segs, x = wl.random_case(seed=950, M=M, K=K, seg_rows=(160,))
    packed, gammas = twd.prepare_weights(W, segs)
    wp = torch.from_numpy(packed).cuda()
    ws = torch.full((twd.linear_bf16_workspace_bytes(M, K),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    acc, y = twd.ternary_linear_bf16_ws(wp, segs, gammas, dev_bf16(torch, x), workspace=ws,
                                        kernel=twd.KERNEL_MFMA_STAGED)
    torch.cuda.synchronize()
    ref = orc.forward(W, segs, x)
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(y.cpu().numpy(), ref["y"], "forced kernel")
    assert bool((ws == 0x5A).all())


def test_linear_bf16_ws_graph_replays_match_oracle(env):
    """Both launches of the two-launch form captured into one graph: three
    replays, with eager work between them, each equal to the oracle."""
    torch, twd, orc = env
    M, K = 16, 6912
    W, segs, x = wl.random_case(seed=960, M=M, K=K, seg_rows=(300,))
    packed, gammas = twd.prepare_weights(W, segs)
    wp = torch.from_numpy(packed).cuda()
    xd = dev_bf16(torch, x)
    ref = orc.forward(W, segs, x)
    ws = torch.empty(twd.linear_bf16_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    acc = torch.empty((M, 300), dtype=torch.int32, device="cuda")
    y = torch.empty((M, 300), device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        twd.ternary_linear_bf16_ws(wp, segs, gammas, xd, workspace=ws, acc=acc, y=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            twd.ternary_linear_bf16_ws(wp, segs, gammas, xd, workspace=ws, acc=acc, y=y)
    for rep in range(3):
        acc.fill_(-1)
        y.fill_(float("nan"))
        ws.fill_(0x77)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
        check_y(y.cpu().numpy(), ref["y"], f"replay {rep}")
        _ = float(y.sum())  # eager work between replays
