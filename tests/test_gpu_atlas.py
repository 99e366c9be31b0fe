"""The finite set of captured decode graphs (BitMTP page, "Methodology in
Plain English": graphs captured ahead of time and picked by width, KV
capacity segment and numerical role), held at once and checked against the
CPU oracle on every replay.

One graph per (role, width), all sharing the same ternary weights, the same
output-projection weights and the same KV segments:
  * critical_mM, M = 1..16: the sweep over a small layer set at width M, the
    critical (bf16) output projection and two accepted-prefix commits of M
    rows (M = 1 an autoregressive step, M > 1 a verification);
  * draft_mM, M = 2..16: the sweep and the fast (E4M3) projection, nothing
    committed.
The graphs are replayed twice each in an interleaved order, with eager work
between replays and every output overwritten before each replay.  After each
replay: sweep accumulators bit-exact and y within 1e-6 relative of the
oracle, the projection within the fp32 summation bound of the oracle's
exact / double value, and the KV state words and every segment byte equal
to the oracle store that took the same commits.
"""
import sys

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6
U = 2.0 ** -24
LAYER = [(256, (48, 16, 16)), (256, (64, 64)), (512, (40,))]  # QKV-, gate/up-, down-like
HEAD_K, HEAD_N = 512, 300
C0, NSEG, LAYERS, ROW = 2, 9, 2, 8  # KV: 1022 positions of 2 layers x (K, V) x 8 bf16


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    from oracle import kv_commit as okv
    import ternary_weight_decode_amd as twd
    oracle.build(force=False)
    return torch, twd, oracle, okv


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def check_y(y, yref, what):
    err = np.abs(np.asarray(y, dtype=np.float64) - yref)
    bad = err > REL_TOL * np.abs(yref)
    assert not bad.any(), f"{what}: {bad.sum()} y values outside 1e-6 relative"


def check_bound(y, yref, yabs, K, what):
    g = K * U / (1 - K * U)
    err = np.abs(np.asarray(y, dtype=np.float64) - yref)
    bad = err > g * yabs + 3 * U * np.abs(yref)
    assert not bad.any(), f"{what}: {bad.sum()} values outside the fp32 summation bound"
    assert np.all(np.asarray(y)[yabs == 0] == 0), f"{what}: nonzero y where every product is zero"


def test_role_width_atlas_replays_match_oracle(env):
    torch, twd, orc, okv = env
    # shared weights: the ternary layer (tiled for the sweep) and the head
    layer = []
    for i, (K, segs) in enumerate(LAYER):
        W, segs, _ = wl.random_case(seed=600 + i, M=1, K=K, seg_rows=segs)
        packed, gammas = twd.prepare_weights(W, segs)
        wt = torch.from_numpy(twd.tile_for_sweep(packed, int(sum(segs)), K)).cuda()
        layer.append((W, segs, gammas, wt))
    Wh, _, _ = wl.random_case(seed=650, M=1, K=HEAD_K, seg_rows=(HEAD_N,), w_sigma=0.02)
    wq, ws = orc.quantize_fp8_rows(Wh)
    wq_d, ws_d = torch.from_numpy(wq).cuda(), torch.from_numpy(ws).cuda()
    wb = wl.f32_to_bf16_bits(Wh)
    wb_d = dev_bf16(torch, wb)
    segs_kv = [torch.zeros(LAYERS * 2 * cap * ROW * 2, dtype=torch.uint8, device="cuda")
               for cap in twd.kv_segment_positions(C0, NSEG)]
    state = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    state[0] = torch.tensor([1, 0, 1, 0], dtype=torch.int32)
    counts = torch.tensor([[m, m] for m in range(17)], dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(651)

    # per width: activations, outputs, oracle results, the KV block
    per = {}
    for M in range(1, 17):
        proj, entries = [], []
        for i, (W, segs, gammas, wt) in enumerate(layer):
            _, _, x = wl.random_case(seed=700 + 31 * M + i, M=M, K=W.shape[1], seg_rows=segs)
            N = int(sum(segs))
            acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
            y = torch.empty((M, N), device="cuda")
            entries.append((wt, segs, gammas, dev_bf16(torch, x), acc, y))
            ref = orc.forward(W, segs, x)
            assert gammas == ref["gammas"]
            proj.append((acc, y, ref))
        _, _, xh = wl.random_case(seed=800 + M, M=M, K=HEAD_K, seg_rows=(HEAD_N,))
        fast = orc.fast_projection(Wh, xh)
        dot, absdot = orc.bf16_linear(xh, wb)
        block = rng.integers(0, 65536, (LAYERS, 2, M, ROW)).astype(np.uint16)
        per[M] = dict(sweep=twd.Sweep(entries), proj=proj, xh=dev_bf16(torch, xh),
                      y_fast=torch.empty((M, HEAD_N), device="cuda"),
                      y_crit=torch.empty((M, HEAD_N), device="cuda"),
                      fast=fast, crit=(dot, absdot), block=block,
                      block_d=torch.from_numpy(block.view(np.uint8).reshape(-1)).cuda())

    def iteration(M, role):
        p = per[M]

        def run():
            p["sweep"].run()
            if role == "draft":
                twd.projection_fp8(wq_d, ws_d, p["xh"], y=p["y_fast"])
            else:
                twd.projection_bf16(wb_d, p["xh"], y=p["y_crit"])
                for j in range(2):  # two commits leave the state on word 0
                    twd.kv_commit(segs_kv, C0, LAYERS, ROW * 2, p["block_d"], M,
                                  counts[M, 0:1], counts[M, 1:2], state[j], state[1 - j])
        return run

    keys = [("critical", M) for M in range(1, 17)] + [("draft", M) for M in range(2, 17)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):  # eager launches of everything but the commits
        for M, p in per.items():
            p["sweep"].run()
            twd.projection_fp8(wq_d, ws_d, p["xh"], y=p["y_fast"])
            twd.projection_bf16(wb_d, p["xh"], y=p["y_crit"])
    torch.cuda.synchronize()
    graphs = {}
    for role, M in keys:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                iteration(M, role)()
        graphs[(role, M)] = g
    torch.cuda.synchronize()
    log(f"atlas of {len(graphs)} graphs held")

    store = okv.KVStore(C0, NSEG, LAYERS, ROW)
    order = list(graphs)
    for rnd in range(2):
        np.random.default_rng(652 + rnd).shuffle(order)
        for role, M in order:
            what = f"{role}_m{M} replay {rnd}"
            p = per[M]
            for acc, y, _ in p["proj"]:
                acc.fill_(-3)
                y.fill_(-3.0)
            p["y_fast"].fill_(float("nan"))
            p["y_crit"].fill_(float("nan"))
            graphs[(role, M)].replay()
            torch.cuda.synchronize()
            for i, (acc, y, ref) in enumerate(p["proj"]):
                np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"],
                                              err_msg=f"{what} projection {i}")
                check_y(y.cpu().numpy(), ref["y"], f"{what} projection {i}")
            if role == "draft":
                check_bound(p["y_fast"].cpu().numpy(), p["fast"]["y"], p["fast"]["yabs"],
                            HEAD_K, f"{what} fast head")
            else:
                check_bound(p["y_crit"].cpu().numpy(), *p["crit"], HEAD_K, f"{what} critical head")
                for _ in range(2):
                    store.commit(p["block"], M, M)
            got = state[0].cpu().numpy().tolist()
            assert got == store.state, (what, got, store.state)
            _ = float(p["proj"][0][1].sum())  # eager work between replays
    assert store.state[3] == 0 and store.state[1] > 0
    for i, (d, o) in enumerate(zip(segs_kv, store.segs)):
        np.testing.assert_array_equal(d.cpu().numpy().view(np.uint16).reshape(o.shape), o,
                                      err_msg=f"KV segment {i}")
    log(f"  {2 * len(graphs)} replays checked; KV length {store.state[1]} of {store.capacity}")
    del graphs
