#!/usr/bin/env python3
"""Benchmark of the W2A8 ternary linear hot path on one MI355X.

A step is one pass of the whole hot path over the 2B-class decode layer set
(30 layers x {fused QKV 2560->3840, O 2560->2560, fused gate/up
2560->13824, down 6912->2560}) at width M: per projection, the per-token
absmax int8 quantization of a fresh bf16 activation block and the ternary
linear with its dequant epilogue.  The step runs as one multi-projection
sweep launch (twd_ternary_sweep) over the 120 projections, whose inputs are
independent; it is recorded once into a HIP graph and replayed.  All weights
(521 MB packed, more than the 256 MB Infinity Cache, so every step streams
cold weights) and activations are resident in HBM before timing starts.

Output: one JSON line.  `value` is packed-weight bytes per second over the
timed steps (wall clock between two synchronizations).  Two HIP events around
the timed replays, on the replaying stream, give the sweep kernel's average
launch duration, from which `roofline` rates it against MI355X's 8 TB/s HBM
peak (its `trace` entry repeats the rocprofv3 kernel-trace figure of the same
command, from profiles/, when it was taken on the current sources).  Also
reported: the same step as one launch per projection (and the two-launch
form), streaming-read references, every width 1..16 on the outlier workload,
the 4B-class stack, the per-width graph atlas, the output projection, the KV
commit, and `cpu_baseline`, the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "ternary_linear weight-stream GB/s and % HBM roofline at M=1,2,4,8,16"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class LayerSetOnDevice:
    """Packed weights of every projection, uploaded once: row-major (the
    per-projection launches) and in the sweep's tiled layout."""

    def __init__(self, twd, torch, ls, layers, tiled=True):
        self.ls = ls
        self.layers = layers
        self.w, self.wt, self.gammas = {}, {}, {}

        def prep(key):
            layer, pi = key
            p = ls.projs[pi]
            W = wl.layer_weights(ls, layer, pi)
            packed, gammas = twd.prepare_weights(W, p.segs)
            t = twd.tile_for_sweep(packed, p.N, p.K) if tiled else None
            return key, packed, t, gammas

        keys = [(l, p) for l in range(layers) for p in range(len(ls.projs))]
        with ThreadPoolExecutor(max_workers=host_threads()) as ex:
            for key, packed, t, gammas in ex.map(prep, keys):
                self.w[key] = torch.from_numpy(packed).cuda()
                if t is not None:
                    self.wt[key] = torch.from_numpy(t).cuda()
                self.gammas[key] = gammas
        torch.cuda.synchronize()

    @property
    def bytes_per_sweep(self):
        return self.layers * self.ls.packed_bytes_per_layer


class Step:
    """Inputs, outputs and launches of one step at width M."""

    def __init__(self, twd, torch, dev_set, workload, M, kernel, outliers=False):
        self.twd, self.torch, self.ds = twd, torch, dev_set
        self.M, self.kernel = M, kernel
        ls = dev_set.ls
        self.x, self.xq, self.xs, self.y = {}, {}, {}, {}
        for layer in range(dev_set.layers):
            for pi, p in enumerate(ls.projs):
                xb = wl.layer_activations(workload, p.K, M, layer, pi, outliers=outliers)
                self.x[(layer, pi)] = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
                self.xq[(layer, pi)] = torch.empty((M, p.K), dtype=torch.int8, device="cuda")
                self.xs[(layer, pi)] = torch.empty((M,), dtype=torch.float32, device="cuda")
                self.y[(layer, pi)] = torch.empty((M, p.N), dtype=torch.float32, device="cuda")
        self._sweep = None
        torch.cuda.synchronize()

    def keys(self):
        return [(l, p) for l in range(self.ds.layers) for p in range(len(self.ds.ls.projs))]

    @property
    def plan(self):
        return self.sweep_obj().plan

    def sweep_obj(self):
        if self._sweep is None:
            self._sweep = self.twd.Sweep(
                [(self.ds.wt[k], self.ds.ls.projs[k[1]].segs, self.ds.gammas[k], self.x[k],
                  None, self.y[k]) for k in self.keys()])
        return self._sweep

    def sweep(self):
        """The step: one multi-projection launch over every projection."""
        self.sweep_obj().run()

    def fused(self):
        """The step as one launch per projection (quantize + linear)."""
        for k in self.keys():
            p = self.ds.ls.projs[k[1]]
            self.twd.ternary_linear_bf16(self.ds.w[k], p.segs, self.ds.gammas[k], self.x[k],
                                         y=self.y[k], want_acc=False, kernel=self.kernel)

    def workspace_form(self):
        """One call per projection of the bf16 linear that runs two launches
        through a workspace where they are faster (one workspace shared by
        the calls, which run in order on one stream)."""
        if getattr(self, "_ws", None) is None:
            K = max(p.K for p in self.ds.ls.projs)
            self._ws = self.torch.empty(self.twd.linear_bf16_workspace_bytes(self.M, K),
                                        dtype=self.torch.uint8, device="cuda")
        for k in self.keys():
            p = self.ds.ls.projs[k[1]]
            self.twd.ternary_linear_bf16_ws(self.ds.w[k], p.segs, self.ds.gammas[k], self.x[k],
                                            workspace=self._ws, y=self.y[k], want_acc=False,
                                            kernel=self.kernel)

    def two_launch(self):
        """Stand-alone quantizer, then the pre-quantized linear."""
        for k in self.keys():
            p = self.ds.ls.projs[k[1]]
            self.twd.quantize_act(self.x[k], self.xq[k], self.xs[k])
            self.twd.ternary_linear_fused(self.ds.w[k], p.segs, self.ds.gammas[k],
                                          self.xq[k], self.xs[k], y=self.y[k],
                                          want_acc=False, kernel=self.kernel)

    def snapshot(self):
        return {k: v.clone() for k, v in self.y.items()}

    def equals(self, snap):
        return all(self.torch.equal(self.y[k].view(self.torch.int32),
                                    snap[k].view(self.torch.int32)) for k in self.keys())

    def clear(self):
        for v in self.y.values():
            v.fill_(-1.0)


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_replays(torch, g, reps):
    """Wall seconds and event seconds for `reps` back-to-back replays."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, start.elapsed_time(end) * 1e-3


def time_launches(torch, fn, reps):
    """Wall seconds and event seconds for reps direct calls of fn on the
    current stream (no graph), synchronized on both sides."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, start.elapsed_time(end) * 1e-3


def time_eager(torch, fn, reps):
    """Wall seconds for `reps` eager calls of fn (no graph), synchronized on
    both sides."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def stream_read_reference(twd, torch, dev_set, reps):
    """The plain streaming-read kernel (every compute unit busy, eight loads
    in flight per lane): once over one contiguous buffer of the step's bytes
    (the sweep's reference: one launch, timed as direct launches like the
    sweep), and over each projection's weight buffer in turn (the
    per-projection launches' reference, graph-replayed like them).  Returns
    ({gbs, us}, {gbs, avg_launch_us})."""
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    keys = [(l, p) for l in range(dev_set.layers) for p in range(len(dev_set.ls.projs))]
    nbytes = dev_set.bytes_per_sweep
    big = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    # direct launches, as the sweep step is timed
    for _ in range(5):
        twd.stream_read(big, nbytes, sink)
    _, sec = time_launches(torch, lambda: twd.stream_read(big, nbytes, sink), reps)
    one = {"gbs": round(nbytes * reps / sec / 1e9, 1), "us": round(sec / reps * 1e6, 2)}
    del big

    def sweep():
        for k in keys:
            w = dev_set.w[k]
            twd.stream_read(w, w.numel(), sink)

    g = capture(torch, sweep)
    g.replay()
    _, sec = time_replays(torch, g, reps)
    per = {"gbs": round(nbytes * reps / sec / 1e9, 1),
           "avg_launch_us": round(sec / (reps * len(keys)) * 1e6, 3)}
    torch.cuda.empty_cache()
    return one, per


def settle(torch, fn, seconds=0.25):
    """Untimed direct launches of fn for about `seconds`: the clocks settle
    before a timed run, as before the headline's."""
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        fn()
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_graph(torch, fn, reps):
    """Capture fn into a graph and time reps replays: (graph, seconds per
    replay)."""
    g = capture(torch, fn)
    g.replay()
    _, sec = time_replays(torch, g, reps)
    return g, sec / reps


def width_entry(twd, torch, dev_set, workload, M, kernel, reps, outliers=False,
                forms=("sweep", "fused", "two_launch", "workspace"), graphs=True):
    """One width.  The sweep (one launch per step) is timed as launched
    directly, back to back, and (graphs) also captured into a graph and
    replayed; the per-projection forms are captured and replayed (graph) and,
    with graphs, also launched directly -- the launch gaps a graph removes.
    The sweep's outputs must equal the per-projection launch's bit for bit."""
    st = Step(twd, torch, dev_set, workload, M, kernel, outliers)
    nbytes = dev_set.bytes_per_sweep
    n = len(st.keys())
    out = {}
    if "fused" in forms:
        st.fused()
        torch.cuda.synchronize()
        ref = st.snapshot()
    if "sweep" in forms:
        st.clear()
        st.sweep()
        torch.cuda.synchronize()
        if "fused" in forms and not st.equals(ref):
            raise SystemExit(f"sweep differs from the per-projection launches at M={M}")
        settle(torch, st.sweep)
        _, sec = time_launches(torch, st.sweep, reps)
        sec /= reps
        e = {"gbs": round(nbytes / sec / 1e9, 1), "frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4),
             "us": round(sec * 1e6, 2), "workgroups": st.plan.nwg}
        if graphs:
            g, gsec = time_graph(torch, st.sweep, reps)
            e["graph_us"] = round(gsec * 1e6, 2)
            del g
        prof = sweep_profile(workload, M, nbytes)
        if prof:
            e["trace"] = prof
        out["sweep"] = e
    if "fused" in forms:
        g, sec = time_graph(torch, st.fused, reps)
        e = {"gbs": round(nbytes / sec / 1e9, 1), "frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4),
             "us_per_launch": round(sec / n * 1e6, 3), "kernels": kernel_map(twd, dev_set.ls, M, kernel)}
        if graphs:
            k = max(3, reps // 3)
            esec = time_eager(torch, st.fused, k) / k
            e["eager_us_per_launch"] = round(esec / n * 1e6, 3)
            e["graph_saves_us_per_launch"] = round((esec - sec) / n * 1e6, 3)
        out["per_launch"] = e
        del g
    if "two_launch" in forms:
        g, sec = time_graph(torch, st.two_launch, reps)
        out["two_launch"] = {"gbs": round(nbytes / sec / 1e9, 1),
                             "kernels": kernel_map(twd, dev_set.ls, M, kernel, False)}
        del g
    if "workspace" in forms:
        # the entry point that picks the form per shape (two launches through
        # a workspace where they are faster); its outputs equal the
        # one-launch form's
        if "fused" in forms:
            st.clear()
            st.workspace_form()
            torch.cuda.synchronize()
            if not st.equals(ref):
                raise SystemExit(f"workspace form differs from the one-launch form at M={M}")
        g, sec = time_graph(torch, st.workspace_form, reps)
        out["workspace_form"] = {"gbs": round(nbytes / sec / 1e9, 1),
                                 "us_per_projection": round(sec / n * 1e6, 3)}
        del g
    if "per_launch" in out and "two_launch" in out:
        # the faster of the two fixed per-projection forms at this width
        best = max(("one_launch", out["per_launch"]["gbs"]), ("two_launch", out["two_launch"]["gbs"]),
                   key=lambda kv: kv[1])
        out["per_projection_best"] = {"form": best[0], "gbs": best[1]}
    del st
    torch.cuda.empty_cache()
    return out


def output_projection_bench(twd, torch, widths, reps):
    """The role-dependent output projection (hidden 2560 -> 128256 rows) in
    both roles: fast (E4M3 weight codes, activations quantized inside) and
    critical (bf16), timed as direct launches that alternate two distinct
    weight copies (656 MB / 1.3 GB, beyond the 256 MB Infinity Cache), so
    every launch reads cold weights (the same launches replayed from a graph
    are reported beside as graph_us); the weights are random on-device values (random
    finite E4M3 codes, N(0, 0.02) bf16), since the kernels' timing does not
    depend on them.  The streaming read over the same buffers is the
    achievable-bandwidth reference."""
    K, N = wl.HEAD_K, wl.HEAD_N
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    copies = 2
    w8 = []
    for _ in range(copies):
        b = torch.randint(0, 256, (N, K), dtype=torch.uint8, device="cuda", generator=gen)
        b[(b & 0x7F) == 0x7F] = 0x38  # no NaN codes
        w8.append(b)
    ws = torch.rand(N, device="cuda", generator=gen) * 1e-3
    w16 = [(torch.randn((N, K), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
           for _ in range(copies)]
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")

    def timed(fn, nbytes):
        # direct launches alternating the copies (as the sweep step is
        # timed), and the same launches replayed from a graph beside them;
        # about 0.25 s of untimed launches first settle the clocks
        t_end = time.perf_counter() + 0.25
        i = 0
        while time.perf_counter() < t_end:
            fn(i % copies)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        n = reps * copies
        state = {"i": 0}

        def one():
            fn(state["i"] % copies)
            state["i"] += 1

        _, sec = time_launches(torch, one, n)
        us = sec / n * 1e6
        g = capture(torch, lambda: [fn(c) for c in range(copies)])
        t_end = time.perf_counter() + 0.1
        while time.perf_counter() < t_end:
            g.replay()
            torch.cuda.synchronize()
        _, gsec = time_replays(torch, g, reps)
        del g
        return {"us": round(us, 2), "gbs": round(nbytes / us / 1e3, 1),
                "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                "graph_us": round(gsec / (reps * copies) * 1e6, 2)}

    out = {"shape": f"K={K} -> N={N} (2B-class output projection)",
           "weights": "random finite E4M3 codes / N(0,0.02) bf16 on device; two copies per graph",
           "fast_fp8": {}, "critical_bf16": {}}
    for M in widths:
        x = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
        y = torch.empty((M, N), device="cuda")
        out["fast_fp8"][str(M)] = timed(lambda c: twd.projection_fp8(w8[c], ws, x, y=y), N * K)
        out["critical_bf16"][str(M)] = timed(lambda c: twd.projection_bf16(w16[c], x, y=y),
                                             2 * N * K)
    rec = None
    path = os.path.join(PROFILES, "output_projection_counters_2b_m1.json")
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_hash") != kernel_source_hash(PROJECTION_SOURCES):
            rec = None
    for role, nbytes in (("fast_fp8", N * K), ("critical_bf16", 2 * N * K)):
        one = out[role].get("1")
        if one:
            out[role]["roofline_m1"] = {
                "bound": "hbm", "achieved": one["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": one["frac"],
                "traffic": rec[role]["hbm_bytes_per_launch"] if rec else None}
    out["stream_read_fp8_bytes"] = timed(lambda c: twd.stream_read(w8[c], N * K, sink), N * K)
    out["stream_read_bf16_bytes"] = timed(lambda c: twd.stream_read(w16[c], 2 * N * K, sink),
                                          2 * N * K)
    del w8, w16
    torch.cuda.empty_cache()
    return out


def cpu_projection_baseline(budget_s, M=1, rows=1024):
    """The CPU oracle of both projection roles (single-threaded C loops:
    E4M3 decode, exact int64 sums / double sums) on a sample of the output
    projection's rows, repeated until budget_s; throughput in weight bytes/s
    of each role."""
    import oracle
    oracle_native()
    W = wl.head_weight_block(0)[:rows]
    x = wl.head_activations(M)
    out = {}
    for role, bpw in (("fast_fp8", 1), ("critical_bf16", 2)):
        if role == "fast_fp8":
            wq, _ = oracle.quantize_fp8_rows(W)
            xq, _ = oracle.quantize_act_fp8(x)
            fn = lambda: oracle.fp8_linear(xq, wq)  # noqa: E731
        else:
            wb = wl.f32_to_bf16_bits(W)
            fn = lambda: oracle.bf16_linear(x, wb)  # noqa: E731
        spent, n = 0.0, 0
        while n == 0 or spent < budget_s:
            t0 = time.perf_counter()
            fn()
            spent += time.perf_counter() - t0
            n += 1
        out[role] = {"value": round(rows * wl.HEAD_K * bpw * n / spent / 1e9, 4), "unit": "GB/s",
                     "cores": 1, "kind": "oracle",
                     "sample": f"{n} pass(es) over {rows} rows of the output projection at M={M} "
                               f"({spent:.1f} s; weight bytes/s)"}
    return out


def cpu_kv_baseline(budget_s, D=8, c0=256, nseg=8, start=1000):
    """The CPU oracle of the KV commit (oracle/kv_commit.py) on the bench's
    geometry and acceptance draws, timed per commit on one thread."""
    from oracle import kv_commit as okv
    ls = wl.SET_2B
    layers, row = ls.layers, ls.projs[0].segs[1]
    store = okv.KVStore(c0, nseg, layers, row, state=(start + 1, start, 1, 0))
    rng = np.random.default_rng(2027)
    block = rng.integers(0, 65536, (layers, 2, D + 1, row)).astype(np.uint16)
    spent, n, moved = 0.0, 0, 0
    while n == 0 or spent < budget_s:
        a = int(rng.integers(0, D + 1))
        t0 = time.perf_counter()
        store.commit(block, 1 + a, a + 1)
        spent += time.perf_counter() - t0
        n += 1
        moved += 2 * (1 + a) * layers * 2 * row * 2
    return {"value": round(spent / n * 1e6, 1), "unit": "us per commit", "cores": 1,
            "kind": "oracle", "gbs": round(moved / spent / 1e9, 3),
            "sample": f"{n} commits of width {D + 1} on the 2B-class KV geometry ({spent:.1f} s)"}


def kv_commit_bench(twd, torch, ls, reps, D=8, steps=64, c0=256, nseg=8, start=1000):
    """Accepted-prefix KV commits on the 2B-class KV geometry (30 layers, K
    and V rows of 640 bf16 = 1280 bytes; segments of 256 * 2^s positions,
    8 segments, 65280 positions): one captured graph of 64 verification
    commits of width D + 1 = 9, the state words alternating, with seeded
    acceptance lengths a ~ uniform{0..D} (n_mat = 1 + a, n_new = a + 1).
    Each replay continues from the state the last one left.  Beside it: the
    time of copying the whole history once (what graphs without a shared KV
    view would pay), as a plain copy of the same bytes."""
    layers, row_bytes = ls.layers, ls.projs[0].segs[1] * 2
    W = D + 1
    pos_bytes = layers * 2 * row_bytes
    segs = [torch.zeros(layers * 2 * cap * row_bytes, dtype=torch.uint8, device="cuda")
            for cap in twd.kv_segment_positions(c0, nseg)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    blocks = [torch.randint(0, 256, (layers * 2 * W * row_bytes,), dtype=torch.uint8,
                            device="cuda", generator=gen) for _ in range(4)]
    rng = np.random.default_rng(2027)
    acc = rng.integers(0, D + 1, steps)
    nm = torch.from_numpy((1 + acc).astype(np.int32)).cuda()
    nn = torch.from_numpy((acc + 1).astype(np.int32)).cuda()
    state = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    state[0] = torch.tensor([start + 1, start, 1, 0], dtype=torch.int32)

    def seq():
        for i in range(steps):
            twd.kv_commit(segs, c0, layers, row_bytes, blocks[i % 4], W, nm[i:i + 1],
                          nn[i:i + 1], state[i % 2], state[(i + 1) % 2])

    per_replay = int((1 + acc).sum())
    reps = max(1, min(reps, (c0 * (2 ** nseg - 1) - start) // per_replay - 2))
    g = capture(torch, seq)   # capture() runs the sequence once eagerly first
    g.replay()
    _, sec = time_replays(torch, g, reps)
    torch.cuda.synchronize()
    final = state[0].cpu().tolist()
    expect_L = start + per_replay * (reps + 2)
    if final[3] != 0 or final[1] != expect_L or final[0] != final[1] + final[2]:
        raise SystemExit(f"kv commit state {final}, expected L={expect_L}")
    us = sec / (reps * steps) * 1e6
    moved = 2 * pos_bytes * per_replay / steps  # bytes read + written per commit
    hist_bytes = final[1] * pos_bytes
    src = torch.empty(hist_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    gc = capture(torch, lambda: twd.stream_copy(src, dst, hist_bytes))
    gc.replay()
    _, csec = time_replays(torch, gc, 5)
    del segs, blocks, src, dst
    torch.cuda.empty_cache()
    return {"geometry": f"{layers} layers x K,V rows of {row_bytes} B; segments of {c0}*2^s "
                        f"positions, {nseg} segments ({c0 * (2 ** nseg - 1)} positions)",
            "width": W, "commits_timed": reps * steps,
            "mean_rows_per_commit": round(per_replay / steps, 3),
            "us_per_commit": round(us, 3),
            "bytes_moved_per_commit": round(moved),
            "gbs": round(moved / us / 1e3, 1),
            "final_state": final,
            "full_history_copy_us": round(csec / 5 * 1e6, 1),
            "full_history_bytes": hist_bytes}


def atlas_bench(twd, torch, dev_set, reps, widths=range(1, 17), c0=256, nseg=8, start=1000):
    """The hot path as a finite set of captured graphs, all held at once and
    sharing the weights and the KV segments, one per (role, width): a decode
    iteration at width M is the sweep over every layer, the output projection
    in the iteration's role and, where tokens are committed, the KV commit.
    For every M: the critical state (M = 1 autoregressive, M > 1 verification:
    bf16 projection, commit of M rows) and, for M > 1, the drafting state
    (fast E4M3 projection, nothing committed).  Each graph is replayed in turn;
    every replay's sweep outputs must equal the eager sweep's."""
    ls = dev_set.ls
    K, N = wl.HEAD_K, wl.HEAD_N
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    w8 = torch.randint(0, 256, (N, K), dtype=torch.uint8, device="cuda", generator=gen)
    w8[(w8 & 0x7F) == 0x7F] = 0x38
    ws = torch.rand(N, device="cuda", generator=gen) * 1e-3
    w16 = (torch.randn((N, K), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    layers, row_bytes = ls.layers, ls.projs[0].segs[1] * 2
    segs = [torch.zeros(layers * 2 * cap * row_bytes, dtype=torch.uint8, device="cuda")
            for cap in twd.kv_segment_positions(c0, nseg)]
    Wmax = max(widths)
    block = torch.randint(0, 256, (layers * 2 * Wmax * row_bytes,), dtype=torch.uint8,
                          device="cuda", generator=gen)
    counts = torch.tensor([[m, m] for m in range(Wmax + 1)], dtype=torch.int32, device="cuda")
    state = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    state[0] = torch.tensor([start + 1, start, 1, 0], dtype=torch.int32)
    steps = {M: Step(twd, torch, dev_set, "2b_sweep_outlier", M, twd.KERNEL_AUTO, True)
             for M in widths}
    heads = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in widths}
    eager = {}
    for M, st in steps.items():
        st.sweep()
        torch.cuda.synchronize()
        eager[M] = st.snapshot()

    def iteration(M, role, commit):
        def run():
            st = steps[M]
            st.sweep()
            xh = st.x[(layers - 1, 0)]  # the last layer's hidden rows stand in
            if role == "fast":
                twd.projection_fp8(w8, ws, xh, y=heads[M])
            else:
                twd.projection_bf16(w16, xh, y=heads[M])
            if commit:
                # two commits per graph keep the state on the first word
                for j in range(2):
                    twd.kv_commit(segs, c0, layers, row_bytes, block, Wmax, counts[M, 0:1],
                                  counts[M, 1:2], state[j], state[1 - j])
        return run

    entries = {}
    for M in widths:
        entries[f"critical_m{M}"] = (M, "critical", True)
        if M > 1:
            entries[f"draft_m{M}"] = (M, "fast", False)
    graphs = {k: capture(torch, iteration(*v)) for k, v in entries.items()}
    out = {"states": "critical_mM: the sweep at width M, the bf16 output projection and two "
                     "KV commits of M rows (M = 1: an autoregressive step, M > 1: "
                     "verification); draft_mM: the sweep and the E4M3 output projection",
           "graphs_held": len(graphs), "sweep_bytes": dev_set.bytes_per_sweep, "us": {}}
    for k, g in graphs.items():
        M = entries[k][0]
        g.replay()
        _, sec = time_replays(torch, g, reps)
        out["us"][k] = round(sec / reps * 1e6, 1)
        steps[M].clear()
        g.replay()
        torch.cuda.synchronize()
        if not steps[M].equals(eager[M]):
            raise SystemExit(f"atlas graph {k}: replayed sweep differs from the eager one")
    torch.cuda.synchronize()
    fin = state[0].cpu().tolist()
    if fin[3] != 0 or fin[0] != fin[1] + fin[2]:
        raise SystemExit(f"atlas KV state {fin}")
    out["replays_checked"] = "every graph: a replay's sweep outputs equal the eager sweep's"
    out["final_kv_state"] = fin
    del steps, heads, segs, w8, w16, graphs
    torch.cuda.empty_cache()
    return out


def kernel_map(twd, ls, M, kernel, bf16_input=True):
    """Kernel family each projection of the set runs at width M, for bf16
    activations (one launch) or int8 ones (the linear of the two-launch
    form); a forced KERNEL_MFMA_TILE runs the staged kernel where K > 3072."""
    out = {}
    for p in ls.projs:
        if kernel == twd.KERNEL_AUTO:
            k = twd.select_kernel(M, p.K, p.N, bf16_input)
        elif kernel == twd.KERNEL_MFMA_TILE and p.K > 3072:
            k = twd.KERNEL_MFMA_STAGED
        else:
            k = kernel
        out[p.name] = twd.KERNEL_NAMES[k]
    return out


def per_projection(twd, torch, ls, M, kernel, reps, target_bytes=640 << 20):
    """Each projection shape on its own, cold: one graph cycles through
    enough distinct weight buffers (random packed bytes; the kernels' timing
    does not depend on the codes) to exceed the 256 MB Infinity Cache.  The
    plain streaming read over the same buffers is timed beside it."""
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    table = {}
    for p in ls.projs:
        nbytes = p.N * p.K // 4
        copies = max(8, -(-target_bytes // nbytes))
        ws = [torch.randint(0, 256, (p.N, p.K // 4), dtype=torch.uint8, device="cuda",
                            generator=gen) for _ in range(copies)]
        x = torch.randn((M, p.K), device="cuda", generator=gen).to(torch.bfloat16)
        y = torch.empty((M, p.N), dtype=torch.float32, device="cuda")
        gam = [1.0] * len(p.segs)

        def lin():
            for w in ws:
                twd.ternary_linear_bf16(w, p.segs, gam, x, y=y, want_acc=False, kernel=kernel)

        def ref():
            for w in ws:
                twd.stream_read(w, nbytes, sink)

        row = {"K": p.K, "N": p.N, "bytes": nbytes}
        for name, fn in (("linear", lin), ("stream_read", ref)):
            g = capture(torch, fn)
            g.replay()
            _, sec = time_replays(torch, g, reps)
            per = sec / (reps * copies)
            row[f"{name}_us"] = round(per * 1e6, 3)
            row[f"{name}_gbs"] = round(nbytes / per / 1e9, 1)
            del g
        table[p.name] = row
        del ws
        torch.cuda.empty_cache()
    return table


def copy_calibration(twd, torch, nbytes=256 << 20, reps=3):
    """Plain copies of known size, for the HBM byte-counter calibration."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    for _ in range(reps):
        twd.stream_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    return nbytes


# The sources the ternary linear kernels are compiled from (the kernels the
# counter record describes); other kernels of the library do not enter.
LINEAR_SOURCES = ("dispatch.hip", "kernel_common.h", "quantize_act.hip", "ternary_narrow.hip",
                  "ternary_rows.hip", "ternary_staged.hip", "ternary_tile.hip")


PROJECTION_SOURCES = ("kernel_common.h", "projection.hip")

SWEEP_SOURCES = ("kernel_common.h", "twd_internal.h", "ternary_sweep.hip", "sweep_plan.cpp")


def sweep_record(workload, M):
    """The sweep's rocprofv3 record (kernel-trace duration, HBM bytes per
    launch) for this workload and width, if it was taken on the current
    sources; else None."""
    path = os.path.join(PROFILES, f"sweep_{workload}_m{M}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(SWEEP_SOURCES):
        return None
    return rec


def sweep_profile(workload, M, nbytes):
    """The committed rocprofv3 figures of the sweep at this workload and
    width (kernel-trace average, the fraction of 8 TB/s it gives, HBM bytes
    per launch, the summary file), or None if none was taken on the current
    sources."""
    rec = sweep_record(workload, M)
    if not rec:
        return None
    return {"avg_us": rec["kernel_trace_avg_us"],
            "frac": round(nbytes / (rec["kernel_trace_avg_us"] * 1e3) / HBM_PEAK_GBS, 4),
            "traffic": rec["hbm_bytes_per_launch"], "summary": rec["summary"]}


def kernel_source_hash(names=LINEAR_SOURCES):
    """Hash of the code (comments and blank space removed) of the given
    kernel sources and of the compile flags: counter records stay valid
    across comment edits and lapse when the code or its build changes."""
    import re
    from ternary_weight_decode_amd import build as twd_build
    h = hashlib.sha256()
    flags = [f for f in twd_build.FLAGS if f != "-I" and not os.path.isabs(f)]
    h.update(" ".join(flags).encode())
    csrc = os.path.join(ROOT, "ternary_weight_decode_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name)) as f:
            code = f.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = " ".join(code.split())
        h.update(name.encode() + code.encode())
    return h.hexdigest()[:16]


def counter_traffic(workload, M, launches_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None.  On the 2B layer
    set the decode (M = 1) and verification (M > 1) workloads launch the same
    kernels over the same weights, so either record serves a width."""
    path = os.path.join(PROFILES, f"ternary_linear_counters_{workload}_m{M}.json")
    if not os.path.exists(path) and workload in ("2b_decode", "2b_verify"):
        other = "2b_verify" if M > 1 else "2b_decode"
        path = os.path.join(PROFILES, f"ternary_linear_counters_{other}_m{M}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def host_cpu():
    """The host CPU model and the logical CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:
        visible = os.cpu_count() or 1
    return f"{model}; {visible} logical CPUs visible to the process"


_NATIVE = None


def oracle_native():
    """Build the oracle for this host (gcc -O3 -march=native, plain loops,
    no fast-math) once per process and use it for the CPU baselines."""
    global _NATIVE
    import oracle
    if _NATIVE is None:
        oracle.select(oracle.build_native())
        _NATIVE = "gcc " + " ".join(oracle.NATIVE_FLAGS) + " -fopenmp -ffp-contract=off"
    return _NATIVE


def cpu_baseline(ls, workload, M, outliers, budget_s, threads=None):
    """The CPU oracle (quantize, int8 x ternary loops, dequant) over the
    layers of the set in order, repeating whole passes until its compute time
    reaches budget_s; timed on the host's cores.  Setup (weight generation and
    the oracle's own ternarization, in a thread pool, all before timing) is
    not timed."""
    import oracle
    native = oracle_native()
    threads = threads or host_threads()

    def prep(key):
        layer, pi = key
        p = ls.projs[pi]
        W = wl.layer_weights(ls, layer, pi)
        t, _, grow = oracle.ternarize_segments(W, p.segs)
        x = wl.layer_activations(workload, p.K, M, layer, pi, outliers=outliers)
        return p, t, grow, x

    keys = [(l, p) for l in range(ls.layers) for p in range(len(ls.projs))]
    done_bytes, spent, passes = 0, 0.0, 0

    def run(item):
        nonlocal done_bytes, spent
        p, t, grow, x = item
        t0 = time.perf_counter()
        q, s = oracle.quantize_act(x)
        acc = oracle.linear(q, t, threads)
        oracle.dequant(acc, s, grow)
        spent += time.perf_counter() - t0
        done_bytes += p.packed_bytes

    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        prepared = list(ex.map(prep, keys))
    while passes == 0 or spent < budget_s:
        for item in prepared:
            run(item)
        passes += 1
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "host": host_cpu(), "build": native,
            "sample": f"{passes} pass(es) over all {ls.layers} layers of the {ls.name.upper()} set "
                      f"at M={M} (4 projections each: quantize + int32 contraction + dequant; "
                      f"{spent:.1f} s of CPU time; throughput in packed-weight bytes/s)"}


# --------------------------------------------------------------------------
# rocprofv3 summaries (no GPU): CSV output of this script under
# `rocprofv3 --kernel-trace --stats -f csv` and two `--pmc` passes
# (FETCH_SIZE, WRITE_SIZE) -> short text summaries plus the counter record
# counter_traffic() reads.

def _csv_rows(d, suffix):
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for path in paths:
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _col(row, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in {list(row)}")


def _short(name):
    return (name.replace("void ", "").replace("twd::(anonymous namespace)::", "")
            .split("(")[0].strip())


def _linear_fused(name):
    """The one-launch (fused quantization) instances of the linear kernels."""
    short = _short(name)
    return (short.startswith(("rows_kernel<", "mfma_kernel<", "tile_kernel<", "staged_kernel<"))
            and short.endswith("true>"))


# The counter calibration copies 256 MiB: 16384 workgroups of 256 threads
# (the benchmark's other copies, e.g. the KV history copy, differ in size).
COPY_GRID_THREADS = (256 << 20) // 16 // 4


def grid(r):
    return int(_col(r, "Grid_Size", "Grid_Size_X", "grid_size"))


def _run_source_hash(path, key="kernel_source_hash"):
    """A kernel-source hash that a bench.py run printed in its JSON line."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("{"):
                return json.loads(line).get(key)
    return None


def summarize_profiles(args):
    trace_dir, fetch_dir, write_dir = args.summarize_profile
    # a counter record is stamped with the sources the profiled run was built
    # from; summarizing a run of other sources would mislabel it
    ran = _run_source_hash(args.profile_run_json)
    if ran is not None and ran != kernel_source_hash():
        raise SystemExit(f"the profiled run used kernel sources {ran}, not the current "
                         f"{kernel_source_hash()}: profile the current sources again")
    cmds = args.profile_commands or ("?", "?", "?")
    ls = wl.LAYER_SETS["4b" if args.workload.startswith("4b") else "2b"]
    M = args.M or wl.workload_widths(args.workload)[0]
    nproj = len(ls.projs)
    out_dir = args.profile_out
    os.makedirs(out_dir, exist_ok=True)
    tag = f"{args.workload}_m{M}"

    # kernel trace: the timed steps are the last steps x launches dispatches
    # of the fused linear kernels (nothing else launches them afterwards)
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    lin = [r for r in trace if _linear_fused(_col(r, "Kernel_Name"))]
    lin.sort(key=lambda r: int(_col(r, "Start_Timestamp")))
    timed = lin[-args.steps * ls.layers * nproj:]
    durs = [int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp")) for r in timed]
    avg_ns = sum(durs) / len(durs)
    span_ns = int(_col(timed[-1], "End_Timestamp")) - int(_col(timed[0], "Start_Timestamp"))
    lines = [f"# ternary linear, {args.workload}, M={M}: rocprofv3 kernel trace", "",
             "Command (from the repository root):", "", "    " + cmds[0], "",
             "## Kernel statistics (rocprofv3 --stats)", "",
             "| kernel | calls | total us | average us | min us | max us |",
             "|---|---|---|---|---|---|"]
    stats.sort(key=lambda r: -float(_col(r, "TotalDurationNs")))
    for r in stats[:12]:
        lines.append(f"| `{_short(_col(r, 'Name'))}` | {_col(r, 'Calls')} | "
                     f"{float(_col(r, 'TotalDurationNs')) / 1e3:.1f} | "
                     f"{float(_col(r, 'AverageNs')) / 1e3:.3f} | {float(_col(r, 'MinNs')) / 1e3:.3f} | "
                     f"{float(_col(r, 'MaxNs')) / 1e3:.3f} |")
    lines += ["", f"## The timed region: the last {len(timed)} fused linear dispatches "
              f"({args.steps} steps x {ls.layers * nproj} launches)", "",
              "| projection | K | N | dispatches | average us | GB/s (K*N/4 bytes) |",
              "|---|---|---|---|---|---|"]
    # within a step the launches go layer by layer, projections in set order
    for pi, p in enumerate(ls.projs):
        ent = durs[pi::nproj]
        a = sum(ent) / len(ent)
        lines.append(f"| {p.name} | {p.K} | {p.N} | {len(ent)} | {a / 1e3:.3f} | "
                     f"{p.packed_bytes / a:.1f} |")
    gaps = [int(_col(b, "Start_Timestamp")) - int(_col(a, "End_Timestamp"))
             for a, b in zip(timed[:-1], timed[1:])]
    gaps.sort()
    lines += ["", f"Average duration over the timed dispatches: **{avg_ns / 1e3:.3f} us** "
              f"(algorithmic bytes per launch {ls.packed_bytes_per_layer / nproj / 1e6:.3f} MB "
              f"-> {ls.packed_bytes_per_layer / nproj / avg_ns:.1f} GB/s); first start to "
              f"last end {span_ns / 1e3:.1f} us; median gap between consecutive dispatches "
              f"{gaps[len(gaps) // 2] / 1e3:.3f} us.", ""]

    def live(path):
        if not path or not os.path.exists(path):
            return None
        with open(path) as f:
            for line in f:
                if line.startswith("{"):
                    return json.loads(line)["roofline"]["avg_launch_us"]
        return None

    prof_live, bench_live = live(args.profile_run_json), live(args.bench_json)
    if prof_live is not None or bench_live is not None:
        lines += ["## Against the live measurement", "",
                  "bench.py times the step with HIP events around back-to-back graph replays, "
                  "so its per-launch figure is elapsed time per launch and includes whatever "
                  "gap separates one kernel from the next.  rocprofv3 reports each kernel "
                  "from its start to its end; under kernel tracing the profiler also spaces "
                  "the dispatches apart.", ""]
        if prof_live is not None:
            lines.append(f"- the profiled run's own live figure: {prof_live:.3f} us per launch "
                         f"(profiler-spaced dispatches)")
        if bench_live is not None:
            gap = bench_live - avg_ns / 1e3
            if gap >= 0:
                lines.append(f"- the unprofiled default run: **{bench_live:.3f} us** per launch; the "
                             f"kernels' own {avg_ns / 1e3:.3f} us plus {gap:.3f} us of inter-kernel "
                             f"gap in back-to-back replay")
            else:
                lines.append(f"- the unprofiled default run: **{bench_live:.3f} us** per launch, "
                             f"{-gap:.3f} us below the kernels' own duration under kernel tracing, "
                             f"so this trace does not back the live per-launch figure: traced "
                             f"dispatches run slower than the same launches back to back (a likely "
                             f"cause, not measured: each back-to-back launch finds the code, "
                             f"kernel arguments and activations the previous ones left in the "
                             f"caches; spacing unprofiled launches apart with idle kernels costs "
                             f"only about 0.1 us per launch). The live figure is backed instead by "
                             f"the HBM counters (traffic per launch, in the counter summary) and "
                             f"by the one-launch sweep, whose trace agrees with its live figure")
        lines.append("")
    trace_path = os.path.join(out_dir, f"ternary_linear_{tag}_kernel_trace.md")
    with open(trace_path, "w") as f:
        f.write("\n".join(lines))

    # counters: KiB per dispatch, scaled by the copy kernel's reading
    def per_kernel(d, counter):
        rows = [r for r in _csv_rows(d, "counter_collection.csv")
                if _col(r, "Counter_Name") == counter]
        agg = {}
        for r in rows:
            name = _col(r, "Kernel_Name")
            g = int(_col(r, "Grid_Size", "Grid_Size_X", "grid_size"))
            agg.setdefault((name, g), []).append(float(_col(r, "Counter_Value")))
        return agg

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = 256 << 20

    def copy_factor(agg):
        vals = [v for (n, g), vs in agg.items()
                if "stream_copy_kernel" in n and g == COPY_GRID_THREADS for v in vs]
        return copy_bytes / (sum(vals) / len(vals) * 1024.0), sum(vals) / len(vals)

    f_fetch, copy_fetch_kib = copy_factor(fetch)
    f_write, copy_write_kib = copy_factor(write)

    def lin_mean(agg):
        vals = [v for (n, _), vs in agg.items() if _linear_fused(n) for v in vs]
        return sum(vals) / len(vals), len(vals)

    lf, nf = lin_mean(fetch)
    lw, nw = lin_mean(write)
    hbm = lf * 1024 * f_fetch + lw * 1024 * f_write
    alg = ls.packed_bytes_per_layer / nproj
    lines = [f"# ternary linear, {args.workload}, M={M}: HBM bytes from rocprofv3 counters", "",
             "Commands (from the repository root), one counter per run:", "",
             "    " + cmds[1], "", "    " + cmds[2], "",
             f"Calibration: the plain copy kernel (`stream_copy_kernel`) moves {copy_bytes} bytes "
             f"each way per dispatch; FETCH_SIZE reads {copy_fetch_kib:.1f} KiB -> factor "
             f"{f_fetch:.4f}; WRITE_SIZE reads {copy_write_kib:.1f} KiB -> factor {f_write:.4f}.", "",
             "| kernel | grid WGs | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) |",
             "|---|---|---|---|---|---|"]
    for (n, g), vs in sorted(fetch.items(), key=lambda kv: _short(kv[0][0])):
        wv = write.get((n, g), [0.0])
        fm, wm = sum(vs) / len(vs), sum(wv) / len(wv)
        lines.append(f"| `{_short(n)}` | {g // 256} | {len(vs)} | {fm:.1f} | {wm:.1f} | "
                     f"{fm * 1024 * f_fetch + wm * 1024 * f_write:,.0f} |")
    lines += ["", f"Fused linear, mean over {nf} dispatches: FETCH {lf:.1f} KiB, WRITE {lw:.1f} KiB "
              f"-> **{hbm:,.0f} HBM bytes per launch** against {alg:,.0f} algorithmic "
              f"(packed weights) = {hbm / alg:.3f}x.", ""]
    cnt_path = os.path.join(out_dir, f"ternary_linear_{tag}_hbm_counters.md")
    with open(cnt_path, "w") as f:
        f.write("\n".join(lines))
    rec = {"source_hash": kernel_source_hash(), "workload": args.workload, "M": M,
           "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": round(alg),
           "fetch_factor": round(f_fetch, 5), "write_factor": round(f_write, 5),
           "summary": os.path.basename(cnt_path)}
    with open(os.path.join(out_dir, f"ternary_linear_counters_{tag}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(trace_path)
    print(cnt_path)


def _sweep_kernel(name):
    return _short(name).startswith("sweep_kernel<")


def summarize_sweep(args):
    """Kernel trace and HBM counters of the headline sweep from three
    rocprofv3 runs of this script with --headline-only (kernel trace + stats;
    FETCH_SIZE; WRITE_SIZE, the counter runs with --copy-calibration) ->
    profiles/sweep_<workload>_m<M>_{kernel_trace,hbm_counters}.md and the
    record sweep_record() reads."""
    trace_dir, fetch_dir, write_dir = args.summarize_sweep
    ran = _run_source_hash(args.profile_run_json, "sweep_source_hash")
    if ran is not None and ran != kernel_source_hash(SWEEP_SOURCES):
        raise SystemExit(f"the profiled run used sweep sources {ran}, not the current "
                         f"{kernel_source_hash(SWEEP_SOURCES)}: profile them again")
    cmds = args.profile_commands or ("?", "?", "?")
    ls = wl.LAYER_SETS["4b" if args.workload.startswith("4b") else "2b"]
    M = args.M or wl.workload_widths(args.workload)[0]
    alg = ls.packed_bytes
    tag = f"{args.workload}_m{M}"
    out_dir = args.profile_out
    os.makedirs(out_dir, exist_ok=True)

    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    sw = [r for r in trace if _sweep_kernel(_col(r, "Kernel_Name"))]
    sw.sort(key=lambda r: int(_col(r, "Start_Timestamp")))
    timed = sw[-args.steps:]
    durs = [int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp")) for r in timed]
    avg_ns = sum(durs) / len(durs)
    kname = _short(_col(timed[0], "Kernel_Name"))
    lines = [f"# multi-projection sweep, {args.workload}, M={M}: rocprofv3 kernel trace", "",
             "Command (from the repository root):", "", "    " + cmds[0], "",
             "## Kernel statistics (rocprofv3 --stats)", "",
             "| kernel | calls | total us | average us | min us | max us |",
             "|---|---|---|---|---|---|"]
    stats.sort(key=lambda r: -float(_col(r, "TotalDurationNs")))
    for r in stats[:10]:
        lines.append(f"| `{_short(_col(r, 'Name'))}` | {_col(r, 'Calls')} | "
                     f"{float(_col(r, 'TotalDurationNs')) / 1e3:.1f} | "
                     f"{float(_col(r, 'AverageNs')) / 1e3:.3f} | {float(_col(r, 'MinNs')) / 1e3:.3f} | "
                     f"{float(_col(r, 'MaxNs')) / 1e3:.3f} |")
    lines += ["", f"## The timed region: the last {len(timed)} dispatches of `{kname}`", "",
              f"Each dispatch runs all {ls.layers * len(ls.projs)} projections of the "
              f"{ls.name.upper()} set: {alg:,} packed-weight bytes.", "",
              f"- average duration **{avg_ns / 1e3:.2f} us** (min {min(durs) / 1e3:.2f}, "
              f"max {max(durs) / 1e3:.2f}) -> {alg / avg_ns:.1f} GB/s, "
              f"{100 * alg / avg_ns / HBM_PEAK_GBS:.1f}% of 8 TB/s", ""]

    def live(path):
        if not path or not os.path.exists(path):
            return None
        with open(path) as f:
            for line in f:
                if line.startswith("{"):
                    return json.loads(line)["roofline"]["avg_launch_us"]
        return None

    prof_live, bench_live = live(args.profile_run_json), live(args.bench_json)
    if prof_live is not None:
        lines.append(f"- the profiled run's own live figure (HIP events around the timed "
                     f"launches): {prof_live:.2f} us per launch")
    if bench_live is not None:
        lines.append(f"- the unprofiled default run: **{bench_live:.2f} us** per launch "
                     f"({100 * (avg_ns / 1e3 - bench_live) / bench_live:+.1f}% for the traced "
                     f"kernel)")
    lines.append("")
    trace_path = os.path.join(out_dir, f"sweep_{tag}_kernel_trace.md")
    with open(trace_path, "w") as f:
        f.write("\n".join(lines))

    def per_kernel(d, counter):
        agg = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if _col(r, "Counter_Name") != counter:
                continue
            name = _col(r, "Kernel_Name")
            if _sweep_kernel(name):
                agg.setdefault("sweep", []).append(float(_col(r, "Counter_Value")))
            elif "stream_copy_kernel" in name and grid(r) == COPY_GRID_THREADS:
                agg.setdefault("copy", []).append(float(_col(r, "Counter_Value")))
        return {k: sum(v) / len(v) for k, v in agg.items()}, len(agg.get("sweep", []))

    fetch, nf = per_kernel(fetch_dir, "FETCH_SIZE")
    write, _ = per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = 256 << 20
    ff = copy_bytes / (fetch["copy"] * 1024.0)
    fw = copy_bytes / (write["copy"] * 1024.0)
    rd = fetch["sweep"] * 1024 * ff
    wr = write["sweep"] * 1024 * fw
    lines = [f"# multi-projection sweep, {args.workload}, M={M}: HBM bytes from rocprofv3 "
             "counters", "", "Commands (from the repository root), one counter per run:", "",
             "    " + cmds[1], "", "    " + cmds[2], "",
             f"Calibration: the plain copy kernel (`stream_copy_kernel`) moves {copy_bytes} bytes "
             f"each way per dispatch; FETCH_SIZE reads {fetch['copy']:.1f} KiB -> factor "
             f"{ff:.4f}; WRITE_SIZE reads {write['copy']:.1f} KiB -> factor {fw:.4f}.", "",
             f"`{kname}`, mean over {nf} dispatches: FETCH_SIZE {fetch['sweep']:.1f} KiB, "
             f"WRITE_SIZE {write['sweep']:.1f} KiB.", "",
             "| | bytes per launch | over the packed weights |", "|---|---|---|",
             f"| read (calibrated FETCH_SIZE) | {rd:,.0f} | {rd / alg:.4f}x |",
             f"| written (calibrated WRITE_SIZE) | {wr:,.0f} | {wr / alg:.4f}x |",
             f"| **HBM traffic** | **{rd + wr:,.0f}** | **{(rd + wr) / alg:.4f}x** |",
             f"| algorithmic (packed weights, K N / 4 summed) | {alg:,} | 1x |", "",
             "Beyond the weights: each workgroup's read of the bf16 activations of the "
             "projections it stages (L2 misses, so also what the Infinity Cache serves), "
             "the fp32 outputs, and the plan table.", ""]
    cnt_path = os.path.join(out_dir, f"sweep_{tag}_hbm_counters.md")
    with open(cnt_path, "w") as f:
        f.write("\n".join(lines))
    rec = {"source_hash": kernel_source_hash(SWEEP_SOURCES), "workload": args.workload, "M": M,
           "kernel": kname, "kernel_trace_avg_us": round(avg_ns / 1e3, 3),
           "hbm_bytes_per_launch": round(rd + wr), "hbm_read_bytes_per_launch": round(rd),
           "algorithmic_bytes_per_launch": alg, "fetch_factor": round(ff, 5),
           "write_factor": round(fw, 5), "summary": os.path.basename(trace_path)}
    with open(os.path.join(out_dir, f"sweep_{tag}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(trace_path)
    print(cnt_path)


def summarize_projection(args):
    """Kernel trace and HBM counters of the output projection (both roles)
    from three rocprofv3 runs of this script with --projection-widths 1
    (trace, FETCH_SIZE, WRITE_SIZE; the counter runs add --copy-calibration)."""
    trace_dir, fetch_dir, write_dir = args.summarize_projection
    ran = _run_source_hash(args.profile_run_json, "projection_source_hash")
    if ran is not None and ran != kernel_source_hash(PROJECTION_SOURCES):
        raise SystemExit(f"the profiled run used projection sources {ran}, not the current "
                         f"{kernel_source_hash(PROJECTION_SOURCES)}: profile them again")
    cmds = args.profile_commands or ("?", "?", "?")
    K, N = wl.HEAD_K, wl.HEAD_N
    roles = (("projection_kernel<true", "fast (E4M3 weights)", N * K),
             ("projection_kernel<false", "critical (bf16 weights)", 2 * N * K))
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    lines = ["# output projection 2560 -> 128256, M=1: rocprofv3 kernel trace and HBM counters",
             "", "Commands (from the repository root):", "", "    " + cmds[0], "",
             "    " + cmds[1], "", "    " + cmds[2], "",
             "bench.py times each role with direct launches alternating two distinct "
             "weight copies (every launch reads cold weights), and the same launches "
             "replayed from a graph beside them; the trace covers all of that run's "
             "dispatches of the kernel, warm-up included.", "",
             "| role | kernel | dispatches | average us | min us | algorithmic bytes | GB/s (avg) |"
             " % of 8 TB/s |", "|---|---|---|---|---|---|---|---|"]
    avg = {}
    for kname, role, nbytes in roles:
        names = {_short(_col(r, "Kernel_Name")) for r in trace
                 if _short(_col(r, "Kernel_Name")).startswith(kname)}
        d = [int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))
             for r in trace if _short(_col(r, "Kernel_Name")).startswith(kname)]
        a = sum(d) / len(d)
        avg[kname] = a
        shown = ", ".join(f"`{n}`" for n in sorted(names))
        lines.append(f"| {role} | {shown} | {len(d)} | {a / 1e3:.2f} | {min(d) / 1e3:.2f} | "
                     f"{nbytes:,} | {nbytes / a:.1f} | {100 * nbytes / a / HBM_PEAK_GBS:.1f} |")

    def per_kernel(d, counter):
        agg = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if _col(r, "Counter_Name") == counter:
                name = _short(_col(r, "Kernel_Name"))
                for kname, _, _ in roles:
                    if name.startswith(kname):
                        name = kname
                if name == "stream_copy_kernel" and grid(r) != COPY_GRID_THREADS:
                    continue  # only the calibration copy of known size
                agg.setdefault(name, []).append(float(_col(r, "Counter_Value")))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = 256 << 20
    ff = copy_bytes / (fetch["stream_copy_kernel"] * 1024.0)
    fw = copy_bytes / (write["stream_copy_kernel"] * 1024.0)
    lines += ["", f"Counter calibration: the plain copy of {copy_bytes} bytes reads "
              f"FETCH_SIZE {fetch['stream_copy_kernel']:.1f} KiB (factor {ff:.4f}) and "
              f"WRITE_SIZE {write['stream_copy_kernel']:.1f} KiB (factor {fw:.4f}).", "",
              "| role | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes read (calibrated) | "
              "over algorithmic | HBM bytes written |", "|---|---|---|---|---|---|"]
    rec = {"source_hash": kernel_source_hash(PROJECTION_SOURCES), "M": 1,
           "fetch_factor": round(ff, 5), "write_factor": round(fw, 5)}
    for kname, role, nbytes in roles:
        rd = fetch[kname] * 1024 * ff
        wr = write[kname] * 1024 * fw
        lines.append(f"| {role} | {fetch[kname]:.1f} | {write[kname]:.1f} | {rd:,.0f} | "
                     f"{rd / nbytes:.3f}x | {wr:,.0f} |")
        rec["fast_fp8" if "true" in kname else "critical_bf16"] = {
            "hbm_bytes_per_launch": round(rd + wr), "algorithmic_bytes_per_launch": nbytes,
            "kernel_trace_avg_us": round(avg[kname] / 1e3, 3)}
    os.makedirs(args.profile_out, exist_ok=True)
    with open(os.path.join(args.profile_out, "output_projection_counters_2b_m1.json"), "w") as f:
        json.dump(rec, f, indent=1)
    # the streaming read of the same bytes, as the profiled run timed it
    # (large reads stride over one workgroup per compute unit, so the trace's
    # grid sizes no longer tell the buffers apart)
    run = None
    if args.profile_run_json and os.path.exists(args.profile_run_json):
        with open(args.profile_run_json) as f:
            for line in f:
                if line.startswith("{"):
                    run = json.loads(line).get("output_projection")
    if run:
        f8, b16 = run["stream_read_fp8_bytes"], run["stream_read_bf16_bytes"]
        lines += ["", "Streaming read of the same bytes in the profiled run (HIP events, direct "
                  f"launches): {f8['us']:.2f} us over the E4M3 weights ({f8['gbs']:.0f} GB/s), "
                  f"{b16['us']:.2f} us over the bf16 weights ({b16['gbs']:.0f} GB/s)."]
    lines.append("")
    path = os.path.join(args.profile_out, "output_projection_2b_m1_trace_and_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(path)


SIMDS = 1024  # MI355X: 256 compute units x 4 SIMDs


def summarize_util(args):
    """Per-kernel means of the utilization counters (one --pmc run).  The
    instruction counts per wave are exact; the MFMA busy share divides
    SQ_VALU_MFMA_BUSY_CYCLES (16 per v_mfma_i32_16x16x64_i8) by the SIMD
    cycles of the dispatch's own duration (2.4 GHz x 1024 SIMDs)."""
    pmc_dir, command = args.summarize_util
    M = args.M or wl.workload_widths(args.workload)[0]
    sweep = args.util_kernels == "sweep"
    agg = {}
    for r in _csv_rows(pmc_dir, "counter_collection.csv"):
        name = _col(r, "Kernel_Name")
        if not (_short(name).startswith("sweep_kernel<") if sweep else _linear_fused(name)):
            continue
        key = (_short(name), int(_col(r, "Grid_Size", "Grid_Size_X", "grid_size")) // 64)
        d = agg.setdefault(key, {})
        d.setdefault(_col(r, "Counter_Name"), []).append(float(_col(r, "Counter_Value")))
        d.setdefault("_dur", {})[_col(r, "Correlation_Id", "Dispatch_Id")] = (
            int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp")))
    what = "multi-projection sweep" if sweep else "ternary linear"
    lines = [f"# {what}, {args.workload}, M={M}: utilization counters", "",
             "Command (from the repository root):", "", "    " + command, "",
             f"Means per dispatch of the {'sweep kernel' if sweep else 'fused linear kernels'} "
             "(one rocprofv3 --pmc run; "
             "dispatches run slower under counter collection than unprofiled).  MFMA busy "
             "share = SQ_VALU_MFMA_BUSY_CYCLES / (dispatch duration x 2.4 GHz x 1024 "
             "SIMDs).", "",
             "| kernel | waves | dispatches | duration us | MFMA i8 instrs | MFMA busy cycles | "
             "MFMA busy % | VALU instrs / wave | LDS instrs / wave | LDS bank-conflict cycles |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for (name, waves_grid), d in sorted(agg.items()):
        durs = list(d.pop("_dur").values())
        dur_ns = sum(durs) / len(durs)
        mean = {k: sum(v) / len(v) for k, v in d.items()}
        waves = mean.get("SQ_WAVES", 0.0) or 1.0
        busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        lines.append(
            f"| `{name}` | {waves_grid} | {len(durs)} | {dur_ns / 1e3:.2f} | "
            f"{mean.get('SQ_INSTS_VALU_MFMA_I8', 0):,.0f} | {busy:,.0f} | "
            f"{100 * busy / (dur_ns * 2.4 * SIMDS):.2f} | "
            f"{mean.get('SQ_INSTS_VALU', 0) / waves:.0f} | "
            f"{mean.get('SQ_INSTS_LDS', 0) / waves:.1f} | "
            f"{mean.get('SQ_LDS_BANK_CONFLICT', 0):,.0f} |")
    lines.append("")
    out = os.path.join(args.profile_out, f"{'sweep' if sweep else 'ternary_linear'}_"
                       f"{args.workload}_m{M}_util.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(out)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="2b_decode",
                    choices=["2b_decode", "2b_verify", "2b_sweep_outlier", "4b_stack"])
    ap.add_argument("--M", type=int, default=None, help="width (default: the workload's first)")
    ap.add_argument("--kernel", default="auto",
                    choices=["auto", "dot", "mfma", "mfma_staged", "mfma_tile"],
                    help="kernel family of the per-projection launches")
    ap.add_argument("--widths", default="1,2,4,8,16",
                    help="widths of the headline set's per-width table ('' to skip)")
    ap.add_argument("--outlier-widths", default=",".join(str(m) for m in range(1, 17)),
                    help="widths of the 2B outlier workload curve ('' to skip)")
    ap.add_argument("--set4b-widths", default="1,4,16",
                    help="widths of the 4B-class stack ('' to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU oracle budget (0 skips the CPU baseline)")
    ap.add_argument("--per-proj", type=int, default=1,
                    help="1: time each projection shape on its own, cold (default)")
    ap.add_argument("--projection-widths", default="1,4,8,16",
                    help="widths of the fast / critical output-projection table ('' skips it)")
    ap.add_argument("--atlas", type=int, default=1,
                    help="time the per-(role, width) iteration graphs (1) or not (0)")
    ap.add_argument("--kv-commit", type=int, default=1,
                    help="time the accepted-prefix KV commit (1) or not (0)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline step only (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with plain copies of 256 MiB (byte-counter calibration)")
    ap.add_argument("--summarize-sweep", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: summarize rocprofv3 runs of the headline sweep into profiles/")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: summarize rocprofv3 CSV output of the per-projection launches")
    ap.add_argument("--profile-commands", nargs=3, metavar=("TRACE_CMD", "FETCH_CMD", "WRITE_CMD"),
                    help="the commands that produced the summarized inputs")
    ap.add_argument("--summarize-projection", nargs=3,
                    metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="summarize rocprofv3 runs of the output-projection table")
    ap.add_argument("--summarize-util", nargs=2, metavar=("PMC_DIR", "COMMAND"),
                    help="no GPU: summarize a rocprofv3 --pmc run of the utilization counters")
    ap.add_argument("--util-kernels", default="linear", choices=["linear", "sweep"],
                    help="with --summarize-util: the fused linear kernels or the sweep")
    ap.add_argument("--profile-out", default=PROFILES)
    ap.add_argument("--profile-run-json", default=None,
                    help="stdout of the profiled kernel-trace run (its own live timing)")
    ap.add_argument("--bench-json", default=None,
                    help="stdout of an unprofiled run of the default command")
    args = ap.parse_args()

    if args.summarize_sweep:
        summarize_sweep(args)
        return
    if args.summarize_profile:
        summarize_profiles(args)
        return
    if args.summarize_util:
        summarize_util(args)
        return
    if args.summarize_projection:
        summarize_projection(args)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the "
              "ternary linear is measured on a single MI355X; the multi-GPU sharding is a "
              "design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import ternary_weight_decode_amd as twd
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kernel = {"auto": twd.KERNEL_AUTO, "dot": twd.KERNEL_DOT, "mfma": twd.KERNEL_MFMA,
              "mfma_staged": twd.KERNEL_MFMA_STAGED, "mfma_tile": twd.KERNEL_MFMA_TILE}[args.kernel]
    set_name = "4b" if args.workload.startswith("4b") else "2b"
    ls = wl.LAYER_SETS[set_name]
    M = args.M or wl.workload_widths(args.workload)[0]
    outliers = args.workload == "2b_sweep_outlier"
    widths_of = lambda v: [int(w) for w in v.split(",") if w]  # noqa: E731

    t_setup = time.perf_counter()
    dev_set = LayerSetOnDevice(twd, torch, ls, ls.layers)
    bytes_step = dev_set.bytes_per_sweep
    log(f"weights ready: {bytes_step / 1e6:.1f} MB packed in "
        f"{time.perf_counter() - t_setup:.1f} s")

    # the headline step: one sweep launch.  Its outputs must equal the
    # per-projection launches' bit for bit, and every graph replay the eager
    # launch's.
    step = Step(twd, torch, dev_set, args.workload, M, kernel, outliers)
    step.fused()
    torch.cuda.synchronize()
    ref = step.snapshot()
    step.clear()
    step.sweep()
    torch.cuda.synchronize()
    if not step.equals(ref):
        raise SystemExit("the sweep differs from the per-projection launches")
    g_sweep = capture(torch, step.sweep)
    for _ in range(2):
        step.clear()
        g_sweep.replay()
        torch.cuda.synchronize()
        if not step.equals(ref):
            raise SystemExit("a graph replay of the sweep differs from the eager launch")
    log(f"headline: sweep of {len(step.keys())} projections, M={M}, "
        f"{step.plan.nwg} workgroups, checked against the per-projection launches")

    # The step is a single launch, so it is timed as launched directly on the
    # stream: back to back, each launch starts as the last one ends.  (A
    # one-kernel graph adds a fixed cost per replay; it is timed beside.)
    reps = max(10, args.steps // 2)
    g_sec = None
    for _ in range(3):  # settle the clocks: about 1.5 s of replays, untimed
        g_sweep.replay()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + 1.5
    while time.perf_counter() < t_end:
        for _ in range(200):
            g_sweep.replay()
        torch.cuda.synchronize()
    _, g_sec = time_replays(torch, g_sweep, reps)
    g_sec /= reps
    for _ in range(args.warmup):
        step.sweep()
    wall, ev_sec = time_launches(torch, step.sweep, args.steps)
    value = bytes_step * args.steps / wall / 1e9
    launch_s = ev_sec / args.steps
    achieved = bytes_step / launch_s / 1e9
    rec = sweep_record(args.workload, M)
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": rec["hbm_bytes_per_launch"] if rec else None,
        "kernel": f"sweep_kernel (M={M}; one launch per step over the {len(step.keys())} "
                  f"projections)",
        "algorithmic_bytes_per_launch": bytes_step,
        "avg_launch_us": round(launch_s * 1e6, 2), "launches_timed": args.steps,
    }
    if rec:
        roofline["trace"] = {"avg_us": rec["kernel_trace_avg_us"],
                             "frac": round(bytes_step / (rec["kernel_trace_avg_us"] * 1e3)
                                           / HBM_PEAK_GBS, 4),
                             "summary": rec["summary"]}
    log(f"headline: {value:.1f} GB/s ({launch_s * 1e6:.1f} us per launch)")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,0.02) weights, absmean-ternarized; N(0,1) bf16 "
                "activations)",
        "config": {
            "workload": args.workload,
            "layer_set": f"{ls.name.upper()}-class, hidden {ls.hidden}, {ls.layers} layers",
            "M": M,
            "packed_weight_bytes_per_step": bytes_step,
            "form": "one multi-projection sweep launch per step (twd_ternary_sweep over the "
                    f"{len(step.keys())} independent projections), tiled weights",
            "launches_per_step": 1,
            "hip_graph": False,
            "sweep_workgroups": step.plan.nwg,
            "sweep_lds_bytes": step.plan.lds_bytes,
        },
        "roofline": roofline,
        "graph_step": {"us": round(g_sec * 1e6, 2),
                       "gbs": round(bytes_step / g_sec / 1e9, 1),
                       "note": "the same step captured into a HIP graph and replayed back to "
                               "back (the timed steps above are direct launches)"},
        "kernel_source_hash": kernel_source_hash(),
        "sweep_source_hash": kernel_source_hash(SWEEP_SOURCES),
        "projection_source_hash": kernel_source_hash(PROJECTION_SOURCES),
    }
    del g_sweep

    if not args.headline_only:
        # the same step as one launch per projection (a decode chain's form)
        pl = width_entry(twd, torch, dev_set, args.workload, M, kernel, reps, outliers,
                         forms=("fused", "two_launch"))
        one, per = stream_read_reference(twd, torch, dev_set, reps)
        pl["per_launch"]["traffic"] = counter_traffic(args.workload, M, bytes_step / len(step.keys()))
        out["per_launch_step"] = {**pl["per_launch"], "two_launch_gbs": pl["two_launch"]["gbs"],
                                  "note": "one launch per projection, 120 per step, graph-replayed"}
        out["stream_read_ref"] = {
            "one_launch": one, "per_projection_launches": per,
            "sweep_over_one_launch": round(achieved / one["gbs"], 4),
            "per_launch_over_per_projection_launches": round(
                pl["per_launch"]["gbs"] / per["gbs"], 4)}
        widths = {}
        for Mw in widths_of(args.widths):
            log(f"width {Mw}")
            widths[str(Mw)] = width_entry(twd, torch, dev_set, args.workload if Mw == 1
                                          else ("2b_verify" if set_name == "2b" else args.workload),
                                          Mw, kernel, reps, outliers)
        out["widths"] = widths
        if set_name == "2b" and args.outlier_widths:
            curve = {}
            for Mw in widths_of(args.outlier_widths):
                log(f"outlier workload, width {Mw}")
                e = width_entry(twd, torch, dev_set, "2b_sweep_outlier", Mw, kernel,
                                max(10, reps // 2), True, forms=("sweep", "fused"), graphs=False)
                curve[str(Mw)] = {"sweep_gbs": e["sweep"]["gbs"], "sweep_frac": e["sweep"]["frac"],
                                  "per_launch_gbs": e["per_launch"]["gbs"]}
            out["outlier_sweep_2b"] = {
                "workload": "2b_sweep_outlier: the 2B set, 1% of channels x20, every width",
                "widths": curve}
        if args.per_proj:
            out["per_projection_cold"] = per_projection(twd, torch, ls, M, kernel, reps)
        if args.kv_commit:
            out["kv_commit"] = kv_commit_bench(twd, torch, ls, reps)
        if args.atlas and set_name == "2b":
            log("graph atlas")
            out["graph_atlas"] = atlas_bench(twd, torch, dev_set, max(5, reps // 4))
        if args.projection_widths:
            out["output_projection"] = output_projection_bench(
                twd, torch, widths_of(args.projection_widths), reps)
        del step
        if set_name == "2b" and args.set4b_widths:
            log("4B-class stack")
            del dev_set
            torch.cuda.empty_cache()
            ds4 = LayerSetOnDevice(twd, torch, wl.SET_4B, wl.SET_4B.layers)
            tab = {}
            for Mw in widths_of(args.set4b_widths):
                e = width_entry(twd, torch, ds4, "4b_stack", Mw, kernel, reps,
                                forms=("sweep", "fused"), graphs=False)
                tab[str(Mw)] = {"sweep_gbs": e["sweep"]["gbs"], "sweep_frac": e["sweep"]["frac"],
                                "sweep_us": e["sweep"]["us"],
                                "per_launch_gbs": e["per_launch"]["gbs"],
                                "per_launch_kernels": e["per_launch"]["kernels"]}
                if "trace" in e["sweep"]:
                    tab[str(Mw)]["sweep_trace"] = e["sweep"]["trace"]
            out["set_4b"] = {"layer_set": "4B-class, hidden 3072, 36 layers",
                             "packed_weight_bytes_per_step": ds4.bytes_per_sweep,
                             "widths": tab}
            del ds4
            torch.cuda.empty_cache()
        if args.cpu_seconds > 0:
            if "output_projection" in out:
                out["output_projection"]["cpu_baseline"] = cpu_projection_baseline(
                    args.cpu_seconds / 5)
            if "kv_commit" in out:
                out["kv_commit"]["cpu_baseline"] = cpu_kv_baseline(args.cpu_seconds / 10)
            out["cpu_baseline"] = cpu_baseline(ls, args.workload, M, outliers, args.cpu_seconds)
            out["cpu_single_thread"] = cpu_baseline(ls, args.workload, M, outliers,
                                                    args.cpu_seconds / 3, threads=1)
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(twd, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
