"""GPU parity of the accepted-prefix KV commit through the C ABI against the
CPU oracle (oracle/kv_commit.py): state words and every segment byte
bit-exact after each commit of seeded sequences (verification, confidence-
only and autoregressive steps, segment boundaries crossed), error paths
(broken identity, bad counts, capacity, a sticky error) write nothing, and a
captured graph of commits replays like the eager calls."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oracle import kv_commit as okv
    import ternary_weight_decode_amd as twd
    return torch, twd, okv


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


class Dev:
    """Device segments, ping-pong state words and count slots."""

    def __init__(self, torch, twd, c0, nseg, layers, row, state=(1, 0, 1, 0), slots=64):
        self.torch, self.twd = torch, twd
        self.c0, self.nseg, self.layers, self.row = c0, nseg, layers, row
        self.segs = [torch.zeros(layers * 2 * cap * row * 2, dtype=torch.uint8, device="cuda")
                     for cap in twd.kv_segment_positions(c0, nseg)]
        self.state = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
        self.state[0] = torch.tensor(state, dtype=torch.int32)
        self.cur = 0
        self.nm = torch.zeros(slots, dtype=torch.int32, device="cuda")
        self.nn = torch.zeros(slots, dtype=torch.int32, device="cuda")

    def commit(self, block_dev, W, slot):
        self.twd.kv_commit(self.segs, self.c0, self.layers, self.row * 2, block_dev, W,
                           self.nm[slot:slot + 1], self.nn[slot:slot + 1],
                           self.state[self.cur], self.state[1 - self.cur])
        self.cur = 1 - self.cur

    def check(self, store):
        got = self.state[self.cur].cpu().numpy().tolist()
        assert got == store.state, (got, store.state)
        for s, (d, o) in enumerate(zip(self.segs, store.segs)):
            np.testing.assert_array_equal(d.cpu().numpy().view(np.uint16).reshape(o.shape), o,
                                          err_msg=f"segment {s}")


def draw(rng, store, W):
    P, L, S, _ = store.state
    mode = int(rng.integers(0, 3))
    if mode == 0 and S <= W:
        a = int(rng.integers(0, W - S + 1))
        return S + a, a + 1
    if mode == 1:
        return 0, int(rng.integers(1, 3))
    return min(1, S, W), 1


@pytest.mark.parametrize("c0,nseg,layers,row", [(8, 6, 30, 640), (2, 4, 3, 8), (1, 8, 1, 8)])
def test_kv_commit_sequences(env, c0, nseg, layers, row):
    torch, twd, okv = env
    log(f"kv commit sequence c0={c0} nseg={nseg} layers={layers} row={row}")
    rng = np.random.default_rng([31, c0, nseg])
    store = okv.KVStore(c0, nseg, layers, row)
    dev = Dev(torch, twd, c0, nseg, layers, row)
    for it in range(60):
        W = int(rng.integers(1, 18))
        n_mat, n_new = draw(rng, store, W)
        if store.state[1] + n_mat > store.capacity:
            break
        block = rng.integers(0, 65536, (layers, 2, W, row)).astype(np.uint16)
        dev.nm[it], dev.nn[it] = n_mat, n_new
        bd = torch.from_numpy(block.view(np.uint8).reshape(-1)).cuda()
        dev.commit(bd, W, it)
        store.commit(block, n_mat, n_new)
        torch.cuda.synchronize()
        got = dev.state[dev.cur].cpu().numpy().tolist()
        assert got == store.state, (it, got, store.state)
    dev.check(store)
    log(f"  reached L={store.state[1]} of capacity {store.capacity}")
    assert store.state[1] > c0  # crossed at least one segment boundary


def test_kv_commit_errors_write_nothing(env):
    torch, twd, okv = env
    c0, nseg, layers, row = 2, 3, 2, 8
    rng = np.random.default_rng(5)
    cases = [((5, 2, 2, 0), 4, 1, 1, okv.ERR_IDENTITY),
             ((1, -2, 3, 0), 4, 1, 1, okv.ERR_IDENTITY),   # negative length
             ((3, 1, 2, 0), 2, 1, 2 ** 31 - 2, okv.ERR_COUNTS),
             ((3, 1, 2, 0), 2, 3, 1, okv.ERR_COUNTS),      # n_mat > W
             ((3, 1, 2, 0), 4, 4, 1, okv.ERR_COUNTS),      # L + n_mat > P + n_new
             ((3, 1, 2, 0), 2, 1, -1, okv.ERR_COUNTS),
             ((14, 13, 1, 0), 2, 2, 1, okv.ERR_CAPACITY),
             ((3, 1, 2, 2), 2, 1, 1, 2)]                   # an error already set
    for state, W, n_mat, n_new, code in cases:
        store = okv.KVStore(c0, nseg, layers, row, state=state)
        dev = Dev(torch, twd, c0, nseg, layers, row, state=state)
        block = rng.integers(1, 65536, (layers, 2, W, row)).astype(np.uint16)
        dev.nm[0], dev.nn[0] = n_mat, n_new
        dev.commit(torch.from_numpy(block.view(np.uint8).reshape(-1)).cuda(), W, 0)
        store.commit(block, n_mat, n_new)
        torch.cuda.synchronize()
        assert store.state[3] == code
        dev.check(store)
        assert not any(s.any().item() for s in dev.segs)


def test_kv_commit_graph_replays(env):
    """A captured sequence of commits (state words alternating, counts read
    from device slots) replays three times, with eager work between the
    replays, and matches the oracle after each."""
    torch, twd, okv = env
    c0, nseg, layers, row, steps = 4, 7, 4, 64, 8
    rng = np.random.default_rng(77)
    store = okv.KVStore(c0, nseg, layers, row)
    dev = Dev(torch, twd, c0, nseg, layers, row)
    W = 9
    blocks = [rng.integers(0, 65536, (layers, 2, W, row)).astype(np.uint16) for _ in range(steps)]
    bdev = [torch.from_numpy(b.view(np.uint8).reshape(-1)).cuda() for b in blocks]
    # counts valid from any state with S = 1 (verification with a accepted)
    accepted = [int(a) for a in rng.integers(0, W, steps)]
    for i, a in enumerate(accepted):
        dev.nm[i], dev.nn[i] = 1 + a, a + 1
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                dev.commit(bdev[i], W, i)
    assert dev.cur == 0  # an even number of commits ends on the first state word
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for i, a in enumerate(accepted):
            store.commit(blocks[i], 1 + a, a + 1)
        dev.check(store)
        _ = (dev.state.sum() + 1).item()  # eager work between replays
    log(f"  after 3 replays: state {store.state}")
