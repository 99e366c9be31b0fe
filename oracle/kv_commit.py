"""CPU oracle of the accepted-prefix KV commit -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may use it; it shares nothing with the HIP library.

What it follows (page "BitMTP: When Multi-Token Prediction Meets Low-Bit
Large Language Models", ai.info AI summary): "Methodology in Plain English",
paragraph 3 -- the runtime tracks a triple (the committed prefix, its
materialized causal KV length, the pending suffix) held consistent by a
length identity, and every captured graph views one physical KV buffer per
segment, the segment capacities growing geometrically; "Key Contributions",
item 1 -- the committed prefix and the materialized KV boundary stay aligned
so that graphs reuse the shared history instead of copying it.  The pages
write out neither the identity nor the layout; the readings taken here:

  state     : P committed tokens, L of them with causal KV rows stored
              (materialized), S = P - L pending; identity P == L + S over
              lengths L, S >= 0 (int32 words, so P stays below 2^31).
  segments  : segment s holds C0 * 2^s positions, following segments 0..s-1,
              so position p lives in the first segment whose cumulative
              capacity exceeds p.  Per segment, one buffer laid out
              [layer][K or V][position in segment][row].
  commit    : a pass computed causal KV rows for W positions starting at L
              (block [layer][K or V][W][row]).  Given n_mat (rows that become
              materialized, the leading ones) and n_new (tokens newly
              committed): L' = L + n_mat, P' = P + n_new, S' = P' - L'.  Valid
              iff the identity holds on entry, no error is set, 0 <= n_mat
              <= W, n_new >= 0, P' < 2^31, L' <= P' and L' fits the segments;
              otherwise nothing is written and the error code is set
              (1 identity, 2 counts, 3 capacity; an error already set is
              kept).
  roles     : a verification pass has n_mat = S + a (the pending tokens and
              the a accepted drafts) and n_new = a + 1 (with the verifier's
              own next token, which stays pending); an autoregressive step
              n_mat = n_new = 1; a confidence-only step commits drafts
              without KV, n_mat = 0.

Parity status: pinned (closed forms of the segment geometry, invariants and
a hand-worked sequence in tests/golden/kv_commit_hand.txt).
"""
from __future__ import annotations

import numpy as np

ERR_IDENTITY, ERR_COUNTS, ERR_CAPACITY = 1, 2, 3


def segment_capacities(c0: int, nseg: int):
    """Positions held by each segment: c0, 2 c0, 4 c0, ..."""
    caps = []
    c = c0
    for _ in range(nseg):
        caps.append(c)
        c *= 2
    return caps


def locate(p: int, c0: int, nseg: int):
    """(segment, offset in segment) of history position p, by walking the
    segments in order; None if p is past the last one."""
    start = 0
    for s, cap in enumerate(segment_capacities(c0, nseg)):
        if p < start + cap:
            return s, p - start
        start += cap
    return None


class KVStore:
    """The segments as numpy arrays [layers][2][cap][row] of uint16 (bf16
    bit patterns; the commit only moves them) plus the state."""

    def __init__(self, c0: int, nseg: int, layers: int, row: int, state=(1, 0, 1, 0)):
        self.c0, self.nseg, self.layers, self.row = c0, nseg, layers, row
        self.segs = [np.zeros((layers, 2, cap, row), np.uint16)
                     for cap in segment_capacities(c0, nseg)]
        self.state = list(state)  # P, L, S, error

    @property
    def capacity(self) -> int:
        return sum(segment_capacities(self.c0, self.nseg))

    def commit(self, block: np.ndarray, n_mat: int, n_new: int):
        """One commit (see the module docstring); block is [layers][2][W][row]."""
        P, L, S, err = self.state
        W = block.shape[2]
        if err:
            return
        if L < 0 or S < 0 or P != L + S:
            self.state[3] = ERR_IDENTITY
            return
        if not (0 <= n_mat <= W) or n_new < 0 or P + n_new > 2 ** 31 - 1 or L + n_mat > P + n_new:
            self.state[3] = ERR_COUNTS
            return
        if L + n_mat > self.capacity:
            self.state[3] = ERR_CAPACITY
            return
        for j in range(n_mat):
            s, o = locate(L + j, self.c0, self.nseg)
            for layer in range(self.layers):
                for kv in range(2):
                    self.segs[s][layer, kv, o, :] = block[layer, kv, j, :]
        P2, L2 = P + n_new, L + n_mat
        self.state = [P2, L2, P2 - L2, 0]

    def history(self):
        """The materialized rows in position order, [layers][2][L][row]."""
        L = self.state[1]
        out = np.zeros((self.layers, 2, L, self.row), np.uint16)
        for p in range(L):
            s, o = locate(p, self.c0, self.nseg)
            out[:, :, p, :] = self.segs[s][:, :, o, :]
        return out
