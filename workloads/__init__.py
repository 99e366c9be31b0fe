"""Seeded synthetic inputs for the W2A8 ternary linear.

This module only draws numbers.  It holds none of the method's arithmetic
(no ternarization, quantization, packing or contraction), so both the CPU
oracle and the HIP path can take their inputs from it.

The layer sets stand in for the ternary backbones the BitMTP page evaluates
(BitNet b1.58-2B and Bonsai 1.7B-4B, "Methodology in Plain English"), whose
weights are not available here.  Shapes follow the usual decoder layout of
those model sizes: a fused Q/K/V projection, the attention output projection,
a fused gate/up projection and the down projection.

Recipe (all draws are numpy ``default_rng`` standard normals in fp32):
  * ``single``: M=1, K=256, N=512, one rng seeded 0; W ~ N(0, 1) of shape
    [512, 256] is drawn first, then x ~ N(0, 1) of shape [1, 256].
  * 2B-class layer set: hidden 2560, projections (K -> N)
    qkv 2560 -> 3840 (segments 2560 | 640 | 640), o 2560 -> 2560,
    gateup 2560 -> 13824 (segments 6912 | 6912), down 6912 -> 2560; 30 layers.
  * 4B-class layer set: hidden 3072, qkv 3072 -> 5120 (3072 | 1024 | 1024),
    o 3072 -> 3072, gateup 3072 -> 16384 (8192 | 8192), down 8192 -> 3072;
    36 layers.
  * Layer-set weights: each segment draws its own N(0, 0.02^2) block from
    ``default_rng([set_seed, layer, proj, seg])`` (set_seed 2 or 4).
  * Layer-set activations: M independent N(0, 1) rows from
    ``default_rng([1002, workload, M, layer, proj])``.
  * Outlier mix: 1% of the K channels (round(0.01 K) indices from
    ``default_rng([3003, layer, proj]).choice(K, .., replace=False)``) are
    scaled by 20 in every row, so per-token absmax scales vary widely.
  * Activations are rounded from fp32 to bf16 with round-to-nearest-even and
    handed over as uint16 bit patterns.
  * Output (vocabulary) projection of the 2B-class set, for the fast and
    critical projection roles: hidden 2560 -> 128256 rows (the size of the
    2B backbone's vocabulary; the pages do not state it).  Rows come in
    blocks of 4096, block b drawn N(0, 0.02^2) from ``default_rng([6, b])``,
    so any row can be regenerated on its own; activations for width M are
    N(0, 1) rows from ``default_rng([1006, M])``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

PROJ_NAMES = ("qkv", "o", "gateup", "down")


@dataclass(frozen=True)
class Proj:
    name: str
    K: int
    segs: tuple  # output rows of each independently scaled segment

    @property
    def N(self) -> int:
        return int(sum(self.segs))

    @property
    def packed_bytes(self) -> int:
        return self.N * self.K // 4


@dataclass(frozen=True)
class LayerSet:
    name: str
    set_seed: int
    hidden: int
    layers: int
    projs: tuple

    @property
    def packed_bytes_per_layer(self) -> int:
        return sum(p.packed_bytes for p in self.projs)

    @property
    def packed_bytes(self) -> int:
        return self.layers * self.packed_bytes_per_layer


def _layer_set(name, set_seed, hidden, kv, inter, layers):
    projs = (
        Proj("qkv", hidden, (hidden, kv, kv)),
        Proj("o", hidden, (hidden,)),
        Proj("gateup", hidden, (inter, inter)),
        Proj("down", inter, (hidden,)),
    )
    return LayerSet(name, set_seed, hidden, layers, projs)


SET_2B = _layer_set("2b", 2, 2560, 640, 6912, 30)
SET_4B = _layer_set("4b", 4, 3072, 1024, 8192, 36)
LAYER_SETS = {"2b": SET_2B, "4b": SET_4B}

# Workload ids used in the activation seeds.
WORKLOADS = {
    "single": 0,        # M=1, K=256, N=512
    "2b_decode": 1,     # 2B set, M=1
    "2b_verify": 2,     # 2B set, M in {2, 4, 8}
    "2b_sweep_outlier": 3,  # 2B set, M = 1..16, 1% outlier channels x20
    "4b_stack": 4,      # 4B set, M in {1, 4, 16}
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def single_case(seed: int = 0, M: int = 1, K: int = 256, N: int = 512):
    """The single-linear case: W ~ N(0,1) [N, K] then x ~ N(0,1) [M, K]."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32)
    x = rng.standard_normal((M, K), dtype=np.float32)
    return W, (N,), f32_to_bf16_bits(x)


def layer_weights(ls: LayerSet, layer: int, proj_index: int, sigma: float = 0.02):
    """fp32 weights [N, K] of one projection, segments stacked along N."""
    p = ls.projs[proj_index]
    blocks = []
    for s, rows in enumerate(p.segs):
        rng = np.random.default_rng([ls.set_seed, layer, proj_index, s])
        w = rng.standard_normal((rows, p.K), dtype=np.float32)
        w *= np.float32(sigma)
        blocks.append(w)
    return np.concatenate(blocks, axis=0) if len(blocks) > 1 else blocks[0]


def outlier_channels(K: int, layer: int, proj_index: int) -> np.ndarray:
    rng = np.random.default_rng([3003, layer, proj_index])
    return np.sort(rng.choice(K, int(round(0.01 * K)), replace=False))


def layer_activations(workload: str, K: int, M: int, layer: int, proj_index: int,
                      outliers: bool = False) -> np.ndarray:
    """bf16 bits [M, K] of N(0,1) rows, optionally with the outlier mix."""
    wid = WORKLOADS[workload]
    rng = np.random.default_rng([1002, wid, M, layer, proj_index])
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        idx = outlier_channels(K, layer, proj_index)
        x[:, idx] *= np.float32(20.0)
    return f32_to_bf16_bits(x)


def random_case(seed: int, M: int, K: int, seg_rows, w_sigma: float = 1.0,
                x_sigma: float = 1.0):
    """A generic seeded case of any shape (parity tests over tile edges and
    ragged tails).  W depends on (seed, K, segments) only, x on (seed, M, K)."""
    N = int(sum(seg_rows))
    rng = np.random.default_rng([77, seed, K, N, len(seg_rows)])
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_sigma)
    rng = np.random.default_rng([78, seed, M, K])
    x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(x_sigma)
    return W, tuple(seg_rows), f32_to_bf16_bits(x)


HEAD_K = 2560
HEAD_N = 128256
HEAD_BLOCK = 4096


def head_weight_block(b: int, K: int = HEAD_K, N: int = HEAD_N, sigma: float = 0.02):
    """fp32 rows [4096 b, min(4096 (b + 1), N)) of the output projection."""
    rows = min(HEAD_BLOCK, N - HEAD_BLOCK * b)
    rng = np.random.default_rng([6, b])
    w = rng.standard_normal((rows, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def head_weights(K: int = HEAD_K, N: int = HEAD_N):
    """The whole output projection, fp32 [N, K]."""
    nb = -(-N // HEAD_BLOCK)
    return np.concatenate([head_weight_block(b, K, N) for b in range(nb)], axis=0)


def head_activations(M: int, K: int = HEAD_K):
    """bf16 bits [M, K] of N(0, 1) rows for the output projection."""
    rng = np.random.default_rng([1006, M])
    return f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


def workload_widths(workload: str):
    return {
        "single": (1,),
        "2b_decode": (1,),
        "2b_verify": (2, 4, 8),
        "2b_sweep_outlier": tuple(range(1, 17)),
        "4b_stack": (1, 4, 16),
    }[workload]
