"""Seeded synthetic inputs for the sharded linear workloads.

This module is shared by the test suite, the oracle side and the GPU side. It
only draws random numbers and converts between float32 and bfloat16 bit
patterns; it holds none of the arithmetic of the sharded multiply itself.

Recipe (every workload):
  * generator: ``numpy.random.default_rng([workload_id, tensor_id])`` with
    tensor ids 0 = X, 1 = W / W1 / Wqkv, 2 = W2 / Wo, 3 = A (the stand-in
    input of the attention output projection);
  * floating inputs: ``standard_normal(float32) * sigma`` (sigma is the
    standard deviation: 1 for activations, 0.02 for weights), then rounded
    to bfloat16 by round-to-nearest-even; both sides receive these exact bits;
  * integer inputs: ``integers(lo, hi + 1)`` stored as float32;
  * sequence-parallel inputs (tensor ids 4 = residual, 5 = dropout keep
    mask, 6 = LayerNorm gamma, 7 = beta): the residual as a floating input;
    the keep mask as ``random() >= p_drop`` stored as 0/1 bytes (the random
    numbers dropout draws are an input, passed to both sides); gamma and
    beta as ``mean + sigma * standard_normal(float32)`` in float32;
  * tensor id 8: the column-parallel outputs of all shards in their own
    buffers (shard-major), the input of the explicit all-gather.
Values are dense and unstructured (no sparsity), as in the dense layers the
tensor-parallelism pages describe.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "rng",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "normal_bf16",
    "int_uniform_f32",
    "normal_f32",
    "keep_mask",
    "Workload",
    "WORKLOADS",
    "sample_rows",
    "stratified_rows",
]


def rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    """The seeded generator for one tensor of one workload."""
    return np.random.default_rng([int(workload_id), int(tensor_id)])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    quiet = (u >> 16) | 0x40
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, sigma: float, workload_id: int, tensor_id: int):
    """N(0, sigma^2) draws rounded to bfloat16: returns (uint16 bits, float32 values)."""
    g = rng(workload_id, tensor_id)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    bits = bf16_bits_from_f32(x)
    return bits, f32_from_bf16_bits(bits)


def int_uniform_f32(shape, lo: int, hi: int, workload_id: int, tensor_id: int) -> np.ndarray:
    """Integers drawn uniformly from lo..hi inclusive, stored as float32."""
    g = rng(workload_id, tensor_id)
    return g.integers(lo, hi + 1, size=shape).astype(np.float32)


def normal_f32(shape, mean: float, sigma: float, workload_id: int, tensor_id: int) -> np.ndarray:
    """float32 draws mean + sigma * N(0, 1) (not rounded to bfloat16)."""
    g = rng(workload_id, tensor_id)
    return (np.float32(mean) + np.float32(sigma) * g.standard_normal(size=shape, dtype=np.float32)).astype(np.float32)


def keep_mask(shape, p_drop: float, workload_id: int, tensor_id: int) -> np.ndarray:
    """A dropout keep mask: uint8 1 where a uniform draw in [0, 1) is >= p_drop, else 0."""
    g = rng(workload_id, tensor_id)
    return (g.random(size=shape) >= p_drop).astype(np.uint8)


def sample_rows(m: int, count: int = 256, seed: int = 0) -> np.ndarray:
    """A seeded, sorted set of distinct row indices that always holds 0 and m - 1."""
    if m <= count:
        return np.arange(m)
    g = np.random.default_rng([0x5EED, int(seed), int(m)])
    inner = g.choice(np.arange(1, m - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, m - 1], inner]))


def stratified_rows(m: int, seed: int = 0, block: int = 32, tile: int = 256) -> np.ndarray:
    """A seeded, sorted set of distinct row indices that covers every block of rows.

    It holds the first and the last row of every `tile`-row tile (the last tile
    may be ragged) and one seeded row inside every `block`-row block, so that
    every tile of an output and every `block`-row band inside each tile has
    rows under check. For m = 16384 that is 512 + 128 rows.
    """
    if m <= 0:
        return np.arange(0)
    g = np.random.default_rng([0x57A7, int(seed), int(m), int(block), int(tile)])
    picks = []
    for t0 in range(0, m, tile):
        picks += [t0, min(t0 + tile, m) - 1]
    for b0 in range(0, m, block):
        picks.append(int(g.integers(b0, min(b0 + block, m))))
    return np.unique(np.asarray(picks, dtype=np.int64))


@dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload (all sizes in elements)."""

    wid: int
    name: str
    M: int            # tokens (rows of X)
    d: int            # model width (columns of X, rows of W1 / Wqkv)
    F: int            # full intermediate width split over N shards (MLP) or full QKV width
    N: int            # number of logical shards
    ns: int           # shards executed in one call
    d_out: int = 0    # output width of the row-parallel layer (defaults to d)
    kind: str = "mlp"  # "mlp", "attn_proj", "split_check"

    @property
    def out(self) -> int:
        return self.d_out or self.d


# Workload table: the tiny exact split check, the Megatron MLP block with all
# 8 shards local, the head-parallel attention projections, one GPU's share of a
# GPT-3-width MLP, and the decode-shaped skinny MLP.
WORKLOADS = {
    "split_check": Workload(1, "split_check", M=4, d=64, F=128, N=2, ns=2, kind="split_check"),
    "megatron_mlp": Workload(2, "megatron_mlp", M=2048, d=4096, F=16384, N=8, ns=8),
    "attn_proj": Workload(3, "attn_proj", M=4096, d=8192, F=24576, N=8, ns=8, d_out=8192,
                          kind="attn_proj"),
    "gpt3_mlp_shard": Workload(4, "gpt3_mlp_shard", M=16384, d=12288, F=49152, N=8, ns=1),
    "decode_mlp": Workload(5, "decode_mlp", M=16, d=8192, F=28672, N=8, ns=8),
}
