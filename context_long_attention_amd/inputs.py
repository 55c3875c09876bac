"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This module holds no attention arithmetic: it draws normal numbers, rounds them
to bfloat16 and samples packed-document lengths.  Both sides of every parity
check receive exactly these arrays.

Recipe (one rank's share is reproducible without materialising the sequence):

* Every tensor X in {Q, K, V, dO} is generated per global chunk.  Chunk k
  (``c`` tokens x H heads x D) is drawn from ``np.random.default_rng([seed_X, k])``
  as float32 N(0, 1), with seed_Q = 1, seed_K = 2, seed_V = 3, seed_dO = 4.
* bf16 inputs are the float32 draws rounded to bfloat16 with round-to-nearest-even;
  the oracle upcasts the rounded values.
* Packed documents (the pages' sequence packing without padding): lengths
  L = clip(round(exp(N(ln 16384, 1))), 256, 524288) are drawn from
  ``np.random.default_rng(seed)`` until they cover S tokens; the last document
  is cut to fit.
* Sliding-window layers (the pages' window layers of models such as Gemma) use
  the same draws; only the visibility changes (window of W tokens).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_Q, SEED_K, SEED_V, SEED_DO = 1, 2, 3, 4


def chunk_normal(seed: int, chunk: int, c: int, heads: int, dim: int) -> np.ndarray:
    """float32 N(0,1) values of global chunk ``chunk``: shape [c, heads, dim]."""
    rng = np.random.default_rng([seed, chunk])
    return rng.standard_normal((c, heads, dim), dtype=np.float32)


def chunks_normal(seed: int, chunks, c: int, heads: int, dim: int) -> np.ndarray:
    """Concatenation of several global chunks along the token axis."""
    return np.concatenate([chunk_normal(seed, k, c, heads, dim) for k in chunks], axis=0)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    # NaN stays NaN (never produced by normal draws, kept for completeness).
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 value (returned as float32)."""
    return bf16_to_f32(bf16_bits(x))


def doc_lengths(total: int, seed: int = 5, median: float = 16384.0, sigma: float = 1.0,
                lo: int = 256, hi: int = 524288) -> np.ndarray:
    """Lognormal document lengths covering exactly ``total`` tokens (int64)."""
    rng = np.random.default_rng(seed)
    lens = []
    acc = 0
    while acc < total:
        L = int(np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma))), lo, hi))
        L = min(L, total - acc)
        lens.append(L)
        acc += L
    return np.asarray(lens, dtype=np.int64)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    """Document start offsets [0, L0, L0+L1, ..., total] as int32."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    assert cu[-1] < 2**31
    return cu.astype(np.int32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named problem shape: one sequence of ``seq_len`` tokens over ``cp`` ranks."""

    name: str
    seq_len: int
    cp: int
    hq: int
    hkv: int
    dim: int
    backward: bool
    packed: bool = False
    input_dtype: str = "bf16"   # "fp32" draws are still cast to bf16 for the kernels
    window: int = 0             # sliding window in tokens (0: none)

    @property
    def chunk(self) -> int:
        return self.seq_len // (2 * self.cp)

    @property
    def local(self) -> int:
        return 2 * self.chunk

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dim)

    def cu_seqlens(self) -> np.ndarray | None:
        if not self.packed:
            return None
        return cu_seqlens_from_lengths(doc_lengths(self.seq_len))


K = 1024
M = 1024 * 1024

WORKLOADS = {
    "tiny": Workload("tiny", 512, 4, 4, 2, 64, backward=True, input_dtype="fp32"),
    "llama3_8b_fwd": Workload("llama3_8b_fwd", 128 * K, 8, 32, 8, 128, backward=False),
    "llama3_8b_fwdbwd": Workload("llama3_8b_fwdbwd", 256 * K, 16, 32, 8, 128, backward=True),
    "llama3_405b_fwd": Workload("llama3_405b_fwd", 1 * M, 16, 128, 8, 128, backward=False),
    "llama3_8b_packed": Workload("llama3_8b_packed", 2 * M, 64, 32, 8, 128, backward=True,
                                 packed=True),
    # window layers: a window inside one chunk (neighbour blocks only) and one spanning chunks
    "tiny_window": Workload("tiny_window", 512, 4, 4, 2, 64, backward=True, window=48),
    "tiny_window_wide": Workload("tiny_window_wide", 512, 4, 4, 2, 64, backward=True, window=150),
    "llama3_8b_window4k": Workload("llama3_8b_window4k", 128 * K, 8, 32, 8, 128, backward=True,
                                   window=4 * K),
}
