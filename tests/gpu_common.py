"""Shared helpers for the GPU parity tests (test infrastructure only)."""
from __future__ import annotations

import sys

import numpy as np

from context_long_attention_amd import inputs

O_ATOL = 2e-2        # max-abs on O, dQ, dK, dV (bf16 inputs)
LSE_RTOL = 1e-3      # |dLSE| <= 1e-3 * max(1, |LSE|)


def note(msg: str) -> None:
    """Print a progress line that names the case, flushed before the GPU work starts."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def device_bf16(x32: np.ndarray):
    """float32 array -> (bf16-rounded float64 copy for the oracle, device bf16 tensor)."""
    import torch
    bits = inputs.bf16_bits(x32)
    dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return inputs.bf16_to_f32(bits).astype(np.float64), dev


class RankInputs:
    """Seeded inputs of one rank: local Q/dO and the KV block of every source rank."""

    def __init__(self, w: inputs.Workload, rank: int, sources=None, want_do=False):
        import oracle
        self.w = w
        c = w.chunk
        R = w.cp
        self.qpos = oracle.zigzag_positions(w.seq_len, R, rank)
        qa, qb = oracle.zigzag_chunks(R, rank)
        self.q64, self.q = device_bf16(inputs.chunks_normal(inputs.SEED_Q, [qa, qb], c, w.hq, w.dim))
        if want_do:
            self.do64, self.do = device_bf16(inputs.chunks_normal(inputs.SEED_DO, [qa, qb], c, w.hq, w.dim))
        self.kv = {}
        self.kv64 = {}
        for s in (range(R) if sources is None else sources):
            ka, kb = oracle.zigzag_chunks(R, s)
            k64, k = device_bf16(inputs.chunks_normal(inputs.SEED_K, [ka, kb], c, w.hkv, w.dim))
            v64, v = device_bf16(inputs.chunks_normal(inputs.SEED_V, [ka, kb], c, w.hkv, w.dim))
            self.kv[s] = (k, v)
            self.kv64[s] = (k64, v64, oracle.zigzag_positions(w.seq_len, R, s))

    def kv_of_source(self, s):
        return self.kv[s]


def assert_o_close(got: np.ndarray, ref: np.ndarray, what: str, live=None):
    """Max-abs check; rows with no visible key (live False) are skipped for O."""
    g = np.asarray(got, dtype=np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    if live is not None:
        g = g[live]
        ref = ref[live]
    diff = np.abs(g - ref)
    err = float(diff.max()) if g.size else 0.0
    if err > O_ATOL:
        where = np.unravel_index(int(np.argmax(diff)), diff.shape)
        bad = int((diff > O_ATOL).sum())
        raise AssertionError(f"{what}: max abs err {err:.3e} > {O_ATOL} at {tuple(int(x) for x in where)} "
                             f"(got {g[where]:.4e}, want {ref[where]:.4e}; {bad} of {diff.size} elements off)")
    return err


def assert_lse_close(got: np.ndarray, ref: np.ndarray, what: str):
    g = np.asarray(got, dtype=np.float64)
    dead = np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), dead), f"{what}: -inf pattern differs"
    assert not np.isnan(g).any(), f"{what}: NaN"
    err = np.abs(g[~dead] - ref[~dead]) / np.maximum(1.0, np.abs(ref[~dead]))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= LSE_RTOL, f"{what}: LSE rel err {worst:.3e} > {LSE_RTOL}"
    return worst
