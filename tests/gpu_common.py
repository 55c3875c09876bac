"""Shared helpers for the GPU parity tests (test infrastructure only)."""
from __future__ import annotations


import numpy as np

from context_long_attention_amd import inputs

O_ATOL = 2e-2        # max-abs on O, dQ, dK, dV (bf16 inputs)
LSE_RTOL = 1e-3      # |dLSE| <= 1e-3 * max(1, |LSE|)


def note(msg: str) -> None:
    """Print a progress line that names the case, flushed before the GPU work starts
    (to the real output, past pytest's capture)."""
    from tests import live
    live.line(f"[gpu-case] {msg}")


def _to_device(bits: np.ndarray):
    import torch
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def device_bf16(x32: np.ndarray):
    """float32 array -> (bf16-rounded float64 copy for the oracle, device bf16 tensor)."""
    bits = inputs.bf16_bits(x32)
    return inputs.bf16_to_f32(bits).astype(np.float64), _to_device(bits)


def widen(bits: np.ndarray) -> np.ndarray:
    return inputs.bf16_to_f32(bits).astype(np.float64)


class RankInputs:
    """Seeded inputs of one rank: local Q/dO and the KV block of every source rank.

    Host copies are kept as bf16 bit patterns and widened to float64 only when
    the oracle asks for them (``q64``, ``kv64[s]``, ``blocks``), so the largest
    workloads fit in host memory.  Sources not listed in ``sources`` get a
    shared all-zero block on the device (use it only for steps with nothing
    visible).
    """

    def __init__(self, w: inputs.Workload, rank: int, sources=None, want_do=False):
        import oracle
        self.w = w
        c = w.chunk
        R = w.cp
        self.qpos = oracle.zigzag_positions(w.seq_len, R, rank)
        qa, qb = oracle.zigzag_chunks(R, rank)
        self.q_bits = inputs.bf16_bits(inputs.chunks_normal(inputs.SEED_Q, [qa, qb], c, w.hq, w.dim))
        self.q = _to_device(self.q_bits)
        if want_do:
            self.do_bits = inputs.bf16_bits(inputs.chunks_normal(inputs.SEED_DO, [qa, qb], c, w.hq, w.dim))
            self.do = _to_device(self.do_bits)
        self.kv = {}
        self.kv_bits = {}
        self.kpos = {}
        self._zero = None
        for s in (range(R) if sources is None else sources):
            ka, kb = oracle.zigzag_chunks(R, s)
            kbits = inputs.bf16_bits(inputs.chunks_normal(inputs.SEED_K, [ka, kb], c, w.hkv, w.dim))
            vbits = inputs.bf16_bits(inputs.chunks_normal(inputs.SEED_V, [ka, kb], c, w.hkv, w.dim))
            self.kv_bits[s] = (kbits, vbits)
            self.kv[s] = (_to_device(kbits), _to_device(vbits))
            self.kpos[s] = oracle.zigzag_positions(w.seq_len, R, s)

    @property
    def q64(self):
        return widen(self.q_bits)

    @property
    def do64(self):
        return widen(self.do_bits)

    @property
    def kv64(self):
        return _Widened(self)

    def blocks(self, schedule):
        """Oracle KV blocks in ring order, widened one at a time (a generator)."""
        for s in schedule:
            if s in self.kv_bits:
                k, v = self.kv_bits[s]
                yield widen(k), widen(v), self.kpos[s]

    def kv_of_source(self, s):
        if s in self.kv:
            return self.kv[s]
        if self._zero is None:
            import torch
            shape = (self.w.local, self.w.hkv, self.w.dim)
            z = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
            self._zero = (z, z)
        return self._zero


class _Widened:
    def __init__(self, inp):
        self.inp = inp

    def __getitem__(self, s):
        k, v = self.inp.kv_bits[s]
        return widen(k), widen(v), self.inp.kpos[s]


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


def sampled_rows(local: int, c: int, n_extra: int, seed: int) -> np.ndarray:
    """Edge rows of both chunks plus uniform random rows."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, 2, c - 1, c, c + 1, local - 2, local - 1]
    return np.unique(np.concatenate([edge, rng.integers(0, local, n_extra)]))


class GroupReference:
    """Whole-tensor float64 oracle results of one rank for the query heads
    ``heads`` (whole GQA groups), started in the background at construction so
    that the GPU ring can run meanwhile.  The backward, when asked for, starts
    from the oracle's own final O and LSE of every local row (never from GPU
    output).  Use as a context manager: the shared input files are removed on
    exit."""

    def __init__(self, inp: RankInputs, order, heads, cu=None, window=0, backward=False):
        from tests import oracle_par
        self._par = oracle_par
        self.order = [int(s) for s in order]
        self.heads = [int(h) for h in heads]
        kv = {s: inp.kv_bits[s] for s in self.order}
        kpos = {s: inp.kpos[s] for s in self.order}
        self.sh = oracle_par.Shared(inp.q_bits, inp.qpos, kv, kpos, inp.w.scale, cu, window,
                                    do_bits=inp.do_bits if backward else None)
        self._fwd = oracle_par.Forward(self.sh, self.heads, self.order)
        self._fwd_res = None
        self._bwd_res = None

    def forward(self):
        """(O [rows, len(heads), D], LSE [len(heads), rows]) in float64."""
        if self._fwd_res is None:
            o, lse, _ = self._fwd.result()
            self._fwd_res = (o, lse)
        return self._fwd_res

    def backward(self):
        """(dQ [rows, len(heads), D], per-step list of {kv head: (dK [m, D], dV [m, D])})."""
        if self._bwd_res is None:
            o, lse = self.forward()
            dq, per_step, _ = self._par.Backward(self.sh, self.heads, self.order, o, lse).result()
            self._bwd_res = (dq, per_step)
        return self._bwd_res

    def close(self):
        self.sh.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def gqa_heads(kv_head: int, hq: int, hkv: int) -> list[int]:
    """The query heads that read KV head ``kv_head``."""
    g = hq // hkv
    return list(range(kv_head * g, (kv_head + 1) * g))
