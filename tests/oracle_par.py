"""Whole-tensor float64 references at full workload sizes (test infrastructure only).

The oracle's step functions treat each query head on its own, and in the
forward each query row on its own.  A whole-tensor reference for one rank's
share of a full-size workload is therefore evaluated here one task per (query
head, ring step, block of local rows), in a pool of worker processes, and the
parent composes the task results the way ``oracle.rank_forward`` and
``oracle.rank_backward`` compose the oracle's step functions:

* forward: the step partials of a head (rows concatenated) are merged in ring
  order with ``oracle.merge``;
* backward: from the final LSE and Delta of every row, dQ is summed over the
  steps in ring order, and each step's dK/dV over the row blocks and the query
  heads of its KV head.

Inside a task the step's keys are taken in blocks of ``_KEY_BLOCK``, so that the
oracle's arrays stay small: the forward folds the partials of the key blocks
with ``oracle.merge`` (a merge over disjoint key sets, as the ring itself does),
and the backward adds the key blocks' dQ terms and places their dK/dV.  A key
block that none of the task's rows can see carries weight exactly zero and is
not evaluated: it leaves O, LSE and dQ unchanged and its dK/dV zero.
``tests/test_oracle_parallel.py`` pins the whole composition against
``oracle.rank_forward`` / ``oracle.rank_backward``.

Inputs travel as bf16 bit patterns in ``.npy`` files (under /dev/shm when it
exists) that the workers memory-map; nothing here touches the GPU, and the
workers import only NumPy, the oracle and the seeded input module.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile
import time
import uuid

import numpy as np

import oracle
from tests import live
from context_long_attention_amd import inputs

_POOL = None
_MAX_WORKERS = 16  # host CPU cores set aside beside one GPU
_KEY_BLOCK = 2048  # keys per oracle call inside a task


def n_workers() -> int:
    return max(1, min(_MAX_WORKERS, len(os.sched_getaffinity(0))))


def _init_worker():
    # one BLAS thread per worker: the pool itself is the parallelism
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # threadpoolctl missing: BLAS keeps its own setting
        pass


def pool(workers: int | None = None) -> cf.ProcessPoolExecutor:
    """The process pool (created once, spawned: the workers start as fresh
    interpreters and never inherit the parent's GPU state)."""
    global _POOL
    if _POOL is None:
        _POOL = cf.ProcessPoolExecutor(max_workers=workers or n_workers(), mp_context=mp.get_context("spawn"),
                                       initializer=_init_worker)
    return _POOL


def _progress(what, done, total, t0):
    live.line(f"[oracle] {what}: {done}/{total} heads, {time.time() - t0:.0f} s")


def shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True, cancel_futures=True)
        _POOL = None


# ----------------------------------------------------------------------------- shared inputs
class Shared:
    """One rank's inputs written once for the workers: local Q (and dO) and the
    KV block of each listed source, as bf16 bit patterns, with their global
    positions, the documents and the window."""

    def __init__(self, q_bits, qpos, kv_bits: dict, kpos: dict, scale: float, cu_seqlens=None, window=0,
                 do_bits=None):
        base = "/dev/shm" if os.path.isdir("/dev/shm") else None
        self.dir = tempfile.mkdtemp(prefix="cpattn_ref_", dir=base)
        self.key = uuid.uuid4().hex
        self.n, self.hq, self.dim = q_bits.shape
        first = next(iter(kv_bits.values()))[0]
        self.hkv = first.shape[1]
        self.group = self.hq // self.hkv
        self.scale = float(scale)
        self.window = int(window or 0)
        self.cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
        self.qpos = np.asarray(qpos, dtype=np.int64)
        self.kpos = {int(s): np.asarray(p, dtype=np.int64) for s, p in kpos.items()}
        self.sources = sorted(int(s) for s in kv_bits)
        np.save(self._path("q"), np.ascontiguousarray(q_bits, dtype=np.uint16))
        if do_bits is not None:
            np.save(self._path("do"), np.ascontiguousarray(do_bits, dtype=np.uint16))
        for s, (kb, vb) in kv_bits.items():
            np.save(self._path(f"k{int(s)}"), np.ascontiguousarray(kb, dtype=np.uint16))
            np.save(self._path(f"v{int(s)}"), np.ascontiguousarray(vb, dtype=np.uint16))
            np.save(self._path(f"p{int(s)}"), self.kpos[int(s)])

    def _path(self, name):
        return os.path.join(self.dir, name + ".npy")

    def spec(self):
        return dict(dir=self.dir, key=self.key, group=self.group, scale=self.scale, window=self.window,
                    cu=self.cu, qpos=self.qpos, key_block=_KEY_BLOCK)

    def close(self):
        shutil.rmtree(self.dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


# ----------------------------------------------------------------------------- worker side
_WCACHE = {"key": None, "arrays": {}}


def _bits(spec, name):
    """Memory-mapped bf16 bits of one input (a worker keeps one input set at a time)."""
    if _WCACHE["key"] != spec["key"]:
        _WCACHE["key"] = spec["key"]
        _WCACHE["arrays"] = {}
    arrs = _WCACHE["arrays"]
    if name not in arrs:
        arrs[name] = np.load(os.path.join(spec["dir"], name + ".npy"), mmap_mode="r")
    return arrs[name]


def _f64(bits) -> np.ndarray:
    return inputs.bf16_to_f32(np.asarray(bits)).astype(np.float64)


def _key_blocks(spec, h, src, r0, r1):
    """(q, visibility, key block [c0, c1)) of a task, for every key block that one
    of its rows can see; q is float64 [r1 - r0, 1, D]."""
    kpos = np.asarray(_bits(spec, f"p{src}"))
    q = _f64(_bits(spec, "q")[r0:r1, h:h + 1, :])
    vis = oracle.visibility(spec["qpos"][r0:r1], kpos, spec["cu"], spec["window"] or None)
    out = []
    kb = spec["key_block"]
    for c0 in range(0, len(kpos), kb):
        c1 = min(len(kpos), c0 + kb)
        if vis[:, c0:c1].any():
            out.append((c0, c1))
    return q, vis, out


def _kv(spec, name, g, c0, c1):
    return _f64(_bits(spec, name)[c0:c1, g:g + 1, :])


def _fwd_task(spec, h, src, r0, r1):
    g = h // spec["group"]
    q, vis, blocks = _key_blocks(spec, h, src, r0, r1)
    o = np.zeros((r1 - r0, 1, q.shape[2]))
    lse = np.full((1, r1 - r0), -np.inf)
    for c0, c1 in blocks:
        o_b, lse_b = oracle.attention_partial(q, _kv(spec, f"k{src}", g, c0, c1), _kv(spec, f"v{src}", g, c0, c1),
                                              vis[:, c0:c1], spec["scale"])
        o, lse = oracle.merge(o, lse, o_b, lse_b)
    return o[:, 0, :], lse[0]


def _bwd_task(spec, h, src, r0, r1, lse_rows, delta_rows):
    g = h // spec["group"]
    q, vis, blocks = _key_blocks(spec, h, src, r0, r1)
    do = _f64(_bits(spec, "do")[r0:r1, h:h + 1, :])
    dq = np.zeros((r1 - r0, q.shape[2]))
    parts = []
    for c0, c1 in blocks:
        dq_b, dk_b, dv_b = oracle.attention_backward_partial(
            q, _kv(spec, f"k{src}", g, c0, c1), _kv(spec, f"v{src}", g, c0, c1), do, lse_rows[None, :],
            delta_rows[None, :], vis[:, c0:c1], spec["scale"])
        dq += dq_b[:, 0, :]
        parts.append((c0, c1, dk_b[:, 0, :], dv_b[:, 0, :]))
    return dq, parts


# ----------------------------------------------------------------------------- parent side
def _row_blocks(n, rows_per_task):
    return [(r0, min(n, r0 + rows_per_task)) for r0 in range(0, n, rows_per_task)]


class Forward:
    """Oracle forward of one rank over the query heads ``heads`` and the sources
    ``order`` (ring order), submitted at construction; ``result()`` composes it.
    ``keep_steps`` also returns each step's partial (O_t, LSE_t)."""

    def __init__(self, sh: Shared, heads, order, rows_per_task=2048, keep_steps=False, workers=None):
        self.sh = sh
        self.heads = [int(h) for h in heads]
        self.order = [int(s) for s in order]
        self.keep_steps = keep_steps
        ex = pool(workers)
        spec = sh.spec()
        self.blocks = _row_blocks(sh.n, rows_per_task)
        self.futs = {(h, t, b): ex.submit(_fwd_task, spec, h, s, r0, r1)
                     for h in self.heads for t, s in enumerate(self.order)
                     for b, (r0, r1) in enumerate(self.blocks)}

    def result(self):
        """(O [n, len(heads), D], LSE [len(heads), n], steps) in float64; steps is a
        list over ring steps of (O_t, LSE_t) in the same layout, when kept."""
        sh = self.sh
        H = len(self.heads)
        o = np.zeros((sh.n, H, sh.dim))
        lse = np.full((H, sh.n), -np.inf)
        steps = [(np.zeros((sh.n, H, sh.dim)), np.full((H, sh.n), -np.inf)) for _ in self.order] \
            if self.keep_steps else None
        t0 = time.time()
        for j, h in enumerate(self.heads):
            acc_o = np.zeros((sh.n, 1, sh.dim))
            acc_l = np.full((1, sh.n), -np.inf)
            for t in range(len(self.order)):
                o_t = np.zeros((sh.n, 1, sh.dim))
                l_t = np.full((1, sh.n), -np.inf)
                for b, (r0, r1) in enumerate(self.blocks):
                    ob, lb = self.futs.pop((h, t, b)).result()
                    o_t[r0:r1, 0] = ob
                    l_t[0, r0:r1] = lb
                if steps is not None:
                    steps[t][0][:, j] = o_t[:, 0]
                    steps[t][1][j] = l_t[0]
                acc_o, acc_l = oracle.merge(acc_o, acc_l, o_t, l_t)
            o[:, j] = acc_o[:, 0]
            lse[j] = acc_l[0]
            _progress("forward", j + 1, H, t0)
        return o, lse, steps


class Backward:
    """Oracle backward of one rank from the final O and LSE of the query heads
    ``heads`` (float64 [n, len(heads), D] and [len(heads), n]), over the sources
    ``order``; Delta comes from that O.  ``heads`` must cover whole GQA groups for
    the dK/dV of their KV heads to be complete."""

    def __init__(self, sh: Shared, heads, order, o, lse, rows_per_task=2048, workers=None):
        self.sh = sh
        self.heads = [int(h) for h in heads]
        self.order = [int(s) for s in order]
        do = _f64(np.load(sh._path("do"), mmap_mode="r")[:, self.heads, :])
        self.delta = oracle.delta_rows(do, o)
        del do
        ex = pool(workers)
        spec = sh.spec()
        self.blocks = _row_blocks(sh.n, rows_per_task)
        self.futs = {(j, t, b): ex.submit(_bwd_task, spec, h, s, r0, r1, lse[j, r0:r1],
                                          self.delta[j, r0:r1])
                     for j, h in enumerate(self.heads) for t, s in enumerate(self.order)
                     for b, (r0, r1) in enumerate(self.blocks)}

    def result(self):
        """(dQ [n, len(heads), D], per-step list of {kv head: (dK [m, D], dV [m, D])}, Delta)."""
        sh = self.sh
        H = len(self.heads)
        dq = np.zeros((sh.n, H, sh.dim))
        kv_heads = sorted({h // sh.group for h in self.heads})
        per_step = []
        t0 = time.time()
        for t, s in enumerate(self.order):
            m = len(sh.kpos[s])
            dkv = {g: (np.zeros((m, sh.dim)), np.zeros((m, sh.dim))) for g in kv_heads}
            for j, h in enumerate(self.heads):
                dk, dv = dkv[h // sh.group]
                for b, (r0, r1) in enumerate(self.blocks):
                    dqb, parts = self.futs.pop((j, t, b)).result()
                    dq[r0:r1, j] += dqb
                    for c0, c1, dkb, dvb in parts:
                        dk[c0:c1] += dkb
                        dv[c0:c1] += dvb
            per_step.append(dkv)
            live.line(f"[oracle] backward: step {t + 1}/{len(self.order)}, {time.time() - t0:.0f} s")
        return dq, per_step, self.delta
